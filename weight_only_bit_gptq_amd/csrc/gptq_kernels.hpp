// Kernel argument blocks and launch entry points (internal to libgptq.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gptq_device.hpp"

namespace gptq {

struct DequantArgs {
  const int32_t* qweight;
  const int32_t* qzeros;
  const _Float16* scales;
  const int32_t* g_idx;     // nullable
  _Float16* out;            // [K, N]
  int N, K, G, group_size, zero_offset;
  int chunks;               // K / 32
  int64_t zrow_words;       // N * bits / 32
};

struct GemmArgs {
  const _Float16* x;        // [M, K]
  const int32_t* qweight;
  const int32_t* qzeros;
  const _Float16* scales;
  const int32_t* g_idx;     // nullable
  _Float16* out;            // [M, N]
  int M, N, K, G, group_size, zero_offset;
  int chunks;               // K / 32
  int64_t zrow_words;       // N * bits / 32
  // decode launch shape: tiles of 16*cpl columns, nw waves per workgroup,
  // K in phases of pc = nw * cpw chunks, cpw chunks per wave per phase,
  // cpg = group_size / 32 chunks per group on the fast path (else 1)
  int tiles, cpl, nw, cpw, pc, phases, cpg;
  // fast path: scale and zero folded once per `fold` consecutive chunks (1, 2
  // or 4; a divisor of cpg, of cpw / 2 and, with ks > 1, of cks)
  int fold;
  // split K: ks workgroups per output tile, each over cks consecutive chunks
  // (the last one over the rest); with ks > 1 every workgroup stores its fp32
  // partial sums to ws [ks, M, N], added in split order by the last decode
  // workgroup of a tile to arrive (counted in cnt[tile], reset to 0 by that
  // workgroup) or, after a prefill launch, by a second kernel
  int ks, cks;
  float* ws;
  uint32_t* cnt;
  // qweight layout: 0 = checkpoint [K*b/32, N]; 1 = tiled [N/16][K/32][b][16]
  // (16-column tiles, each chunk's b packed rows contiguous)
  int wtiled;
  // grouped (mixture-of-experts) GEMM, when n_experts > 0: expert e owns
  // rows [moe_off[e], moe_off[e + 1]) of x and out (tokens sorted by expert,
  // clamped to [0, M]) and the weights at qweight + e * qw_stride (qzeros,
  // scales, g_idx likewise).  Decode: the grid is n_experts x moe_blocks x
  // tiles, each workgroup one block of up to 16 of its expert's rows.
  // Prefill: n_experts x tiles_m x tiles_n, row tiles over the expert's rows.
  // Either way only an expert's first moe_rows rows are computed.
  const int32_t* moe_off;
  int n_experts, moe_blocks, moe_rows;
  int64_t qw_stride, qz_stride, sc_stride, gi_stride;
  // decode over row blocks (M > 16 on a per-element layer): row_blocks x
  // tiles workgroups, workgroup (b, t) computes rows [16 b, 16 b + 16) of
  // column tile t (no K split); 0 or 1 otherwise
  int row_blocks;
  // prefill launch shape: tiles_m x tiles_n workgroup tiles of pbm (32, 64,
  // 128 or 256) rows by 256 columns
  int tiles_m, tiles_n, pbm;
  // activation type: 0 = fp16 (x, scales, out fp16), 1 = bfloat16 (x,
  // scales and out hold bfloat16 bits behind the same pointers)
  int bf16;
};

// LDS carve-up of the decode kernel: one phase buffer (two when K takes
// several phases) holding x fragments and either per-chunk correction sums and
// the phase's scale/zero rows (fast path) or the phase's g_idx slice, then the
// whole scale/zero table (per-element path); the cross-wave reduction buffer
// aliases everything after the main loop.
struct DecodeLayout {
  size_t buf_stride;        // bytes of one phase buffer
  size_t corr_off;          // correction sums inside a buffer (fast path)
  size_t gidx_off;          // per-row table byte offsets of a buffer's chunks (per-element path)
  size_t ptab_off;          // the phase's scale/zero rows inside a buffer (fast path)
  int ptab_rows;            // groups a phase covers (fast path)
  size_t tab_off;           // whole scale/zero table (per-element path)
  bool fits_staging;        // the table quads fit the staging registers
  size_t total;
};

// Group of row k: g_idx[k] (clamped into [0, G) so a bad entry cannot read out
// of bounds) or k / group_size.
__device__ __forceinline__ int group_of(const int32_t* __restrict__ g_idx, int k, int group_size, int G) {
  if (g_idx) {
    const int g = g_idx[k];
    return g < 0 ? 0 : (g >= G ? G - 1 : g);
  }
  return k / group_size;
}

hipError_t launch_dequant(int bits, const DequantArgs& a, bool bf16, hipStream_t stream);

// Decode (M <= 16).  `per_elem` selects the per-element scale/zero path (act
// order or group_size % 32 != 0).
// LDS bytes of a launch shape (SIZE_MAX if its table cannot be staged)
size_t decode_lds_bytes(int M, int pc, int nw, int cpl, bool per_elem, int G, int cpg, int phases,
                        bool bf16 = false);
int decode_max_x_pieces(int M);   // 16-byte x pieces each thread may stage per phase
// per instantiation: workgroup size limit, waves per SIMD it is compiled for,
// and whether that chunks-per-wave value is compiled at all
int decode_max_threads_for(int bits, bool per_elem, int cpl, int cpw, int M);
int decode_waves_per_simd_for(int bits, bool per_elem, int cpl, int cpw, int M);
bool decode_cpw_allowed(int bits, bool per_elem, int cpl, int cpw, int M, bool bf16 = false);
hipError_t launch_decode(int bits, bool per_elem, const GemmArgs& a, hipStream_t stream);

// Prefill (any M, used for M > 16).
// big_ok: the 256-row tile may be used (fast path, fp16)
void prefill_shape(int M, int N, bool big_ok, int* tiles_m, int* tiles_n, int* bm);
hipError_t launch_prefill(int bits, bool per_elem, const GemmArgs& a, hipStream_t stream);

// Min/max quantize + pack (fp32 W -> qweight, qzeros, scales).
hipError_t launch_quantize(const float* w, const int32_t* g_idx, int bits, int group_size, int sym, int is_v2,
                           int N, int K, int32_t* qweight, int32_t* qzeros, void* scales, hipStream_t stream);

// qweight checkpoint layout <-> tiled layout (to_tiled = 1: forward).
hipError_t launch_repack(const int32_t* in, int32_t* out, int bits, int64_t N, int64_t K, int to_tiled,
                         hipStream_t stream);

// Act-order rows sorted by group (qweight rows permuted bit-exactly) and x
// gathered into the sorted row order.
hipError_t launch_sort_rows(const int32_t* in, const int32_t* perm, int32_t* out, int bits, int64_t N, int64_t K,
                            hipStream_t stream);
hipError_t launch_gather_cols(const void* x, const int32_t* perm, void* xg, int64_t M, int64_t K, hipStream_t stream);

// Zero `words` int32 words with a kernel (capture-safe, unlike a memset node).
hipError_t launch_zero_words(void* p, int64_t words, hipStream_t stream);

// Memory-read reference: reads `bytes` (a multiple of 16) at buf once.
hipError_t launch_read_ceiling(const void* buf, int64_t bytes, void* sink, hipStream_t stream);

// GPTQv1 <-> GPTQv2 stored zero conversion of a packed qzeros [G, N*b/32].
hipError_t launch_convert_zeros(const int32_t* in, int32_t* out, int bits, int64_t G, int64_t N, int to_v2,
                                int32_t* lossy_count, hipStream_t stream);

}  // namespace gptq
