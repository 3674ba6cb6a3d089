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
  float* partial;           // decode split-K partial sums (nullable when splits == 1)
  int* counters;            // decode per-tile arrival counters (nullable when splits == 1)
  int M, N, K, G, group_size, zero_offset;
  int chunks;               // K / 32
  int64_t zrow_words;       // N * bits / 32
  // decode launch shape
  int tiles;                // ceil(N / 64)
  int splits;               // K slices reduced across workgroups
  int wg_chunks;            // 32-row chunks per workgroup (multiple of 4)
  // prefill launch shape
  int tiles_m, tiles_n;
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

hipError_t launch_dequant(int bits, const DequantArgs& a, hipStream_t stream);

// Decode (M <= 16).  `per_elem` selects the per-element scale/zero path (act
// order or group_size % 32 != 0).  LDS bytes needed for a launch shape:
size_t decode_lds_bytes(int M, int wg_chunks, bool per_elem);
hipError_t launch_decode(int bits, bool per_elem, const GemmArgs& a, hipStream_t stream);

// Prefill (any M, used for M > 16).
void prefill_shape(int M, int N, int* tiles_m, int* tiles_n);
hipError_t launch_prefill(int bits, bool per_elem, const GemmArgs& a, hipStream_t stream);

// Min/max quantize + pack (fp32 W -> qweight, qzeros, scales).
hipError_t launch_quantize(const float* w, const int32_t* g_idx, int bits, int group_size, int sym, int is_v2,
                           int N, int K, int32_t* qweight, int32_t* qzeros, void* scales, hipStream_t stream);

}  // namespace gptq
