// Decode kernel (M <= 16): y[M, N] = x[M, K] . W^[K, N], the memory-bound case
// (page "Weight-only INT4 quantization: GPTQ, AWQ and the Marlin kernel",
// section 1.1: decode reads every weight once per token).
//
// Work split.  A workgroup owns a column tile of TN = 16 * CPL columns for the
// whole of K, so no partial sum ever leaves the workgroup: its waves split K,
// each wave takes CPW consecutive 32-row chunks per phase (lane = one 8-row
// block of CPL adjacent columns, CPL = 1, 2 or 4 words per load), and the
// waves reduce through LDS at the end.  Tile width, wave count and CPW are
// chosen per shape so the grid covers all 256 CUs with little padding;
// consecutive tiles are placed on the same XCD so neighbouring row pieces
// share that XCD's L2 lines.
//
// Memory-level parallelism.  CPW is a compile-time constant and the chunk loop
// is straight-line and branch-free: a wave issues the loads of its small
// operands (x, the scale/zero rows, for act order the g_idx slice), then all
// CPW of its weight loads back to back (buffer loads: one per-lane offset, the
// chunk's offset in a scalar register), and each chunk waits only for its own
// load.  For M = 1 every decode layer here takes a single phase, so a
// workgroup's whole weight tile is in flight right after launch.  Larger
// M * K runs in K-phases whose x is staged in alternating LDS buffers.
//
// Contraction: one v_mfma_f32_16x16x32_f16 per (32-row chunk, column slot):
// A = 16 rows of x (rows >= M are zero), B = the block each lane unpacked.
//
// Fast path (group_size % 32 == 0, no g_idx): a chunk lies in one group, so
// its scale s and zero z are constant over it.  B holds each field as the fp16
// subnormal MUL*q*2^-24 (a plain mask of the packed word; the MFMA keeps
// subnormal inputs exactly) and x is pre-divided by MUL, so
//   D = sum x' B = 2^-24 sum x q
//   y += (s 2^24) D + (-s z) sum x = s sum x (q - z)
// i.e. the dequant formula with the scale and the zero point factored out of
// the chunk's sum (page "Enhancing vLLM's support for the GPTQv2 format",
// section "Weight quantization of LLMs").  Per-element path (act order or
// other groups): B is the exact fp16 dequantized weight, built with each
// row's own scale and zero.
#include <type_traits>

#include "gptq_kernels.hpp"

namespace gptq {

// 16-byte x pieces a thread stages per phase: a phase holds nw * CPW chunks of
// M rows, so CPW * M <= 16 * XP must hold (the host checks it).
__host__ __device__ constexpr int decode_x_pieces_of(int mv) { return mv == 1 ? 2 : 8; }
constexpr int kDecodeTQuads = 4;   // at most this many scale/zero quads (4 columns of a group) per thread per round

// Table quads a thread stages per round: enough for the rows a wave's run of
// cpw chunks touches with 32-row groups, at most kDecodeTQuads (the host
// rejects shapes whose rows do not fit).
__host__ __device__ constexpr int decode_table_quads(bool per_elem, int cpl, int cpw) {
  return per_elem ? kDecodeTQuads
                  : ((cpw + 1) * 4 * cpl + 63) / 64 < kDecodeTQuads ? ((cpw + 1) * 4 * cpl + 63) / 64 : kDecodeTQuads;
}

__host__ __device__ constexpr int decode_words(int bits, bool per_elem, int cpl, int cpw, int mv) {
  return cpw * cpl * ((bits == 3 || bits == 8) ? 2 : 1);
}

// Waves per SIMD each instantiation is compiled for (a register budget of
// 512 / W per lane, met without spills): M = 1 runs 4 while a lane holds at
// most 32 weight words and 3 above; M > 1 runs 2.
__host__ __device__ constexpr int decode_waves_per_simd(int bits, bool per_elem, int cpl, int cpw, int mv) {
  return mv != 1 ? 2 : (decode_words(bits, per_elem, cpl, cpw, mv) <= 32 ? 4 : 3);
}

// A workgroup's waves spread over the CU's 4 SIMDs, so at most 4 W of them.
__host__ __device__ constexpr int decode_max_threads(int bits, bool per_elem, int cpl, int cpw, int mv) {
  return 256 * decode_waves_per_simd(bits, per_elem, cpl, cpw, mv) < 1024
             ? 256 * decode_waves_per_simd(bits, per_elem, cpl, cpw, mv) : 1024;
}

// CPW values compiled: at most 64 weight words per lane in flight where that
// leaves room for the rest (M = 1, 32- and 64-column tiles), 32 otherwise.
// bfloat16 at M = 1 has no 64-column tiles (they spill in its register budget).
__host__ __device__ constexpr bool decode_cpw_ok(int bits, bool per_elem, int cpl, int cpw, int mv, bool bf16 = false) {
  return (cpw == 8 || cpw == 16 || cpw == 32) &&
         decode_words(bits, per_elem, cpl, cpw, mv) <= ((mv == 1 && cpl > 1) ? 64 : 32) &&
         !(bf16 && (!per_elem || (mv == 1 && cpl == 4)));
}

template <int CPL> struct WordVec;
template <> struct WordVec<1> { typedef uint32_t T; };
template <> struct WordVec<2> { typedef u32x2_t T; };
template <> struct WordVec<4> { typedef u32x4_t T; };

template <int CPL> __device__ __forceinline__ uint32_t word_of(const typename WordVec<CPL>::T& v, int j) {
  if constexpr (CPL == 1) return v;
  else return v[j];
}

// Packed weights are read exactly once per call: nontemporal loads (cache
// policy bit 2, `nt` on gfx950) keep them from displacing x and the
// scale/zero rows in the caches (measured on MI355X: the Llama-7B decode
// layers 4-9% faster, a plain read of the same bytes 5-9%).
constexpr int kWeightLoadPolicy = 2;

template <int CPL>
__device__ __forceinline__ typename WordVec<CPL>::T buffer_words(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (CPL == 1) return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, kWeightLoadPolicy);
  else if constexpr (CPL == 2) return __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kWeightLoadPolicy);
  else return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kWeightLoadPolicy);
}

__host__ __device__ inline size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

// v / d and v % d for v >= 0, d > 0: a shift or a mask when d is a power of
// two (every whole-chunk group size of 2^j * 32 rows), so the kernel's
// prologue spends no integer-division sequence on them
__host__ __device__ inline int div_pos(int v, int d) {
  return (d & (d - 1)) == 0 ? v >> __builtin_ctz((unsigned)d) : v / d;
}
__host__ __device__ inline int mod_pos(int v, int d) { return (d & (d - 1)) == 0 ? v & (d - 1) : v % d; }

// rows of x a chunk's sums are laid out for (multiple of 4 for M > 1)
__host__ __device__ inline int decode_corr_rows(int M) { return M == 1 ? 1 : (M + 3) & ~3; }

// LDS carve-up.  Fast path: one region per wave holding only that wave's
// chunks of a phase (x fragments, per-chunk sums of x, the scale/zero rows of
// the groups they touch), so a wave stages and reads its own data and never
// waits for the others before the final reduction.  Per-element path: a phase buffer shared
// by the workgroup (two when K takes several phases: x fragments and the
// phase's g_idx slice) plus the whole scale/zero table, behind a barrier.
__host__ __device__ inline DecodeLayout decode_layout(int M, int pc, int nw, int cpl, bool per_elem, int G, int cpg,
                                                      int phases, bool bf16 = false, int cpw_known = 0) {
  DecodeLayout L;
  const size_t tn = (size_t)16 * cpl;
  const int cpw = cpw_known > 0 ? cpw_known : pc / nw;   // the kernel passes its compile-time value
  // several rows (fp16): the A fragments come straight from x in global
  // memory (no x staging; on the fast path the sums of x come from an MFMA),
  // and every wave stages its own chunks' small operands in its own region
  const bool xdirect = M > 1 && !bf16;
  const bool per_wave = !per_elem || xdirect;
  const int chunks = per_wave ? cpw : pc;                // chunks one staging region holds
  const size_t frag = xdirect ? 0 : align16((size_t)chunks * 4 * M * 16);
  L.corr_off = frag;
  const size_t corr = (per_elem || xdirect) ? 0 : align16((size_t)chunks * decode_corr_rows(M) * 4);
  L.gidx_off = frag + corr;
  // per-element path: each row's byte offset of its group's table row (4
  // bytes per row, so that a lookup is one add to the lane's column offset)
  const size_t gidx = per_elem ? align16((size_t)chunks * 32 * 4) : 0;
  L.ptab_off = L.gidx_off + gidx;
  // fast path: the groups a run of cpw consecutive chunks can touch
  L.ptab_rows = per_elem ? 0 : div_pos(cpw - 1, cpg) + 2;
  L.buf_stride = align16(L.ptab_off + (size_t)L.ptab_rows * tn * 8);
  const int regions = per_wave ? nw : (phases > 1 ? 2 : 1);
  L.tab_off = (size_t)regions * L.buf_stride;            // whole table (per-element path)
  // per-element table entry: (zero << 16 | fp16 scale), or the fp32 pair
  // (s, -z s) for bfloat16
  const size_t tab = per_elem ? (size_t)G * tn * (bf16 ? 8 : 4) : 0;
  // a wave stages its rows in one round; the whole table (per-element path) loops
  L.fits_staging = per_elem || (size_t)L.ptab_rows * tn / 4 <= (size_t)decode_table_quads(per_elem, cpl, cpw) * 64;
  const size_t data = L.tab_off + tab;
  const size_t red = (size_t)nw * M * tn * 4;
  L.total = data > red ? data : red;
  return L;
}

size_t decode_lds_bytes(int M, int pc, int nw, int cpl, bool per_elem, int G, int cpg, int phases, bool bf16) {
  const DecodeLayout L = decode_layout(M, pc, nw, cpl, per_elem, G, cpg, phases, bf16);
  return L.fits_staging ? L.total : ~(size_t)0;
}

int decode_max_x_pieces(int M) { return decode_x_pieces_of(M == 1 ? 1 : 4); }
int decode_waves_per_simd_for(int bits, bool per_elem, int cpl, int cpw, int M) {
  return decode_waves_per_simd(bits, per_elem, cpl, cpw, M == 1 ? 1 : 4);
}
int decode_max_threads_for(int bits, bool per_elem, int cpl, int cpw, int M) {
  return decode_max_threads(bits, per_elem, cpl, cpw, M == 1 ? 1 : 4);
}
bool decode_cpw_allowed(int bits, bool per_elem, int cpl, int cpw, int M, bool bf16) {
  return decode_cpw_ok(bits, per_elem, cpl, cpw, M == 1 ? 1 : 4, bf16);
}

// The kernel body; BF16 (per-element path only): x, scales and out are
// bfloat16, B is the element-wise bfloat16 dequant and the MFMA the bf16 one.
// FOLD (fast path): the scale and zero are folded into the sums once per
// block of FOLD consecutive chunks of one group (the MFMAs accumulate the
// block's chunks, also the multi-row sums of x) instead of once per chunk;
// needs group_size % (32 FOLD) == 0 and every wave's run and K split starting
// on a multiple of FOLD chunks.
template <int BITS, bool PER_ELEM, bool BF16, int MV, int CPL, int CPW, int FOLD>
__device__ __forceinline__ void decode_body(GemmArgs a) {
  static_assert(!BF16 || PER_ELEM, "bfloat16 decode runs the per-element path");
  static_assert(FOLD == 1 || (!PER_ELEM && CPW % (2 * FOLD) == 0), "block fold: fast path");
  extern __shared__ __align__(16) unsigned char lds[];
  // one output element, rounded to the activation type (nearest even)
  auto store_out = [](_Float16* out, int64_t i, float v) __attribute__((always_inline)) {
    if constexpr (BF16) reinterpret_cast<__bf16*>(out)[i] = (__bf16)v;
    else out[i] = (_Float16)v;
  };
  // workgroup -> (column tile t, K split sk); consecutive units share an XCD
  int unit = blockIdx.x;
  if (a.n_experts > 0) {
    // grouped decode: (expert, block of up to 16 of its rows, column tile);
    // blocks without rows leave at once (the expert's rows are clamped to M
    // and to its first moe_rows)
    const int per_expert = a.tiles * a.moe_blocks;
    const int e = blockIdx.x / per_expert;
    const int rest = blockIdx.x - e * per_expert;
    const int b = rest / a.tiles;
    unit = rest - b * a.tiles;
    const int e0 = min(max(a.moe_off[e], 0), a.M);
    const int r_end = min(min(max(a.moe_off[e + 1], 0), a.M), e0 + min(a.moe_rows, a.M));
    const int r0 = e0 + 16 * b;
    const int rows = min(16, r_end - r0);
    if (rows <= 0) return;
    a.M = rows;
    a.x += (int64_t)r0 * a.K;
    a.out += (int64_t)r0 * a.N;
    a.qweight += e * a.qw_stride;
    a.qzeros += e * a.qz_stride;
    a.scales += e * a.sc_stride;
    if (a.g_idx) a.g_idx += e * a.gi_stride;
  } else if (a.row_blocks > 1) {
    // rows in blocks of 16 (no K split): workgroup (b, unit) takes rows
    // [16 b, 16 b + 16) of column tile `unit`.  With whole eighths of tiles,
    // the row blocks of one tile run on one XCD, back to back, so its L2
    // serves their repeated reads of the tile's weights.
    int b;
    if ((a.tiles & 7) == 0) {
      const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
      b = slot % a.row_blocks;
      unit = (slot / a.row_blocks) * 8 + xcd;
    } else {
      b = blockIdx.x / a.tiles;
      unit = blockIdx.x - b * a.tiles;
    }
    a.M = min(16, a.M - 16 * b);
    a.x += (int64_t)(16 * b) * a.K;
    a.out += (int64_t)(16 * b) * a.N;
  } else {
    const int units = a.tiles * a.ks;
    if ((units & 7) == 0) unit = (blockIdx.x & 7) * (units >> 3) + (blockIdx.x >> 3);
  }
  constexpr int XP = decode_x_pieces_of(MV);
  // the zero term's per-chunk sums of x: dot products at staging for one row,
  // an extra MFMA per chunk for several rows (for one row the extra MFMA in
  // every chunk's chain measured slower on MI355X; for 4 and 16 rows the
  // staging work it removes made the layers 5-21% faster)
  constexpr bool kSumsByMfma = MV != 1;
  // several rows on the fast path: each lane loads its A fragment (row q,
  // block kb of a chunk: 16 bytes of x) with the chunk's weights and puts it in
  // the unpack's field order in registers, instead of the wave staging x
  // through LDS per phase (as many bytes per chunk as 2-bit weights at 16
  // rows); the per-element path keeps its shared staging
  constexpr bool XD = !BF16 && MV != 1;
  // staging per wave (own chunks, own LDS region, no workgroup barrier per
  // phase): the fast path, and the per-element path with several rows (whose
  // whole scale/zero table is staged once, behind one barrier)
  constexpr bool PW = !PER_ELEM || XD;
  constexpr int GP = (CPW + 7) / 8;                  // g_idx pieces: 8 * CPW rows <= 64 * GP pieces of 4
  constexpr int TQ = decode_table_quads(PER_ELEM, CPL, CPW);
  constexpr int TN = 16 * CPL;
  constexpr int L = Block<BITS>::LOADS;
  typedef typename WordVec<CPL>::T wvec;
  typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));

  const int M = MV == 1 ? 1 : a.M;
  const int nthreads = (int)blockDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int kb = lane >> 4;          // 8-row block of the chunk (A and B operands)
  const int q = lane & 15;           // column slot (B) and x row (A)
  const int t = a.ks == 1 ? unit : unit / a.ks;
  const int sk = unit - t * a.ks;
  const int c0 = sk * a.cks;                         // first chunk of this split
  const int n0 = t * TN;
  const int n = n0 + CPL * q;
  const int nc = n < a.N ? n : 0;                    // lanes past N read column 0 (result unused)
  const int C = min(a.chunks - c0, a.cks);          // chunks of this split (>= 1)
  const int pc = a.pc, phases = a.phases, cpg = a.cpg;
  // rows the LDS layout is sized for: the multi-row instantiation reads its
  // per-chunk sums of x in groups of four rows, so it lays out at least two
  // rows (four sums) even for a one-row block of a grouped launch
  const int ML = MV == 1 ? 1 : max(M, 2);
  const DecodeLayout lay = decode_layout(ML, pc, a.nw, CPL, PER_ELEM, a.G, cpg, phases, BF16, CPW);
  const int Mp = decode_corr_rows(ML);
  const uint32_t sel = block_sel<BITS>(kb);
  // every row of a 32-row chunk in one group (no g_idx, whole-chunk groups)
  const bool rows_share_group = a.g_idx == nullptr && (a.group_size & 31) == 0;
  // 4-bit words of the tiled layout hold their fields in pair order, so the
  // unpack's register v holds fields (2v, 2v + 1) instead of (F[2v], F[2v + 1])
  const bool pairs4 = BITS == 4 && a.wtiled != 0;

  // ---- staging scope: the fast path stages per wave (its own CPW chunks, in
  // its own LDS region), the per-element path per workgroup (the phase's pc
  // chunks, shared).  st / sn: this thread's index and the staging threads.
  const int st = PW ? lane : tid;
  const int sn = PW ? 64 : nthreads;
  const int sc = PW ? CPW : pc;                      // chunks one staging region holds
  // scale/zero table: the fast path stages its rows per wave, the per-element
  // path the whole table once with the whole workgroup
  const int tst = PER_ELEM ? tid : lane;
  const int tsn = PER_ELEM ? nthreads : 64;
  // Chunk u of wave w in phase p is p*pc + w*CPW + u: each wave reads a run of
  // consecutive packed rows.
  auto stage_chunk = [&](int p, int cl) __attribute__((always_inline)) { return PW ? p * pc + wave * CPW + cl : p * pc + cl; };
  auto stage_base = [&](int p) __attribute__((always_inline)) {
    return lds + (size_t)(PW ? wave : (phases > 1 ? (p & 1) : 0)) * lay.buf_stride;
  };

  // ---- small operands of a phase: x, g_idx slice, scale/zero rows.  The loads
  // are unconditional (out-of-range indices are clamped, the value replaced by
  // zero when it is stored) and keep raw words, so they issue as one burst.
  half8_t xr[XP];
  const int xpieces = sc * M * 4;
  // piece i of this thread: e = st + i sn, kbe = e & 3, rest = e >> 2 = cl M + m
  // (row m, chunk cl).  rest grows by sn / 4 per piece, so (m, cl) advance by
  // (dm, dcl) with at most one carry: no integer division per piece
  const int xr0 = st >> 2, xrd = sn >> 2;
  const int xcl0 = MV == 1 ? xr0 : xr0 / M, xm0 = xr0 - xcl0 * M;
  const int xdcl = MV == 1 ? xrd : xrd / M, xdm = xrd - xdcl * M;
  auto x_next = [&](int& m, int& cl) __attribute__((always_inline)) {
    m += xdm;
    cl += xdcl;
    if (m >= M) {
      m -= M;
      ++cl;
    }
  };
  auto load_x = [&](int p) __attribute__((always_inline)) {
    if constexpr (XD) return;
    int m = xm0, cl = xcl0;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int e = st + i * sn;
      const bool ok = e < xpieces && stage_chunk(p, cl) < C;
      const int c = ok ? stage_chunk(p, cl) : 0;
      xr[i] = *reinterpret_cast<const half8_t*>(a.x + (int64_t)(ok ? m : 0) * a.K + 32 * (c0 + c) + 8 * (e & 3));
      x_next(m, cl);
    }
  };
  i32x4_t gr[PER_ELEM ? GP : 1];
  const int gpieces = sc * 8;                        // 4 rows per piece
  auto load_g = [&](int p) __attribute__((always_inline)) {
    if constexpr (PER_ELEM) {
#pragma unroll
      for (int i = 0; i < GP; ++i) {
        const int e = st + i * sn;
        const int k = 32 * stage_chunk(p, 0) + 4 * e;   // row within the split
        const int kk = (e < gpieces && k < 32 * C) ? 32 * c0 + k : 0;
        if (a.g_idx) gr[i] = *reinterpret_cast<const i32x4_t*>(a.g_idx + kk);
        else gr[i] = i32x4_t{kk / a.group_size, (kk + 1) / a.group_size, (kk + 2) / a.group_size,
                             (kk + 3) / a.group_size};
      }
    }
  };
  auto store_xg = [&](int p) __attribute__((always_inline)) {
    unsigned char* base = stage_base(p);
    _Float16* frag = reinterpret_cast<_Float16*>(base);
    float* corr = reinterpret_cast<float*>(base + lay.corr_off);
    int m_next = xm0, cl_next = xcl0;
#pragma unroll
    for (int i = 0; i < (XD ? 0 : XP); ++i) {
      const int m = m_next, cl = cl_next, kbe = (st + i * sn) & 3;
      x_next(m_next, cl_next);
      const bool ok = st + i * sn < xpieces && stage_chunk(p, cl) < C;
      if (st + i * sn >= xpieces) continue;          // xpieces % 4 == 0: groups of four stay together
      half8_t av;
      float xs = 0.f;                                // sum of x' MUL over the piece
      const half8_t xv = ok ? xr[i] : half8_t{};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        // the pair of register v in field order; x' = x / MUL is exact in fp16
        // (a power-of-two scaling) up to subnormal rounding, like the scalar form
        half2_t pr = pairs4 ? half2_t{xv[2 * v], xv[2 * v + 1]}
                            : half2_t{xv[Block<BITS>::F[2 * v]], xv[Block<BITS>::F[2 * v + 1]]};
        if constexpr (!PER_ELEM) {
          const _Float16 inv = (_Float16)(1.0f / (float)Block<BITS>::MUL[v]);
          const _Float16 mul = (_Float16)Block<BITS>::MUL[v];
          pr = pr * half2_t{inv, inv};
          if constexpr (!kSumsByMfma) xs = __builtin_amdgcn_fdot2(pr, half2_t{mul, mul}, xs, false);
        }
        av[2 * v] = pr[0];
        av[2 * v + 1] = pr[1];
      }
      *reinterpret_cast<half8_t*>(frag + (((cl * 4 + kbe) * M + m) << 3)) = av;
      // one-row instantiation: the chunk's (with FOLD > 1 the fold block's)
      // sum of x (x' MUL) for the zero term; lanes 4 cl .. 4 cl + 3 hold
      // chunk cl, so a block of FOLD chunks is 4 FOLD aligned lanes of one
      // 16-lane row.  Summed into the block's last lane by DPP row shifts
      // (lanes shifted in from outside the row read 0): the same pairwise
      // sums as a butterfly of lane swaps, without their LDS round trips
      // (measured on MI355X: the Llama-7B step 1.7% faster).  The multi-row
      // instantiation gets its sums from an MFMA at compute time
      if constexpr (!PER_ELEM && !kSumsByMfma) {
        auto shr = [](float v, auto n_c) __attribute__((always_inline)) {
          return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                      0x110 + decltype(n_c)::value, 0xF, 0xF, true));
        };
        xs += shr(xs, std::integral_constant<int, 1>{});     // row_shr:1
        xs += shr(xs, std::integral_constant<int, 2>{});
        if constexpr (FOLD >= 2) xs += shr(xs, std::integral_constant<int, 4>{});
        if constexpr (FOLD >= 4) xs += shr(xs, std::integral_constant<int, 8>{});
        if (kbe == 3 && cl % FOLD == FOLD - 1) corr[(cl / FOLD) * Mp + m] = xs;
      }
    }
    if constexpr (PER_ELEM) {
      // row -> byte offset of its group's row in the whole table (groups
      // clamped into [0, G))
      u32x4_t* gl = reinterpret_cast<u32x4_t*>(base + lay.gidx_off);
#pragma unroll
      for (int i = 0; i < GP; ++i) {
        const int e = st + i * sn;
        if (e < gpieces) {
          const bool ok = 32 * stage_chunk(p, 0) + 4 * e < 32 * C;
          u32x4_t go;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int g = ok ? gr[i][r] : 0;
            g = g < 0 ? 0 : (g >= a.G ? a.G - 1 : g);
            go[r] = (uint32_t)g * (uint32_t)(TN * (BF16 ? 8 : 4));
          }
          gl[e] = go;
        }
      }
    }
  };

  // Fast-path table row: entry (s 2^24, -s z) of column col at float offset
  // tab_pos(col).  64-column tiles split a row into two planes (columns 4q,
  // 4q+1 | 4q+2, 4q+3) so that the 16 lanes of a read fetch consecutive
  // 16-byte pieces (no LDS bank conflicts); narrower tiles are contiguous.
  auto tab_pos = [](int col) __attribute__((always_inline)) {
    if constexpr (CPL == 4) return (((col & 3) >> 1) * 16 + (col >> 2)) * 4 + (col & 1) * 2;
    else return col * 2;
  };

  // scale/zero table rows r < rows holding group group_of_row(r), four columns
  // per quad: raw scale and zero words in registers, unpacked when stored.
  // Groups past G and columns past N are stored as zero.
  u32x2_t tsr[TQ];
  uint32_t tz0[TQ], tz1[TQ];
  const uint32_t* qz = reinterpret_cast<const uint32_t*>(a.qzeros);
  auto table_quad = [&](int rows, int e0, int i, int& r, int& c4) __attribute__((always_inline)) {
    const int e = e0 + tst + i * tsn;
    r = e / (TN / 4);
    c4 = e - r * (TN / 4);
    return e < rows * (TN / 4);
  };
  auto load_table = [&](auto group_of_row, int rows, int e0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TQ; ++i) {
      if (i > 0 && e0 + i * tsn >= rows * (TN / 4)) break;   // wave-uniform: no quad of this round left
      int r, c4;
      const bool in = table_quad(rows, e0, i, r, c4);
      const int nn = n0 + 4 * c4;
      const int gr = group_of_row(r);
      const bool ok = in && gr < a.G && nn < a.N;
      const int g = ok ? gr : 0, nq = ok ? nn : 0;
      tsr[i] = *reinterpret_cast<const u32x2_t*>(a.scales + (int64_t)g * a.N + nq);
      const uint32_t* row = qz + (int64_t)g * a.zrow_words;
      if constexpr (BITS == 3) {                     // 12 bits, possibly across two words
        const int w = 3 * (nq >> 5) + ((3 * (nq & 31)) >> 5);
        tz0[i] = row[w];
        tz1[i] = row[((3 * (nq & 31)) >> 5) < 2 ? w + 1 : w];
      } else {
        tz0[i] = row[(nq * BITS) >> 5];
      }
    }
  };
  // four columns' (zero + offset) of quad i
  auto quad_zeros = [&](int i, int c4) __attribute__((always_inline)) {
    const int nq = n0 + 4 * c4;
    if constexpr (BITS == 3) return __builtin_amdgcn_alignbit(tz1[i], tz0[i], (uint32_t)((3 * (nq & 31)) & 31));
    else return tz0[i] >> ((nq * BITS) & 31);
  };
  auto store_table = [&](unsigned char* tw, auto group_of_row, int rows, int e0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TQ; ++i) {
      if (i > 0 && e0 + i * tsn >= rows * (TN / 4)) break;
      int r, c4;
      if (!table_quad(rows, e0, i, r, c4)) continue;
      const bool real = group_of_row(r) < a.G && n0 + 4 * c4 < a.N;
      const uint32_t zw = quad_zeros(i, c4);
      uint32_t sb[4], z[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sb[j] = (j & 1) ? (tsr[i][j >> 1] >> 16) : (tsr[i][j >> 1] & 0xFFFFu);
        z[j] = ((zw >> (BITS * j)) & ((1u << BITS) - 1u)) + (uint32_t)a.zero_offset;
      }
      if constexpr (BF16) {                          // (s, -s (zero + offset)) as fp32, exact
        f32x4_t v0, v1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float sc = real ? bf16_to_f32(sb[j]) : 0.f;
          f32x4_t& v = j < 2 ? v0 : v1;
          v[2 * (j & 1)] = sc;
          v[2 * (j & 1) + 1] = -sc * (float)z[j];
        }
        *reinterpret_cast<f32x4_t*>(tw + (r * TN + 4 * c4) * 8) = v0;
        *reinterpret_cast<f32x4_t*>(tw + (r * TN + 4 * c4) * 8 + 16) = v1;
      } else if constexpr (PER_ELEM) {               // fp16 pair (s, -(zero + offset)), both exact
        u32x4_t v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t nz = __builtin_bit_cast(uint16_t, (_Float16)(-(float)z[j]));
          v[j] = real ? ((nz << 16) | sb[j]) : 0u;
        }
        *reinterpret_cast<u32x4_t*>(tw + (r * TN + 4 * c4) * 4) = v;
      } else {                                       // (s 2^24, -s (zero + offset)) as fp32, exact
        f32x4_t v0, v1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float sc = real ? (float)__builtin_bit_cast(_Float16, (uint16_t)sb[j]) : 0.f;
          f32x4_t& v = j < 2 ? v0 : v1;
          v[2 * (j & 1)] = sc * 16777216.0f;
          v[2 * (j & 1) + 1] = -sc * (float)z[j];
        }
        *reinterpret_cast<f32x4_t*>(tw + r * TN * 8 + tab_pos(4 * c4) * 4) = v0;
        *reinterpret_cast<f32x4_t*>(tw + r * TN * 8 + tab_pos(4 * c4 + 2) * 4) = v1;
      }
    }
  };
  // fast path: row r of a wave's table holds group stage_chunk(p, 0) / cpg + r
  auto chunk_group = [&](int p) __attribute__((always_inline)) {
    const int g0 = div_pos(c0 + stage_chunk(p, 0), cpg);
    return [g0](int r) __attribute__((always_inline)) { return g0 + r; };
  };
  auto whole_table = [](int r) { return r; };
  auto stage_next = [&](int p) __attribute__((always_inline)) {                    // loads for phase p (registers)
    load_x(p);
    load_g(p);
    if constexpr (!PER_ELEM) load_table(chunk_group(p), lay.ptab_rows, 0);
  };
  auto store_stage = [&](int p) __attribute__((always_inline)) {                    // ... and their LDS stores
    store_xg(p);
    if constexpr (!PER_ELEM) store_table(stage_base(p) + lay.ptab_off, chunk_group(p), lay.ptab_rows, 0);
  };

  // ---- packed words: block kb of chunk c lives in packed rows BITS * c +
  // row0(kb) (+ row1), i.e. at the lane's offset in chunk 0 plus the
  // wave-uniform c * BITS row strides.  A packed row is N * 4 bytes apart in
  // the checkpoint layout and 64 bytes apart in the tiled one, where column n
  // lies in 16-column tile n / 16 (starting at (n / 16) * chunks * BITS * 64
  // bytes); a lane's CPL adjacent columns never cross a 16-column tile.
  // Chunks past K re-read the last chunk: they meet zero x (and a zero table
  // row) and add exactly nothing.
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(a.qweight), (short)0, (int)((int64_t)a.chunks * BITS * a.N * 4), 0x00020000);
  const uint32_t wrow = a.wtiled ? 64u : (uint32_t)a.N * 4u;
  const uint32_t wcol = a.wtiled ? (uint32_t)(nc >> 4) * (uint32_t)a.chunks * (uint32_t)BITS * 64u +
                                       (uint32_t)(nc & 15) * 4u
                                 : (uint32_t)nc * 4u;
  const uint32_t off0 = (uint32_t)block_row0<BITS>(0, kb) * wrow + wcol;
  const uint32_t off1 = (uint32_t)block_row1<BITS>(0, kb) * wrow + wcol;
  const uint32_t cbytes = (uint32_t)BITS * wrow;
  wvec w0[1][CPW], w1[1][L == 2 ? CPW : 1];
  // several rows (XD): the lane's A fragment of chunk c is x[min(q, M - 1)]
  // [32 c + 8 kb, + 8).  For a chunk past the split's end the lane offset is
  // moved 1 GiB past the end of x (at most 32 MiB here): the buffer's range
  // check, which covers the lane offset, returns zeros and reads nothing, so
  // the chunk adds nothing
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16*>(a.x), (short)0, XD ? (int)((uint32_t)M * (uint32_t)a.K * 2u) : 0, 0x00020000);
  const uint32_t xoff = ((uint32_t)min(q, M - 1) * (uint32_t)a.K + 8u * (uint32_t)kb) * 2u;
  u32x4_t xa[XD ? CPW : 1];
  // chunks [U0, U1) of this wave in phase p
  auto load_w = [&](int p, auto set_c, auto u0_c, auto u1_c) __attribute__((always_inline)) {
    constexpr int set = decltype(set_c)::value;
#pragma unroll
    for (int u = decltype(u0_c)::value; u < decltype(u1_c)::value; ++u) {
      const int cw = p * pc + wave * CPW + u;
      if constexpr (XD)
        xa[u] = __builtin_amdgcn_raw_buffer_load_b128(xrsrc, (int)(cw < C ? xoff : xoff + 0x40000000u),
                                                      (c0 + min(cw, C - 1)) * 64, 0);
      const uint32_t so = (uint32_t)(c0 + min(cw, C - 1)) * cbytes;
      w0[set][u] = buffer_words<CPL>(wrsrc, off0, so);
      if constexpr (L == 2) w1[set][u] = buffer_words<CPL>(wrsrc, off1, so);
      // issue in chunk order, so chunk u waits only for loads 0..u
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  floatx4_t accg[CPL];                               // per-element path: MFMA accumulators
  float acc[CPL][MV];                                // fast path: scaled sums
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    accg[j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < MV; ++v) acc[j][v] = 0.f;
  }
  // fast path: the previous chunk's MFMA results and scales, folded one chunk
  // later; the empty asm pins each fold in place (otherwise the whole chain is
  // sunk past the loop and every chunk's results stay live)
  constexpr bool kDeferFold = CPL < 4 || FOLD > 1;
  floatx4_t d_prev[CPL];
  float s_prev[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    d_prev[j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    s_prev[j] = 0.f;
  }
  auto fold_prev = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
#pragma unroll
      for (int v = 0; v < MV; ++v) {
        acc[j][v] = __builtin_fmaf(s_prev[j], d_prev[j][v], acc[j][v]);
        asm volatile("" : "+v"(acc[j][v]));
      }
    }
  };
  // block fold: the previous block's zero term too (its sums of x come from
  // the block's MFMAs for several rows)
  float s2_prev[CPL];
  floatx4_t x_prev = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < CPL; ++j) s2_prev[j] = 0.f;
  auto fold_prev_block = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
#pragma unroll
      for (int v = 0; v < MV; ++v) {
        acc[j][v] = __builtin_fmaf(s_prev[j], d_prev[j][v], __builtin_fmaf(s2_prev[j], x_prev[v], acc[j][v]));
        asm volatile("" : "+v"(acc[j][v]));
      }
    }
  };
  // XD: chunk u's A fragment from the lane's x words (natural k order), put in
  // the unpack's field order and divided by each register's MUL, exactly as
  // the staging writes it (a power-of-two scaling, exact up to subnormals)
  auto direct_A = [&](int u) __attribute__((always_inline)) {
    const half8_t xv = __builtin_bit_cast(half8_t, xa[XD ? u : 0]);
    half8_t av;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      half2_t pr = pairs4 ? half2_t{xv[2 * v], xv[2 * v + 1]}
                          : half2_t{xv[Block<BITS>::F[2 * v]], xv[Block<BITS>::F[2 * v + 1]]};
      if (!PER_ELEM && Block<BITS>::MUL[v] != 1) {   // a constant per unrolled v
        const _Float16 inv = (_Float16)(1.0f / (float)Block<BITS>::MUL[v]);
        pr = pr * half2_t{inv, inv};
      }
      av[2 * v] = pr[0];
      av[2 * v + 1] = pr[1];
    }
    return av;
  };
  const int kbc = MV == 1 ? 0 : min(kb, Mp / 4 - 1);  // rows 4 kbc + v of the correction sums

  // fast path: a chunk's LDS operands (A fragment, sum of x, the group row's
  // table entries), read one chunk ahead of their use so that LDS latency
  // overlaps the previous chunk's work
  struct FastOps {
    half8_t A;
    float X[1];                                      // one-row instantiation only
    float s1[CPL], s2[CPL];
  };
  auto fast_ops = [&](int p, int u, int row) __attribute__((always_inline)) {
    FastOps o;
    const unsigned char* base = stage_base(p);
    const _Float16* frag = reinterpret_cast<const _Float16*>(base);
    // rows >= M of A only feed rows >= M of D, which are never used
    if constexpr (!XD) o.A = *reinterpret_cast<const half8_t*>(frag + (((u * 4 + kb) * M + min(q, M - 1)) << 3));
    if constexpr (!kSumsByMfma) {
      const float* corr = reinterpret_cast<const float*>(base + lay.corr_off) + u * Mp + 4 * kbc;
      o.X[0] = corr[0];
    }
    // the group row is wave-uniform: keep its offset in a scalar register
    const int row_bytes = __builtin_amdgcn_readfirstlane(row * TN * 8);
    const float* te = reinterpret_cast<const float*>(base + lay.ptab_off + row_bytes);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      o.s1[j] = te[tab_pos(CPL * q + j)];
      o.s2[j] = te[tab_pos(CPL * q + j) + 1];
    }
    return o;
  };

  // chunk u of this wave in phase p (cl = its index in the staging region,
  // row = its group's row in the wave's table), words from register set `set`;
  // the fast path takes its LDS operands from `fo`
  auto compute_chunk = [&](int p, int u, int row, auto set_c, const FastOps& fo) __attribute__((always_inline)) {
    constexpr int set = decltype(set_c)::value;
    const unsigned char* base = stage_base(p);
    uint32_t w1j[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) w1j[j] = L == 2 ? word_of<CPL>(w1[set][L == 2 ? u : 0], j) : 0u;

    if constexpr (PER_ELEM) {
      const int cl = PW ? u : wave * CPW + u;        // the chunk's place in its staging region
      const _Float16* frag = reinterpret_cast<const _Float16*>(base);
      // rows >= M of A only feed rows >= M of D, which are never used
      const half8_t A = XD ? direct_A(u)
                           : *reinterpret_cast<const half8_t*>(frag + (((cl * 4 + kb) * M + min(q, M - 1)) << 3));
      // per-row scale and zero: the block's 8 rows each carry their own group,
      // staged as the byte offset of the group's table row
      const u32x4_t* gl = reinterpret_cast<const u32x4_t*>(base + lay.gidx_off) + 8 * cl + 2 * kb;
      const u32x4_t gv0 = gl[0], gv1 = gl[1];
      const uint32_t gv[8] = {gv0[0], gv0[1], gv0[2], gv0[3], gv1[0], gv1[1], gv1[2], gv1[3]};
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        if constexpr (BF16) {
          // fields in the staging's order (F, or pairs for 4-bit tiled
          // words), each with its row's (s, -z s); without g_idx and with
          // groups of whole chunks the block's rows share one group: one
          // table read.  r[2v], r[2v + 1]: register v's two fields.
          const unsigned char* tab2 = lds + lay.tab_off + (size_t)(CPL * q + j) * 8;
          float r[8];
          if constexpr (BITS == 4) {
            block4_regs_f32(word_of<CPL>(w0[set][u], j), r);
          } else {
            float f[8];
            block_fields_f32<BITS>(word_of<CPL>(w0[set][u], j), w1j[j], kb, f);
#pragma unroll
            for (int i = 0; i < 8; ++i) r[i] = f[Block<BITS>::F[i]];
          }
          u32x4_t bw;
          if (rows_share_group) {
            const f32x2_t t = *reinterpret_cast<const f32x2_t*>(tab2 + gv[0]);
#pragma unroll
            for (int v = 0; v < 4; ++v)
              bw[v] = bf16_pair(__builtin_fmaf(r[2 * v], t[0], t[1]), __builtin_fmaf(r[2 * v + 1], t[0], t[1]));
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              // the rows of register v's fields
              const uint32_t ga = pairs4 ? gv[2 * v] : gv[Block<BITS>::F[2 * v]];
              const uint32_t gb = pairs4 ? gv[2 * v + 1] : gv[Block<BITS>::F[2 * v + 1]];
              const f32x2_t ta = *reinterpret_cast<const f32x2_t*>(tab2 + ga);
              const f32x2_t tb = *reinterpret_cast<const f32x2_t*>(tab2 + gb);
              bw[v] = bf16_pair(__builtin_fmaf(r[2 * v], ta[0], ta[1]), __builtin_fmaf(r[2 * v + 1], tb[0], tb[1]));
            }
          }
          accg[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A),
                                                            __builtin_bit_cast(bf16x8_t, bw), accg[j], 0, 0, 0);
        }
      }
      if constexpr (!BF16) {
        // each field with its own row's group: the table row of (group, the
        // lane's CPL columns) is one contiguous LDS vector of fp16 pairs
        // (s, -z), read once per field for all CPL columns; per register pair
        //   q   = (1024 + MUL q) / MUL - 1024 / MUL    (one packed FMA, exact)
        //   W^  = (q - z) * s                          (packed add, packed multiply:
        //                                               exact, then one rounding)
        uint32_t pr[CPL][4];
#pragma unroll
        for (int j = 0; j < CPL; ++j) unpack_block<BITS>(word_of<CPL>(w0[set][u], j), w1j[j], sel, pr[j]);
        u32x4_t bw[CPL];
        const unsigned char* tab_lane = lds + lay.tab_off + (size_t)(CPL * q) * 4;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t ga = pairs4 ? gv[2 * v] : gv[Block<BITS>::F[2 * v]];
          const uint32_t gb = pairs4 ? gv[2 * v + 1] : gv[Block<BITS>::F[2 * v + 1]];
          const wvec ea = *reinterpret_cast<const wvec*>(tab_lane + ga);
          const wvec eb = *reinterpret_cast<const wvec*>(tab_lane + gb);
          const _Float16 inv = (_Float16)(1.0f / (float)Block<BITS>::MUL[v]);
          const _Float16 off = (_Float16)(-kMagic / (float)Block<BITS>::MUL[v]);
#pragma unroll
          for (int j = 0; j < CPL; ++j) {
            const uint32_t eaj = word_of<CPL>(ea, j), ebj = word_of<CPL>(eb, j);
            const half2_t nz = as_half2(__builtin_amdgcn_perm(ebj, eaj, 0x07060302u));   // (-z_a, -z_b)
            const half2_t sc = as_half2(__builtin_amdgcn_perm(ebj, eaj, 0x05040100u));   // (s_a, s_b)
            const half2_t qv = as_half2(pr[j][v]) * half2_t{inv, inv} + half2_t{off, off};
            bw[j][v] = as_u32((qv + nz) * sc);
          }
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j)
          accg[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(half8_t, bw[j]), accg[j], 0, 0, 0);
      }
    } else {
      // sums of x over the chunk for every row: one MFMA against a B operand
      // holding each register's MUL, i.e. sum x' MUL = what the one-row
      // staging computes with dot products (D rows 4 kb + v = this lane's rows)
      float X[MV];
      if constexpr (!kSumsByMfma) {
        X[0] = fo.X[0];
      } else {
        half8_t ones;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          ones[2 * v] = (_Float16)Block<BITS>::MUL[v];
          ones[2 * v + 1] = (_Float16)Block<BITS>::MUL[v];
        }
        const floatx4_t dx = __builtin_amdgcn_mfma_f32_16x16x32_f16(fo.A, ones, floatx4_t{0.f, 0.f, 0.f, 0.f},
                                                                    0, 0, 0);
#pragma unroll
        for (int v = 0; v < MV; ++v) X[v] = dx[v];
      }
      floatx4_t d[CPL];
      float s1[CPL];
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        s1[j] = fo.s1[j];
        uint32_t pr[4];
        unpack_block<BITS>(word_of<CPL>(w0[set][u], j), w1j[j], sel, pr, 0u);
        const u32x4_t bw = {pr[0], pr[1], pr[2], pr[3]};
        d[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fo.A, __builtin_bit_cast(half8_t, bw),
                                                      floatx4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < MV; ++v) acc[j][v] = __builtin_fmaf(fo.s2[j], X[v], acc[j][v]);
      }
      // with one or two MFMAs per chunk the previous chunk's products are
      // folded in while this chunk's MFMAs run; four cover their own latency
      if constexpr (kDeferFold) fold_prev();
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        d_prev[j] = d[j];
        s_prev[j] = s1[j];
      }
      if constexpr (!kDeferFold) fold_prev();
    }
  };

  using S0 = std::integral_constant<int, 0>;       // register set index, compile-time
  constexpr int H = CPW / 2;                        // the two halves of a wave's run of a phase
  using U0 = std::integral_constant<int, 0>;
  using UH = std::integral_constant<int, H>;
  using UE = std::integral_constant<int, CPW>;
  auto wave_fence = [&]() __attribute__((always_inline)) {
    // the wave reads back only what its own lanes wrote: LDS operations of one
    // wave complete in order, the fences keep the compiler's order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // chunks [U0, U1) of phase p; row / rem track the group row of the next chunk
  auto compute_range = [&](int p, auto u0_c, auto u1_c, int& row, int& rem) __attribute__((always_inline)) {
    constexpr int u0 = decltype(u0_c)::value, u1 = decltype(u1_c)::value;
    if constexpr (PER_ELEM) {
#pragma unroll
      for (int u = u0; u < u1; ++u) {
        compute_chunk(p, u, row, S0{}, FastOps{});
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (FOLD > 1) {
      // blocks of FOLD chunks of one group: the block's MFMAs accumulate its
      // sum of x' B (and, for several rows, its sums of x against the MUL
      // pattern), and its scale and zero are applied once, with the block's
      // sum of x (staged for one row).  The previous block's fold is issued
      // after this block's first MFMA (its results are not waited on at
      // once).  A fragments are read one chunk ahead, the block's table
      // entries and sum of x one block ahead.  row / rem (the group row and
      // the position in the group of chunk u0, a multiple of FOLD) are
      // wave-uniform and advance once per block.
      struct BlockOps {
        float X;
        float s1[CPL], s2[CPL];
      };
      auto block_ops = [&](int u, int r) __attribute__((always_inline)) {
        BlockOps o;
        const unsigned char* base = stage_base(p);
        o.X = kSumsByMfma ? 0.f : reinterpret_cast<const float*>(base + lay.corr_off)[u / FOLD];
        const int row_bytes = __builtin_amdgcn_readfirstlane(r * TN * 8);
        const float* te = reinterpret_cast<const float*>(base + lay.ptab_off + row_bytes);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          o.s1[j] = te[tab_pos(CPL * q + j)];
          o.s2[j] = te[tab_pos(CPL * q + j) + 1];
        }
        return o;
      };
      auto frag_A = [&](int u) __attribute__((always_inline)) {
        // rows >= M of A only feed rows >= M of D, which are never used
        if constexpr (XD) return direct_A(u);
        const _Float16* frag = reinterpret_cast<const _Float16*>(stage_base(p));
        return *reinterpret_cast<const half8_t*>(frag + (((u * 4 + kb) * M + min(q, M - 1)) << 3));
      };
      half8_t ones;                                  // each register's MUL (sums of x, several rows)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        ones[2 * v] = (_Float16)Block<BITS>::MUL[v];
        ones[2 * v + 1] = (_Float16)Block<BITS>::MUL[v];
      }
      row = __builtin_amdgcn_readfirstlane(row);
      rem = __builtin_amdgcn_readfirstlane(rem);
      BlockOps cur = block_ops(u0, row);
      // A fragments: from LDS one chunk ahead; with XD from registers at the
      // chunk itself (ahead would wait for the next chunk's loads too)
      half8_t A = XD ? half8_t{} : frag_A(u0);
#pragma unroll
      for (int b = u0 / FOLD; b < u1 / FOLD; ++b) {
        const int inc = 1 - (int)min(1u, (uint32_t)((rem + FOLD) ^ cpg));
        row = __builtin_amdgcn_readfirstlane(row + inc);
        rem = __builtin_amdgcn_readfirstlane((rem + FOLD) * (1 - inc));
        BlockOps nxt = cur;
        if (b + 1 < u1 / FOLD) nxt = block_ops(FOLD * (b + 1), row);
        floatx4_t d[CPL];
        floatx4_t dx = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < FOLD; ++i) {
          const int u = FOLD * b + i;
          if constexpr (XD) A = frag_A(u);
          half8_t An = A;
          if (!XD && u + 1 < u1) An = frag_A(u + 1);
          if constexpr (kSumsByMfma) dx = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ones, dx, 0, 0, 0);
#pragma unroll
          for (int j = 0; j < CPL; ++j) {
            uint32_t pr[4];
            const uint32_t w1j = L == 2 ? word_of<CPL>(w1[0][L == 2 ? u : 0], j) : 0u;
            unpack_block<BITS>(word_of<CPL>(w0[0][u], j), w1j, sel, pr, 0u);
            const u32x4_t bw = {pr[0], pr[1], pr[2], pr[3]};
            d[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(half8_t, bw),
                                                          i == 0 ? floatx4_t{0.f, 0.f, 0.f, 0.f} : d[j], 0, 0, 0);
          }
          if (i == 0) fold_prev_block();
          __builtin_amdgcn_sched_barrier(0);
          A = An;
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          d_prev[j] = d[j];
          s_prev[j] = cur.s1[j];
          s2_prev[j] = cur.s2[j];
        }
        if constexpr (kSumsByMfma) x_prev = dx;
        else x_prev = floatx4_t{cur.X, 0.f, 0.f, 0.f};
        cur = nxt;
      }
    } else {
      // the LDS operands of chunk u + 1 are read before chunk u is computed
      // (one chunk ahead only: hoisting all of them ahead of the weight waits
      // would cost ~10 registers per chunk).  row / rem are wave-uniform.
      row = __builtin_amdgcn_readfirstlane(row);
      rem = __builtin_amdgcn_readfirstlane(rem);
      FastOps cur = fast_ops(p, u0, row);
#pragma unroll
      for (int u = u0; u < u1; ++u) {
        // inc = (rem + 1 == cpg), in integer arithmetic so that it stays in
        // scalar registers (a compare would go through a vector select)
        const int inc = 1 - (int)min(1u, (uint32_t)((rem + 1) ^ cpg));
        row = __builtin_amdgcn_readfirstlane(row + inc);
        rem = __builtin_amdgcn_readfirstlane((rem + 1) * (1 - inc));
        FastOps nxt = cur;
        if (u + 1 < u1) nxt = fast_ops(p, u + 1, row);
        if constexpr (XD) cur.A = direct_A(u);        // waits for this chunk's loads only
        compute_chunk(p, u, row, S0{}, cur);
        __builtin_amdgcn_sched_barrier(0);
        cur = nxt;
      }
    }
  };
  // issue phase p's loads: small operands strictly before the weights, so
  // waiting for the former never waits for the latter
  auto issue = [&](int p) __attribute__((always_inline)) {
    stage_next(p);
    __builtin_amdgcn_sched_barrier(0);
    load_w(p, S0{}, U0{}, UE{});
  };

  if constexpr (PER_ELEM) {
    // ---- prologue: the first table round, phase 0's small operands and
    // weights, then the rest of the whole table before the first barrier
    load_table(whole_table, a.G, 0);
    issue(0);
    unsigned char* tw = lds + lay.tab_off;
    store_table(tw, whole_table, a.G, 0);
    const int quads = a.G * (TN / 4);
    for (int e0 = TQ * nthreads; e0 < quads; e0 += TQ * nthreads) {   // rare: very many groups
      load_table(whole_table, a.G, e0);
      store_table(tw, whole_table, a.G, e0);
    }
    if constexpr (!PW) {
      // ---- per phase: stage (one barrier), compute, issue the next phase
      for (int p = 0; p < phases; ++p) {
        store_stage(p);
        __syncthreads();
        int row = 0, rem = 0;
        compute_range(p, U0{}, UE{}, row, rem);
        if (p + 1 < phases) issue(p + 1);
      }
    }
  }
  if constexpr (PW) {
    // ---- per phase (staging wave-local): while the second half of phase p's
    // run is computed, the next phase's small operands and first half of
    // words are in flight; its second half is issued once the first half of
    // the register set is free.  So the bytes a wave has in flight stay at
    // about one run, and compute overlaps the memory stream.  The last phase
    // is peeled off so that every issued load is consumed and every wait is
    // exact (no branch between a load and its use).  The per-element path
    // has issued phase 0 already and passes one barrier, for its table.
    if constexpr (!PER_ELEM) issue(0);
    store_stage(0);
    if constexpr (PER_ELEM) __syncthreads();
    else wave_fence();
    int p = 0;
    for (; p + 1 < phases; ++p) {
      int row = 0, rem = mod_pos(c0 + stage_chunk(p, 0), cpg);
      compute_range(p, U0{}, UH{}, row, rem);
      stage_next(p + 1);
      __builtin_amdgcn_sched_barrier(0);
      load_w(p + 1, S0{}, U0{}, UH{});
      compute_range(p, UH{}, UE{}, row, rem);
      store_stage(p + 1);
      wave_fence();
      load_w(p + 1, S0{}, UH{}, UE{});
    }
    int row = 0, rem = mod_pos(c0 + stage_chunk(p, 0), cpg);
    compute_range(p, U0{}, UE{}, row, rem);
  }
  if constexpr (!PER_ELEM && FOLD > 1) fold_prev_block();
  else if constexpr (!PER_ELEM && kDeferFold) fold_prev();

  // ---- reduce the waves through LDS (rows < M), write fp16
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
#pragma unroll
    for (int v = 0; v < MV; ++v) {
      const int m = 4 * kb + v;
      if (m < M) red[(wave * M + m) * TN + CPL * q + j] = PER_ELEM ? accg[j][v] : acc[j][v];
    }
  }
  __syncthreads();
  const int nw = nthreads >> 6;
  if (a.ks == 1) {
    for (int e = tid; e < M * TN; e += nthreads) {
      const int m = e / TN, col = e - m * TN;
      if (n0 + col < a.N) {
        float s = 0.f;
        for (int w = 0; w < nw; ++w) s += red[(w * M + m) * TN + col];
        store_out(a.out, (int64_t)m * a.N + n0 + col, s);
      }
    }
    return;
  }
  // ---- split K: publish this split's sums, count the tile's arrivals; the
  // last split to arrive adds all of them in split order (deterministic) and
  // re-arms the counter.  The partial sums move only through agent-scope
  // atomic stores and loads, which are coherent across the XCDs' L2s by
  // themselves; the one ordering needed, every store of the workgroup
  // complete before its arrival is counted, comes from each wave waiting for
  // its stores (vmcnt 0) before the barrier.  (A full release/acquire fence
  // would also write back and invalidate the whole L2, which only plain
  // accesses need and which stalls every workgroup on that XCD.)
  for (int e = tid; e < M * TN; e += nthreads) {
    const int m = e / TN, col = e - m * TN;
    if (n0 + col < a.N) {
      float s = 0.f;
      for (int w = 0; w < nw; ++w) s += red[(w * M + m) * TN + col];
      __hip_atomic_store(a.ws + ((int64_t)sk * M + m) * a.N + n0 + col, s, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0): this wave's stores are complete
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __shared__ int last_split;
  __syncthreads();
  if (tid == 0)
    last_split = __hip_atomic_fetch_add(a.cnt + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (uint32_t)(a.ks - 1);
  __syncthreads();
  if (!last_split) return;
  for (int e = tid; e < M * TN; e += nthreads) {
    const int m = e / TN, col = e - m * TN;
    if (n0 + col < a.N) {
      float s = 0.f;
      for (int k = 0; k < a.ks; ++k)
        s += __hip_atomic_load(a.ws + ((int64_t)k * M + m) * a.N + n0 + col, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      store_out(a.out, (int64_t)m * a.N + n0 + col, s);
    }
  }
  if (tid == 0) __hip_atomic_store(a.cnt + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Each instantiation is compiled for a fixed number of waves per SIMD, which
// the host uses to size the grid and to know how many workgroups a CU holds.
template <int BITS, bool PER_ELEM, int MV, int CPL, int CPW, int FOLD>
__global__ __attribute__((amdgpu_flat_work_group_size(64, decode_max_threads(BITS, PER_ELEM, CPL, CPW, MV))))
__attribute__((amdgpu_waves_per_eu(decode_waves_per_simd(BITS, PER_ELEM, CPL, CPW, MV))))
void decode_kernel(GemmArgs a) {
  decode_body<BITS, PER_ELEM, false, MV, CPL, CPW, FOLD>(a);
}

// bfloat16 activations: the per-element path's launch shapes and registers
template <int BITS, int MV, int CPL, int CPW>
__global__ __attribute__((amdgpu_flat_work_group_size(64, decode_max_threads(BITS, true, CPL, CPW, MV))))
__attribute__((amdgpu_waves_per_eu(decode_waves_per_simd(BITS, true, CPL, CPW, MV))))
void decode_bf16_kernel(GemmArgs a) {
  decode_body<BITS, true, true, MV, CPL, CPW, 1>(a);
}

template <int BITS, bool PER_ELEM, int MV, int CPL, int CPW, int FOLD>
static hipError_t launch_decode_k(const GemmArgs& a, hipStream_t stream) {
  if constexpr (!decode_cpw_ok(BITS, PER_ELEM, CPL, CPW, MV)) {
    return hipErrorInvalidValue;
  } else {
    const size_t lds = decode_lds_bytes((a.n_experts > 0 || a.row_blocks > 1) ? 16 : a.M, a.pc, a.nw, CPL, PER_ELEM,
                                        a.G, a.cpg, a.phases, a.bf16 != 0);
    auto kern = decode_kernel<BITS, PER_ELEM, MV, CPL, CPW, FOLD>;
    if constexpr (FOLD == 1 && decode_cpw_ok(BITS, PER_ELEM, CPL, CPW, MV, true)) {
      if (a.bf16) kern = decode_bf16_kernel<BITS, MV, CPL, CPW>;
    } else {
      if (a.bf16) return hipErrorInvalidValue;
    }
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    if (a.row_blocks > 1 && (a.ks != 1 || a.n_experts > 0)) return hipErrorInvalidValue;
    const int grid = a.n_experts > 0 ? a.n_experts * a.moe_blocks * a.tiles
                                     : a.tiles * a.ks * (a.row_blocks > 1 ? a.row_blocks : 1);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * a.nw), lds, stream, a);
    return hipGetLastError();
  }
}

// block fold (a.fold > 1): fast path only
template <int BITS, bool PER_ELEM, int MV, int CPL, int CPW>
static hipError_t launch_decode_fold(const GemmArgs& a, hipStream_t stream) {
  if constexpr (!PER_ELEM) {
    switch (a.fold) {
      case 1: return launch_decode_k<BITS, PER_ELEM, MV, CPL, CPW, 1>(a, stream);
      case 2: return launch_decode_k<BITS, PER_ELEM, MV, CPL, CPW, 2>(a, stream);
      case 4: return launch_decode_k<BITS, PER_ELEM, MV, CPL, CPW, 4>(a, stream);
      default: return hipErrorInvalidValue;
    }
  } else {
    return a.fold == 1 ? launch_decode_k<BITS, PER_ELEM, MV, CPL, CPW, 1>(a, stream) : hipErrorInvalidValue;
  }
}

template <int BITS, bool PER_ELEM, int MV, int CPL>
static hipError_t launch_decode_cpw(const GemmArgs& a, hipStream_t stream) {
  switch (a.cpw) {
    case 8: return launch_decode_fold<BITS, PER_ELEM, MV, CPL, 8>(a, stream);
    case 16: return launch_decode_fold<BITS, PER_ELEM, MV, CPL, 16>(a, stream);
    case 32: return launch_decode_fold<BITS, PER_ELEM, MV, CPL, 32>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS, bool PER_ELEM, int MV>
static hipError_t launch_decode_cpl(const GemmArgs& a, hipStream_t stream) {
  switch (a.cpl) {
    case 1: return launch_decode_cpw<BITS, PER_ELEM, MV, 1>(a, stream);
    case 2: return launch_decode_cpw<BITS, PER_ELEM, MV, 2>(a, stream);
    default: return launch_decode_cpw<BITS, PER_ELEM, MV, 4>(a, stream);
  }
}

template <int BITS, bool PER_ELEM>
static hipError_t launch_decode_pe(const GemmArgs& a, hipStream_t stream) {
  // grouped decode: up to 16 rows per workgroup whatever the total
  return a.M == 1 && a.n_experts == 0 ? launch_decode_cpl<BITS, PER_ELEM, 1>(a, stream)
                                      : launch_decode_cpl<BITS, PER_ELEM, 4>(a, stream);
}

template <int BITS>
static hipError_t launch_decode_bits(bool per_elem, const GemmArgs& a, hipStream_t stream) {
  return per_elem ? launch_decode_pe<BITS, true>(a, stream) : launch_decode_pe<BITS, false>(a, stream);
}

hipError_t launch_decode(int bits, bool per_elem, const GemmArgs& a, hipStream_t stream) {
  switch (bits) {
    case 2: return launch_decode_bits<2>(per_elem, a, stream);
    case 3: return launch_decode_bits<3>(per_elem, a, stream);
    case 4: return launch_decode_bits<4>(per_elem, a, stream);
    default: return launch_decode_bits<8>(per_elem, a, stream);
  }
}

}  // namespace gptq
