// Decode kernel (M <= 16): y[M, N] = x[M, K] . W^[K, N], the memory-bound case
// (page "Weight-only INT4 quantization: GPTQ, AWQ and the Marlin kernel",
// section 1.1: decode reads every weight once per token).
//
// Work split.  A workgroup owns a column tile of TN = 16 * CPL columns for the
// whole of K, so no partial sum ever leaves the workgroup: its NW waves split
// K, each wave streams its share of the packed words (lane = one 8-row block
// of CPL adjacent columns, CPL = 1, 2 or 4 words per load), and the waves
// reduce through LDS at the end.  Tile width and wave count are chosen per
// shape so the grid covers all 256 CUs; consecutive tiles are placed on the
// same XCD so neighbouring row pieces share that XCD's L2 lines.
//
// Latency.  Everything a workgroup needs besides its weights is small and is
// staged in LDS by a prologue: x (permuted into the unpack's field order, in
// K-phases when M * K does not fit), the tile's scale/zero table (G x TN), and
// for act order the phase's g_idx slice.  Those loads go out first, then each
// wave fills a ring of two batches of packed words; afterwards every batch
// that is consumed is refilled two batches ahead, so a wave keeps 4-8 KB of
// weights in flight and never waits on a scale or a zero point.
//
// Contraction: one v_mfma_f32_16x16x32_f16 per (32-row chunk, column slot):
// A = 16 rows of x (rows >= M are zero), B = the block each lane unpacked.
//
// Fast path (group_size % 32 == 0, no g_idx): B holds the raw magic pairs
// 1024 + MUL*q, x is pre-divided by MUL, and the zero point and the magic
// offset are removed per group through the accumulator's initial value:
//   acc_g = -(1024 * sum x' + z * sum x' MUL) + sum x' * B = sum x (q - z)
//   y    += s * acc_g                    (s, z constant over a group)
// i.e. the dequant formula with the scale factored out of the group's sum
// (page "Enhancing vLLM's support for the GPTQv2 format", section "Weight
// quantization of LLMs").  Per-element path (act order or small groups): B is
// the exact fp16 dequantized weight, built with each row's own scale and zero.
#include "gptq_kernels.hpp"

namespace gptq {

// chunks per load batch: 16-column tiles load one word per chunk, so they use
// longer batches to keep the same bytes in flight
// (and 64-column tiles of two-word blocks use shorter ones to fit registers;
// 8 * batch * M <= 64 * x pieces keeps a phase's x within the staging registers)
__host__ __device__ constexpr int decode_batch_of(int cpl, int loads, int mv) {
  return cpl == 1 ? (mv <= 2 ? 8 : 4) : (cpl == 4 && loads == 2 ? 2 : 4);
}
// 16-byte x pieces a thread stages per phase (more rows of x -> more pieces)
__host__ __device__ constexpr int decode_x_pieces_of(int mv) { return mv <= 2 ? 4 : 8; }
constexpr int kDecodeGPieces = 4;  // 16-byte g_idx pieces (4 rows) a thread stages per phase
constexpr int kDecodeTQuads = 4;   // scale/zero table quads (4 columns of a group) per thread

template <int CPL> struct WordVec;
template <> struct WordVec<1> { typedef uint32_t T; };
template <> struct WordVec<2> { typedef u32x2_t T; };
template <> struct WordVec<4> { typedef u32x4_t T; };

template <int CPL> __device__ __forceinline__ uint32_t word_of(const typename WordVec<CPL>::T& v, int j) {
  if constexpr (CPL == 1) return v;
  else return v[j];
}

// Zero points of the CPL adjacent columns n .. n+CPL-1 (n % CPL == 0) of group
// row g, as CPL b-bit fields in the low CPL*b bits.
template <int BITS, int CPL>
__device__ __forceinline__ uint32_t load_zeros(const int32_t* __restrict__ qzeros, int64_t row_words, int g, int n) {
  const uint32_t* row = reinterpret_cast<const uint32_t*>(qzeros) + (int64_t)g * row_words;
  constexpr uint32_t mask = (CPL * BITS >= 32) ? 0xFFFFFFFFu : ((1u << (CPL * BITS)) - 1u);
  if constexpr (BITS == 3) {
    const int base = 3 * (n >> 5);
    const int bit = 3 * (n & 31);
    const int w = bit >> 5;
    const uint32_t lo = row[base + w];
    const uint32_t hi = row[base + (w < 2 ? w + 1 : 2)];
    return __builtin_amdgcn_alignbit(hi, lo, (uint32_t)(bit & 31)) & mask;
  } else {
    const int bit = n * BITS;
    return (row[bit >> 5] >> (bit & 31)) & mask;
  }
}

__host__ __device__ inline size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

__host__ __device__ inline DecodeLayout decode_layout(int M, int pc, int nw, int cpl, bool per_elem, int G, int cpg) {
  DecodeLayout L;
  const size_t tn = (size_t)16 * cpl;
  const size_t frag = (size_t)pc * 4 * M * 16;
  L.corr_off = frag;
  const size_t corr = per_elem ? 0 : (size_t)pc * M * 8;
  L.gidx_off = align16(frag + corr);
  const size_t gidx = per_elem ? (size_t)pc * 32 * 2 : 0;
  L.ptab_off = align16(L.gidx_off + gidx);
  L.ptab_rows = per_elem ? 0 : (pc + cpg - 1) / cpg;    // groups a phase covers (fast path)
  L.buf_stride = align16(L.ptab_off + (size_t)L.ptab_rows * tn * 4);
  L.tab_off = 2 * L.buf_stride;                          // whole table (per-element path)
  const size_t tab = per_elem ? (size_t)G * tn * 4 : 0;
  // the phase table is staged in one round; the whole table (per-element path) loops
  L.fits_staging = per_elem || (size_t)L.ptab_rows * tn / 4 <= (size_t)kDecodeTQuads * 64 * nw;
  const size_t data = L.tab_off + tab;
  const size_t red = (size_t)nw * M * tn * 4;
  L.total = data > red ? data : red;
  return L;
}

size_t decode_lds_bytes(int M, int pc, int nw, int cpl, bool per_elem, int G, int cpg) {
  const DecodeLayout L = decode_layout(M, pc, nw, cpl, per_elem, G, cpg);
  return L.fits_staging ? L.total : ~(size_t)0;
}

int decode_max_x_pieces(int M) { return decode_x_pieces_of(M <= 2 ? M : 4); }
int decode_max_g_pieces() { return kDecodeGPieces; }
int decode_max_waves(int) { return 8; }
int decode_batch(int cpl, int bits, int M) {
  return decode_batch_of(cpl, (bits == 3 || bits == 8) ? 2 : 1, M <= 2 ? M : 4);
}

// At most 8 waves per workgroup, so every lane has 256 registers for the
// weight ring, the staging registers and the accumulators.
template <int BITS, bool PER_ELEM, int MV, int CPL>
__global__ __launch_bounds__(512) void decode_kernel(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int U = decode_batch_of(CPL, Block<BITS>::LOADS, MV);
  constexpr int XP = decode_x_pieces_of(MV);
  constexpr int GP = kDecodeGPieces;
  constexpr int TQ = kDecodeTQuads;
  constexpr int TN = 16 * CPL;
  typedef typename WordVec<CPL>::T wvec;

  const int M = a.M;
  const int nthreads = (int)blockDim.x;
  const int nw = nthreads >> 6;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int kb = lane >> 4;          // 8-row block of the chunk (A and B operands)
  const int q = lane & 15;           // column slot (B) and x row (A)
  int t = blockIdx.x;
  if ((a.tiles & 7) == 0) t = (blockIdx.x & 7) * (a.tiles >> 3) + (blockIdx.x >> 3);
  const int n0 = t * TN;
  const int n = n0 + CPL * q;
  const bool col_ok = n < a.N;
  const int C = a.chunks;
  const int pc = a.pc, cpw = a.cpw, phases = a.phases;
  const DecodeLayout lay = decode_layout(M, pc, nw, CPL, PER_ELEM, a.G, a.cpg);

  const uint32_t* qw = reinterpret_cast<const uint32_t*>(a.qweight);
  const uint32_t sel = block_sel<BITS>(kb);

  // ---- prologue loads: x (phase 0), g_idx slice (phase 0), scale/zero table
  half8_t xr[XP];
  const int xpieces = pc * M * 4;
  auto load_x = [&](int p) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int e = tid + i * nthreads;
      xr[i] = half8_t{};
      if (e < xpieces) {
        const int kbe = e & 3, rest = e >> 2;
        const int m = rest % M, cl = rest / M;
        const int c = p * pc + cl;
        if (c < C) xr[i] = *reinterpret_cast<const half8_t*>(a.x + (int64_t)m * a.K + 32 * c + 8 * kbe);
      }
    }
  };
  typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
  i32x4_t gr[PER_ELEM ? GP : 1];
  const int gpieces = pc * 8;                        // 4 rows per piece
  auto load_g = [&](int p) {
    if constexpr (PER_ELEM) {
#pragma unroll
      for (int i = 0; i < GP; ++i) {
        const int e = tid + i * nthreads;
        gr[i] = i32x4_t{0, 0, 0, 0};
        if (e < gpieces) {
          const int k = 32 * p * pc + 4 * e;
          if (k < a.K) {
            if (a.g_idx) gr[i] = *reinterpret_cast<const i32x4_t*>(a.g_idx + k);
            else gr[i] = i32x4_t{k / a.group_size, (k + 1) / a.group_size, (k + 2) / a.group_size,
                                 (k + 3) / a.group_size};
          }
        }
      }
    }
  };
  auto store_xg = [&](int buf) {
    unsigned char* base = lds + (size_t)buf * lay.buf_stride;
    _Float16* frag = reinterpret_cast<_Float16*>(base);
    float* corr = reinterpret_cast<float*>(base + lay.corr_off);
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int e = tid + i * nthreads;
      if (e >= xpieces) continue;                    // xpieces % 4 == 0: groups of four stay together
      const int kbe = e & 3, rest = e >> 2;
      const int m = rest % M, cl = rest / M;
      half8_t av;
      float o = 0.f, xs = 0.f;
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const _Float16 xf = xr[i][Block<BITS>::F[h]];
        if constexpr (PER_ELEM) {
          av[h] = xf;
        } else {
          const float mul = (float)Block<BITS>::MUL[h >> 1];
          const _Float16 xp = (_Float16)((float)xf / mul);
          av[h] = xp;
          o += (float)xp;
          xs += (float)xp * mul;
        }
      }
      *reinterpret_cast<half8_t*>(frag + (((cl * 4 + kbe) * M + m) << 3)) = av;
      if constexpr (!PER_ELEM) {
        o += __shfl_xor(o, 1);
        xs += __shfl_xor(xs, 1);
        o += __shfl_xor(o, 2);
        xs += __shfl_xor(xs, 2);
        if (kbe == 0) {
          corr[(cl * M + m) * 2] = kMagic * o;
          corr[(cl * M + m) * 2 + 1] = xs;
        }
      }
    }
    if constexpr (PER_ELEM) {
      uint16_t* gl = reinterpret_cast<uint16_t*>(base + lay.gidx_off);
#pragma unroll
      for (int i = 0; i < GP; ++i) {
        const int e = tid + i * nthreads;
        if (e < gpieces) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int g = gr[i][r];
            g = g < 0 ? 0 : (g >= a.G ? a.G - 1 : g);
            gl[4 * e + r] = (uint16_t)g;
          }
        }
      }
    }
  };

  // scale/zero table rows [g0, g0 + rows): entry (g, col) = (zero + offset) << 16 |
  // fp16 scale bits, four columns per quad; staged like x (loads, then stores)
  u32x2_t tsr[TQ];
  uint32_t tzr[TQ];
  int tg0 = 0, trows = 0;
  auto load_table = [&](int g0, int rows, int e0) {
    tg0 = g0;
    trows = max(0, min(rows, a.G - g0));
#pragma unroll
    for (int i = 0; i < TQ; ++i) {
      const int e = e0 + tid + i * nthreads;
      tsr[i] = u32x2_t{0u, 0u};
      tzr[i] = 0;
      if (e < trows * (TN / 4)) {
        const int gr_ = e / (TN / 4), c4 = e - gr_ * (TN / 4);
        const int nn = n0 + 4 * c4;
        if (nn < a.N) {
          tsr[i] = *reinterpret_cast<const u32x2_t*>(a.scales + (int64_t)(g0 + gr_) * a.N + nn);
          tzr[i] = load_zeros<BITS, 4>(a.qzeros, a.zrow_words, g0 + gr_, nn);
        }
      }
    }
  };
  auto store_table = [&](uint32_t* tw, int rows, int e0) {  // rows past G are written as zero
#pragma unroll
    for (int i = 0; i < TQ; ++i) {
      const int e = e0 + tid + i * nthreads;
      if (e < rows * (TN / 4)) {
        const int gr_ = e / (TN / 4), c4 = e - gr_ * (TN / 4);
        u32x4_t v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t sb = (j & 1) ? (tsr[i][j >> 1] >> 16) : (tsr[i][j >> 1] & 0xFFFFu);
          const uint32_t z = ((tzr[i] >> (BITS * j)) & ((1u << BITS) - 1u)) + (uint32_t)a.zero_offset;
          v[j] = (z << 16) | sb;
        }
        *reinterpret_cast<u32x4_t*>(tw + gr_ * TN + 4 * c4) = v;
      }
    }
  };

  // ---- packed words: block kb of chunk c lives in rows BITS * c + row0(kb) (+ row1),
  // so a chunk advances every lane's pointer by BITS rows.  Lanes past N read
  // column 0 and slots past K re-read the last chunk: loads stay in bounds
  // without branches and those results are never used.
  const int nc = col_ok ? n : 0;
  const uint32_t* p0 = qw + (int64_t)block_row0<BITS>(0, kb) * a.N + nc;
  const uint32_t* p1 = qw + (int64_t)block_row1<BITS>(0, kb) * a.N + nc;
  const int64_t cstride = (int64_t)BITS * a.N;      // words per chunk
  int lp = 0, li = 0;                                // next chunk to load: phase, index in range
  auto load_batch = [&](wvec* w0, wvec* w1) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(lp * pc + wave * cpw + li, C - 1);
      w0[u] = *reinterpret_cast<const wvec*>(p0 + c * cstride);
      if constexpr (Block<BITS>::LOADS == 2) w1[u] = *reinterpret_cast<const wvec*>(p1 + c * cstride);
      if (++li == cpw) {
        li = 0;
        ++lp;
      }
    }
  };

  // (scale, zero + offset) of column slot j of table row r
  auto group_param = [&](const uint32_t* tab, int r, int j, float& s, int& z) {
    const uint32_t v = tab[r * TN + CPL * q + j];
    s = (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
    z = (int)(v >> 16);
  };

  floatx4_t accg[CPL];
  float acc[CPL][MV];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    accg[j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < MV; ++v) acc[j][v] = 0.f;
  }
  float s_cur[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) s_cur[j] = 0.f;

  // one chunk: c is the chunk, cl its index inside the phase buffer, gi its
  // index inside its group (wave ranges hold whole groups on the fast path)
  const uint32_t* full_tab = reinterpret_cast<const uint32_t*>(lds + lay.tab_off);
  auto compute_chunk = [&](int c, int cl, int gi, const unsigned char* base, uint32_t w0j[CPL], uint32_t w1j[CPL]) {
    const _Float16* frag = reinterpret_cast<const _Float16*>(base);
    half8_t A = {};
    if (q < M) A = *reinterpret_cast<const half8_t*>(frag + (((cl * 4 + kb) * M + q) << 3));

    if constexpr (PER_ELEM) {
      // per-row scale and zero: the block's 8 rows each carry their own group
      const uint16_t* gl = reinterpret_cast<const uint16_t*>(base + lay.gidx_off);
      typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
      const u16x8_t gv = *reinterpret_cast<const u16x8_t*>(gl + 32 * cl + 8 * kb);
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        uint32_t p[4];
        unpack_block<BITS>(w0j[j], w1j[j], sel, p);
        u32x4_t bw;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int fa = Block<BITS>::F[2 * v], fb = Block<BITS>::F[2 * v + 1];
          float sa, sb;
          int za, zb;
          group_param(full_tab, (int)gv[fa], j, sa, za);
          group_param(full_tab, (int)gv[fb], j, sb, zb);
          const half2_t neg = {neg_offset<BITS>(v, za), neg_offset<BITS>(v, zb)};
          const half2_t d = pair_minus_zero<BITS>(p[v], v, neg);
          bw[v] = as_u32(d * half2_t{(_Float16)sa, (_Float16)sb});
        }
        accg[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(half8_t, bw), accg[j], 0, 0, 0);
      }
    } else {
      if (gi == 0) {                                 // a group starts: its scale/zero from the
        const float* corr = reinterpret_cast<const float*>(base + lay.corr_off);   // phase table,
        const uint32_t* ptab = reinterpret_cast<const uint32_t*>(base + lay.ptab_off);  // and the
        const int r = cl / a.cpg;                    // accumulators start at -(correction)
        int z[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) group_param(ptab, r, j, s_cur[j], z[j]);
        float O[MV], X[MV];
#pragma unroll
        for (int v = 0; v < MV; ++v) {
          O[v] = 0.f;
          X[v] = 0.f;
          const int m = 4 * kb + v;
          if (m < M) {
            for (int i = 0; i < a.cpg; ++i) {
              O[v] += corr[((cl + i) * M + m) * 2];
              X[v] += corr[((cl + i) * M + m) * 2 + 1];
            }
          }
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const float zj = (float)z[j];
#pragma unroll
          for (int v = 0; v < 4; ++v) accg[j][v] = (v < MV) ? -(O[v < MV ? v : 0] + zj * X[v < MV ? v : 0]) : 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        uint32_t p[4];
        unpack_block<BITS>(w0j[j], w1j[j], sel, p);
        const u32x4_t bw = {p[0], p[1], p[2], p[3]};
        accg[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(half8_t, bw), accg[j], 0, 0, 0);
      }
      if (gi == a.cpg - 1) {                         // group ends: fold in its scale
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
#pragma unroll
          for (int v = 0; v < MV; ++v) acc[j][v] += s_cur[j] * accg[j][v];
        }
      }
    }
  };

  auto stage_next = [&](int p) {                    // loads for phase p (registers)
    load_x(p);
    load_g(p);
    if constexpr (!PER_ELEM) load_table(p * pc / a.cpg, lay.ptab_rows, 0);
  };
  auto store_stage = [&](int p) {                    // ... and their LDS stores
    store_xg(p & 1);
    if constexpr (!PER_ELEM)
      store_table(reinterpret_cast<uint32_t*>(lds + (size_t)(p & 1) * lay.buf_stride + lay.ptab_off),
                  lay.ptab_rows, 0);
  };
  // One batch: chunks [ci, ci + U) of this wave's range in phase p.  Chunks
  // past K hold zero x and a zero table row, so they add exactly nothing and
  // need no branch.
  auto consume_batch = [&](int p, int ci, const wvec* w0, const wvec* w1) {
    const unsigned char* base = lds + (size_t)(p & 1) * lay.buf_stride;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int cl = wave * cpw + ci + u;
      uint32_t w0j[CPL], w1j[CPL];
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        w0j[j] = word_of<CPL>(w0[u], j);
        w1j[j] = word_of<CPL>(w1[u], j);
      }
      int gi = 0;
      if constexpr (!PER_ELEM) gi = (ci + u) % a.cpg;   // ranges hold whole groups
      compute_chunk(p * pc + cl, cl, gi, base, w0j, w1j);
    }
  };

  // ---- prologue: small operands first, then two batches of weights in flight
  wvec wA0[U], wA1[U], wB0[U], wB1[U];
  if constexpr (PER_ELEM) {                         // whole table, in rounds, before the first barrier
    const int quads = a.G * (TN / 4);
    for (int e0 = 0; e0 < quads; e0 += TQ * nthreads) {
      load_table(0, a.G, e0);
      store_table(const_cast<uint32_t*>(full_tab), a.G, e0);
    }
  }
  stage_next(0);
  load_batch(wA0, wA1);
  load_batch(wB0, wB1);

  // ---- per phase: stage (one barrier), then pairs of batches; every consumed
  // batch is refilled two batches ahead (addresses past K are clamped)
  for (int p = 0; p < phases; ++p) {
    store_stage(p);
    __syncthreads();
    if (p + 1 < phases) stage_next(p + 1);
    for (int ci = 0; ci < cpw; ci += 2 * U) {
      consume_batch(p, ci, wA0, wA1);
      __builtin_amdgcn_sched_barrier(0);
      load_batch(wA0, wA1);
      __builtin_amdgcn_sched_barrier(0);
      consume_batch(p, ci + U, wB0, wB1);
      __builtin_amdgcn_sched_barrier(0);
      load_batch(wB0, wB1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

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
  for (int e = tid; e < M * TN; e += nthreads) {
    const int m = e / TN, col = e - m * TN;
    if (n0 + col < a.N) {
      float s = 0.f;
      for (int w = 0; w < nw; ++w) s += red[(w * M + m) * TN + col];
      a.out[(int64_t)m * a.N + n0 + col] = (_Float16)s;
    }
  }
}

template <int BITS, bool PER_ELEM, int MV, int CPL>
static hipError_t launch_decode_k(const GemmArgs& a, hipStream_t stream) {
  const size_t lds = decode_lds_bytes(a.M, a.pc, a.nw, CPL, PER_ELEM, a.G, a.cpg);
  auto kern = decode_kernel<BITS, PER_ELEM, MV, CPL>;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(a.tiles), dim3(64 * a.nw), lds, stream, a);
  return hipGetLastError();
}

template <int BITS, bool PER_ELEM, int MV>
static hipError_t launch_decode_cpl(const GemmArgs& a, hipStream_t stream) {
  switch (a.cpl) {
    case 1: return launch_decode_k<BITS, PER_ELEM, MV, 1>(a, stream);
    case 2: return launch_decode_k<BITS, PER_ELEM, MV, 2>(a, stream);
    default: return launch_decode_k<BITS, PER_ELEM, MV, 4>(a, stream);
  }
}

template <int BITS, bool PER_ELEM>
static hipError_t launch_decode_pe(const GemmArgs& a, hipStream_t stream) {
  if (a.M == 1) return launch_decode_cpl<BITS, PER_ELEM, 1>(a, stream);
  if (a.M == 2) return launch_decode_cpl<BITS, PER_ELEM, 2>(a, stream);
  return launch_decode_cpl<BITS, PER_ELEM, 4>(a, stream);
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
