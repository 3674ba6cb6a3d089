// Decode kernel (M <= 16): y[M, N] = x[M, K] . W^[K, N], the memory-bound case
// (page "Weight-only INT4 quantization: GPTQ, AWQ and the Marlin kernel",
// section 1.1: decode reads every weight once per token).
//
// Work split: a wave owns 64 output columns (16 lanes x one 128-bit load of
// four adjacent columns) and a contiguous run of 32-row chunks; the four waves
// of a workgroup split the workgroup's K slice, reduce through LDS, and when K
// is also split across workgroups the last workgroup to finish a column tile
// sums the fp32 partials in a fixed order (deterministic) and writes fp16.
//
// Contraction: one v_mfma_f32_16x16x32_f16 per (chunk, column quad slot j):
// A = 16 rows of x (rows >= M are zero), B = the 8-row block each lane
// unpacked from its word(s).  x is staged once per workgroup in LDS, already
// permuted into the unpack's field order.
//
// Fast path (group_size % 32 == 0, no g_idx): B holds the raw magic pairs
// 1024 + MUL*q, x is pre-divided by MUL, and the zero point and the magic
// offset are removed per group through the accumulator's initial value:
//   acc_g = -(1024 * sum x' + z * sum x' MUL) + sum x' * B = sum x (q - z)
//   y    += s * acc_g                    (s, z constant over a group)
// which is the dequant formula with the scale factored out of the group sum
// (page "Enhancing vLLM's support for the GPTQv2 format", section "Weight
// quantization of LLMs").  Per-element path (act order or small groups): B is
// the exact fp16 dequantized weight, built with each row's own scale and zero.
#include "gptq_kernels.hpp"

namespace gptq {

constexpr int kDecodeThreads = 256;

__host__ __device__ static inline size_t decode_region0(int M, int wg_chunks) {
  const size_t a = (size_t)wg_chunks * 4 * M * 16;   // staged x fragments
  const size_t red = (size_t)4 * M * 64 * 4;          // cross-wave reduction
  return a > red ? a : red;
}

size_t decode_lds_bytes(int M, int wg_chunks, bool per_elem) {
  return decode_region0(M, wg_chunks) + (per_elem ? 0 : (size_t)wg_chunks * M * 8);
}

template <int BITS, bool PER_ELEM, int MV, int U>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int s_is_last;

  const int M = a.M;
  const int tile = blockIdx.x % a.tiles;
  const int split = blockIdx.x / a.tiles;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kb = lane >> 4;          // 8-row block of the chunk (B and A operand)
  const int col4 = lane & 15;        // column quad (B operand / output column)
  const int mA = lane & 15;          // x row held for the A operand
  const int n0 = tile * 64;
  const int n = n0 + 4 * col4;
  const bool col_ok = n < a.N;
  const int cb = split * a.wg_chunks;
  const int ce = min(cb + a.wg_chunks, a.chunks);
  const int nch = ce - cb;
  const int per_wave = a.wg_chunks >> 2;
  const int wb = min(cb + wave * per_wave, ce);
  const int we = min(wb + per_wave, ce);

  _Float16* a_lds = reinterpret_cast<_Float16*>(lds);
  float* corr = reinterpret_cast<float*>(lds + decode_region0(M, a.wg_chunks));

  // ---- stage this workgroup's K slice of x (rows < M), permuted (and scaled)
  for (int e = tid; e < nch * M * 4; e += kDecodeThreads) {
    const int kbe = e & 3;
    const int rest = e >> 2;
    const int m = rest % M;
    const int cl = rest / M;
    const half8_t xv = *reinterpret_cast<const half8_t*>(a.x + (int64_t)m * a.K + 32 * (cb + cl) + 8 * kbe);
    half8_t av;
    float o = 0.f, xs = 0.f;
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const _Float16 xf = xv[Block<BITS>::F[h]];
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
    *reinterpret_cast<half8_t*>(a_lds + (((cl * 4 + kbe) * M + m) << 3)) = av;
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
  __syncthreads();

  const uint32_t sel = block_sel<BITS>(kb);
  const uint32_t* qw = reinterpret_cast<const uint32_t*>(a.qweight);
  floatx4_t accg[4];
  float acc[4][MV];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    accg[j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < MV; ++v) acc[j][v] = 0.f;
  }
  half4_t s4 = {};

  for (int c0 = wb; c0 < we; c0 += U) {
    u32x4_t w0[U], w1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u;
      w0[u] = u32x4_t{0u, 0u, 0u, 0u};
      w1[u] = w0[u];
      if (c < we && col_ok) {
        w0[u] = *reinterpret_cast<const u32x4_t*>(qw + (int64_t)block_row0<BITS>(c, kb) * a.N + n);
        if constexpr (Block<BITS>::LOADS == 2)
          w1[u] = *reinterpret_cast<const u32x4_t*>(qw + (int64_t)block_row1<BITS>(c, kb) * a.N + n);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u;
      if (c >= we) break;
      const int k = 32 * c;
      if constexpr (!PER_ELEM) {
        const int g = k / a.group_size;
        if (c == wb || k % a.group_size == 0) {          // group starts in this wave
          uint32_t z4 = 0;
          if (col_ok) {
            z4 = load_zero4<BITS>(a.qzeros, a.zrow_words, g, n);
            s4 = *reinterpret_cast<const half4_t*>(a.scales + (int64_t)g * a.N + n);
          }
          const int cend = min(we, ((g + 1) * a.group_size) >> 5);
          float O[MV], X[MV];
#pragma unroll
          for (int v = 0; v < MV; ++v) {
            O[v] = 0.f;
            X[v] = 0.f;
            const int m = 4 * kb + v;
            if (m < M) {
              for (int cc = c; cc < cend; ++cc) {
                O[v] += corr[((cc - cb) * M + m) * 2];
                X[v] += corr[((cc - cb) * M + m) * 2 + 1];
              }
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float zj = (float)(field_of4(z4, j, BITS) + a.zero_offset);
#pragma unroll
            for (int v = 0; v < 4; ++v) accg[j][v] = (v < MV) ? -(O[v < MV ? v : 0] + zj * X[v < MV ? v : 0]) : 0.f;
          }
        }
      }

      half8_t A = {};
      if (mA < M) A = *reinterpret_cast<const half8_t*>(a_lds + ((((c - cb) * 4 + kb) * M + mA) << 3));

      if constexpr (PER_ELEM) {
        const int k0 = k + 8 * kb;
        uint32_t z4h[8];
        half4_t s4h[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          z4h[h] = 0;
          s4h[h] = half4_t{};
          if (col_ok) {
            const int g = group_of(a.g_idx, k0 + h, a.group_size, a.G);
            z4h[h] = load_zero4<BITS>(a.qzeros, a.zrow_words, g, n);
            s4h[h] = *reinterpret_cast<const half4_t*>(a.scales + (int64_t)g * a.N + n);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t p[4];
          unpack_block<BITS>(w0[u][j], w1[u][j], sel, p);
          u32x4_t bw;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int fa = Block<BITS>::F[2 * v], fb = Block<BITS>::F[2 * v + 1];
            const half2_t neg = {neg_offset<BITS>(v, field_of4(z4h[fa], j, BITS) + a.zero_offset),
                                 neg_offset<BITS>(v, field_of4(z4h[fb], j, BITS) + a.zero_offset)};
            const half2_t d = pair_minus_zero<BITS>(p[v], v, neg);
            bw[v] = as_u32(d * half2_t{s4h[fa][j], s4h[fb][j]});
          }
          accg[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(half8_t, bw), accg[j], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t p[4];
          unpack_block<BITS>(w0[u][j], w1[u][j], sel, p);
          const u32x4_t bw = {p[0], p[1], p[2], p[3]};
          accg[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(half8_t, bw), accg[j], 0, 0, 0);
        }
        if (c == we - 1 || (k + 32) % a.group_size == 0) {   // group ends in this wave
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float sj = (float)s4[j];
#pragma unroll
            for (int v = 0; v < MV; ++v) acc[j][v] += sj * accg[j][v];
          }
        }
      }
    }
  }

  // ---- reduce the four waves through LDS (rows < M only)
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int v = 0; v < MV; ++v) {
      const int m = 4 * kb + v;
      if (m < M && col_ok) red[(wave * M + m) * 64 + 4 * col4 + j] = PER_ELEM ? accg[j][v] : acc[j][v];
    }
  }
  __syncthreads();

  const int total = M * 64;
  if (a.splits == 1) {
    for (int e = tid; e < total; e += kDecodeThreads) {
      const int m = e >> 6, col = e & 63;
      if (n0 + col < a.N) {
        const float s = red[(0 * M + m) * 64 + col] + red[(1 * M + m) * 64 + col] +
                        red[(2 * M + m) * 64 + col] + red[(3 * M + m) * 64 + col];
        a.out[(int64_t)m * a.N + n0 + col] = (_Float16)s;
      }
    }
    return;
  }

  // ---- split-K: publish this slice's partial tile; the last arrival reduces
  float* part = a.partial + (int64_t)(tile * a.splits + split) * total;
  for (int e = tid; e < total; e += kDecodeThreads) {
    const int m = e >> 6, col = e & 63;
    const float s = red[(0 * M + m) * 64 + col] + red[(1 * M + m) * 64 + col] +
                    red[(2 * M + m) * 64 + col] + red[(3 * M + m) * 64 + col];
    __hip_atomic_store(part + e, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(a.counters + tile, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_is_last = (prev == a.splits - 1);
  }
  __syncthreads();
  if (!s_is_last) return;
  __threadfence();
  const float* base = a.partial + (int64_t)tile * a.splits * total;
  for (int e = tid; e < total; e += kDecodeThreads) {
    const int m = e >> 6, col = e & 63;
    float s = 0.f;
    for (int sp = 0; sp < a.splits; ++sp)
      s += __hip_atomic_load(base + (int64_t)sp * total + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (n0 + col < a.N) a.out[(int64_t)m * a.N + n0 + col] = (_Float16)s;
  }
  if (tid == 0) __hip_atomic_store(a.counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int BITS, bool PER_ELEM, int MV>
static hipError_t launch_decode_mv(const GemmArgs& a, hipStream_t stream) {
  constexpr int U = (Block<BITS>::LOADS == 2) ? 4 : 8;
  const size_t lds = decode_lds_bytes(a.M, a.wg_chunks, PER_ELEM);
  hipLaunchKernelGGL((decode_kernel<BITS, PER_ELEM, MV, U>), dim3(a.tiles * a.splits), dim3(kDecodeThreads),
                     lds, stream, a);
  return hipGetLastError();
}

template <int BITS, bool PER_ELEM>
static hipError_t launch_decode_pe(const GemmArgs& a, hipStream_t stream) {
  switch (a.M) {
    case 1: return launch_decode_mv<BITS, PER_ELEM, 1>(a, stream);
    case 2: return launch_decode_mv<BITS, PER_ELEM, 2>(a, stream);
    case 3: return launch_decode_mv<BITS, PER_ELEM, 3>(a, stream);
    default: return launch_decode_mv<BITS, PER_ELEM, 4>(a, stream);
  }
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
