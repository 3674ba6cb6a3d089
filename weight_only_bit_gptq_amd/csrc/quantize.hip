// gptq_quantize: min/max round-to-nearest quantization of W [K, N] (fp32) into
// the packed GPTQ tensors (qweight, qzeros, scales).
//
// Formulas (page "Enhancing vLLM's support for the GPTQv2 format", section
// "Weight quantization of LLMs"): scale = (wmax - wmin) / (2^b - 1),
// zero = -round(wmin / scale), q = clamp(round(w / scale) + zero); symmetric
// groups take wmax = -wmin = max|w| and zero = round((2^b - 1) / 2).  Storage
// of the zero (section "From GPTQv1 to GPTQv2"): v2 stores zero, v1 stores
// clamp(zero - 1).  Readings of what the page leaves open: round() is
// round-half-even; zero and q are clamped to [0, 2^b - 1]; the scale is
// computed in fp64, stored as fp16 (nearest-even) and the stored value is the
// one used for zero and q; a stored scale of 0 becomes 1; every division and
// rounding that decides an integer runs in fp64.
//
// Two kernels on the caller's stream:
//   params: one thread per (group, column): min/max over the group's rows,
//           scale, true zero (to a stream-ordered temporary), and the packed
//           stored zeros of the block's 256 columns.
//   pack:   one thread per (32-row chunk, column): the chunk's 32 codes packed
//           LSB-first into b consecutive qweight rows.
#include <hip/hip_runtime.h>

#include "gptq_kernels.hpp"

namespace gptq {

// fp64 -> fp16 bits, round to nearest even, subnormals kept, overflow to inf.
__device__ __forceinline__ uint16_t f64_to_f16_bits(double d) {
  const uint64_t u = (uint64_t)__double_as_longlong(d);
  const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  const int exp = (int)((u >> 52) & 0x7FF);
  const uint64_t mant = u & ((1ull << 52) - 1);
  if (exp == 0x7FF) return sign | 0x7C00u | (mant ? 0x200u : 0u);
  if (exp == 0) return sign;                      // fp64 subnormal: far below fp16 range
  const int e = exp - 1023;
  if (e > 15) return sign | 0x7C00u;
  const uint64_t sig = mant | (1ull << 52);
  const int shift = (e >= -14) ? 42 : 28 - e;     // keep 11 bits, or align to 2^-24
  if (shift >= 64) return sign;
  uint64_t q = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (e >= -14) {
    int he = e + 15;
    if (q == (1ull << 11)) { q = 1ull << 10; ++he; }
    if (he >= 31) return sign | 0x7C00u;
    return (uint16_t)(sign | (he << 10) | (uint16_t)(q & 0x3FF));
  }
  return (uint16_t)(sign | q);                    // q == 1024 is the smallest normal
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  return (double)__builtin_bit_cast(_Float16, h);
}

struct QuantArgs {
  const float* w;          // [K, N]
  const int32_t* g_idx;    // nullable
  int32_t* qweight;        // [K*b/32, N]
  int32_t* qzeros;         // [G, N*b/32]
  uint16_t* scales;        // [G, N] fp16 bits
  uint8_t* zero_tmp;       // [G, N] true zero points
  int N, K, G, group_size, bits, sym, is_v2;
};

__global__ __launch_bounds__(256) void quant_params_kernel(QuantArgs a) {
  __shared__ int32_t gl[256];
  __shared__ uint32_t zs[256];
  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * 256;
  const int n = n0 + tid;
  const int g = blockIdx.y;
  const bool ok = n < a.N;
  const int qmax = (1 << a.bits) - 1;

  float wmin = 0.f, wmax = 0.f;
  bool any = false;
  auto take = [&](int k) {
    if (!ok) return;
    const float v = a.w[(int64_t)k * a.N + n];
    if (!any) { wmin = v; wmax = v; any = true; }
    else { wmin = fminf(wmin, v); wmax = fmaxf(wmax, v); }
  };
  if (a.g_idx) {
    for (int k0 = 0; k0 < a.K; k0 += 256) {
      __syncthreads();
      gl[tid] = (k0 + tid < a.K) ? a.g_idx[k0 + tid] : -1;
      __syncthreads();
      const int kn = min(256, a.K - k0);
      for (int i = 0; i < kn; ++i)
        if (gl[i] == g) take(k0 + i);
    }
  } else {
    for (int k = g * a.group_size; k < (g + 1) * a.group_size; ++k) take(k);
  }

  double lo = (double)wmin, hi = (double)wmax;     // an empty group acts as all-zero
  if (a.sym) {
    const double wabs = fmax(fabs(lo), fabs(hi));
    hi = wabs;
    lo = -wabs;
  }
  uint16_t sbits = f64_to_f16_bits((hi - lo) / (double)qmax);
  if ((sbits & 0x7FFFu) == 0) sbits = 0x3C00u;       // degenerate group: scale 1.0
  const double s = f16_bits_to_f64(sbits);
  int zero;
  if (a.sym) {
    zero = (int)rint((double)qmax / 2.0);
  } else {
    double z = -rint(lo / s);
    z = z < 0.0 ? 0.0 : (z > (double)qmax ? (double)qmax : z);
    zero = (int)z;
  }
  if (ok) {
    a.scales[(int64_t)g * a.N + n] = sbits;
    a.zero_tmp[(int64_t)g * a.N + n] = (uint8_t)zero;
  }
  int stored = a.is_v2 ? zero : zero - 1;
  stored = stored < 0 ? 0 : stored;
  zs[tid] = (uint32_t)stored;
  __syncthreads();

  // pack the stored zeros of this block's columns: word t = stream bits [32t, 32t+32)
  const int ncols = min(256, a.N - n0);
  const int nwords = ncols * a.bits / 32;
  if (tid < nwords) {
    uint32_t word = 0;
    const int bit0 = 32 * tid;
    const int f_first = bit0 / a.bits;
    const int f_last = (bit0 + 31) / a.bits;
    for (int f = f_first; f <= f_last && f < ncols; ++f) {
      const int pos = f * a.bits - bit0;            // may be negative (straddles in from below)
      const uint64_t v = (uint64_t)zs[f];
      word |= (uint32_t)(pos >= 0 ? (v << pos) : (v >> -pos));
    }
    a.qzeros[(int64_t)g * (a.N * a.bits / 32) + (n0 * a.bits) / 32 + tid] = (int32_t)word;
  }
}

__global__ __launch_bounds__(256) void quant_pack_kernel(QuantArgs a) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y;
  if (n >= a.N) return;
  const int qmax = (1 << a.bits) - 1;
  uint32_t words[8] = {0, 0, 0, 0, 0, 0, 0, 0};   // 32 fields * b bits = b words
  for (int i = 0; i < 32; ++i) {
    const int k = 32 * c + i;
    const int g = group_of(a.g_idx, k, a.group_size, a.G);
    const double s = f16_bits_to_f64(a.scales[(int64_t)g * a.N + n]);
    const int zero = a.zero_tmp[(int64_t)g * a.N + n];
    double qd = rint((double)a.w[(int64_t)k * a.N + n] / s) + (double)zero;
    qd = qd < 0.0 ? 0.0 : (qd > (double)qmax ? (double)qmax : qd);
    const uint64_t q = (uint64_t)qd;
    const int bit = i * a.bits;
    const int wi = bit >> 5, off = bit & 31;
    words[wi] |= (uint32_t)(q << off);
    if (off + a.bits > 32) words[wi + 1] |= (uint32_t)(q >> (32 - off));
  }
  for (int i = 0; i < a.bits; ++i) a.qweight[(int64_t)(c * a.bits + i) * a.N + n] = (int32_t)words[i];
}

hipError_t launch_quantize(const float* w, const int32_t* g_idx, int bits, int group_size, int sym, int is_v2,
                           int N, int K, int32_t* qweight, int32_t* qzeros, void* scales, hipStream_t stream) {
  QuantArgs a{};
  a.w = w;
  a.g_idx = g_idx;
  a.qweight = qweight;
  a.qzeros = qzeros;
  a.scales = static_cast<uint16_t*>(scales);
  a.N = N;
  a.K = K;
  a.G = K / group_size;
  a.group_size = group_size;
  a.bits = bits;
  a.sym = sym;
  a.is_v2 = is_v2;
  hipError_t err = hipMallocAsync(reinterpret_cast<void**>(&a.zero_tmp), (size_t)a.G * N, stream);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(quant_params_kernel, dim3((N + 255) / 256, a.G), dim3(256), 0, stream, a);
  err = hipGetLastError();
  if (err == hipSuccess) {
    hipLaunchKernelGGL(quant_pack_kernel, dim3((N + 255) / 256, K / 32), dim3(256), 0, stream, a);
    err = hipGetLastError();
  }
  const hipError_t ferr = hipFreeAsync(a.zero_tmp, stream);
  return err != hipSuccess ? err : ferr;
}

// ---------------------------------------------------------------------------
// Zero-point format conversion (page "Enhancing vLLM's support for the GPTQv2
// format", section "From GPTQv1 to GPTQv2"): GPTQv1 stores clamp(zero - 1) and
// adds 1 at run time, GPTQv2 stores the zero itself.  v1 -> v2 adds 1 to every
// stored field, v2 -> v1 subtracts 1 clamped at 0.  A v1 field of 2^b - 1 (a
// zero of 2^b, which no v1 writer produces) has no v2 encoding and saturates to
// 2^b - 1; a v2 zero of 0 becomes the v1 field 0 (run-time zero 1).  Both are
// counted as lossy.
//
// One thread per unit of whole fields: one word for b in {2, 4, 8}, the three
// words of a 32-field chunk for b = 3 (fields 10 and 21 straddle words).  Rows
// hold N*b/32 words with N % 32 == 0, so units never cross a row and the
// tensor is converted as one flat array.  A thread reads all of its words
// before writing them, so in == out is allowed.

template <int BITS>
__device__ __forceinline__ uint32_t convert_field(uint32_t f, int to_v2, int* lossy) {
  constexpr uint32_t kMax = (1u << BITS) - 1u;
  if (to_v2) {
    *lossy += (f == kMax);
    return f == kMax ? kMax : f + 1u;
  }
  *lossy += (f == 0u);
  return f == 0u ? 0u : f - 1u;
}

template <int BITS>
__global__ void __launch_bounds__(256) convert_zeros_kernel(const int32_t* __restrict__ in, int32_t* out,
                                                            int64_t units, int to_v2, int32_t* lossy_count) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int lossy = 0;
  if (u < units) {
    if constexpr (BITS == 3) {
      const uint32_t w0 = (uint32_t)in[3 * u], w1 = (uint32_t)in[3 * u + 1], w2 = (uint32_t)in[3 * u + 2];
      const uint64_t lo = (uint64_t)w0 | ((uint64_t)w1 << 32);
      uint64_t olo = 0;
      uint32_t ohi = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int p = 3 * i;  // bit position in the 96-bit chunk
        uint32_t f;
        if (p + 3 <= 64) f = (uint32_t)(lo >> p) & 7u;
        else if (p >= 64) f = (w2 >> (p - 64)) & 7u;
        else f = (uint32_t)(lo >> p) | ((w2 << (64 - p)) & 7u);
        const uint32_t g = convert_field<3>(f, to_v2, &lossy);
        if (p + 3 <= 64) olo |= (uint64_t)g << p;
        else if (p >= 64) ohi |= g << (p - 64);
        else { olo |= (uint64_t)g << p; ohi |= g >> (64 - p); }
      }
      out[3 * u] = (int32_t)(uint32_t)olo;
      out[3 * u + 1] = (int32_t)(uint32_t)(olo >> 32);
      out[3 * u + 2] = (int32_t)ohi;
    } else {
      const uint32_t w = (uint32_t)in[u];
      uint32_t o = 0;
#pragma unroll
      for (int i = 0; i < 32 / BITS; ++i)
        o |= convert_field<BITS>((w >> (BITS * i)) & ((1u << BITS) - 1u), to_v2, &lossy) << (BITS * i);
      out[u] = (int32_t)o;
    }
  }
  if (lossy_count) {
    // wave sum, then one vector atomic per wave
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lossy += __shfl_xor(lossy, off, 64);
    if ((threadIdx.x & 63) == 0 && lossy) atomicAdd(lossy_count, lossy);
  }
}

hipError_t launch_convert_zeros(const int32_t* in, int32_t* out, int bits, int64_t G, int64_t N, int to_v2,
                                int32_t* lossy_count, hipStream_t stream) {
  const int64_t words = G * (N * bits / 32);
  const int64_t units = bits == 3 ? words / 3 : words;
  const dim3 grid((unsigned)((units + 255) / 256)), block(256);
  switch (bits) {
    case 2: hipLaunchKernelGGL(convert_zeros_kernel<2>, grid, block, 0, stream, in, out, units, to_v2, lossy_count); break;
    case 3: hipLaunchKernelGGL(convert_zeros_kernel<3>, grid, block, 0, stream, in, out, units, to_v2, lossy_count); break;
    case 4: hipLaunchKernelGGL(convert_zeros_kernel<4>, grid, block, 0, stream, in, out, units, to_v2, lossy_count); break;
    default: hipLaunchKernelGGL(convert_zeros_kernel<8>, grid, block, 0, stream, in, out, units, to_v2, lossy_count); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// qweight re-layout.  Checkpoint layout: int32 [K*b/32, N] (packed row r,
// column n).  Tiled layout: int32 [N/16][K/32][b][16]: word (t, c, r, j) is
// packed row c*b + r of column 16 t + j, so a 16-column tile's words are one
// contiguous run, chunk (32 rows of K) after chunk.  2/3/8-bit words move
// unchanged; 4-bit words also get their fields in pair order (below).
// One thread per word of the tiled array (its writes coalesce; its reads are
// 64-byte pieces of checkpoint rows).
// 4-bit words of the tiled layout hold their eight fields in pair order:
// field 2i in nibble i and field 2i + 1 in nibble i + 4 (i < 4), so that one
// mask per 16-bit half gives two consecutive fields.  to_pairs = 0 inverts.
__device__ __forceinline__ uint32_t pair_order_nibbles(uint32_t w, int to_pairs) {
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int f = i < 4 ? 2 * i : 2 * (i - 4) + 1;  // field held by tiled nibble i
    if (to_pairs) out |= ((w >> (4 * f)) & 0xFu) << (4 * i);
    else out |= ((w >> (4 * i)) & 0xFu) << (4 * f);
  }
  return out;
}

__global__ void __launch_bounds__(256) repack_kernel(const int32_t* __restrict__ in, int32_t* __restrict__ out,
                                                     int bits, int64_t N, int64_t K, int to_tiled) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;     // tiled index
  const int64_t rows = K / 32 * bits;
  if (i >= rows * N) return;
  const int64_t j = i & 15;
  const int64_t rest = i >> 4;                     // (t * (K/32) + c) * bits + r
  const int64_t cr = rest % rows;                  // c * bits + r: the packed row
  const int64_t t = rest / rows;
  const int64_t src = cr * N + 16 * t + j;         // checkpoint index
  if (to_tiled) out[i] = bits == 4 ? (int32_t)pair_order_nibbles((uint32_t)in[src], 1) : in[src];
  else out[src] = bits == 4 ? (int32_t)pair_order_nibbles((uint32_t)in[i], 0) : in[i];
}

hipError_t launch_repack(const int32_t* in, int32_t* out, int bits, int64_t N, int64_t K, int to_tiled,
                         hipStream_t stream) {
  const int64_t words = K / 32 * bits * N;
  hipLaunchKernelGGL(repack_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream, in, out, bits, N, K,
                     to_tiled);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Act-order row sort.  perm[i] is the original row of sorted row i (rows
// ordered by group).  One thread per (32-row chunk of the sorted layer,
// column): it gathers the 32 fields of rows perm[32c .. 32c + 32) of its
// column from the packed checkpoint layout and packs them into the chunk's
// BITS words.  Reads are scattered; this runs once per layer.
template <int BITS>
__device__ __forceinline__ uint32_t field_of_row(const uint32_t* __restrict__ q, int64_t N, int64_t n, int r) {
  if constexpr (BITS == 3) {
    const int c = r >> 5, f = r & 31;                      // chunk, field: bit 3f of the chunk's 96 bits
    const int w = 3 * c + ((3 * f) >> 5), off = (3 * f) & 31;
    uint32_t v = q[(int64_t)w * N + n] >> off;
    if (off > 29) v |= q[(int64_t)(w + 1) * N + n] << (32 - off);
    return v & 7u;
  } else {
    constexpr int PER = 32 / BITS;
    return (q[(int64_t)(r / PER) * N + n] >> (BITS * (r % PER))) & ((1u << BITS) - 1u);
  }
}

template <int BITS>
__global__ void __launch_bounds__(256) sort_rows_kernel(const int32_t* __restrict__ in, const int32_t* __restrict__ perm,
                                                        int32_t* __restrict__ out, int64_t N, int chunks) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y;
  if (n >= N || c >= chunks) return;
  const uint32_t* q = reinterpret_cast<const uint32_t*>(in);
  uint32_t w[BITS];
#pragma unroll
  for (int i = 0; i < BITS; ++i) w[i] = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t f = field_of_row<BITS>(q, N, n, perm[32 * c + i]);
    const int bit = BITS * i;                              // LSB-first stream of the chunk
    w[bit >> 5] |= f << (bit & 31);
    if ((bit & 31) + BITS > 32) w[(bit >> 5) + 1] |= f >> (32 - (bit & 31));
  }
#pragma unroll
  for (int i = 0; i < BITS; ++i) out[((int64_t)c * BITS + i) * N + n] = (int32_t)w[i];
}

hipError_t launch_sort_rows(const int32_t* in, const int32_t* perm, int32_t* out, int bits, int64_t N, int64_t K,
                            hipStream_t stream) {
  const dim3 grid((unsigned)((N + 255) / 256), (unsigned)(K / 32)), block(256);
  const int chunks = (int)(K / 32);
  switch (bits) {
    case 2: hipLaunchKernelGGL(sort_rows_kernel<2>, grid, block, 0, stream, in, perm, out, N, chunks); break;
    case 3: hipLaunchKernelGGL(sort_rows_kernel<3>, grid, block, 0, stream, in, perm, out, N, chunks); break;
    case 4: hipLaunchKernelGGL(sort_rows_kernel<4>, grid, block, 0, stream, in, perm, out, N, chunks); break;
    default: hipLaunchKernelGGL(sort_rows_kernel<8>, grid, block, 0, stream, in, perm, out, N, chunks); break;
  }
  return hipGetLastError();
}

// x gathered into the sorted row order: xg[m, i] = x[m, perm[i]].  One thread
// per 8 consecutive i (one 16-byte store).
__global__ void __launch_bounds__(256) gather_cols_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
                                                          uint16_t* __restrict__ xg, int64_t M, int64_t K) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (m, i / 8)
  const int64_t per_row = K / 8;
  if (t >= M * per_row) return;
  const int64_t m = t / per_row, i0 = (t - m * per_row) * 8;
  typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
  u16x8_t v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = x[m * K + perm[i0 + j]];
  *reinterpret_cast<u16x8_t*>(xg + m * K + i0) = v;
}

hipError_t launch_gather_cols(const void* x, const int32_t* perm, void* xg, int64_t M, int64_t K, hipStream_t stream) {
  const int64_t threads = M * (K / 8);
  hipLaunchKernelGGL(gather_cols_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), perm, static_cast<uint16_t*>(xg), M, K);
  return hipGetLastError();
}

// Zero `words` 32-bit words (a fill kernel rather than hipMemsetAsync, so the
// clear is an ordinary kernel node when the caller captures the stream).
__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* __restrict__ p, int64_t words) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < words) p[i] = 0u;
}

hipError_t launch_zero_words(void* p, int64_t words, hipStream_t stream) {
  if (words <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                     static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace gptq
