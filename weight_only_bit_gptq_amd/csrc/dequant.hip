// gptq_dequant: W^[k, n] = fp16((q - z) * s) written as fp16 [K, N].
//
// The "reconstruct" kernel of page "Enhancing vLLM's support for the GPTQv2
// format", section "Adjustment details": one 128-bit load carries the same
// packed word of four adjacent columns, each column gets its own zero point
// (stored value + zero_offset, zero_offset = is_v2 ? 0 : 1), and the fp16 rows
// are written with stride N.  The per-element arithmetic is the one the fused
// GEMM kernels use (unpack_block -> pair_minus_zero -> one fp16 multiply), so
// this bit-exact observable also checks their unpack.
//
// Grid: x = 64-column tiles, y = groups of four 32-row chunks; one wave per
// (chunk, tile); lane = (8-row block kb, column quad).
#include "gptq_kernels.hpp"

namespace gptq {

template <int BITS>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  const int lane = threadIdx.x & 63;
  const int kb = lane >> 4;
  const int col4 = lane & 15;
  const int c = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int n = blockIdx.x * 64 + 4 * col4;
  if (c >= a.chunks || n >= a.N) return;

  const uint32_t* qw = reinterpret_cast<const uint32_t*>(a.qweight);
  const u32x4_t r0 = *reinterpret_cast<const u32x4_t*>(qw + (int64_t)block_row0<BITS>(c, kb) * a.N + n);
  u32x4_t r1 = r0;
  if constexpr (Block<BITS>::LOADS == 2)
    r1 = *reinterpret_cast<const u32x4_t*>(qw + (int64_t)block_row1<BITS>(c, kb) * a.N + n);
  const uint32_t sel = block_sel<BITS>(kb);
  const int k0 = 32 * c + 8 * kb;

  // zero points (4 columns) and scales (4 columns) of each of the block's 8 rows
  uint32_t z4[8];
  half4_t s4[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const int g = group_of(a.g_idx, k0 + h, a.group_size, a.G);
    z4[h] = load_zero4<BITS>(a.qzeros, a.zrow_words, g, n);
    s4[h] = *reinterpret_cast<const half4_t*>(a.scales + (int64_t)g * a.N + n);
  }

  _Float16 w[8][4];   // [field h][column j]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t p[4];
    unpack_block<BITS>(r0[j], r1[j], sel, p);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int fa = Block<BITS>::F[2 * v], fb = Block<BITS>::F[2 * v + 1];
      const half2_t neg = {neg_offset<BITS>(v, field_of4(z4[fa], j, BITS) + a.zero_offset),
                           neg_offset<BITS>(v, field_of4(z4[fb], j, BITS) + a.zero_offset)};
      const half2_t d = pair_minus_zero<BITS>(p[v], v, neg);       // exact q - z
      const half2_t r = d * half2_t{s4[fa][j], s4[fb][j]};          // one rounding
      w[fa][j] = r[0];
      w[fb][j] = r[1];
    }
  }
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const half4_t o = {w[h][0], w[h][1], w[h][2], w[h][3]};
    *reinterpret_cast<half4_t*>(a.out + (int64_t)(k0 + h) * a.N + n) = o;
  }
}

// bfloat16 layer (scales and W^ bfloat16): same grid and loads, the field
// unpack and bfloat16 rounding of the bfloat16 GEMM kernels.  (q - z) s is
// formed as written (the GEMM kernels' fma(q, s, -z s) gives the same value,
// except that an exact zero there is always +0, which no sum can see).
template <int BITS>
__global__ __launch_bounds__(256) void dequant_bf16_kernel(DequantArgs a) {
  const int lane = threadIdx.x & 63;
  const int kb = lane >> 4;
  const int col4 = lane & 15;
  const int c = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int n = blockIdx.x * 64 + 4 * col4;
  if (c >= a.chunks || n >= a.N) return;

  const uint32_t* qw = reinterpret_cast<const uint32_t*>(a.qweight);
  const u32x4_t r0 = *reinterpret_cast<const u32x4_t*>(qw + (int64_t)block_row0<BITS>(c, kb) * a.N + n);
  u32x4_t r1 = r0;
  if constexpr (Block<BITS>::LOADS == 2)
    r1 = *reinterpret_cast<const u32x4_t*>(qw + (int64_t)block_row1<BITS>(c, kb) * a.N + n);
  const int k0 = 32 * c + 8 * kb;
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(a.scales);

  uint32_t w[8][2];   // [row h][column pair]
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const int g = group_of(a.g_idx, k0 + h, a.group_size, a.G);
    const uint32_t z4 = load_zero4<BITS>(a.qzeros, a.zrow_words, g, n);
    const u32x2_t s4 = *reinterpret_cast<const u32x2_t*>(sc + (int64_t)g * a.N + n);
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float f[8];
      block_fields_f32<BITS>(r0[j], r1[j], kb, f);
      const float s = bf16_to_f32((s4[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
      const float z = (float)(field_of4(z4, j, BITS) + a.zero_offset);
      o[j] = (f[h] - z) * s;                     // both steps exact in fp32 (<= 9 + 8 bits)
    }
    w[h][0] = bf16_pair(o[0], o[1]);
    w[h][1] = bf16_pair(o[2], o[3]);
  }
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
  for (int h = 0; h < 8; ++h)
    *reinterpret_cast<u32x2_t*>(out + (int64_t)(k0 + h) * a.N + n) = u32x2_t{w[h][0], w[h][1]};
}

template <int BITS>
static hipError_t launch_dequant_bits(const DequantArgs& a, bool bf16, hipStream_t stream) {
  const dim3 grid((a.N + 63) / 64, (a.chunks + 3) / 4);
  if (bf16) hipLaunchKernelGGL(dequant_bf16_kernel<BITS>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(dequant_kernel<BITS>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dequant(int bits, const DequantArgs& a, bool bf16, hipStream_t stream) {
  switch (bits) {
    case 2: return launch_dequant_bits<2>(a, bf16, stream);
    case 3: return launch_dequant_bits<3>(a, bf16, stream);
    case 4: return launch_dequant_bits<4>(a, bf16, stream);
    default: return launch_dequant_bits<8>(a, bf16, stream);
  }
}

}  // namespace gptq
