// Device-side building blocks shared by the dequant, decode and prefill kernels.
//
// Packed layout (page "Enhancing vLLM's support for the GPTQv2 format",
// sections "Weight quantization of LLMs" and "Adjustment details"): qweight is
// int32 [K*b/32, N], each column's K b-bit fields an LSB-first bitstream, so one
// 128-bit load of row r gives the same packed word of four adjacent columns.
//
// The unit of work is a 32-row chunk c (k in [32c, 32c+32)) split into four
// 8-row blocks kb.  An 8-row block of one column is exactly the B operand one
// lane holds for a gfx950 16x16x32 (or 32x32x16) f16 MFMA: eight k values of
// one column.  The block's eight b-bit fields sit in:
//   b = 2: half (kb & 1) of word 2c + (kb >> 1)
//   b = 3: bits [24kb, 24kb+24) of the 96-bit chunk in words 3c .. 3c+2
//   b = 4: word 4c + kb
//   b = 8: words 8c + 2kb and 8c + 2kb + 1
//
// Fields become fp16 with the exponent trick: OR-ing a field (shifted by s
// bits) into the mantissa of 1024.0 gives exactly 1024 + 2^s * q.  Each 32-bit
// result holds two fields of one column ("magic pair"); the eight halves of a
// block come out in the field order F[] below, with multiplier MUL[v] for the
// pair in register v.  Callers reorder and scale the other MFMA operand (x) to
// match, so no instruction is spent putting fields back in k order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gptq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kMagicPair = 0x64006400u;   // fp16 1024.0 in both halves
constexpr float kMagic = 1024.0f;

// Field order of the eight halves of a block and the power-of-two multiplier of
// each register's pair, per bit width.
template <int BITS> struct Block;
template <> struct Block<2> {
  static constexpr int F[8] = {0, 4, 1, 5, 2, 6, 3, 7};
  static constexpr int MUL[4] = {1, 4, 16, 64};
  static constexpr int LOADS = 1;               // 128-bit qweight rows per block
};
template <> struct Block<3> {
  static constexpr int F[8] = {0, 4, 1, 5, 2, 6, 3, 7};
  static constexpr int MUL[4] = {1, 8, 64, 8};
  static constexpr int LOADS = 2;
};
template <> struct Block<4> {
  static constexpr int F[8] = {0, 4, 1, 5, 2, 6, 3, 7};
  static constexpr int MUL[4] = {1, 16, 1, 16};
  static constexpr int LOADS = 1;
};
template <> struct Block<8> {
  static constexpr int F[8] = {0, 2, 1, 3, 4, 6, 5, 7};
  static constexpr int MUL[4] = {1, 1, 1, 1};
  static constexpr int LOADS = 2;
};

// qweight rows holding block kb of chunk c (second row only for LOADS == 2).
template <int BITS> __device__ __forceinline__ int block_row0(int c, int kb) {
  if constexpr (BITS == 2) return 2 * c + (kb >> 1);
  else if constexpr (BITS == 3) return 3 * c + ((24 * kb) >> 5);
  else if constexpr (BITS == 4) return 4 * c + kb;
  else return 8 * c + 2 * kb;
}
template <int BITS> __device__ __forceinline__ int block_row1(int c, int kb) {
  if constexpr (BITS == 3) { int w = (24 * kb) >> 5; return 3 * c + (w < 2 ? w + 1 : 2); }
  else if constexpr (BITS == 8) return 8 * c + 2 * kb + 1;
  else return block_row0<BITS>(c, kb);
}

// Lane-constant selector for unpack_block: byte selector (b = 2) or funnel
// shift (b = 3); unused otherwise.
template <int BITS> __device__ __forceinline__ uint32_t block_sel(int kb) {
  if constexpr (BITS == 2) return (kb & 1) ? 0x0C030C02u : 0x0C010C00u;
  else if constexpr (BITS == 3) return (uint32_t)((24 * kb) & 31);
  else return 0u;
}

// Eight fields of one column's block -> four magic pairs (see file comment).
// w0 / w1 are the column's words from block_row0 / block_row1.  With
// magic = 0 the pairs are instead the fp16 subnormals MUL * q * 2^-24 (every
// shifted field stays inside the 10 mantissa bits), exact inputs for the
// MFMA, which keeps fp16 subnormals.
template <int BITS>
__device__ __forceinline__ void unpack_block(uint32_t w0, uint32_t w1, uint32_t sel, uint32_t p[4],
                                             uint32_t magic = kMagicPair) {
  if constexpr (BITS == 4) {
    const uint32_t t = w0 >> 8;
    p[0] = (w0 & 0x000F000Fu) | magic;   // f0, f4
    p[1] = (w0 & 0x00F000F0u) | magic;   // 16 f1, 16 f5
    p[2] = (t & 0x000F000Fu) | magic;    // f2, f6
    p[3] = (t & 0x00F000F0u) | magic;    // 16 f3, 16 f7
  } else if constexpr (BITS == 2) {
    // spread the block's two bytes to bytes 0 and 2 (f0..f3 low, f4..f7 high)
    const uint32_t t = __builtin_amdgcn_perm(0u, w0, sel);
    p[0] = (t & 0x00030003u) | magic;    // f0, f4
    p[1] = (t & 0x000C000Cu) | magic;    // 4 f1, 4 f5
    p[2] = (t & 0x00300030u) | magic;    // 16 f2, 16 f6
    p[3] = (t & 0x00C000C0u) | magic;    // 64 f3, 64 f7
  } else if constexpr (BITS == 3) {
    // 24-bit block: f0..f3 in bits 0..11 stay, f4..f7 (bits 12..23) move to 16..27
    const uint32_t s = __builtin_amdgcn_alignbit(w1, w0, sel);
    const uint32_t t = (s & 0x0000FFFFu) | ((s << 4) & 0xFFFF0000u);
    const uint32_t t6 = t >> 6;
    p[0] = (t & 0x00070007u) | magic;    // f0, f4
    p[1] = (t & 0x00380038u) | magic;    // 8 f1, 8 f5
    p[2] = (t & 0x01C001C0u) | magic;    // 64 f2, 64 f6
    p[3] = (t6 & 0x00380038u) | magic;   // 8 f3, 8 f7
  } else {
    p[0] = (w0 & 0x00FF00FFu) | magic;          // f0, f2
    p[1] = ((w0 >> 8) & 0x00FF00FFu) | magic;   // f1, f3
    p[2] = (w1 & 0x00FF00FFu) | magic;          // f4, f6
    p[3] = ((w1 >> 8) & 0x00FF00FFu) | magic;   // f5, f7
  }
}

// Natural-order variant: the eight halves of a block come out as the pairs
// (f0, f1), (f2, f3), (f4, f5), (f6, f7), each half of register v with its
// own power-of-two multiplier MULN<BITS>::LO[v] / HI[v], so that the other
// MFMA operand can be x in its natural k order.
template <int BITS> struct MULN;
template <> struct MULN<2> { static constexpr int LO[4] = {1, 16, 1, 16}, HI[4] = {4, 64, 4, 64}; };
template <> struct MULN<3> { static constexpr int LO[4] = {1, 64, 1, 64}, HI[4] = {1, 64, 1, 64}; };
template <> struct MULN<4> { static constexpr int LO[4] = {1, 1, 1, 1}, HI[4] = {16, 16, 16, 16}; };
template <> struct MULN<8> { static constexpr int LO[4] = {1, 1, 1, 1}, HI[4] = {1, 1, 1, 1}; };

// Byte selector copying byte b of the source into bytes 0 and 2 (zeros elsewhere).
__device__ __forceinline__ uint32_t dup_byte_sel(int b) { return 0x0C000C00u | (uint32_t)b | ((uint32_t)b << 16); }

// `magic` is kMagicPair held in a register the compiler cannot see through,
// so that mask-and-or is one v_and_or_b32 (the mask from a scalar register;
// these VOP3 forms take no literal).
template <int BITS>
__device__ __forceinline__ void unpack_block_natural(uint32_t w0, uint32_t w1, int kb, uint32_t p[4],
                                                     uint32_t kMagicPair) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
      p[v] = (__builtin_amdgcn_perm(0u, w0, dup_byte_sel(v)) & 0x00F0000Fu) | kMagicPair;
  } else if constexpr (BITS == 8) {
    // one byte permute per register: field bytes b, b + 1 of the word into
    // bytes 0 and 2, and the magic's 0x64 (its byte 1, selector 5) into bytes
    // 1 and 3, i.e. the fp16 pair (1024 + f_b, 1024 + f_{b+1})
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t b = 2 * (v & 1);
      p[v] = __builtin_amdgcn_perm(kMagicPair, v < 2 ? w0 : w1, 0x05000500u | b | ((b + 1) << 16));
    }
  } else if constexpr (BITS == 2) {
    const int b0 = 2 * (kb & 1);                 // the block's two bytes: f0..f3, f4..f7
    const uint32_t t0 = __builtin_amdgcn_perm(0u, w0, dup_byte_sel(b0));
    const uint32_t t1 = __builtin_amdgcn_perm(0u, w0, dup_byte_sel(b0 + 1));
    p[0] = (t0 & 0x000C0003u) | kMagicPair;    // f0, 4 f1
    p[1] = (t0 & 0x00C00030u) | kMagicPair;    // 16 f2, 64 f3
    p[2] = (t1 & 0x000C0003u) | kMagicPair;    // f4, 4 f5
    p[3] = (t1 & 0x00C00030u) | kMagicPair;    // 16 f6, 64 f7
  } else {
    // 24-bit block: fields 0..3 in bits 0..11, fields 4..7 in bits 12..23;
    // u = lo12 | lo12 << 13 puts f1 at bits 16..18 and f3 at 22..24
    const uint32_t t = __builtin_amdgcn_alignbit(w1, w0, (uint32_t)((24 * kb) & 31));
    const uint32_t lo = t & 0xFFFu, hi = (t >> 12) & 0xFFFu;
    const uint32_t u0 = lo | (lo << 13), u1 = hi | (hi << 13);
    p[0] = (u0 & 0x00070007u) | kMagicPair;    // f0, f1
    p[1] = (u0 & 0x01C001C0u) | kMagicPair;    // 64 f2, 64 f3
    p[2] = (u1 & 0x00070007u) | kMagicPair;    // f4, f5
    p[3] = (u1 & 0x01C001C0u) | kMagicPair;    // 64 f6, 64 f7
  }
}

// Natural-order magic pair of register v -> exact (q - z) in both halves.
template <int BITS>
__device__ __forceinline__ half2_t pair_minus_zero_natural(uint32_t p, int v, half2_t neg_off) {
  const half2_t inv = {(_Float16)(1.0f / (float)MULN<BITS>::LO[v]), (_Float16)(1.0f / (float)MULN<BITS>::HI[v])};
  return __builtin_bit_cast(half2_t, p) * inv + neg_off;
}

// -(1024 / MUL + z) for both halves of natural register v.
template <int BITS>
__device__ __forceinline__ half2_t neg_offset_natural(int v, int zlo, int zhi) {
  return half2_t{(_Float16)(-(kMagic / (float)MULN<BITS>::LO[v] + (float)zlo)),
                 (_Float16)(-(kMagic / (float)MULN<BITS>::HI[v] + (float)zhi))};
}

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// Magic pair of register v -> exact (q - z) in both halves:
// (1024 + MUL q) / MUL - (1024 / MUL + z); every step is exact in fp16.
template <int BITS>
__device__ __forceinline__ half2_t pair_minus_zero(uint32_t p, int v, half2_t neg_off) {
  const _Float16 inv = (_Float16)(1.0f / (float)Block<BITS>::MUL[v]);
  return as_half2(p) * half2_t{inv, inv} + neg_off;
}

// -(1024 / MUL_v + z) for a zero point z (exact in fp16 for every bit width).
template <int BITS>
__device__ __forceinline__ _Float16 neg_offset(int v, int z) {
  return (_Float16)(-(kMagic / (float)Block<BITS>::MUL[v] + (float)z));
}

// Zero points of the four adjacent columns n .. n+3 (n % 4 == 0) of group row g,
// as four b-bit fields in the low 4b bits of the result.
template <int BITS>
__device__ __forceinline__ uint32_t load_zero4(const int32_t* __restrict__ qzeros, int64_t row_words,
                                               int g, int n) {
  const uint32_t* row = reinterpret_cast<const uint32_t*>(qzeros) + (int64_t)g * row_words;
  if constexpr (BITS == 3) {
    const int base = 3 * (n >> 5);
    const int bit = 3 * (n & 31);
    const int w = bit >> 5;
    const uint32_t lo = row[base + w];
    const uint32_t hi = row[base + (w < 2 ? w + 1 : 2)];
    return __builtin_amdgcn_alignbit(hi, lo, (uint32_t)(bit & 31)) & 0xFFFu;
  } else {
    const int bit = n * BITS;
    const uint32_t word = row[bit >> 5];
    if constexpr (BITS == 8) return word;
    else return (word >> (bit & 31)) & ((1u << (4 * BITS)) - 1u);
  }
}

__device__ __forceinline__ int field_of4(uint32_t z4, int j, int bits) {
  return (int)((z4 >> (bits * j)) & ((1u << bits) - 1u));
}

// ---- bfloat16 activations (the other 16-bit activation type of page
// "Weight-only INT4 quantization: GPTQ, AWQ and the Marlin kernel", section
// 1.2).  bfloat16 has 8 significant bits, too few for the fp16 exponent trick
// (a 4-bit field shifted by 4 would run into the exponent), so these paths
// dequantize element by element in fp32: a field becomes an exact float (a
// byte conversion), W^ = fma(q, s, -z s) is exact in fp32 (q s and z s have
// at most 8 + 9 significant bits, and so does their difference (q - z) s;
// z s stays finite for |s| < 2^119), and one hardware conversion rounds a
// pair to bfloat16, nearest-even -- the same single rounding as
// bf16_RNE((q - z) s), up to the sign of an exact zero (always +0 here).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// The eight fields of one column's block kb as exact floats, natural order
// f[0..7]; w0 / w1 are the column's words from block_row0 / block_row1.
template <int BITS>
__device__ __forceinline__ void block_fields_f32(uint32_t w0, uint32_t w1, int kb, float f[8]) {
  if constexpr (BITS == 4) {
    const uint32_t lo = w0 & 0x0F0F0F0Fu, hi = (w0 >> 4) & 0x0F0F0F0Fu;   // f0 f2 f4 f6 | f1 f3 f5 f7
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = (float)((lo >> (8 * i)) & 0xFFu);
      f[2 * i + 1] = (float)((hi >> (8 * i)) & 0xFFu);
    }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = (float)((w0 >> (8 * i)) & 0xFFu);
      f[4 + i] = (float)((w1 >> (8 * i)) & 0xFFu);
    }
  } else if constexpr (BITS == 2) {
    const uint32_t t = w0 >> (16 * (kb & 1));                               // the block's 16 bits
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t u = (t >> (2 * j)) & 0x0303u;                          // f_j in byte 0, f_{j+4} in byte 1
      f[j] = (float)(u & 0xFFu);
      f[j + 4] = (float)((u >> 8) & 0xFFu);
    }
  } else {
    const uint32_t t = __builtin_amdgcn_alignbit(w1, w0, (uint32_t)((24 * kb) & 31));   // 24-bit block
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)((t >> (3 * i)) & 7u);
  }
}

// A 4-bit block's fields in MFMA register order, for either qweight layout:
// r[2v], r[2v + 1] are the nibbles at bits 4v and 16 + 4v, i.e. fields
// (v, v + 4) of a checkpoint word (the unpack order F) or (2v, 2v + 1) of a
// tiled word, whose fields are stored in pair order.
__device__ __forceinline__ void block4_regs_f32(uint32_t w, float r[8]) {
  // even nibbles (0, 2, 4, 6) and odd nibbles (1, 3, 5, 7) spread to bytes:
  // every field is then one byte-to-float conversion
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t nib[8] = {lo, hi, lo >> 8, hi >> 8, lo >> 16, hi >> 16, lo >> 24, hi >> 24};   // nibble i in byte 0
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    r[2 * v] = (float)(nib[v] & 0xFFu);
    r[2 * v + 1] = (float)(nib[v + 4] & 0xFFu);
  }
}

// Two fp32 values -> a bfloat16 pair (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round-to-nearest-even fp32 -> fp16 with subnormals (hardware conversion).
__device__ __forceinline__ _Float16 f32_to_f16(float f) { return (_Float16)f; }

}  // namespace gptq
