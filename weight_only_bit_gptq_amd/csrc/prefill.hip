// Prefill kernel (large M): y[M, N] = x[M, K] . W^[K, N] as a dense MFMA GEMM.
//
// Prefill is compute-bound with 16-bit activations (page "Weight-only INT4
// quantization: GPTQ, AWQ and the Marlin kernel", section 1.2), so this is the
// one place the path is a dense contraction; dequantization runs inside the
// pipeline, in registers, next to the MFMAs (same page, section 6.1).
//
// Tiling: workgroup tile 128 x 256, four waves splitting the 256 columns (no
// two waves dequantize the same weights), wave tile 128 x 64 = four 32-row
// by two 32-column v_mfma_f32_32x32x16_f16 tiles, so every dequantized B
// fragment feeds four MFMAs.  K advances in 64-row tiles; the x tile goes
// global -> registers -> LDS (double buffered, permuted into the unpack's
// field order, XOR-swizzled 16-byte slots), while every lane loads its own
// packed words (one 64-bit load = two adjacent columns) and turns them into
// B operands: unpack_block -> exact (q - z) -> one fp16 multiply by the
// scale, the same bits gptq_dequant produces.
//
// Grid: one workgroup per output tile; when the tile count is a multiple of 8,
// consecutive tiles of the column-major tile order go to the same XCD
// (workgroup ids are dealt round-robin over the 8 XCDs), so an XCD's L2 holds
// a few weight column tiles and the x row tiles they share.
#include "gptq_kernels.hpp"

namespace gptq {

constexpr int kPrefillBM = 128;
constexpr int kPrefillBN = 256;
constexpr int kPrefillBK = 64;
constexpr int kPrefillMS = kPrefillBM / 32;      // 32-row MFMA subtiles per wave

void prefill_shape(int M, int N, int* tiles_m, int* tiles_n) {
  *tiles_m = (M + kPrefillBM - 1) / kPrefillBM;
  *tiles_n = (N + kPrefillBN - 1) / kPrefillBN;
}

// Two workgroups per CU: 256 registers per lane for the 128 accumulators, the
// B and A fragments and the next tile's loads.
template <int BITS, bool PER_ELEM>
__global__ __launch_bounds__(256, 2) void prefill_kernel(GemmArgs a) {
  constexpr int BM = kPrefillBM;
  constexpr int BK = kPrefillBK;
  constexpr int MS = kPrefillMS;
  constexpr int A_PER_THREAD = BM * (BK / 8) / 256;      // 16-byte x pieces per thread per tile
  __shared__ __align__(16) _Float16 a_lds[2][BM * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  int t = blockIdx.x;
  const int ntiles = a.tiles_m * a.tiles_n;
  if ((ntiles & 7) == 0) t = (blockIdx.x & 7) * (ntiles >> 3) + (blockIdx.x >> 3);
  const int tm = t % a.tiles_m, tn = t / a.tiles_m;
  const int m0 = tm * BM;
  const int q = lane & 31;           // A row in a subtile / B column pair
  const int kb2 = lane >> 5;         // 8-row block within a 16-row k step
  const int n = tn * kPrefillBN + wave * 64 + 2 * q;   // this lane's two columns n, n + 1
  const bool col_ok = n < a.N;

  const uint32_t* qw = reinterpret_cast<const uint32_t*>(a.qweight);
  const int ktiles = (a.K + BK - 1) / BK;

  // ---- x tile staging: global -> registers (permuted) -> LDS
  half8_t xr[A_PER_THREAD];
  auto load_x = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_PER_THREAD; ++i) {
      const int e = tid + 256 * i;
      const int m = e >> 3, kblk = e & 7;
      const int row = m0 + m, kk = kt * BK + 8 * kblk;
      half8_t v = {};
      if (row < a.M && kk < a.K) {
        const half8_t raw = *reinterpret_cast<const half8_t*>(a.x + (int64_t)row * a.K + kk);
#pragma unroll
        for (int h = 0; h < 8; ++h) v[h] = raw[Block<BITS>::F[h]];
      }
      xr[i] = v;
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER_THREAD; ++i) {
      const int e = tid + 256 * i;
      const int m = e >> 3, kblk = e & 7;
      *reinterpret_cast<half8_t*>(&a_lds[buf][(m * 8 + (kblk ^ (m & 7))) * 8]) = xr[i];
    }
  };

  // ---- packed weight words of one k tile (4 steps of 16 rows), two columns per load
  u32x2_t w0[4], w1[4];
  auto load_w = [&](int kt) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = kt * BK + 16 * s;
      w0[s] = u32x2_t{0u, 0u};
      w1[s] = w0[s];
      if (col_ok && k < a.K) {
        const int c = k >> 5, kb = 2 * (s & 1) + kb2;
        w0[s] = *reinterpret_cast<const u32x2_t*>(qw + (int64_t)block_row0<BITS>(c, kb) * a.N + n);
        if constexpr (Block<BITS>::LOADS == 2)
          w1[s] = *reinterpret_cast<const u32x2_t*>(qw + (int64_t)block_row1<BITS>(c, kb) * a.N + n);
      }
    }
  };

  // ---- group parameters (fast path: one group per k tile, group_size % 64 == 0)
  uint32_t zg = 0, zg_next = 0;
  half2_t sg = {}, sg_next = {};
  auto load_group = [&](int kt, uint32_t& z2, half2_t& s2) {
    if (col_ok && kt * BK < a.K) {
      const int g = (kt * BK) / a.group_size;
      z2 = load_zero4<BITS>(a.qzeros, a.zrow_words, g, n & ~3) >> (BITS * (n & 3));
      s2 = *reinterpret_cast<const half2_t*>(a.scales + (int64_t)g * a.N + n);
    }
  };

  floatx16_t acc[MS][2];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  load_x(0);
  load_w(0);
  if constexpr (!PER_ELEM) load_group(0, zg, sg);
  store_x(0);
  __syncthreads();

  for (int kt = 0; kt < ktiles; ++kt) {
    const int buf = kt & 1;
    u32x2_t cw0[4], cw1[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) { cw0[s] = w0[s]; cw1[s] = w1[s]; }
    if (kt + 1 < ktiles) {
      load_x(kt + 1);
      load_w(kt + 1);
      if constexpr (!PER_ELEM) load_group(kt + 1, zg_next, sg_next);
    }

    // B operand constants of this tile's group (fast path)
    half2_t negp[2][4], sp[2];
    if constexpr (!PER_ELEM) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int z = field_of4(zg, j, BITS) + a.zero_offset;
        sp[j] = half2_t{sg[j], sg[j]};
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const _Float16 o = neg_offset<BITS>(v, z);
          negp[j][v] = half2_t{o, o};
        }
      }
    }

    const int ksteps = min(4, (a.K - kt * BK) >> 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s >= ksteps) break;
      const int kb = 2 * (s & 1) + kb2;
      const uint32_t sel = block_sel<BITS>(kb);

      half8_t B[2];
      if constexpr (PER_ELEM) {
        const int k0 = kt * BK + 16 * s + 8 * kb2;
        uint32_t z2h[8];
        half2_t s2h[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          z2h[h] = 0;
          s2h[h] = half2_t{};
          if (col_ok) {
            const int g = group_of(a.g_idx, k0 + h, a.group_size, a.G);
            z2h[h] = load_zero4<BITS>(a.qzeros, a.zrow_words, g, n & ~3) >> (BITS * (n & 3));
            s2h[h] = *reinterpret_cast<const half2_t*>(a.scales + (int64_t)g * a.N + n);
          }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t p[4];
          unpack_block<BITS>(cw0[s][j], cw1[s][j], sel, p);
          u32x4_t bw;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int fa = Block<BITS>::F[2 * v], fb = Block<BITS>::F[2 * v + 1];
            const half2_t neg = {neg_offset<BITS>(v, field_of4(z2h[fa], j, BITS) + a.zero_offset),
                                 neg_offset<BITS>(v, field_of4(z2h[fb], j, BITS) + a.zero_offset)};
            bw[v] = as_u32(pair_minus_zero<BITS>(p[v], v, neg) * half2_t{s2h[fa][j], s2h[fb][j]});
          }
          B[j] = __builtin_bit_cast(half8_t, bw);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t p[4];
          unpack_block<BITS>(cw0[s][j], cw1[s][j], sel, p);
          u32x4_t bw;
#pragma unroll
          for (int v = 0; v < 4; ++v) bw[v] = as_u32(pair_minus_zero<BITS>(p[v], v, negp[j][v]) * sp[j]);
          B[j] = __builtin_bit_cast(half8_t, bw);
        }
      }

#pragma unroll
      for (int i = 0; i < MS; ++i) {
        const int m = 32 * i + q;
        const int kblk = 2 * s + kb2;
        const half8_t A = *reinterpret_cast<const half8_t*>(&a_lds[buf][(m * 8 + (kblk ^ (m & 7))) * 8]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B[j], acc[i][j], 0, 0, 0);
      }
    }

    if (kt + 1 < ktiles) {
      store_x(buf ^ 1);
      if constexpr (!PER_ELEM) { zg = zg_next; sg = sg_next; }
    }
    __syncthreads();
  }

  // ---- epilogue: fp32 -> fp16, two adjacent columns per store
  if (!col_ok) return;
#pragma unroll
  for (int i = 0; i < MS; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = m0 + 32 * i + 8 * (v >> 2) + 4 * kb2 + (v & 3);
      if (row < a.M) {
        const half2_t o = {(_Float16)acc[i][0][v], (_Float16)acc[i][1][v]};
        *reinterpret_cast<half2_t*>(a.out + (int64_t)row * a.N + n) = o;
      }
    }
  }
}

template <int BITS, bool PER_ELEM>
static hipError_t launch_prefill_pe(const GemmArgs& a, hipStream_t stream) {
  const dim3 grid(a.tiles_m * a.tiles_n);
  hipLaunchKernelGGL((prefill_kernel<BITS, PER_ELEM>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_prefill_bits(bool per_elem, const GemmArgs& a, hipStream_t stream) {
  return per_elem ? launch_prefill_pe<BITS, true>(a, stream) : launch_prefill_pe<BITS, false>(a, stream);
}

hipError_t launch_prefill(int bits, bool per_elem, const GemmArgs& a, hipStream_t stream) {
  switch (bits) {
    case 2: return launch_prefill_bits<2>(per_elem, a, stream);
    case 3: return launch_prefill_bits<3>(per_elem, a, stream);
    case 4: return launch_prefill_bits<4>(per_elem, a, stream);
    default: return launch_prefill_bits<8>(per_elem, a, stream);
  }
}

}  // namespace gptq
