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
// fragment feeds four MFMAs.  K advances in 64-row tiles.
//
// Pipeline, two tiles deep: x tiles go from global memory straight into LDS
// (buffer loads with the LDS destination, three stages, XOR-swizzled 16-byte
// slots, no registers), the packed words of a tile into one of three
// register sets (one 64-bit load = two adjacent columns); at the start of tile
// kt the loads of tile kt + 2 are issued.  Every load is a buffer load:
// offsets past the tensor read zero without touching memory, so the loop has
// no branch around a load and every wait is exact.  B operands: the
// natural-order unpack (x needs no permutation) -> exact (q - z) -> one fp16
// multiply by the scale, the same bits gptq_dequant produces.
//
// Grid: one workgroup per output tile; when the tile count is a multiple of 8,
// consecutive tiles of the column-major tile order go to the same XCD
// (workgroup ids are dealt round-robin over the 8 XCDs), so an XCD's L2 holds
// a few weight column tiles and the x row tiles they share.  A grid of few
// tiles (small M) splits K: ks workgroups per tile store fp32 partial sums
// and a second, chip-wide kernel adds them in split order.
#include <type_traits>

#include "gptq_kernels.hpp"

namespace gptq {

constexpr int kPrefillBN = 256;
constexpr int kPrefillBK = 64;
constexpr int kPrefillStages = 3;                 // x tiles in LDS: current + two in flight
// Rows per workgroup tile: 128 (two workgroups per CU, each dequantized B
// fragment feeds four MFMAs), or 256 (a wave tile of 256 x 64: each B fragment
// feeds eight MFMAs, the 256 accumulators per lane fill the accumulation
// registers, one workgroup per CU).  Measured on MI355X (70B-MLP shapes, M =
// 2048, 4-bit): 256 rows win when all their tiles run in one round on the 256
// CUs (28672 -> 8192: 1159 -> 1207 TFLOP/s) but lose when the grid takes
// several rounds, whose last one runs partly empty and, at one workgroup per
// CU, exposes every workgroup's prologue and epilogue (8192 -> 28672: 1160 ->
// 1107).  8-bit takes them with its pipelined body, which only they hold
// without spills (28672 -> 8192: 993 -> 1042, 8192 -> 8192: 1009 -> 1083
// TFLOP/s against the 128-row tile's plain body).  They also lose when their one round leaves many CUs idle: 4096 -> 4096 at M =
// 1024 .. 2048 (64 .. 128 tiles) and 11008 -> 4096 ran at 340-710 TFLOP/s, so
// they are taken only with at least 3/4 of the CUs busy.
constexpr int kPrefillCUs = 256;

// Up to 64 rows: 32- or 64-row tiles, so that the MFMAs of rows past M are
// not computed (a k tile's dequant is the same, its MFMAs a quarter or half).
void prefill_shape(int M, int N, bool big_ok, int* tiles_m, int* tiles_n, int* bm) {
  const int64_t big_tiles = (int64_t)((M + 255) / 256) * ((N + kPrefillBN - 1) / kPrefillBN);
  *bm = (big_ok && M >= 1024 && big_tiles <= kPrefillCUs && 4 * big_tiles >= 3 * kPrefillCUs) ? 256 : 128;
  if (M <= 64) *bm = M <= 32 ? 32 : 64;
  *tiles_m = (M + *bm - 1) / *bm;
  *tiles_n = (N + kPrefillBN - 1) / kPrefillBN;
}

// Two workgroups per CU: 256 registers per lane for the 128 accumulators, the
// B and A fragments and three tiles of packed words.
// FULL (fast path, K % 64 == 0): every k tile has its four 16-row steps and
// runs the software-pipelined tile body; otherwise (act order, other group
// sizes, a last half tile) the plain body with a step count per tile.  Two
// separate instantiations: one body with both paths behind a branch spills.
// BF16: x, scales and out are bfloat16; B is the element-wise bfloat16
// dequant of gptq_device.hpp and the MFMA the bf16 one (same tiles).
// PAIRS (4-bit, tiled layout): the words hold their fields in pair order, so
// one shift and four mask-ors make the four registers (fields 2v, 2v + 1,
// multiplier 1, 16, 1, 16 for both halves) instead of four byte permutes.
template <int BITS, bool PER_ELEM, bool FULL, bool BF16, bool PAIRS, int BM>
__device__ __forceinline__ void prefill_body(GemmArgs a) {
  static_assert(!PAIRS || BITS == 4, "pair-order words: 4-bit");
  static_assert(BM == 32 || BM == 64 || BM == 128 || BM == 256, "workgroup tile rows");
  constexpr int BK = kPrefillBK;
  constexpr int MS = BM / 32;                       // 32-row MFMA subtiles per wave
  constexpr int NST = kPrefillStages;
  constexpr int L = Block<BITS>::LOADS;
  constexpr int XI = BM * (BK / 8) / 256;          // 16-byte x pieces per thread (per wave: XI loads of 1 KB)
  // three separate arrays (not one indexed by a runtime stage), so that the
  // compiler can tell the stages apart and does not wait for the x tiles in
  // flight before reading the current one
  __shared__ __align__(16) _Float16 a_lds0[BM * BK];
  __shared__ __align__(16) _Float16 a_lds1[BM * BK];
  __shared__ __align__(16) _Float16 a_lds2[BM * BK];
  auto stage_lds = [&](auto st_c) __attribute__((always_inline)) -> _Float16* {
    constexpr int st = decltype(st_c)::value % NST;
    if constexpr (st == 0) return a_lds0;
    else if constexpr (st == 1) return a_lds1;
    else return a_lds2;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // workgroup -> tile t (column-major over tiles_m x tiles_n); a grouped launch
  // first picks the expert (ntiles workgroups each), a split-K launch the
  // split sk of K (ks consecutive workgroups per tile)
  const int ntiles = a.tiles_m * a.tiles_n;
  const int ks = (BM > 128 || a.n_experts > 0) ? 1 : max(a.ks, 1);   // tiles of up to 128 rows
  int b = blockIdx.x, e = 0, sk = 0;
  if (a.n_experts > 0) {
    e = b / ntiles;
    b -= e * ntiles;
  } else if (ks > 1) {
    sk = b % ks;
    b /= ks;
  }
  int t = b;
  if ((ntiles & 7) == 0) t = (b & 7) * (ntiles >> 3) + (b >> 3);
  const int tm = t % a.tiles_m, tn = t / a.tiles_m;
  int m0 = tm * BM;
  if (a.n_experts > 0) {
    // grouped (mixture-of-experts) prefill: expert e owns rows [moe_off[e],
    // moe_off[e + 1]) of x and out (clamped to [0, M], and to its first
    // moe_rows) and its own weights; row tile tm is rows tm BM .. of those, a
    // tile past them leaves at once.
    // x and out are moved to the tile's first row, M becomes its row count,
    // so the body below runs unchanged on a tile at row 0.
    const int e0 = min(max(a.moe_off[e], 0), a.M);
    const int r_end = min(min(max(a.moe_off[e + 1], 0), a.M), e0 + min(a.moe_rows, a.M));
    const int r0 = e0 + m0;
    const int rows = min(BM, r_end - r0);
    if (rows <= 0) return;
    a.M = rows;
    a.x += (int64_t)r0 * a.K;
    a.out += (int64_t)r0 * a.N;
    a.qweight += e * a.qw_stride;
    a.qzeros += e * a.qz_stride;
    a.scales += e * a.sc_stride;
    if (a.g_idx) a.g_idx += e * a.gi_stride;
    m0 = 0;
  }
  const int q = lane & 31;           // A row in a subtile / B column pair
  const int kb2 = lane >> 5;         // 8-row block within a 16-row k step
  const int n = tn * kPrefillBN + wave * 64 + 2 * q;   // this lane's two columns n, n + 1
  const bool col_ok = n < a.N;
  const int nc = col_ok ? n : 0;
  // this workgroup's k tiles: [kt0, kt0 + ktiles) of the whole K (a split
  // covers cks chunks, an even count, the last split the rest)
  const int ktiles_all = (a.K + BK - 1) / BK;
  const int kt0 = ks > 1 ? sk * (a.cks / 2) : 0;
  const int ktiles = ks > 1 ? min(a.cks / 2, ktiles_all - kt0) : ktiles_all;

  // ---- x tiles: slot s = m * 8 + (kblk ^ ((m >> 1) & 7)) of a stage holds
  // x[m0 + m, 8 kblk .. 8 kblk + 8) of the tile.  The swizzle puts the 16
  // rows one 128-bit LDS read serves per cycle (16 lanes) in 16 different
  // 16-byte bank groups of gfx950's 64 banks (rows m and m + 1 sit 128 bytes
  // apart, so only every other row needs a distinct column block).  Load i of wave w fills slots
  // (4 w + i) * 64 + lane, so each lane fetches the piece that lands there.
  // Rows past M read zero (past the end of x); k past K is never used.
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16*>(a.x), (short)0, (int)((uint32_t)a.M * (uint32_t)a.K * 2u), 0x00020000);
  uint32_t xoff[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int s = (XI * wave + i) * 64 + lane;
    const int m = s >> 3, kblk = (s & 7) ^ ((m >> 1) & 7);
    xoff[i] = ((uint32_t)(m0 + m) * (uint32_t)a.K + 8u * kblk) * 2u;
    // rows past M: an offset past the end of x (plus at most the K bytes of
    // a tile offset it stays past it, or wraps to valid data of row 0); such
    // rows only feed output rows that are never stored
    if (m0 + m >= a.M) xoff[i] = 0xF0000000u;
  }
  // Tiles past this workgroup's last (the loop runs in threes) load from
  // offsets past the end of x and of qweight: they read zero without a
  // memory access, so the step that waits for them does not wait for memory
  // (their stage and registers are never used).
  // x holds M K < 2^31 elements, K % 32 == 0: at most 2^32 - 64 bytes;
  // qweight N K b / 8 < 2^31 bytes
  constexpr uint32_t kPastEndX = 0xFFFFFFF0u, kPastEnd = 0x80000000u;
  auto load_x = [&](int kt, auto st_c) __attribute__((always_inline)) {
    _Float16* sl = stage_lds(st_c);
    const bool live = kt < ktiles;
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrsrc, (__attribute__((address_space(3))) void*)(sl + (XI * wave + i) * 64 * 8), 16,
          live ? xoff[i] + (uint32_t)(kt0 + kt) * BK * 2u : kPastEndX, 0, 0, 0);
    }
  };

  // ---- packed words of a tile (4 steps of 16 rows), three register sets
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(a.qweight), (short)0, (int)((uint32_t)(a.K / 32 * BITS) * (uint32_t)a.N * 4u), 0x00020000);
  // three register sets on the fast path (tiles kt, kt + 1, kt + 2); the
  // per-element path, whose scale/zero lookups need the registers, keeps one
  constexpr int NSR = PER_ELEM ? 1 : NST;
  u32x2_t w0[NSR][4], w1[NSR][L == 2 ? 4 : 1];
  // byte offsets of the lane's words for the 4 steps of tile 0; a tile is
  // BK * BITS / 32 packed rows further on.  A packed row is N * 4 bytes in
  // the checkpoint layout; in the tiled one it is 64 bytes (16 columns) and
  // column n sits in tile n / 16, which starts at (n / 16) * chunks * BITS * 64.
  const uint32_t wrow = a.wtiled ? 64u : (uint32_t)a.N * 4u;
  const uint32_t wcol = a.wtiled ? (uint32_t)(nc >> 4) * (uint32_t)a.chunks * (uint32_t)BITS * 64u +
                                       (uint32_t)(nc & 15) * 4u
                                 : (uint32_t)nc * 4u;
  const uint32_t tile_bytes = (uint32_t)(BK / 32 * BITS) * wrow;
  uint32_t woff0[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = (16 * s) >> 5, kb = 2 * (s & 1) + kb2;
    woff0[s] = (uint32_t)block_row0<BITS>(c, kb) * wrow + wcol;
  }
  // second word of a two-word block: (row1 - row0) rows further on
  auto woff1 = [&](int s) __attribute__((always_inline)) {
    const int c = (16 * s) >> 5, kb = 2 * (s & 1) + kb2;
    return woff0[s] + (uint32_t)(block_row1<BITS>(c, kb) - block_row0<BITS>(c, kb)) * wrow;
  };
  // the tile's group parameters (fast path: one group per k tile) travel with
  // its words, so waiting for a tile never waits for a newer load
  uint32_t zw0[NSR], zw1[NSR];
  half2_t sw[NSR];
  const uint32_t* qzr = reinterpret_cast<const uint32_t*>(a.qzeros);
  auto load_w = [&](int kt, auto set_c) __attribute__((always_inline)) {
    constexpr int set = decltype(set_c)::value % NSR;
    if constexpr (!PER_ELEM) {
      const int g = min(((kt0 + kt) * BK) / a.group_size, a.G - 1);
      const uint32_t* zrow = qzr + (int64_t)g * a.zrow_words;
      const int n4 = nc & ~3;
      if constexpr (BITS == 3) {
        const int w = 3 * (n4 >> 5) + ((3 * (n4 & 31)) >> 5);
        zw0[set] = zrow[w];
        zw1[set] = zrow[((3 * (n4 & 31)) >> 5) < 2 ? w + 1 : w];
      } else {
        zw0[set] = zrow[(n4 * BITS) >> 5];
      }
      sw[set] = *reinterpret_cast<const half2_t*>(a.scales + (int64_t)g * a.N + nc);
    }
    // rows past K lie past the end of qweight and read zero; tiles past this
    // workgroup's last read nothing (see load_x)
    const bool live = kt < ktiles;
    const uint32_t tile_off = (uint32_t)(kt0 + kt) * tile_bytes;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      w0[set][s] = __builtin_amdgcn_raw_buffer_load_b64(wrsrc, (int)(live ? woff0[s] + tile_off : kPastEnd), 0, 0);
      if constexpr (L == 2)
        w1[set][s] = __builtin_amdgcn_raw_buffer_load_b64(wrsrc, (int)(live ? woff1(s) + tile_off : kPastEnd), 0, 0);
    }
  };

  uint32_t magic;                                    // kMagicPair in a register (see unpack_block_natural)
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));
  // a block's four magic pairs, each pair (fields 2v, 2v + 1) -> exact (q - z),
  // and the offsets -(1024 / MUL + z) of both halves of register v
  auto unpack_B = [&](uint32_t w0v, uint32_t w1v, int kb, uint32_t p[4]) __attribute__((always_inline)) {
    if constexpr (PAIRS) unpack_block<4>(w0v, 0u, 0u, p, magic);
    else unpack_block_natural<BITS>(w0v, w1v, kb, p, magic);
  };
  auto minus_zero = [](uint32_t pv, int v, half2_t neg) __attribute__((always_inline)) {
    if constexpr (PAIRS) return pair_minus_zero<4>(pv, v, neg);
    else return pair_minus_zero_natural<BITS>(pv, v, neg);
  };
  auto neg_off = [](int v, int zlo, int zhi) __attribute__((always_inline)) {
    if constexpr (PAIRS) return half2_t{neg_offset<4>(v, zlo), neg_offset<4>(v, zhi)};
    else return neg_offset_natural<BITS>(v, zlo, zhi);
  };
  auto mfma = [](const half8_t& A, const half8_t& B, const floatx16_t& c) __attribute__((always_inline)) {
    if constexpr (BF16)
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, A), __builtin_bit_cast(bf16x8_t, B),
                                                     c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B, c, 0, 0, 0);
  };

  floatx16_t acc[MS][2];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // scale/zero of the lane's two columns for the tile's group (fast path),
  // from register set `set`
  auto group_consts = [&](int set, half2_t negp[2][4], half2_t sp[2]) __attribute__((always_inline)) {
    const int n4 = nc & ~3;
    uint32_t z4;
    if constexpr (BITS == 3) z4 = __builtin_amdgcn_alignbit(zw1[set], zw0[set], (uint32_t)((3 * (n4 & 31)) & 31));
    else z4 = zw0[set] >> ((n4 * BITS) & 31);
    const uint32_t z2 = z4 >> (BITS * (nc & 3));
    const half2_t s2 = sw[set];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int z = field_of4(z2, j, BITS) + a.zero_offset;
      sp[j] = half2_t{s2[j], s2[j]};
#pragma unroll
      for (int v = 0; v < 4; ++v) negp[j][v] = neg_off(v, z, z);
    }
  };

  // bfloat16: the lane's two columns' s and -z s for the tile's group
  auto group_consts_bf16 = [&](int set, float bs[2], float bc[2]) __attribute__((always_inline)) {
    const int n4 = nc & ~3;
    uint32_t z4;
    if constexpr (BITS == 3) z4 = __builtin_amdgcn_alignbit(zw1[set], zw0[set], (uint32_t)((3 * (n4 & 31)) & 31));
    else z4 = zw0[set] >> ((n4 * BITS) & 31);
    const uint32_t z2 = z4 >> (BITS * (nc & 3));
    const uint32_t s2 = as_u32(sw[set]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float sc = bf16_to_f32((s2 >> (16 * j)) & 0xFFFFu);
      bs[j] = sc;
      bc[j] = -(float)(field_of4(z2, j, BITS) + a.zero_offset) * sc;
    }
  };
  // B fragment j of block kb from the words, bfloat16 with one (s, -z s)
  auto make_B_bf16 = [&](uint32_t w0j, uint32_t w1j, int kb, float s, float c) __attribute__((always_inline)) {
    float f[8];                                      // fields in k order
    if constexpr (PAIRS) block4_regs_f32(w0j, f);    // a pair-order word's register order is k order
    else block_fields_f32<BITS>(w0j, w1j, kb, f);
    u32x4_t bw;
#pragma unroll
    for (int v = 0; v < 4; ++v) bw[v] = bf16_pair(__builtin_fmaf(f[2 * v], s, c), __builtin_fmaf(f[2 * v + 1], s, c));
    return __builtin_bit_cast(half8_t, bw);
  };

  // fast path, a whole k tile: the B operands of step s + 1 are made (VALU)
  // while the MFMAs of step s run, in the same wave, so the two pipes overlap
  // without relying on the other wave of the SIMD
  auto compute_full_tile = [&](auto set_c) __attribute__((always_inline)) {
    constexpr int set = decltype(set_c)::value % NSR;
    const _Float16* sl = stage_lds(set_c);
    half2_t negp[2][4], sp[2];
    float bs[2], bc[2];
    if constexpr (BF16) group_consts_bf16(set, bs, bc);
    else group_consts(set, negp, sp);
    auto make_B = [&](int s, half8_t (&B)[2]) __attribute__((always_inline)) {
      const int kb = 2 * (s & 1) + kb2;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (BF16) {
          B[j] = make_B_bf16(w0[set][s][j], L == 2 ? w1[set][L == 2 ? s : 0][j] : 0u, kb, bs[j], bc[j]);
          continue;
        }
        uint32_t p[4];
        unpack_B(w0[set][s][j], L == 2 ? w1[set][L == 2 ? s : 0][j] : 0u, kb, p);
        u32x4_t bw;
#pragma unroll
        for (int v = 0; v < 4; ++v) bw[v] = as_u32(minus_zero(p[v], v, negp[j][v]) * sp[j]);
        B[j] = __builtin_bit_cast(half8_t, bw);
      }
    };
    half8_t Bc[2], Bn[2];
    make_B(0, Bc);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) make_B(s + 1, Bn);
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        const int m = 32 * i + q;
        const int kblk = 2 * s + kb2;
        const half8_t A = *reinterpret_cast<const half8_t*>(sl + (m * 8 + (kblk ^ ((m >> 1) & 7))) * 8);
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma(A, Bc[j], acc[i][j]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j) Bc[j] = Bn[j];
    }
  };

  // one k tile from LDS stage `stage` and register set `set`
  auto compute_tile = [&](int kt, auto set_c) __attribute__((always_inline)) {
    constexpr int set = decltype(set_c)::value % NSR;
    if constexpr (FULL) {
      // the loop runs tiles in threes: tiles past the end compute nothing
      if (kt < ktiles) compute_full_tile(set_c);
      return;
    }
    // tiles past the split (the loop runs in threes) compute nothing
    const int ksteps = kt < ktiles ? min(4, (a.K - (kt0 + kt) * BK) >> 4) : 0;
    const _Float16* sl = stage_lds(set_c);
    half2_t negp[2][4], sp[2];
    float bs[2], bc[2];
    if constexpr (!PER_ELEM && BF16) group_consts_bf16(set, bs, bc);
    else if constexpr (!PER_ELEM) group_consts(set, negp, sp);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s >= ksteps) break;
      const int kb = 2 * (s & 1) + kb2;
      half8_t B[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (BF16) {
          const uint32_t w0j = w0[set][s][j], w1j = L == 2 ? w1[set][L == 2 ? s : 0][j] : 0u;
          if constexpr (PER_ELEM) {
            // each row its own group: (s, -z s) per field
            const uint16_t* scb = reinterpret_cast<const uint16_t*>(a.scales);
            const int k0 = (kt0 + kt) * BK + 16 * s + 8 * kb2;
            float f[8];                              // fields in k order
            if constexpr (PAIRS) block4_regs_f32(w0j, f);
            else block_fields_f32<BITS>(w0j, w1j, kb, f);
            u32x4_t bw;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              float o[2];
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const int g = group_of(a.g_idx, k0 + 2 * v + h, a.group_size, a.G);
                const uint32_t z = load_zero4<BITS>(a.qzeros, a.zrow_words, g, nc & ~3) >> (BITS * ((nc & 3) + j));
                const float sc = bf16_to_f32(scb[(int64_t)g * a.N + nc + j]);
                const float zf = (float)((int)(z & ((1u << BITS) - 1u)) + a.zero_offset);
                o[h] = __builtin_fmaf(f[2 * v + h], sc, -zf * sc);
              }
              bw[v] = bf16_pair(o[0], o[1]);
            }
            B[j] = __builtin_bit_cast(half8_t, bw);
          } else {
            B[j] = make_B_bf16(w0j, w1j, kb, bs[j], bc[j]);
          }
          continue;
        }
        uint32_t p[4];
        unpack_B(w0[set][s][j], L == 2 ? w1[set][L == 2 ? s : 0][j] : 0u, kb, p);
        u32x4_t bw;
        if constexpr (PER_ELEM) {
          const int k0 = (kt0 + kt) * BK + 16 * s + 8 * kb2;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int ga = group_of(a.g_idx, k0 + 2 * v, a.group_size, a.G);
            const int gb = group_of(a.g_idx, k0 + 2 * v + 1, a.group_size, a.G);
            const uint32_t za = load_zero4<BITS>(a.qzeros, a.zrow_words, ga, nc & ~3) >> (BITS * ((nc & 3) + j));
            const uint32_t zb = load_zero4<BITS>(a.qzeros, a.zrow_words, gb, nc & ~3) >> (BITS * ((nc & 3) + j));
            const half2_t neg = neg_off(v, (int)(za & ((1u << BITS) - 1u)) + a.zero_offset,
                                        (int)(zb & ((1u << BITS) - 1u)) + a.zero_offset);
            const half2_t sc = {a.scales[(int64_t)ga * a.N + nc + j], a.scales[(int64_t)gb * a.N + nc + j]};
            bw[v] = as_u32(minus_zero(p[v], v, neg) * sc);
          }
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) bw[v] = as_u32(minus_zero(p[v], v, negp[j][v]) * sp[j]);
        }
        B[j] = __builtin_bit_cast(half8_t, bw);
      }
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        const int m = 32 * i + q;
        const int kblk = 2 * s + kb2;
        const half8_t A = *reinterpret_cast<const half8_t*>(sl + (m * 8 + (kblk ^ ((m >> 1) & 7))) * 8);
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma(A, B[j], acc[i][j]);
      }
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  constexpr int LOADS_PER_TILE = XI + 4 * L + (BITS == 3 ? 3 : 2);
  // s_waitcnt immediate: vmcnt <= n, no wait on the other counters
  constexpr int kWaitOneTile = (LOADS_PER_TILE & 15) | ((LOADS_PER_TILE >> 4) << 14) | 0x70 | 0xF00;
  // tile kt: wait until its loads (issued two tiles earlier) are done while
  // the next tile's stay in flight, barrier (every wave's x pieces are in LDS
  // and the stage of tile kt - 1 is free), issue tile kt + 2, compute tile kt
  auto step = [&](int kt, auto set_c, auto next_c) __attribute__((always_inline)) {
    if constexpr (PER_ELEM) {
      // one register set: the words of tile kt were the last loads issued
      __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);
      __syncthreads();
      load_x(kt + 2, next_c);
      compute_tile(kt, set_c);
      load_w(kt + 1, S0{});
    } else {
      // a plain s_barrier: __syncthreads() would also wait for the x tiles
      // still in flight (its fence covers every LDS write, DMA included); the
      // compiler-only fences keep LDS reads and loads on their side of it
      __builtin_amdgcn_s_waitcnt(kWaitOneTile);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      load_x(kt + 2, next_c);
      load_w(kt + 2, next_c);
      compute_tile(kt, set_c);
    }
  };

  load_x(0, S0{});
  if constexpr (PER_ELEM) {
    load_x(1, S1{});
    load_w(0, S0{});
  } else {
    load_w(0, S0{});
    load_x(1, S1{});
    load_w(1, S1{});
  }
  for (int kt = 0; kt < ktiles; kt += 3) {
    step(kt, S0{}, S2{});
    step(kt + 1, S1{}, S0{});
    step(kt + 2, S2{}, S1{});
  }

  // ---- split K: this split's fp32 sums (rows < M) go to its slice of ws
  // [ks, M, N]; launch_prefill then runs split_sum_kernel on the same stream,
  // which adds the slices in split order (deterministic) and rounds once
  if (BM <= 128 && ks > 1) {
    if (!col_ok) return;
#pragma unroll
    for (int i = 0; i < MS; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + 32 * i + 8 * (v >> 2) + 4 * kb2 + (v & 3);
        if (row < a.M) {
          float* w = a.ws + ((int64_t)sk * a.M + row) * a.N + n;
          w[0] = acc[i][0][v];
          w[1] = acc[i][1][v];
        }
      }
    }
    return;
  }

  // ---- epilogue: fp32 -> fp16 (bfloat16), two adjacent columns per store
  if (!col_ok) return;
#pragma unroll
  for (int i = 0; i < MS; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = m0 + 32 * i + 8 * (v >> 2) + 4 * kb2 + (v & 3);
      if (row < a.M) {
        if constexpr (BF16) {
          *reinterpret_cast<uint32_t*>(a.out + (int64_t)row * a.N + n) = bf16_pair(acc[i][0][v], acc[i][1][v]);
        } else {
          const half2_t o = {(_Float16)acc[i][0][v], (_Float16)acc[i][1][v]};
          *reinterpret_cast<half2_t*>(a.out + (int64_t)row * a.N + n) = o;
        }
      }
    }
  }
}

template <int BITS, bool PER_ELEM, bool FULL, bool PAIRS>
__global__ __launch_bounds__(256, 2) void prefill_kernel(GemmArgs a) {
  prefill_body<BITS, PER_ELEM, FULL, false, PAIRS, 128>(a);
}

// 256-row tiles: one workgroup (one wave per SIMD) per CU
template <int BITS, bool FULL, bool PAIRS>
__global__ __launch_bounds__(256, 1) void prefill_big_kernel(GemmArgs a) {
  prefill_body<BITS, false, FULL, false, PAIRS, 256>(a);
}

template <int BITS, bool PER_ELEM, bool FULL, bool PAIRS>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(GemmArgs a) {
  prefill_body<BITS, PER_ELEM, FULL, true, PAIRS, 128>(a);
}

// 32- and 64-row tiles (M <= 64), fp16 and bfloat16
template <int BITS, bool PER_ELEM, bool FULL, bool PAIRS, int BM>
__global__ __launch_bounds__(256, 2) void prefill_small_kernel(GemmArgs a) {
  prefill_body<BITS, PER_ELEM, FULL, false, PAIRS, BM>(a);
}
template <int BITS, bool PER_ELEM, bool FULL, bool PAIRS, int BM>
__global__ __launch_bounds__(256, 2) void prefill_bf16_small_kernel(GemmArgs a) {
  prefill_body<BITS, PER_ELEM, FULL, true, PAIRS, BM>(a);
}

template <int BITS, bool PER_ELEM, bool FULL, bool PAIRS>
static void launch_small(const GemmArgs& a, dim3 grid, hipStream_t stream) {
  if (a.bf16) {
    if (a.pbm == 32) hipLaunchKernelGGL((prefill_bf16_small_kernel<BITS, PER_ELEM, FULL, PAIRS, 32>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((prefill_bf16_small_kernel<BITS, PER_ELEM, FULL, PAIRS, 64>), grid, dim3(256), 0, stream, a);
  } else {
    if (a.pbm == 32) hipLaunchKernelGGL((prefill_small_kernel<BITS, PER_ELEM, FULL, PAIRS, 32>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((prefill_small_kernel<BITS, PER_ELEM, FULL, PAIRS, 64>), grid, dim3(256), 0, stream, a);
  }
}

template <int BITS, bool PER_ELEM, bool FULL>
static hipError_t launch_prefill_pe(const GemmArgs& a, hipStream_t stream) {
  const dim3 grid(a.tiles_m * a.tiles_n * (a.n_experts > 0 ? a.n_experts : (a.ks > 1 ? a.ks : 1)));
  if (a.pbm < 128) {
    // 4-bit tiled words hold their fields in pair order
    if (BITS == 4 && a.wtiled) launch_small<BITS, PER_ELEM, FULL, BITS == 4>(a, grid, stream);
    else launch_small<BITS, PER_ELEM, FULL, false>(a, grid, stream);
  } else if (a.bf16) {
    if (BITS == 4 && a.wtiled)                     // pair-order words
      hipLaunchKernelGGL((prefill_bf16_kernel<BITS, PER_ELEM, FULL, BITS == 4>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_bf16_kernel<BITS, PER_ELEM, FULL, false>), grid, dim3(256), 0, stream, a);
  } else if (a.pbm == 256) {
    if constexpr (PER_ELEM) {
      return hipErrorInvalidValue;                 // 256-row tiles: fast path only
    } else if (BITS == 4 && a.wtiled) {
      hipLaunchKernelGGL((prefill_big_kernel<BITS, FULL, BITS == 4>), grid, dim3(256), 0, stream, a);
    } else {
      hipLaunchKernelGGL((prefill_big_kernel<BITS, FULL, false>), grid, dim3(256), 0, stream, a);
    }
  } else if (BITS == 4 && a.wtiled) {
    // 4-bit tiled words hold their fields in pair order
    hipLaunchKernelGGL((prefill_kernel<BITS, PER_ELEM, FULL, BITS == 4>), grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((prefill_kernel<BITS, PER_ELEM, FULL, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

// Split-K sum: y[r, c] = sum over s = 0 .. ks - 1, in that order, of ws[s, r, c],
// rounded once to fp16 (bfloat16).  One thread per 4 adjacent columns (N is a
// multiple of 32), 16-byte loads, all KB >= ks splits' loads in flight at once
// (unconditional: loads j >= ks repeat split ks - 1 and are not added, so the
// code has no branch between the loads and their waits).
template <bool BF16, int KB>
__global__ __launch_bounds__(128) void split_sum_kernel(const float* __restrict__ ws, _Float16* __restrict__ out,
                                                        int64_t quads, int64_t split_elems, int ks) {
  const int64_t qd = (int64_t)blockIdx.x * 128 + threadIdx.x;
  if (qd >= quads) return;
  const floatx4_t* p = reinterpret_cast<const floatx4_t*>(ws) + qd;
  const int64_t stride = split_elems >> 2;
  floatx4_t v[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j) v[j] = p[(int64_t)min(j, ks - 1) * stride];
  floatx4_t sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KB; ++j)
    if (j < ks) sum += v[j];
  _Float16* o = out + 4 * qd;
  if constexpr (BF16) {
    *reinterpret_cast<u32x2_t*>(o) = u32x2_t{bf16_pair(sum[0], sum[1]), bf16_pair(sum[2], sum[3])};
  } else {
    typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
    *reinterpret_cast<half4_t*>(o) = half4_t{(_Float16)sum[0], (_Float16)sum[1], (_Float16)sum[2], (_Float16)sum[3]};
  }
}

template <int KB>
static void launch_split_sum_kb(const GemmArgs& a, hipStream_t stream) {
  const int64_t elems = (int64_t)a.M * a.N;
  const int64_t quads = elems >> 2;
  const dim3 grid((unsigned)((quads + 127) / 128));
  if (a.bf16) hipLaunchKernelGGL((split_sum_kernel<true, KB>), grid, dim3(128), 0, stream, a.ws, a.out, quads, elems, a.ks);
  else hipLaunchKernelGGL((split_sum_kernel<false, KB>), grid, dim3(128), 0, stream, a.ws, a.out, quads, elems, a.ks);
}

static hipError_t launch_split_sum(const GemmArgs& a, hipStream_t stream) {
  if (a.ks <= 4) launch_split_sum_kb<4>(a, stream);
  else if (a.ks <= 8) launch_split_sum_kb<8>(a, stream);
  else if (a.ks <= 16) launch_split_sum_kb<16>(a, stream);
  else launch_split_sum_kb<32>(a, stream);
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_prefill_bits(bool per_elem, const GemmArgs& a, hipStream_t stream) {
  if (per_elem) return launch_prefill_pe<BITS, true, false>(a, stream);
  // 8-bit: the pipelined body needs more registers than 2 workgroups per CU
  // leave (it spills), so the 128-row and smaller tiles keep the plain body;
  // the 256-row tile (one workgroup per CU, accumulators in AGPRs) holds it
  if constexpr (BITS == 8) {
    if (a.pbm == 256 && a.K % 64 == 0) {
      if (a.ks > 1 || a.n_experts > 0) return hipErrorInvalidValue;   // never planned for 256-row tiles
      hipLaunchKernelGGL((prefill_big_kernel<8, true, false>), dim3(a.tiles_m * a.tiles_n), dim3(256), 0, stream, a);
      return hipGetLastError();
    }
    return launch_prefill_pe<BITS, false, false>(a, stream);
  }
  else
    return a.K % 64 == 0 ? launch_prefill_pe<BITS, false, true>(a, stream)
                         : launch_prefill_pe<BITS, false, false>(a, stream);
}

hipError_t launch_prefill(int bits, bool per_elem, const GemmArgs& a, hipStream_t stream) {
  const bool split = a.ks > 1 && a.n_experts == 0 && a.pbm <= 128;
  if (split && a.ks > 32) return hipErrorInvalidValue;   // the sum kernel adds at most 32 splits
  hipError_t err;
  switch (bits) {
    case 2: err = launch_prefill_bits<2>(per_elem, a, stream); break;
    case 3: err = launch_prefill_bits<3>(per_elem, a, stream); break;
    case 4: err = launch_prefill_bits<4>(per_elem, a, stream); break;
    default: err = launch_prefill_bits<8>(per_elem, a, stream); break;
  }
  if (err != hipSuccess || !split || a.M == 0) return err;
  return launch_split_sum(a, stream);
}

}  // namespace gptq
