// extern "C" entry points of libgptq.so: argument checks, kernel choice and
// launch shape, and launches on the caller's stream.  No exception leaves this
// file; every failure is a gptq_status code.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "gptq.h"
#include "gptq_kernels.hpp"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_weights(const int32_t* qweight, const int32_t* qzeros, const void* scales, const int32_t* g_idx,
                  int bits, int group_size, int is_v2, int64_t N, int64_t K) {
  if (!qweight || !qzeros || !scales) return GPTQ_ERR_NULL_PTR;
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return GPTQ_ERR_BAD_BITS;
  if (N <= 0 || K <= 0 || N % 32 != 0 || K % 32 != 0) return GPTQ_ERR_BAD_SHAPE;
  if (N > ((int64_t)1 << 20) || K > ((int64_t)1 << 20) || N * K >= kMaxElems) return GPTQ_ERR_BAD_SHAPE;
  if (group_size <= 0 || K % group_size != 0) return GPTQ_ERR_BAD_GROUP;
  if (is_v2 != 0 && is_v2 != 1) return GPTQ_ERR_BAD_ARG;
  if (!aligned(qweight, 16) || !aligned(scales, 8) || !aligned(qzeros, 4) || (g_idx && !aligned(g_idx, 16)))
    return GPTQ_ERR_MISALIGNED;
  return GPTQ_OK;
}

int check_gemm(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
               const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
               const void* out) {
  if (M < 0) return GPTQ_ERR_BAD_SHAPE;
  if (M > 0 && (!x || !out)) return GPTQ_ERR_NULL_PTR;
  const int rc = check_weights(qweight, qzeros, scales, g_idx, bits, group_size, is_v2, N, K);
  if (rc != GPTQ_OK) return rc;
  if (M > ((int64_t)1 << 24) || M * K >= kMaxElems || M * N >= kMaxElems) return GPTQ_ERR_BAD_SHAPE;
  if (M > 0 && (!aligned(x, 16) || !aligned(out, 16))) return GPTQ_ERR_MISALIGNED;
  return GPTQ_OK;
}

// Decode launch shape: column tiles of 16 * cpl columns (cpl = 4 or 2 only
// while that still gives >= 192 workgroups), waves per workgroup and chunks
// per wave.  Every instantiation is compiled for a fixed number of waves per
// SIMD, so the number of workgroups a CU holds at once is known here.
// Measured on MI355X, a decode GEMV streams fastest with ~8-13 MB of weights
// in flight across the chip (more only queues; the rows of a whole matrix
// requested at once run slower) and every workgroup resident.  The choice
// therefore minimises, in order: rounds of workgroups; whether the bytes in
// flight exceed kInflightCap; their distance below it; the distance of the
// wave count from 8; then prefers wider tiles, fewer K phases and less padding.
// Limits: the LDS budget and the x staging registers (cpw * M <= 16 * x
// pieces).  The fast path needs group_size % 32 == 0 (a chunk inside one
// group); otherwise, or when no fast-path shape fits, the per-element path.
// dynamic LDS per workgroup (the kernel adds a few bytes of static LDS)
constexpr size_t kDecodeLdsBudget = 160 * 1024 - 256;
constexpr int kCUs = 256;
constexpr int64_t kInflightCap = 13ll << 20;
constexpr int kNoDecodePlan = 1;
constexpr int kMinSplitChunks = 32;                  // a K split covers at least 1024 rows
constexpr int kMinSplitK = 8192;                     // ... of a K this long (shorter: not worth the reduction)
constexpr int64_t kSplitWsCap = 16ll << 20;          // fp32 partial sums of all splits, bytes (decode)
constexpr int64_t kPrefillSplitWsCap = 64ll << 20;   // ... of a prefill launch

struct DecodeChoice {
  int rounds;
  bool over;          // bytes in flight above kInflightCap
  int64_t inflight;
  int nw, cpl, cpw, ks, tiles, phases, waste;
  int busy;           // CUs with at least one workgroup
};

bool better_choice(const DecodeChoice& a, const DecodeChoice& b) {
  if (a.rounds != b.rounds) return a.rounds < b.rounds;
  if (a.over != b.over) return !a.over;
  if (a.inflight != b.inflight) return a.over ? a.inflight < b.inflight : a.inflight > b.inflight;
  if (std::abs(a.nw - 8) != std::abs(b.nw - 8)) return std::abs(a.nw - 8) < std::abs(b.nw - 8);
  if (a.cpl != b.cpl) return a.cpl > b.cpl;
  if (a.busy != b.busy) return a.busy > b.busy;
  if (a.ks != b.ks) return a.ks < b.ks;
  if (a.phases != b.phases) return a.phases < b.phases;
  return a.waste < b.waste;
}

// Launch shape of one (cpl, nw, cpw, ks) candidate, or false when it does not
// fit (registers, LDS, x staging, split sizes).
bool decode_candidate(int bits, int M, int N, int K, int G, bool per_elem, int cpl, int nw, int cpw, int ks,
                      DecodeChoice* c, size_t* lds_out, bool bf16 = false, int64_t ws_cap = kSplitWsCap) {
  const int C = K / 32;
  const int cpg = per_elem ? 1 : (K / G) / 32;
  if (!gptq::decode_cpw_allowed(bits, per_elem, cpl, cpw, M, bf16)) return false;
  // x staged per phase (one row, or bfloat16): the staging registers bound
  // the chunks per wave; several rows (fp16) load their A fragments directly
  const bool x_direct = M > 1 && !bf16;
  if (!x_direct && cpw * M > 16 * gptq::decode_max_x_pieces(M)) return false;
  if (nw < 1 || 64 * nw > gptq::decode_max_threads_for(bits, per_elem, cpl, cpw, M)) return false;
  const int cks = (C + ks - 1) / ks;
  if (ks < 1 || (ks - 1) * cks >= C || (ks > 1 && cks < kMinSplitChunks)) return false;
  if (ks > 1 && (int64_t)ks * M * N * 4 > ws_cap) return false;
  const int pc = nw * cpw;
  const int phases = (cks + pc - 1) / pc;
  const size_t lds = gptq::decode_lds_bytes(M, pc, nw, cpl, per_elem, G, cpg, phases, bf16);
  if (lds > kDecodeLdsBudget) return false;
  const int tiles = (N + 16 * cpl - 1) / (16 * cpl);
  const int units = tiles * ks;
  const int simd_waves = gptq::decode_waves_per_simd_for(bits, per_elem, cpl, cpw, M);
  const int by_waves = simd_waves / ((nw + 3) / 4);
  const int by_lds = (int)(kDecodeLdsBudget / std::max<size_t>(lds, 1));
  const int resident = std::max(1, std::min({by_waves, by_lds, 16})) * kCUs;
  // weight bytes one phase of the resident workgroups has in flight
  const int64_t loads = (bits == 3 || bits == 8) ? 2 : 1;
  // bytes in flight matter where the stream is the bound; the per-element
  // path with several rows is bound by its dequant work, which the cap does
  // not describe (measured: a 3-bit act-order M = 16 layer ran 36% faster
  // with 4 waves per workgroup than with the 2 the cap chose; one row, e.g.
  // bfloat16 decode, keeps the cap: 20% slower without it)
  const bool work_bound = per_elem && M > 1;
  const int64_t inflight = work_bound ? 0 : (int64_t)std::min(units, resident) * std::min(pc, cks) * 64 * cpl * loads * 4;
  *c = DecodeChoice{(units + resident - 1) / resident, inflight > kInflightCap, inflight,
                    nw, cpl, cpw, ks, tiles, phases, phases * pc - cks, std::min(units, kCUs)};
  *lds_out = lds;
  return true;
}

void apply_choice(const DecodeChoice& c, int M, int K, int G, bool per_elem, bool bf16, gptq::GemmArgs* a) {
  const int C = K / 32;
  a->tiles = c.tiles;
  a->cpl = c.cpl;
  a->nw = c.nw;
  a->cpw = c.cpw;
  a->pc = c.nw * c.cpw;
  a->phases = c.phases;
  a->cpg = per_elem ? 1 : (K / G) / 32;
  a->ks = c.ks;
  a->cks = (C + c.ks - 1) / c.ks;
  // fast path: fold scale and zero once per block of 4 (or 2) chunks of one
  // group; every wave's run (cpw chunks, halved at a phase's midpoint) and
  // every K split must start on a block boundary
  a->fold = 1;
  if (!per_elem && !bf16) {
    for (int f : {4, 2}) {
      if (a->cpg % f == 0 && (c.cpw / 2) % f == 0 && (c.ks == 1 || a->cks % f == 0)) {
        a->fold = f;
        break;
      }
    }
  }
}

bool decode_plan_for(int bits, int M, int N, int K, int G, int waves, bool per_elem, bool allow_split,
                     bool tiled, gptq::GemmArgs* a, bool bf16, int64_t ws_cap) {
  bool found = false;
  DecodeChoice best{};
  // tiled layout, M = 1, full-width: 16 chunks per wave over 16-column tiles
  // (32-column tiles from N = 16384 on) were the fastest or within 2% of it
  // on every Llama-7B decode layer in MI355X sweeps, where the general rules
  // below lose up to 10%; the wave count (8..16, also 4 for K <= 2048) keeps
  // the fewest rounds of resident workgroups, then pads K the least, then
  // takes the fewest phases, then the fewest waves (8 when K is a multiple of
  // 4096: one phase,
  // no padding; 11 for K = 11008 at N = 4096: 2 phases of 176 chunks for 344,
  // 5% faster than 8 waves in 3 phases of 128; 4 for K = 2048: one phase with
  // no padded waves, 11-12% faster than 8 at N = 4096, 2- and 4-bit)
  // tiled layout, 2..16 rows, full-width: 8 chunks per wave, 64-column tiles
  // for 2/4-bit layers from N = 8192 on (32-column otherwise), 8 or 4 waves,
  // whichever pads K less (8 on a tie), two K splits for N <= 4096 with
  // K >= 8192 -- the fastest shapes of MI355X sweeps at M = 4 and 16, where
  // the general rules below are up to 40% slower.  Two-word blocks (3 and 8
  // bits) and the per-element path (either layout, several rows): 32-column
  // tiles of 4 waves, three K splits for K >= 8192 (3-bit act-order layers at
  // M = 16, sorted or not: the fastest shape of the sweeps on both shapes,
  // 10-13% ahead of the next on 13824 -> 5120)
  const bool two_word = bits == 3 || bits == 8;
  if (((tiled && !per_elem) || (per_elem && !bf16)) && M > 1 && waves == 0 && N / 16 >= kCUs / 2) {
    const int C = K / 32;
    const bool narrow = two_word || per_elem;
    const int cpl = !narrow && N >= 8192 ? 4 : 2;
    const int ks = !allow_split ? 1 : narrow ? (K >= 8192 ? 3 : 1) : (N <= 4096 && K >= 8192 ? 2 : 1);
    const int cks = (C + ks - 1) / ks;
    const int waste8 = (cks + 63) / 64 * 64 - cks, waste4 = (cks + 31) / 32 * 32 - cks;
    const int nw = narrow ? 4 : waste4 < waste8 ? 4 : 8;
    size_t lds;
    if (decode_candidate(bits, M, N, K, G, per_elem, cpl, nw, 8, ks, &best, &lds, bf16, ws_cap)) {
      apply_choice(best, M, K, G, per_elem, bf16, a);
      return true;
    }
  }
  if (tiled && M == 1 && !per_elem && waves == 0 && N / 16 >= kCUs / 2) {
    size_t lds;
    const bool wide = N >= 16384;
    int64_t best_slots = 0;
    // 4 waves only where 8 would leave half of their chunk slots empty
    for (int nw = K / 32 <= 64 ? 4 : 8; nw <= 16; nw += nw == 4 ? 4 : 1) {
      DecodeChoice c;
      if (!decode_candidate(bits, M, N, K, G, per_elem, wide ? 2 : 1, nw, 16, 1, &c, &lds, bf16, ws_cap)) continue;
      const int64_t slots = (int64_t)c.phases * nw * 16;
      if (!found || c.rounds < best.rounds ||
          (c.rounds == best.rounds && (slots < best_slots || (slots == best_slots && c.phases < best.phases)))) {
        best = c;
        best_slots = slots;
        found = true;
      }
    }
    if (found) {
      apply_choice(best, M, K, G, per_elem, bf16, a);
      return true;
    }
  }
  for (int cpl : {4, 2, 1}) {
    const int tiles = (N + 16 * cpl - 1) / (16 * cpl);
    for (int ks : {1, 2, 3, 4, 6, 8}) {
      // K splits pay for their cross-workgroup reduction (about 2 us) only
      // when the narrowest column tiles leave most CUs idle and K is long
      // (measured on MI355X: at N >= 4096, or K = 4096, every split shape was
      // slower than the best unsplit one; at N <= 1536 with K >= 8192 they
      // were 10-25% faster)
      if (ks > 1 && (!allow_split || N / 16 >= kCUs / 2 || K < kMinSplitK)) continue;
      // wide tiles only while they leave enough workgroups for the stream (the
      // per-element path with several rows, bound by its dequant work, takes
      // them regardless: a 3-bit act-order 13824 -> 5120 layer at M = 16 ran
      // 30% faster on 160 32-column tiles than on 320 16-column ones)
      if (cpl > 1 && tiles * ks < 192 && !(per_elem && M > 1)) continue;
      for (int cpw : {8, 16, 32}) {
        const int maxw = gptq::decode_max_threads_for(bits, per_elem, cpl, cpw, M) / 64;
        const int lo = waves > 0 ? std::min(waves, maxw) : 1, hi = waves > 0 ? lo : maxw;
        for (int nw = lo; nw <= hi; ++nw) {
          if (waves == 0 && (nw & (nw - 1)) != 0) continue;   // automatic: 1, 2, 4, 8, 16 waves
          DecodeChoice c;
          size_t lds;
          if (!decode_candidate(bits, M, N, K, G, per_elem, cpl, nw, cpw, ks, &c, &lds, bf16, ws_cap)) continue;
          if (!found || better_choice(c, best)) {
            best = c;
            found = true;
          }
        }
      }
    }
  }
  if (!found) return false;
  apply_choice(best, M, K, G, per_elem, bf16, a);
  return true;
}

int decode_shape(int bits, int M, int N, int K, int G, int waves, bool allow_split, bool tiled, bool* per_elem,
                 gptq::GemmArgs* a, bool bf16 = false, int64_t ws_cap = kSplitWsCap) {
  if ((K / G) % 32 != 0) *per_elem = true;
  for (int pe = *per_elem ? 1 : 0; pe < 2; ++pe) {
    if (decode_plan_for(bits, M, N, K, G, waves, pe == 1, allow_split, tiled, a, bf16, ws_cap)) {
      *per_elem = pe == 1;
      return GPTQ_OK;
    }
  }
  return kNoDecodePlan;                              // the scale/zero table does not fit LDS
}

// Prefill split K for small grids of 32-, 64- or 128-row tiles (small M, or
// N of a few thousand columns): ks workgroups per tile each take a slice of
// K and store fp32 partial sums, which a second kernel adds.  The split count
// minimises a time model (us) fitted to measurements on MI355X (4-bit,
// 4096 -> 4096 / 12288 / 22016 and 11008 -> 4096, M = 17 .. 512, 1 .. 32
// splits: the pick is on average 1.9% slower than the best count): a
// workgroup's k tiles run as a chain of t_tile each (0.53 / 0.67 / 0.93 us
// for 32 / 64 / 128 rows at one workgroup per CU), stretched by (workgroups
// per CU)^0.75 above that for the small tiles and by (rounds of one
// workgroup per CU)^1.25 for the 128-row ones (the last round's CUs set the
// time); a split launch costs about 4.3 us more (the sum kernel's launch and
// latency) plus the partial sums' traffic, ks * M * N fp32 written and read
// back, at 8 bytes per ns.  No split with 256-row tiles or in a grouped
// launch.
constexpr int kPrefillMinSplitTiles = 2;               // k tiles (128 rows of K) per split at least
constexpr int kPrefillMaxSplits = 32;                  // the sum kernel's loads in flight per thread

// Model time of a launch whose splits take `per` k tiles each (ks splits).
double prefill_time_model(const gptq::GemmArgs& a, int per, int ks) {
  const double per_cu = (double)a.tiles_m * a.tiles_n * ks / kCUs;
  double t = per;
  if (a.pbm < 128) t *= (a.pbm == 32 ? 0.53 : 0.67) * std::pow(std::max(1.0, per_cu), 0.75);
  else t *= 0.93 * std::pow(std::ceil(per_cu - 1e-9), 1.25);
  if (ks > 1) t += 4.3 + 2.0 * ks * a.M * a.N * 4 / 8.0e6;
  return t;
}

void plan_prefill_split(gptq::GemmArgs* a, bool allow_split, int64_t ws_cap) {
  a->ks = 1;
  a->cks = a->chunks;
  if (!allow_split || a->pbm > 128) return;
  const int ktiles = (a->K + 63) / 64;
  int ks = 1;
  double best = prefill_time_model(*a, ktiles, 1);
  for (int k = 2; k <= std::min(kPrefillMaxSplits, ktiles / kPrefillMinSplitTiles); ++k) {
    const int per = (ktiles + k - 1) / k;             // k tiles per split
    const int eks = (ktiles + per - 1) / per;          // splits with no empty one
    if ((int64_t)eks * a->M * a->N * 4 > ws_cap) break;
    const double t = prefill_time_model(*a, per, eks);
    if (t < best) {
      best = t;
      ks = eks;
    }
  }
  if (ks < 2) return;
  const int per = (ktiles + ks - 1) / ks;
  a->ks = (ktiles + per - 1) / per;
  a->cks = 2 * per;                                    // in 32-row chunks
}

// Per-element layers (act-order g_idx, or groups that are not whole 64-row
// k tiles) at up to this many rows run the decode kernel over blocks of 16
// rows: the prefill kernel's per-element path looks up g_idx, zeros and
// scales per element in global memory, while the decode kernel stages the
// layer's scale/zero table per workgroup and the row blocks of a column tile
// share its weights through one XCD's L2.  Measured on MI355X (tiled, act
// order unless noted), decode over row blocks vs the prefill kernel, us:
// 4096 -> 12288 4-bit 22 / 39 / 128 / 253 / 1089 vs 111 / 149 / 354 / 678 /
// 1441 at M = 17 / 64 / 256 / 512 / 2048; 3-bit 5120 -> 13824 38 / 205 /
// 1694 vs 152 / 482 / 2288 at M = 17 / 256 / 2048; 4096 -> 4096 4-bit g32
// (no g_idx) 8.6 / 81 / 325 vs 38 / 137 / 477 at M = 17 / 512 / 2048; 8192
// -> 28672 4-bit at M = 2048 5254 vs 6072.  The bound keeps the grid (row
// blocks x column tiles) far below 2^31.
constexpr int64_t kRowBlockMaxRows = 4096;

// Small fast-path layers (N <= 4096, K <= 8192, fp16) at 17..64 rows: the
// decode kernel over row blocks when its plan has at most 128 column tiles
// (at most two rounds of the CUs for four blocks).  The prefill grid there
// is 16 column tiles or fewer, so its split launch's fixed costs dominate.
// Measured on MI355X (tiled, 4-bit unless noted, us, decode vs prefill, at
// M = 17 / 32 / 64): 4096 -> 4096 8.1 / 8.2 / 12.7 vs 10.9 / 13.5 / 16.2;
// 4096 -> 1024 6.7 / 6.9 / 6.9 vs 9.1 / 10.4 / 13.7; 2048 -> 4096 5.2 /
// 5.4 / 7.7 vs 9.6 / 10.6 / 13.9; 5120 -> 4096 9.7 / 9.8 / 16.0 vs 11.6 /
// 13.9 / 19.6; 8192 -> 4096 12.8 / 12.7 vs 12.7 / 15.4 at 17 / 32; 2-bit
// and 8-bit 4096 -> 4096 alike.  Excluded by measurement: the checkpoint
// layout of 4096 -> 4096 (256 tiles: 13.8 vs 11.4 at 17 rows), 11008 ->
// 4096 (a tie at 17, 1.4x slower at 64) and wider layers (4096 -> 12288 /
// 22016: up to 1.6x slower).
constexpr int64_t kSmallLayerMaxN = 4096, kSmallLayerMaxK = 8192;

// Argument checks plus kernel choice and launch shape: pure host code.
int plan_gemm(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
              const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
              const void* out, int path, int decode_waves, bool tiled, gptq::GemmArgs* a, bool* use_decode,
              bool* per_elem, bool allow_split = true, bool bf16 = false, int64_t ws_cap = kPrefillSplitWsCap) {
  if (path < 0 || path > 2 || decode_waves < 0 || decode_waves > 16) return GPTQ_ERR_BAD_ARG;
  int rc = check_gemm(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out);
  if (rc != GPTQ_OK) return rc;
  if (path == 1 && M > 16) return GPTQ_ERR_BAD_ARG;
  *a = gptq::GemmArgs{};
  a->x = static_cast<const _Float16*>(x);
  a->qweight = qweight;
  a->qzeros = qzeros;
  a->scales = static_cast<const _Float16*>(scales);
  a->g_idx = g_idx;
  a->out = static_cast<_Float16*>(const_cast<void*>(out));
  a->M = (int)M;
  a->N = (int)N;
  a->K = (int)K;
  a->G = (int)(K / group_size);
  a->group_size = group_size;
  a->zero_offset = is_v2 ? 0 : 1;
  a->chunks = (int)(K / 32);
  a->zrow_words = N * bits / 32;
  a->wtiled = tiled ? 1 : 0;
  a->bf16 = bf16 ? 1 : 0;
  *use_decode = (path == 1) || (path == 0 && M <= 16);
  if (M == 0) return GPTQ_OK;
  if (path == 0 && M > 16 && M <= kRowBlockMaxRows && (g_idx != nullptr || group_size % 64 != 0)) {
    // the prefill kernel would take its per-element path: the decode kernel
    // over blocks of 16 rows instead (no K split)
    bool pe = bf16 || g_idx != nullptr || group_size % 32 != 0;
    if (decode_shape(bits, 16, a->N, a->K, a->G, decode_waves, false, tiled, &pe, a, bf16) == GPTQ_OK) {
      *per_elem = pe;
      *use_decode = true;
      a->row_blocks = (int)((M + 15) / 16);
      return GPTQ_OK;
    }
  }
  if (path == 0 && !bf16 && M > 16 && M <= 64 && N <= kSmallLayerMaxN && K <= kSmallLayerMaxK) {
    gptq::GemmArgs b = *a;
    bool pe = group_size % 32 != 0;
    if (decode_shape(bits, 16, b.N, b.K, b.G, decode_waves, false, tiled, &pe, &b, false) == GPTQ_OK &&
        2 * b.tiles <= kCUs) {
      *a = b;
      *per_elem = pe;
      *use_decode = true;
      a->row_blocks = (int)((M + 15) / 16);
      return GPTQ_OK;
    }
  }
  if (*use_decode) {
    // bfloat16: always the element-wise dequant (the fp16 exponent trick of
    // the fast path does not carry over)
    *per_elem = bf16 || (g_idx != nullptr) || (group_size % 32 != 0);
    const int rc2 = decode_shape(bits, a->M, a->N, a->K, a->G, decode_waves, allow_split, tiled, per_elem, a, bf16,
                                 std::min(ws_cap, kSplitWsCap));
    if (rc2 != kNoDecodePlan) return rc2;
    if (path == 1) return GPTQ_ERR_BAD_ARG;         // forced decode, but no launch shape fits
    *use_decode = false;                             // very many groups: the prefill kernel
  }
  *per_elem = (g_idx != nullptr) || (group_size % 64 != 0);
  // 256-row tiles: the fp16 fast path (8-bit only with whole 64-row k tiles,
  // its pipelined body)
  gptq::prefill_shape(a->M, a->N, !*per_elem && !bf16 && (bits != 8 || K % 64 == 0), &a->tiles_m, &a->tiles_n,
                      &a->pbm);
  plan_prefill_split(a, allow_split, ws_cap);
  return GPTQ_OK;
}

// Split-K arrival counters a plan needs (one per column tile in the decode
// kernel; a prefill split is summed by a second kernel and counts nothing).
size_t split_counter_bytes(const gptq::GemmArgs& a, bool use_decode) {
  if (a.ks <= 1 || !use_decode) return 0;
  return (size_t)a.tiles * 4;
}

// Split-K workspace, one per (device, stream): the per-tile arrival counters
// at a fixed place (the first kCounterBytes, enough for every tile count),
// then the fp32 partial sums.  Counters are zeroed once at allocation and
// every kernel leaves them at zero, so calls of any shape can share them.
// Grown when a call needs more; never allocated while the stream is being
// captured.  A superseded buffer is not freed: a HIP graph captured earlier on
// that stream holds its address and keeps using it on every replay, so it is
// kept on a retired list until gptq_release.
constexpr size_t kCounterBytes = (size_t)4 << 16;   // N <= 2^20 columns: at most 2^16 tiles
struct SplitWorkspace {
  int device;
  hipStream_t stream;
  char* base;
  size_t bytes;
};
struct RetiredBuffer {
  int device;
  char* base;
};
std::mutex g_ws_mu;
std::vector<SplitWorkspace> g_ws;
std::vector<RetiredBuffer> g_retired;

// Test hook: with GPTQ_TEST_FAIL_WORKSPACE=1 in the environment every
// workspace allocation fails, so tests can reach the no-memory paths (the
// unsplit fallback, GPTQ_ERR_NO_MEM) without exhausting device memory.
bool workspace_alloc_disabled() {
  const char* v = std::getenv("GPTQ_TEST_FAIL_WORKSPACE");
  return v != nullptr && v[0] == '1';
}

// x_bytes > 0 also reserves a buffer after the partial sums (the gathered x
// of gptq_gemm_sorted), returned in *xbuf.
bool split_workspace(hipStream_t stream, size_t ws_bytes, size_t cnt_bytes, float** ws, uint32_t** cnt,
                     size_t x_bytes = 0, void** xbuf = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || cnt_bytes > kCounterBytes) return false;
  const size_t ws_al = (ws_bytes + 255) & ~(size_t)255;
  const size_t need = kCounterBytes + ws_al + x_bytes;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  SplitWorkspace* e = nullptr;
  for (auto& w : g_ws)
    if (w.device == dev && w.stream == stream) e = &w;
  if (e == nullptr || e->bytes < need) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess || st != hipStreamCaptureStatusNone) return false;
    if (workspace_alloc_disabled()) return false;
    size_t bytes = std::max(need, (size_t)1 << 20);
    if (e != nullptr) bytes = std::max(bytes, 2 * e->bytes);
    char* base = nullptr;
    if (hipMalloc(reinterpret_cast<void**>(&base), bytes) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    if (hipMemsetAsync(base, 0, bytes, stream) != hipSuccess) {
      (void)hipFree(base);
      return false;
    }
    if (e == nullptr) {
      g_ws.push_back(SplitWorkspace{dev, stream, base, bytes});
      e = &g_ws.back();
    } else {
      // kernels queued on the stream and graphs captured on it may still use
      // the old buffer: retire it (freed by gptq_release), never free it here
      g_retired.push_back(RetiredBuffer{dev, e->base});
      e->base = base;
      e->bytes = bytes;
    }
  }
  *cnt = reinterpret_cast<uint32_t*>(e->base);
  *ws = reinterpret_cast<float*>(e->base + kCounterBytes);
  if (xbuf) *xbuf = e->base + kCounterBytes + ws_al;
  return true;
}

// Scratch of gptq_gemm_noalloc: a static device array (each device holds its
// own copy for the life of the process) instead of the allocated workspace:
// the split-K arrival counters in the first kScratchCounterBytes, the fp32
// partial sums after them.  Host code never uses the array's name as an
// address (on the host it is only a stand-in): the device address comes from
// hipGetSymbolAddress, once per device, and is kept in g_scratch_ptr.
constexpr size_t kScratchBytes = (size_t)2 << 20;
constexpr size_t kScratchCounterBytes = (size_t)64 << 10;   // 16384 tiles
constexpr int64_t kScratchSumBytes = (int64_t)(kScratchBytes - kScratchCounterBytes);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // device address of `scratch`, per device

// The calling thread's current device's scratch address; on first use on a
// device the counters are cleared by a kernel on `stream` (the array also
// starts zeroed when the code object loads; every split-K kernel leaves the
// counters it used at zero).
int scratch_for_device(hipStream_t stream, char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GPTQ_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (g_scratch_ptr[(size_t)dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return GPTQ_ERR_DEVICE;
    }
    if (gptq::launch_zero_words(p, (int64_t)(kScratchCounterBytes / 4), stream) != hipSuccess) return GPTQ_ERR_LAUNCH;
    g_scratch_ptr[(size_t)dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[(size_t)dev]);
  return GPTQ_OK;
}

// x_perm (nullable): rows of qweight are sorted by act-order group and x is
// gathered into that order first (x_perm[i] = original row of sorted row i).
int gemm_impl(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
              const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
              void* out, void* stream_ptr, int path, int decode_waves, bool tiled, const int32_t* x_perm = nullptr,
              bool bf16 = false) {
  gptq::GemmArgs a;
  bool use_decode = false, per_elem = false;
  const int rc = plan_gemm(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, path,
                           decode_waves, tiled, &a, &use_decode, &per_elem, true, bf16);
  if (rc != GPTQ_OK || M == 0) return rc;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  if (x_perm) {
    // one workspace request for the gathered x and (if planned) the split sums
    const size_t xb = (size_t)M * K * 2;
    const bool split = a.ks > 1;
    void* xg = nullptr;
    bool ok = split_workspace(stream, split ? (size_t)a.ks * a.M * a.N * 4 : 0, split_counter_bytes(a, use_decode),
                              &a.ws, &a.cnt, xb, &xg);
    if (!ok && split) {
      const int rc2 = plan_gemm(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, path,
                                decode_waves, tiled, &a, &use_decode, &per_elem, false, bf16);
      if (rc2 != GPTQ_OK) return rc2;
      ok = split_workspace(stream, 0, 0, &a.ws, &a.cnt, xb, &xg);
    }
    if (!ok) return GPTQ_ERR_NO_MEM;
    if (gptq::launch_gather_cols(x, x_perm, xg, M, K, stream) != hipSuccess) return GPTQ_ERR_LAUNCH;
    a.x = static_cast<const _Float16*>(xg);
    const hipError_t err = use_decode ? gptq::launch_decode(bits, per_elem, a, stream)
                                      : gptq::launch_prefill(bits, per_elem, a, stream);
    return err == hipSuccess ? GPTQ_OK : GPTQ_ERR_LAUNCH;
  }
  if (a.ks > 1 &&
      !split_workspace(stream, (size_t)a.ks * a.M * a.N * 4, split_counter_bytes(a, use_decode), &a.ws, &a.cnt)) {
    // no workspace (first use under stream capture, or out of memory): one split
    const int rc2 = plan_gemm(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, path,
                              decode_waves, tiled, &a, &use_decode, &per_elem, false, bf16);
    if (rc2 != GPTQ_OK) return rc2;
  }
  const hipError_t err = use_decode ? gptq::launch_decode(bits, per_elem, a, stream)
                                    : gptq::launch_prefill(bits, per_elem, a, stream);
  return err == hipSuccess ? GPTQ_OK : GPTQ_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int gptq_gemm_check(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                    const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
                    const void* out) {
  gptq::GemmArgs a;
  bool use_decode = false, per_elem = false;
  return plan_gemm(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, 0, 0, false, &a,
                   &use_decode, &per_elem);
}

int gptq_gemm_ex_check(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                       const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
                       const void* out, int path, int decode_waves) {
  gptq::GemmArgs a;
  bool use_decode = false, per_elem = false;
  return plan_gemm(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, path, decode_waves,
                   false, &a, &use_decode, &per_elem);
}

}  // extern "C"

namespace {
int describe_impl(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                  const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
                  const void* out, int path, int decode_waves, bool tiled, char* buf, int64_t buflen,
                  bool bf16 = false) {
  if (!buf || buflen <= 0) return GPTQ_ERR_NULL_PTR;
  buf[0] = '\0';
  gptq::GemmArgs a;
  bool use_decode = false, per_elem = false;
  const int rc = plan_gemm(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, path,
                           decode_waves, tiled, &a, &use_decode, &per_elem, true, bf16);
  if (rc != GPTQ_OK) return rc;
  const char* pe = per_elem ? "true" : "false";
  if (M == 0) {
    std::snprintf(buf, (size_t)buflen, "none (M = 0)");
  } else if (use_decode) {
    const int rb = a.row_blocks > 1 ? a.row_blocks : 1;
    int len;
    if (bf16)
      len = std::snprintf(buf, (size_t)buflen,
                          "gptq::decode_bf16_kernel<%d, %d, %d, %d> grid=%d block=%d phases=%d chunks_per_phase=%d "
                          "k_splits=%d",
                          bits, M == 1 ? 1 : 4, a.cpl, a.cpw, a.tiles * a.ks * rb, 64 * a.nw, a.phases, a.pc, a.ks);
    else
      len = std::snprintf(buf, (size_t)buflen,
                          "gptq::decode_kernel<%d, %s, %d, %d, %d, %d> grid=%d block=%d phases=%d chunks_per_phase=%d "
                          "k_splits=%d",
                          bits, pe, M == 1 ? 1 : 4, a.cpl, a.cpw, a.fold, a.tiles * a.ks * rb, 64 * a.nw, a.phases,
                          a.pc, a.ks);
    if (rb > 1 && len > 0 && len < buflen)
      std::snprintf(buf + len, (size_t)(buflen - len), " row_blocks=%d", rb);
  } else {
    // the pipelined full-tile body: fast path, K % 64 == 0, 8-bit only on the
    // 256-row tile
    const bool full = !per_elem && K % 64 == 0 && (bits != 8 || a.pbm == 256);
    if (a.pbm < 128)         // 32- or 64-row tiles (M <= 64)
      std::snprintf(buf, (size_t)buflen, "gptq::%s<%d, %s, %s, %s, %d> grid=%dx%d block=256 k_splits=%d",
                    bf16 ? "prefill_bf16_small_kernel" : "prefill_small_kernel", bits, pe, full ? "true" : "false",
                    (bits == 4 && tiled) ? "true" : "false", a.pbm, a.tiles_n, a.tiles_m, a.ks);
    else if (bf16)
      std::snprintf(buf, (size_t)buflen, "gptq::prefill_bf16_kernel<%d, %s, %s> grid=%dx%d block=256 k_splits=%d",
                    bits, pe, full ? "true" : "false", a.tiles_n, a.tiles_m, a.ks);
    else if (a.pbm == 256)   // last argument: 4-bit tiled words with fields in pair order
      std::snprintf(buf, (size_t)buflen, "gptq::prefill_big_kernel<%d, %s, %s> grid=%dx%d block=256 k_splits=%d",
                    bits, full ? "true" : "false", (bits == 4 && tiled) ? "true" : "false", a.tiles_n, a.tiles_m,
                    a.ks);
    else
      std::snprintf(buf, (size_t)buflen, "gptq::prefill_kernel<%d, %s, %s, %s> grid=%dx%d block=256 k_splits=%d",
                    bits, pe, full ? "true" : "false", (bits == 4 && tiled) ? "true" : "false", a.tiles_n,
                    a.tiles_m, a.ks);
  }
  return GPTQ_OK;
}
}  // namespace

extern "C" {

int gptq_gemm_describe(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                       const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
                       const void* out, int path, int decode_waves, char* buf, int64_t buflen) {
  return describe_impl(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, path,
                       decode_waves, false, buf, buflen);
}

int gptq_gemm_tiled_describe(const void* x, const int32_t* qweight_tiled, const int32_t* qzeros,
                             const void* scales, const int32_t* g_idx, int bits, int group_size, int is_v2,
                             int64_t M, int64_t N, int64_t K, const void* out, int path, int decode_waves, char* buf,
                             int64_t buflen) {
  return describe_impl(x, qweight_tiled, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, path,
                       decode_waves, true, buf, buflen);
}

int gptq_dequant_check(const int32_t* qweight, const int32_t* qzeros, const void* scales, const int32_t* g_idx,
                       int bits, int group_size, int is_v2, int64_t N, int64_t K, const void* w_out) {
  if (!w_out) return GPTQ_ERR_NULL_PTR;
  const int rc = check_weights(qweight, qzeros, scales, g_idx, bits, group_size, is_v2, N, K);
  if (rc != GPTQ_OK) return rc;
  if (!aligned(w_out, 16)) return GPTQ_ERR_MISALIGNED;
  return GPTQ_OK;
}

int gptq_gemm_ex(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                 const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
                 void* out, void* stream, int path, int decode_waves) {
  try {
    return gemm_impl(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, stream, path,
                     decode_waves, false);
  } catch (const std::bad_alloc&) {
    return GPTQ_ERR_NO_MEM;
  } catch (...) {
    return GPTQ_ERR_DEVICE;
  }
}

int gptq_gemm_tiled_ex(const void* x, const int32_t* qweight_tiled, const int32_t* qzeros, const void* scales,
                       const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
                       void* out, void* stream, int path, int decode_waves) {
  try {
    return gemm_impl(x, qweight_tiled, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, stream, path,
                     decode_waves, true);
  } catch (const std::bad_alloc&) {
    return GPTQ_ERR_NO_MEM;
  } catch (...) {
    return GPTQ_ERR_DEVICE;
  }
}

int gptq_gemm_tiled(const void* x, const int32_t* qweight_tiled, const int32_t* qzeros, const void* scales,
                    const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
                    void* out, void* stream) {
  return gptq_gemm_tiled_ex(x, qweight_tiled, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, stream,
                            0, 0);
}

namespace {
// Grouped GEMM path: expert batches of one decode block (up to 16 rows) run
// on the decode kernel, larger ones on the prefill kernel (tiles of 32 to 128
// rows, each reading its expert's weights once, where every further block of
// 16 rows of the decode kernel reads them again).  Measured on MI355X, 8
// experts 4096 -> 14336, 4-bit: decode 64 / 103 / 112 us at 16 / 24 / 32 rows
// per expert, prefill with 128-row tiles 106 / 101 / 98 us (the 32- and
// 64-row tiles now taken at such row counts skip the MFMAs of absent rows).
constexpr int kMoePrefillRows = 16;

int moe_impl(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales, const int32_t* g_idx,
             const int32_t* expert_offsets, int n_experts, int max_tokens_per_expert, int bits, int group_size,
             int is_v2, int64_t T, int64_t N, int64_t K, void* out, void* stream, int path) {
  int rc = check_weights(qweight, qzeros, scales, g_idx, bits, group_size, is_v2, N, K);
  if (rc != GPTQ_OK) return rc;
  if (!expert_offsets) return GPTQ_ERR_NULL_PTR;
  if (n_experts < 1 || n_experts > (1 << 16) || max_tokens_per_expert < 0) return GPTQ_ERR_BAD_ARG;
  if (path < 0 || path > 2) return GPTQ_ERR_BAD_ARG;
  if (T < 0 || T > ((int64_t)1 << 24) || T * K >= kMaxElems || T * N >= kMaxElems) return GPTQ_ERR_BAD_SHAPE;
  if ((int64_t)n_experts * (K / 32 * bits) * N >= kMaxElems) return GPTQ_ERR_BAD_SHAPE;
  if (T == 0 || max_tokens_per_expert == 0) return GPTQ_OK;
  if (!x || !out) return GPTQ_ERR_NULL_PTR;
  // an expert has at most T rows: a looser bound only adds empty blocks
  max_tokens_per_expert = (int)std::min<int64_t>(max_tokens_per_expert, T);
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(expert_offsets, 4)) return GPTQ_ERR_MISALIGNED;
  gptq::GemmArgs a{};
  a.x = static_cast<const _Float16*>(x);
  a.qweight = qweight;
  a.qzeros = qzeros;
  a.scales = static_cast<const _Float16*>(scales);
  a.g_idx = g_idx;
  a.out = static_cast<_Float16*>(out);
  a.M = (int)T;
  a.N = (int)N;
  a.K = (int)K;
  a.G = (int)(K / group_size);
  a.group_size = group_size;
  a.zero_offset = is_v2 ? 0 : 1;
  a.chunks = (int)(K / 32);
  a.zrow_words = N * bits / 32;
  a.moe_off = expert_offsets;
  a.n_experts = n_experts;
  a.moe_rows = max_tokens_per_expert;
  a.qw_stride = K / 32 * bits * N;
  a.qz_stride = a.G * a.zrow_words;
  a.sc_stride = (int64_t)a.G * N;
  a.gi_stride = K;
  const bool prefill = path == 2 || (path == 0 && max_tokens_per_expert > kMoePrefillRows);
  bool per_elem;
  if (prefill) {
    // one launch of prefill tiles per expert: row tiles over the largest batch
    per_elem = (g_idx != nullptr) || (group_size % 64 != 0);
    gptq::prefill_shape(max_tokens_per_expert, a.N, false, &a.tiles_m, &a.tiles_n, &a.pbm);
    if ((int64_t)n_experts * a.tiles_m * a.tiles_n >= ((int64_t)1 << 31)) return GPTQ_ERR_BAD_SHAPE;
    const hipError_t err = gptq::launch_prefill(bits, per_elem, a, reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? GPTQ_OK : GPTQ_ERR_LAUNCH;
  }
  per_elem = (g_idx != nullptr) || (group_size % 32 != 0);
  // launch shape for blocks of up to 16 rows, no K split (one workgroup per
  // expert block and column tile)
  if (decode_shape(bits, 16, a.N, a.K, a.G, 0, false, false, &per_elem, &a) != GPTQ_OK) return GPTQ_ERR_BAD_SHAPE;
  a.moe_blocks = (max_tokens_per_expert + 15) / 16;
  if ((int64_t)n_experts * a.moe_blocks * a.tiles >= ((int64_t)1 << 31)) return GPTQ_ERR_BAD_SHAPE;
  const hipError_t err = gptq::launch_decode(bits, per_elem, a, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? GPTQ_OK : GPTQ_ERR_LAUNCH;
}

int repack_impl(const int32_t* in, int32_t* out, int bits, int64_t N, int64_t K, int to_tiled, void* stream) {
  if (!in || !out) return GPTQ_ERR_NULL_PTR;
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return GPTQ_ERR_BAD_BITS;
  if (N <= 0 || K <= 0 || N % 32 != 0 || K % 32 != 0) return GPTQ_ERR_BAD_SHAPE;
  if (N > ((int64_t)1 << 20) || K > ((int64_t)1 << 20) || N * K >= kMaxElems) return GPTQ_ERR_BAD_SHAPE;
  if (!aligned(in, 16) || !aligned(out, 16)) return GPTQ_ERR_MISALIGNED;
  const int64_t bytes = K / 32 * bits * N * 4;
  const uintptr_t a = (uintptr_t)in, b = (uintptr_t)out;
  if (a < b + bytes && b < a + bytes) return GPTQ_ERR_BAD_ARG;          // no overlap, not even in place
  const hipError_t err = gptq::launch_repack(in, out, bits, N, K, to_tiled, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? GPTQ_OK : GPTQ_ERR_LAUNCH;
}
}  // namespace

int gptq_sort_act_order(const int32_t* qweight, const int32_t* g_idx, int bits, int group_size, int64_t N,
                        int64_t K, int32_t* qweight_sorted, int32_t* perm, void* stream_ptr) {
  try {
    if (!g_idx || !qweight_sorted || !perm) return GPTQ_ERR_NULL_PTR;
    // scales/qzeros are not read: pass qweight in their place for the checks
    int rc = check_weights(qweight, qweight, qweight, nullptr, bits, group_size, 1, N, K);
    if (rc != GPTQ_OK) return rc;
    if (!aligned(qweight_sorted, 16) || !aligned(perm, 16) || !aligned(g_idx, 4)) return GPTQ_ERR_MISALIGNED;
    const int64_t bytes = K / 32 * bits * N * 4;
    const uintptr_t a0 = (uintptr_t)qweight, b0 = (uintptr_t)qweight_sorted;
    if (a0 < b0 + bytes && b0 < a0 + bytes) return GPTQ_ERR_BAD_ARG;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess || st != hipStreamCaptureStatusNone) return GPTQ_ERR_BAD_ARG;
    // the order is decided on the host: a stable sort of g_idx (read back)
    std::vector<int32_t> g((size_t)K), p((size_t)K);
    if (hipMemcpyAsync(g.data(), g_idx, (size_t)K * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return GPTQ_ERR_DEVICE;
    const int64_t G = K / group_size;
    std::vector<int64_t> count((size_t)G + 1, 0);
    for (int64_t k = 0; k < K; ++k) {
      if (g[k] < 0 || g[k] >= G) return GPTQ_ERR_BAD_ARG;
      ++count[(size_t)g[k] + 1];
    }
    for (int64_t i = 0; i < G; ++i) {
      if (count[(size_t)i + 1] != group_size) return GPTQ_ERR_BAD_ARG;   // every group exactly group_size rows
      count[(size_t)i + 1] += count[(size_t)i];
    }
    for (int64_t k = 0; k < K; ++k) p[(size_t)count[(size_t)g[k]]++] = (int32_t)k;   // stable counting sort
    if (hipMemcpyAsync(perm, p.data(), (size_t)K * 4, hipMemcpyHostToDevice, stream) != hipSuccess)
      return GPTQ_ERR_DEVICE;
    if (gptq::launch_sort_rows(qweight, perm, qweight_sorted, bits, N, K, stream) != hipSuccess) return GPTQ_ERR_LAUNCH;
    // the host vector must outlive the copy
    return hipStreamSynchronize(stream) == hipSuccess ? GPTQ_OK : GPTQ_ERR_DEVICE;
  } catch (const std::bad_alloc&) {
    return GPTQ_ERR_NO_MEM;
  } catch (...) {
    return GPTQ_ERR_DEVICE;
  }
}

int gptq_gemm_sorted(const void* x, const int32_t* qweight_sorted, const int32_t* qzeros, const void* scales,
                     const int32_t* perm, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
                     void* out, void* stream, int layout, int path, int decode_waves) {
  try {
    if (!perm) return GPTQ_ERR_NULL_PTR;
    if (!aligned(perm, 4)) return GPTQ_ERR_MISALIGNED;
    if (layout != 0 && layout != 1) return GPTQ_ERR_BAD_ARG;
    if (K % 8 != 0) return GPTQ_ERR_BAD_SHAPE;
    return gemm_impl(x, qweight_sorted, qzeros, scales, nullptr, bits, group_size, is_v2, M, N, K, out, stream, path,
                     decode_waves, layout == 1, perm);
  } catch (const std::bad_alloc&) {
    return GPTQ_ERR_NO_MEM;
  } catch (...) {
    return GPTQ_ERR_DEVICE;
  }
}

int gptq_moe_gemm_ex(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                     const int32_t* g_idx, const int32_t* expert_offsets, int n_experts, int max_tokens_per_expert,
                     int bits, int group_size, int is_v2, int64_t T, int64_t N, int64_t K, void* out, void* stream,
                     int path) {
  try {
    return moe_impl(x, qweight, qzeros, scales, g_idx, expert_offsets, n_experts, max_tokens_per_expert, bits,
                    group_size, is_v2, T, N, K, out, stream, path);
  } catch (...) {
    return GPTQ_ERR_DEVICE;
  }
}

int gptq_moe_gemm(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                  const int32_t* g_idx, const int32_t* expert_offsets, int n_experts, int max_tokens_per_expert,
                  int bits, int group_size, int is_v2, int64_t T, int64_t N, int64_t K, void* out, void* stream) {
  return gptq_moe_gemm_ex(x, qweight, qzeros, scales, g_idx, expert_offsets, n_experts, max_tokens_per_expert, bits,
                          group_size, is_v2, T, N, K, out, stream, 0);
}

int gptq_repack_tiled(const int32_t* qweight, int32_t* qweight_tiled, int bits, int64_t N, int64_t K,
                      void* stream) {
  return repack_impl(qweight, qweight_tiled, bits, N, K, 1, stream);
}

int gptq_unrepack_tiled(const int32_t* qweight_tiled, int32_t* qweight, int bits, int64_t N, int64_t K,
                        void* stream) {
  return repack_impl(qweight_tiled, qweight, bits, N, K, 0, stream);
}

int gptq_gemm(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
              const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K, void* out,
              void* stream) {
  return gptq_gemm_ex(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, stream, 0, 0);
}

int gptq_gemm_bf16_ex(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                      const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
                      void* out, void* stream, int path, int decode_waves) {
  try {
    return gemm_impl(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, stream, path,
                     decode_waves, false, nullptr, true);
  } catch (const std::bad_alloc&) {
    return GPTQ_ERR_NO_MEM;
  } catch (...) {
    return GPTQ_ERR_DEVICE;
  }
}

int gptq_gemm_bf16(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                   const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
                   void* out, void* stream) {
  return gptq_gemm_bf16_ex(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, stream, 0, 0);
}

int gptq_gemm_bf16_describe(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                            const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N,
                            int64_t K, const void* out, int path, int decode_waves, char* buf, int64_t buflen) {
  return describe_impl(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, path,
                       decode_waves, false, buf, buflen, true);
}

int gptq_gemm_tiled_bf16_ex(const void* x, const int32_t* qweight_tiled, const int32_t* qzeros, const void* scales,
                            const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N,
                            int64_t K, void* out, void* stream, int path, int decode_waves) {
  try {
    return gemm_impl(x, qweight_tiled, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, stream, path,
                     decode_waves, true, nullptr, true);
  } catch (const std::bad_alloc&) {
    return GPTQ_ERR_NO_MEM;
  } catch (...) {
    return GPTQ_ERR_DEVICE;
  }
}

int gptq_gemm_tiled_bf16(const void* x, const int32_t* qweight_tiled, const int32_t* qzeros, const void* scales,
                         const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
                         void* out, void* stream) {
  return gptq_gemm_tiled_bf16_ex(x, qweight_tiled, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out,
                                 stream, 0, 0);
}

int gptq_gemm_tiled_bf16_describe(const void* x, const int32_t* qweight_tiled, const int32_t* qzeros,
                                  const void* scales, const int32_t* g_idx, int bits, int group_size, int is_v2,
                                  int64_t M, int64_t N, int64_t K, const void* out, int path, int decode_waves,
                                  char* buf, int64_t buflen) {
  return describe_impl(x, qweight_tiled, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, path,
                       decode_waves, true, buf, buflen, true);
}

namespace {
int dequant_impl(const int32_t* qweight, const int32_t* qzeros, const void* scales, const int32_t* g_idx, int bits,
                 int group_size, int is_v2, int64_t N, int64_t K, void* w_out, void* stream, bool bf16) {
  const int rc = gptq_dequant_check(qweight, qzeros, scales, g_idx, bits, group_size, is_v2, N, K, w_out);
  if (rc != GPTQ_OK) return rc;
  gptq::DequantArgs a{};
  a.qweight = qweight;
  a.qzeros = qzeros;
  a.scales = static_cast<const _Float16*>(scales);
  a.g_idx = g_idx;
  a.out = static_cast<_Float16*>(w_out);
  a.N = (int)N;
  a.K = (int)K;
  a.G = (int)(K / group_size);
  a.group_size = group_size;
  a.zero_offset = is_v2 ? 0 : 1;
  a.chunks = (int)(K / 32);
  a.zrow_words = N * bits / 32;
  const hipError_t err = gptq::launch_dequant(bits, a, bf16, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? GPTQ_OK : GPTQ_ERR_LAUNCH;
}
}  // namespace

int gptq_dequant(const int32_t* qweight, const int32_t* qzeros, const void* scales, const int32_t* g_idx, int bits,
                 int group_size, int is_v2, int64_t N, int64_t K, void* w_out, void* stream) {
  return dequant_impl(qweight, qzeros, scales, g_idx, bits, group_size, is_v2, N, K, w_out, stream, false);
}

int gptq_dequant_bf16(const int32_t* qweight, const int32_t* qzeros, const void* scales, const int32_t* g_idx,
                      int bits, int group_size, int is_v2, int64_t N, int64_t K, void* w_out, void* stream) {
  return dequant_impl(qweight, qzeros, scales, g_idx, bits, group_size, is_v2, N, K, w_out, stream, true);
}

int gptq_quantize(const float* w, const int32_t* g_idx, int bits, int group_size, int sym, int is_v2, int64_t N,
                  int64_t K, int32_t* qweight, int32_t* qzeros, void* scales, void* stream) {
  if (!w || !qweight || !qzeros || !scales) return GPTQ_ERR_NULL_PTR;
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return GPTQ_ERR_BAD_BITS;
  if (N <= 0 || K <= 0 || N % 32 != 0 || K % 32 != 0) return GPTQ_ERR_BAD_SHAPE;
  if (N > ((int64_t)1 << 20) || K > ((int64_t)1 << 20) || N * K >= kMaxElems) return GPTQ_ERR_BAD_SHAPE;
  if (group_size <= 0 || K % group_size != 0) return GPTQ_ERR_BAD_GROUP;
  if ((sym != 0 && sym != 1) || (is_v2 != 0 && is_v2 != 1)) return GPTQ_ERR_BAD_ARG;
  if (!aligned(w, 4) || !aligned(qweight, 4) || !aligned(qzeros, 4) || !aligned(scales, 2) ||
      (g_idx && !aligned(g_idx, 4)))
    return GPTQ_ERR_MISALIGNED;
  const hipError_t err = gptq::launch_quantize(w, g_idx, bits, group_size, sym, is_v2, (int)N, (int)K, qweight,
                                               qzeros, scales, reinterpret_cast<hipStream_t>(stream));
  if (err == hipErrorOutOfMemory) return GPTQ_ERR_NO_MEM;
  return err == hipSuccess ? GPTQ_OK : GPTQ_ERR_LAUNCH;
}

int gptq_convert_zeros_check(const int32_t* qzeros_in, const int32_t* qzeros_out, int bits, int64_t G, int64_t N,
                             int to_v2, const int32_t* lossy_count) {
  if (!qzeros_in || !qzeros_out) return GPTQ_ERR_NULL_PTR;
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return GPTQ_ERR_BAD_BITS;
  if (G <= 0 || N <= 0 || N % 32 != 0 || N > ((int64_t)1 << 20) || G > ((int64_t)1 << 20) ||
      G * (N * bits / 32) >= kMaxElems)
    return GPTQ_ERR_BAD_SHAPE;
  if (to_v2 != 0 && to_v2 != 1) return GPTQ_ERR_BAD_ARG;
  if (!aligned(qzeros_in, 4) || !aligned(qzeros_out, 4) || (lossy_count && !aligned(lossy_count, 4)))
    return GPTQ_ERR_MISALIGNED;
  const int64_t bytes = G * (N * bits / 32) * 4;
  const uintptr_t a = (uintptr_t)qzeros_in, b = (uintptr_t)qzeros_out;
  if (a != b && a < b + bytes && b < a + bytes) return GPTQ_ERR_BAD_ARG;  // partial overlap
  return GPTQ_OK;
}

int gptq_convert_zeros(const int32_t* qzeros_in, int32_t* qzeros_out, int bits, int64_t G, int64_t N, int to_v2,
                       int32_t* lossy_count, void* stream) {
  const int rc = gptq_convert_zeros_check(qzeros_in, qzeros_out, bits, G, N, to_v2, lossy_count);
  if (rc != GPTQ_OK) return rc;
  const hipError_t err = gptq::launch_convert_zeros(qzeros_in, qzeros_out, bits, G, N, to_v2, lossy_count,
                                                    reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? GPTQ_OK : GPTQ_ERR_LAUNCH;
}

const char* gptq_strerror(int code) {
  switch (code) {
    case GPTQ_OK: return "ok";
    case GPTQ_ERR_NULL_PTR: return "a required pointer is NULL";
    case GPTQ_ERR_BAD_BITS: return "bits must be 2, 3, 4 or 8";
    case GPTQ_ERR_BAD_SHAPE: return "bad shape: need M >= 0, N and K positive multiples of 32, within size limits";
    case GPTQ_ERR_BAD_GROUP: return "group_size must be positive and divide K";
    case GPTQ_ERR_MISALIGNED: return "misaligned pointer (x, qweight, g_idx, out: 16 B; scales: 8 B; qzeros: 4 B)";
    case GPTQ_ERR_NO_MEM: return "device memory allocation failed (a temporary or workspace; none is allocated during stream capture)";
    case GPTQ_ERR_LAUNCH: return "kernel launch failed";
    case GPTQ_ERR_DEVICE: return "HIP runtime call failed";
    case GPTQ_ERR_BAD_ARG: return "option out of range (is_v2, sym, to_v2, path or decode_waves) or overlapping buffers";
    default: return "unknown error";
  }
}

void gptq_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  int cur = 0;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  for (auto& w : g_ws) {
    if (hipSetDevice(w.device) == hipSuccess) {
      (void)hipDeviceSynchronize();
      (void)hipFree(w.base);
    }
  }
  for (auto& r : g_retired) {
    if (hipSetDevice(r.device) == hipSuccess) {
      (void)hipDeviceSynchronize();
      (void)hipFree(r.base);
    }
  }
  g_ws.clear();
  g_retired.clear();
  if (have) (void)hipSetDevice(cur);
}

int gptq_gemm_noalloc(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                      const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
                      void* out, void* stream_ptr) {
  try {
    gptq::GemmArgs a;
    bool use_decode = false, per_elem = false;
    // the same plan as gptq_gemm, with split-K partial sums limited to what
    // the scratch holds (the planner never needs more than about 1 MiB)
    const int rc = plan_gemm(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, 0, 0, false,
                             &a, &use_decode, &per_elem, true, false, kScratchSumBytes);
    if (rc != GPTQ_OK || M == 0) return rc;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
    if (a.ks > 1) {
      if (split_counter_bytes(a, use_decode) > kScratchCounterBytes ||
          (int64_t)a.ks * a.M * a.N * 4 > kScratchSumBytes)
        return GPTQ_ERR_NO_MEM;                      // beyond the static scratch (not reached by the planner)
      char* p = nullptr;
      const int rs = scratch_for_device(stream, &p);
      if (rs != GPTQ_OK) return rs;
      a.cnt = reinterpret_cast<uint32_t*>(p);
      a.ws = reinterpret_cast<float*>(p + kScratchCounterBytes);
    }
    const hipError_t err = use_decode ? gptq::launch_decode(bits, per_elem, a, stream)
                                      : gptq::launch_prefill(bits, per_elem, a, stream);
    return err == hipSuccess ? GPTQ_OK : GPTQ_ERR_LAUNCH;
  } catch (const std::bad_alloc&) {
    return GPTQ_ERR_NO_MEM;
  } catch (...) {
    return GPTQ_ERR_DEVICE;
  }
}

int gptq_read_ceiling(const void* buf, int64_t bytes, void* sink, void* stream) {
  if (!buf || !sink) return GPTQ_ERR_NULL_PTR;
  if (bytes < 0 || bytes % 16 != 0 || bytes > ((int64_t)1 << 40)) return GPTQ_ERR_BAD_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return GPTQ_ERR_MISALIGNED;
  if (bytes == 0) return GPTQ_OK;
  const hipError_t err = gptq::launch_read_ceiling(buf, bytes, sink, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? GPTQ_OK : GPTQ_ERR_LAUNCH;
}

int gptq_abi_version(void) { return 1; }

}  // extern "C"
