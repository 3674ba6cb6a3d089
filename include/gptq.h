/*
 * gptq.h -- C ABI of libgptq.so, the MI355X (gfx950) GPTQ weight-only GEMM.
 *
 * What it computes (page "Enhancing vLLM's support for the GPTQv2 format:
 * analysis and implementation", sections "Weight quantization of LLMs",
 * "From GPTQv1 to GPTQv2" and "Adjustment details"):
 *
 *   g(k)      = g_idx ? g_idx[k] : k / group_size
 *   q[k,n]    = b-bit field k of column n of qweight
 *   z[g,n]    = b-bit field n of row g of qzeros  + (is_v2 ? 0 : 1)
 *   W^[k,n]   = fp16_round((q[k,n] - z[g(k),n]) * scales[g(k),n])
 *   out[m,n]  = fp16_round( sum_k x[m,k] * W^[k,n] )   (fp32 accumulation)
 *
 * Data layout (all row-major, caller-owned device memory):
 *   x        fp16  [M, K]
 *   qweight  int32 [K*bits/32, N]  packed along K: column n's K fields form one
 *                                  LSB-first bitstream of bits-wide fields;
 *                                  word r holds stream bits [32r, 32r+32).  For
 *                                  bits = 3 one 32-value chunk spans three
 *                                  consecutive rows (fields 10 and 21 straddle).
 *   qzeros   int32 [G, N*bits/32]  packed along N, same bitstream rule per row.
 *   scales   fp16  [G, N]
 *   g_idx    int32 [K] or NULL     group of every row k (act-order); NULL means
 *                                  k / group_size.
 *   out      fp16  [M, N]          written, never accumulated into.
 * with G = K / group_size.  The int32 words are bit containers (no sign).
 *
 * Ownership and streams: the library keeps no caller pointer after a call
 * returns.  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and is asynchronous: buffers must stay valid until that work
 * completes, and a device-side fault surfaces at the caller's next
 * synchronisation.  The library's own device memory: a workspace per
 * (device, stream) -- split-K partial sums and arrival counters, and the
 * gathered x of gptq_gemm_sorted -- allocated (hipMalloc, zeroed on the
 * stream) by the first call on that stream that needs it, and replaced by a
 * larger one when a later call needs more; a replaced buffer is not freed
 * until gptq_release, because work queued earlier and graphs captured earlier
 * on that stream keep its address.  gptq_quantize uses a stream-ordered
 * temporary freed on the same stream.
 * HIP graphs: calls on one stream may be captured.  A capture never allocates
 * (a split-K call captured before its stream has a workspace runs unsplit
 * instead; gptq_gemm_sorted returns GPTQ_ERR_NO_MEM), and the graph keeps
 * using the workspace its capture stream had at capture time.  So a replay
 * shares that workspace with every other call on the capture stream: replays
 * (on any stream) must not overlap such calls or each other, and
 * gptq_release must not run while such a graph may still replay.
 * Concurrent calls on different streams are otherwise safe; two host threads
 * enqueuing on the same stream at once are not.
 *
 * Errors: every function returns GPTQ_OK (0) or a negative gptq_status code;
 * nothing is launched when an argument check fails, and no C++ exception
 * crosses the ABI.  M == 0 returns GPTQ_OK without launching.
 *
 * Preconditions that are not checked: g_idx entries lie in [0, G) (an entry
 * outside is clamped into range, so memory stays in bounds but the result is
 * unspecified); scales are finite; out does not alias an input.
 */
#ifndef GPTQ_H_
#define GPTQ_H_

#include <stdint.h>

#if defined(__GNUC__)
#define GPTQ_API __attribute__((visibility("default")))
#else
#define GPTQ_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gptq_status {
  GPTQ_OK = 0,
  GPTQ_ERR_NULL_PTR = -1,    /* a required pointer is NULL */
  GPTQ_ERR_BAD_BITS = -2,    /* bits not in {2, 3, 4, 8} */
  GPTQ_ERR_BAD_SHAPE = -3,   /* M < 0, N <= 0, K <= 0, K % 32, N % 32, or a size limit */
  GPTQ_ERR_BAD_GROUP = -4,   /* group_size <= 0 or K % group_size != 0 */
  GPTQ_ERR_MISALIGNED = -5,  /* x, qweight, g_idx, out not 16-byte aligned; scales not 8; qzeros not 4 */
  GPTQ_ERR_NO_MEM = -6,      /* a temporary or workspace could not be allocated */
  GPTQ_ERR_LAUNCH = -7,      /* a kernel launch failed */
  GPTQ_ERR_DEVICE = -8,      /* no current HIP device or a HIP runtime call failed */
  GPTQ_ERR_BAD_ARG = -9      /* is_v2 / sym / to_v2 not 0 or 1, a gptq_gemm_ex option out of range,
                                or partially overlapping conversion buffers */
} gptq_status;

/* Size limits (GPTQ_ERR_BAD_SHAPE beyond them): M <= 2^24, N and K <= 2^20,
 * and M*K, K*N, M*N each below 2^31 elements. */

/*
 * y = x . dequant(W): the GPTQ weight-only GEMM (the `gptq_gemm` call of the
 * page above, whose `use_v2_format` flag is `is_v2` here).
 *   bits        2, 3, 4 or 8.
 *   group_size  rows per quantization group; K % group_size == 0.
 *   is_v2       1: zeros are stored as is (GPTQv2); 0: stored zero + 1 (GPTQv1).
 *               Mandatory: there is no default and no format detection.
 *   M, N, K     x is [M,K], out is [M,N]; N % 32 == 0 and K % 32 == 0.
 *   stream      hipStream_t as void*.
 * M <= 16 runs the decode kernel (workgroups own column tiles, MFMA with M
 * padded to 16; for narrow N with K >= 8192 the workgroups of a tile split K
 * and the last to finish adds the fp32 partial sums, in a fixed order, so
 * results are deterministic either way); larger M runs the MFMA prefill
 * kernel (32-, 64-, 128- or 256-row tiles; when the tiles of up to 128 rows
 * are too few to fill the GPU, e.g. M <= 512 with N of a few thousand, their
 * workgroups split K and store fp32 partial sums, which a second kernel on
 * the same stream adds in split order, so results are deterministic too).
 * Exception: a layer the prefill kernel would dequantize element by element
 * (g_idx given, or group_size % 64 != 0) runs the decode kernel over blocks
 * of 16 rows for 16 < M <= 4096, without a K split.
 */
GPTQ_API int gptq_gemm(const void* x, const int32_t* qweight, const int32_t* qzeros,
              const void* scales, const int32_t* g_idx, int bits, int group_size,
              int is_v2, int64_t M, int64_t N, int64_t K, void* out, void* stream);

/*
 * gptq_gemm for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and checks as gptq_gemm; it calls no hipMalloc / hipFree.  Where
 * gptq_gemm splits K over workgroups (decode with narrow N and long K,
 * prefill with few tiles), the decode arrival counters and the fp32 partial
 * sums live in a static device array of 2 MiB that the library holds on every device it
 * runs on until the process ends (gptq_release does not free it); the plan
 * keeps the partial sums within it (at most ks * M * N * 4 bytes of 2 MiB -
 * 64 KiB, and 4 bytes per decode tile in the first 64 KiB), and a plan that needed
 * more would return GPTQ_ERR_NO_MEM before launching.  Decode plans are the
 * same as gptq_gemm's and so is the result, bit for bit; a prefill launch
 * whose partial sums would exceed the array splits K fewer times than
 * gptq_gemm (or not at all), which changes only the order of the fp32 sums.  The counters
 * are cleared by a kernel on `stream` at the first call on a device (the
 * array also starts zeroed) and every split-K decode kernel leaves them at zero.
 * All calls on one device share that one array: calls that may overlap on a
 * device (concurrent streams, or graph replays overlapping each other or
 * eager calls) race on it and must be serialized by the caller.
 */
GPTQ_API int gptq_gemm_noalloc(const void* x, const int32_t* qweight, const int32_t* qzeros,
                               const void* scales, const int32_t* g_idx, int bits, int group_size,
                               int is_v2, int64_t M, int64_t N, int64_t K, void* out, void* stream);

/*
 * gptq_gemm with explicit kernel choice, for tests and tuning.
 *   path          0 = automatic (as gptq_gemm), 1 = decode kernel (requires
 *                 M <= 16), 2 = prefill kernel (any M).
 *   decode_waves  0 = automatic; 1..16 = waves per decode workgroup (each
 *                 workgroup owns a column tile for all of K; its waves split K;
 *                 values above the kernel's limit, 16 for M = 1 with 16-column
 *                 tiles and 8 otherwise, are clamped to it).
 * Other values give GPTQ_ERR_BAD_ARG.
 */
GPTQ_API int gptq_gemm_ex(const void* x, const int32_t* qweight, const int32_t* qzeros,
                 const void* scales, const int32_t* g_idx, int bits, int group_size,
                 int is_v2, int64_t M, int64_t N, int64_t K, void* out, void* stream,
                 int path, int decode_waves);

/*
 * W^ = dequant(W) into w_out, fp16 [K, N] row-major (the "reconstruct" kernel
 * of the page's "Adjustment details" section).  Bit-exact: one round-to-
 * nearest-even of the exact product (q - z) * s per element, fp16 subnormals
 * kept.  Same arguments and checks as gptq_gemm minus x and M.
 */
GPTQ_API int gptq_dequant(const int32_t* qweight, const int32_t* qzeros, const void* scales,
                 const int32_t* g_idx, int bits, int group_size, int is_v2,
                 int64_t N, int64_t K, void* w_out, void* stream);

/*
 * Argument checks of gptq_gemm / gptq_gemm_ex / gptq_dequant only (the GEMM
 * checks also pick the kernel and its launch shape): pure host code, touches
 * no device and no pointer target.  Returns the code the full call would return for these
 * arguments before any HIP call.
 */
GPTQ_API int gptq_gemm_check(const void* x, const int32_t* qweight, const int32_t* qzeros,
                    const void* scales, const int32_t* g_idx, int bits, int group_size,
                    int is_v2, int64_t M, int64_t N, int64_t K, const void* out);
GPTQ_API int gptq_gemm_ex_check(const void* x, const int32_t* qweight, const int32_t* qzeros,
                       const void* scales, const int32_t* g_idx, int bits, int group_size,
                       int is_v2, int64_t M, int64_t N, int64_t K, const void* out,
                       int path, int decode_waves);
/*
 * Names the kernel instantiation and launch shape gptq_gemm_ex would use for
 * these arguments, as a NUL-terminated string in buf (at most buflen bytes,
 * truncated if longer), e.g. for profiles.  Pure host code like the checks
 * above; returns the same code they do (GPTQ_ERR_NULL_PTR also for a NULL buf
 * or buflen <= 0).
 */
GPTQ_API int gptq_gemm_describe(const void* x, const int32_t* qweight, const int32_t* qzeros,
                       const void* scales, const int32_t* g_idx, int bits, int group_size,
                       int is_v2, int64_t M, int64_t N, int64_t K, const void* out,
                       int path, int decode_waves, char* buf, int64_t buflen);
GPTQ_API int gptq_dequant_check(const int32_t* qweight, const int32_t* qzeros, const void* scales,
                       const int32_t* g_idx, int bits, int group_size, int is_v2,
                       int64_t N, int64_t K, const void* w_out);

/*
 * Min/max round-to-nearest quantization of W (fp32 [K, N] row-major, device)
 * into qweight, qzeros and scales with the layout above (page "Enhancing
 * vLLM's support for the GPTQv2 format", sections "Weight quantization of
 * LLMs" and "From GPTQv1 to GPTQv2"):
 *   scale = fp16((wmax - wmin) / (2^b - 1)), computed in fp64 (0 becomes 1.0)
 *   zero  = clamp(-round(wmin / scale), 0, 2^b - 1)   (sym: wmax = -wmin =
 *           max|w| and zero = round((2^b - 1) / 2) = 2^(b-1))
 *   q     = clamp(round(w / scale) + zero, 0, 2^b - 1)
 *   stored zero = is_v2 ? zero : clamp(zero - 1, 0, 2^b - 1)
 * round() is half-to-even and every division that decides an integer is done
 * in fp64 with the stored fp16 scale.  g_idx (nullable) assigns rows to groups
 * as in gptq_gemm.  sym and is_v2 are 0 or 1.  Alignment: 4 bytes for w,
 * qweight, qzeros, g_idx; 2 bytes for scales.  Enqueues two kernels and a
 * stream-ordered temporary of G*N bytes on `stream`.
 */
GPTQ_API int gptq_quantize(const float* w, const int32_t* g_idx, int bits, int group_size,
                           int sym, int is_v2, int64_t N, int64_t K, int32_t* qweight,
                           int32_t* qzeros, void* scales, void* stream);

/*
 * GPTQv1 <-> GPTQv2 conversion of packed zero points, qzeros [G, N*bits/32]
 * int32 (layout as for gptq_gemm), device memory (page "Enhancing vLLM's
 * support for the GPTQv2 format", section "From GPTQv1 to GPTQv2": v1 stores
 * clamp(zero - 1) and adds 1 at run time, v2 stores zero).
 *   to_v2 = 1: every stored b-bit field f becomes f + 1; a field of 2^b - 1
 *              (zero 2^b, never written by a v1 quantizer) saturates at 2^b - 1.
 *   to_v2 = 0: f becomes max(f - 1, 0); a v2 zero of 0 is stored as 0 and
 *              reads back as zero 1 (the format's documented loss).
 * Saturated (to_v2 = 1) or clamped (to_v2 = 0) fields are lossy: when
 * lossy_count (device int32, nullable) is given, their number is added to it
 * (the caller zeroes it first).  qzeros_out may equal qzeros_in (in place);
 * any other overlap is GPTQ_ERR_BAD_ARG.  N % 32 == 0, G >= 1; pointers 4-byte
 * aligned.  Enqueues one kernel on `stream`; allocates nothing.
 */
GPTQ_API int gptq_convert_zeros(const int32_t* qzeros_in, int32_t* qzeros_out, int bits, int64_t G, int64_t N,
                                int to_v2, int32_t* lossy_count, void* stream);
/* Argument checks of gptq_convert_zeros only (pure host, no launch). */
GPTQ_API int gptq_convert_zeros_check(const int32_t* qzeros_in, const int32_t* qzeros_out, int bits, int64_t G,
                                      int64_t N, int to_v2, const int32_t* lossy_count);

/*
 * Tiled qweight layout: the words of the checkpoint layout, reordered so
 * that each 16-column tile is one contiguous run (an offline re-layout in the
 * spirit of the page "Weight-only INT4 quantization: GPTQ, AWQ and the Marlin
 * kernel", section 6.1; the order is this library's own):
 *   qweight_tiled int32 [N/16][K/32][bits][16],
 *   qweight_tiled[t][c][r][j] = qweight[c*bits + r][16*t + j]
 * for 2, 3 and 8 bits; a 4-bit word also has its eight fields in pair order
 * (field 2i of the checkpoint word in nibble i, field 2i + 1 in nibble i + 4,
 * i < 4), so that one mask per 16-bit half gives two consecutive fields (the
 * prefill kernel builds its MFMA operand with one shift and four masks per
 * word instead of four byte permutes).
 * The decode kernel then streams each workgroup's weights from one contiguous
 * region instead of 64-256-byte pieces of rows N*4 bytes apart (measured on
 * MI355X: 5-11% less time per Llama-7B-shaped decode layer at M = 1).
 * qzeros, scales and g_idx are unchanged.
 *
 * gptq_repack_tiled / gptq_unrepack_tiled convert between the layouts on
 * `stream` (one kernel).  Same N, K, bits rules as
 * gptq_gemm; both buffers 16-byte aligned, K*bits/32*N int32 words each,
 * and they must not overlap (GPTQ_ERR_BAD_ARG, also for in == out).
 */
GPTQ_API int gptq_repack_tiled(const int32_t* qweight, int32_t* qweight_tiled, int bits, int64_t N, int64_t K,
                               void* stream);
GPTQ_API int gptq_unrepack_tiled(const int32_t* qweight_tiled, int32_t* qweight, int bits, int64_t N, int64_t K,
                                 void* stream);

/* gptq_gemm / gptq_gemm_ex / gptq_gemm_describe with qweight in the tiled
 * layout: same arguments, results and error codes (decode workgroups then
 * own 16-column tiles). */
GPTQ_API int gptq_gemm_tiled(const void* x, const int32_t* qweight_tiled, const int32_t* qzeros,
                             const void* scales, const int32_t* g_idx, int bits, int group_size, int is_v2,
                             int64_t M, int64_t N, int64_t K, void* out, void* stream);
GPTQ_API int gptq_gemm_tiled_ex(const void* x, const int32_t* qweight_tiled, const int32_t* qzeros,
                                const void* scales, const int32_t* g_idx, int bits, int group_size, int is_v2,
                                int64_t M, int64_t N, int64_t K, void* out, void* stream, int path,
                                int decode_waves);
GPTQ_API int gptq_gemm_tiled_describe(const void* x, const int32_t* qweight_tiled, const int32_t* qzeros,
                                      const void* scales, const int32_t* g_idx, int bits, int group_size,
                                      int is_v2, int64_t M, int64_t N, int64_t K, const void* out, int path,
                                      int decode_waves, char* buf, int64_t buflen);

/*
 * Act-order layers with their rows sorted by group (page "GPTQ quantization
 * principles and engineering practice", section 3.4: act order quantizes
 * rows out of order, so g_idx scatters each group's rows over K).  Sorting
 * the rows by group makes every group contiguous again, and
 *   y = x . W^ = x[:, perm] . W^[perm, :]
 * so the layer runs on the grouped fast path with x gathered by perm.
 *
 * gptq_sort_act_order: perm[i] = original row of sorted row i (a stable sort
 * of g_idx, decided on the host: g_idx is read back, so the call synchronizes
 * `stream`), and qweight_sorted [K*bits/32, N] = qweight's packed rows in that
 * order (bit-exact field moves).  Requires every group to hold exactly
 * group_size rows and g_idx entries in [0, G) (else GPTQ_ERR_BAD_ARG: use
 * gptq_gemm with g_idx instead); not during stream capture (GPTQ_ERR_BAD_ARG).
 * qzeros and scales are unchanged.  qweight_sorted must not overlap qweight;
 * qweight_sorted and perm 16-byte aligned.
 *
 * gptq_gemm_sorted: gptq_gemm for such a layer: x is gathered by perm into
 * the stream's library workspace (M*K*2 bytes, allocated on first use outside
 * stream capture, else GPTQ_ERR_NO_MEM) and the grouped GEMM runs on it.
 * layout: 0 = qweight_sorted in the checkpoint layout, 1 = tiled (after
 * gptq_repack_tiled).  path / decode_waves as for gptq_gemm_ex.
 */
GPTQ_API int gptq_sort_act_order(const int32_t* qweight, const int32_t* g_idx, int bits, int group_size, int64_t N,
                                 int64_t K, int32_t* qweight_sorted, int32_t* perm, void* stream);
GPTQ_API int gptq_gemm_sorted(const void* x, const int32_t* qweight_sorted, const int32_t* qzeros,
                              const void* scales, const int32_t* perm, int bits, int group_size, int is_v2,
                              int64_t M, int64_t N, int64_t K, void* out, void* stream, int layout, int path,
                              int decode_waves);

/*
 * bfloat16 activations (page "Weight-only INT4 quantization: GPTQ, AWQ and
 * the Marlin kernel", section 1.2: activations stay 16-bit, fp16 or bf16).
 * Same arguments, layouts, checks, return codes and workspace rules as
 * gptq_gemm / gptq_gemm_ex / gptq_gemm_describe / gptq_dequant, with x,
 * scales and out (w_out) holding bfloat16 instead of fp16:
 *   W^[k, n] = bf16_RNE((q - z) * s),  y = x . W^ (fp32 accumulate, one
 *   bfloat16 rounding of each output).
 * gptq_dequant_bf16 is bit-exact with that formula.  The GEMM kernels form
 * the same W^ values as fma(q, s, -z s) in fp32, exact while |s| < 2^119 (so
 * that z s stays finite; real scales are many orders below).  Decode (M <= 16) always
 * dequantizes element by element (act order or not); prefill uses the same
 * tiles as the fp16 kernel.  The gptq_gemm_tiled_bf16* calls take the tiled
 * qweight layout of gptq_repack_tiled (as gptq_gemm_tiled*); there are no
 * sorted or grouped bfloat16 variants.
 */
GPTQ_API int gptq_gemm_bf16(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                            const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N,
                            int64_t K, void* out, void* stream);
GPTQ_API int gptq_gemm_bf16_ex(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                               const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N,
                               int64_t K, void* out, void* stream, int path, int decode_waves);
GPTQ_API int gptq_gemm_bf16_describe(const void* x, const int32_t* qweight, const int32_t* qzeros,
                                     const void* scales, const int32_t* g_idx, int bits, int group_size, int is_v2,
                                     int64_t M, int64_t N, int64_t K, const void* out, int path, int decode_waves,
                                     char* buf, int64_t buflen);
GPTQ_API int gptq_dequant_bf16(const int32_t* qweight, const int32_t* qzeros, const void* scales,
                               const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t N, int64_t K,
                               void* w_out, void* stream);
GPTQ_API int gptq_gemm_tiled_bf16(const void* x, const int32_t* qweight_tiled, const int32_t* qzeros,
                                  const void* scales, const int32_t* g_idx, int bits, int group_size, int is_v2,
                                  int64_t M, int64_t N, int64_t K, void* out, void* stream);
GPTQ_API int gptq_gemm_tiled_bf16_ex(const void* x, const int32_t* qweight_tiled, const int32_t* qzeros,
                                     const void* scales, const int32_t* g_idx, int bits, int group_size, int is_v2,
                                     int64_t M, int64_t N, int64_t K, void* out, void* stream, int path,
                                     int decode_waves);
GPTQ_API int gptq_gemm_tiled_bf16_describe(const void* x, const int32_t* qweight_tiled, const int32_t* qzeros,
                                           const void* scales, const int32_t* g_idx, int bits, int group_size,
                                           int is_v2, int64_t M, int64_t N, int64_t K, const void* out, int path,
                                           int decode_waves, char* buf, int64_t buflen);

/*
 * Grouped (mixture-of-experts) GEMM: for every expert e,
 *   out[r, :] = x[r, :] . dequant(expert e's weights)   for r in [off[e], off[e+1])
 * i.e. one gptq_gemm per expert over the tokens routed to it, in one launch
 * (page "Weight-only INT4 quantization: GPTQ, AWQ and the Marlin kernel",
 * section 7: GPTQ quantizes the expert weights of MoE models too).
 *   x               fp16 [T, K], tokens sorted by expert (device)
 *   qweight         int32 [E][K*bits/32][N]  (checkpoint layout per expert)
 *   qzeros          int32 [E][G][N*bits/32],  scales fp16 [E][G][N]
 *   g_idx           int32 [E][K] or NULL
 *   expert_offsets  int32 [E+1] device: expert e's rows are [off[e], off[e+1]),
 *                   nondecreasing, off[0] = 0, off[E] <= T (values are clamped
 *                   to [0, T], so bad offsets never reach outside x / out)
 *   max_tokens_per_expert  host bound on off[e+1] - off[e]: only the first
 *                   max_tokens_per_expert rows of each expert are computed;
 *                   rows beyond them keep their out contents
 *   out             fp16 [T, N]; rows of no expert are left as they were.
 * Same bits / group_size / is_v2 / N / K rules and alignment as gptq_gemm.
 * Batches of up to 16 rows per expert (max_tokens_per_expert <= 16) run the
 * decode kernel (one block of up to 16 rows per expert, MFMA with rows padded
 * to 16); larger ones the prefill kernel in 128-row tiles per expert (each
 * tile reads its expert's weights once).  Allocates nothing;
 * deterministic.  T == 0 or max_tokens_per_expert == 0 launches nothing.
 */
GPTQ_API int gptq_moe_gemm(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                           const int32_t* g_idx, const int32_t* expert_offsets, int n_experts,
                           int max_tokens_per_expert, int bits, int group_size, int is_v2, int64_t T, int64_t N,
                           int64_t K, void* out, void* stream);

/*
 * gptq_moe_gemm with the kernel chosen by the caller: path 0 = as
 * gptq_moe_gemm, 1 = the decode kernel (blocks of 16 rows) whatever the batch,
 * 2 = the prefill kernel (128-row tiles) whatever the batch.  Other path values
 * give GPTQ_ERR_BAD_ARG.  Results of either kernel meet the gptq_gemm bar.
 */
GPTQ_API int gptq_moe_gemm_ex(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                              const int32_t* g_idx, const int32_t* expert_offsets, int n_experts,
                              int max_tokens_per_expert, int bits, int group_size, int is_v2, int64_t T,
                              int64_t N, int64_t K, void* out, void* stream, int path);

/*
 * Memory-read reference for the decode kernels: reads `bytes` bytes at buf
 * (device memory) exactly once with 16-byte nontemporal loads and does
 * nothing else (decode reads every packed weight once per call, page
 * "Weight-only INT4 quantization: GPTQ, AWQ and the Marlin kernel", section
 * 1.1, so a plain read of a layer's weight bytes is the achievable floor of
 * its decode launch).  bytes is a multiple of 16, at most 2^40; buf is 16-byte
 * aligned.  sink is a 4-byte aligned device word that the kernel writes only
 * for contents it never meets in practice (it keeps the loads from being
 * optimized away); its value is meaningless.  Enqueues one kernel on
 * `stream`; bytes == 0 launches nothing.
 */
GPTQ_API int gptq_read_ceiling(const void* buf, int64_t bytes, void* sink, void* stream);

/* Static text for a gptq_status code ("unknown error" for other values). */
GPTQ_API const char* gptq_strerror(int code);

/* Releases library-owned device memory (the split-K workspaces of every device
 * and stream), after synchronising those devices.  Later calls allocate again
 * as needed.  Not to be called while another thread is calling the library or
 * while a captured graph that used a workspace may still replay. */
GPTQ_API void gptq_release(void);

/* Library ABI version: 1. */
GPTQ_API int gptq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_H_ */
