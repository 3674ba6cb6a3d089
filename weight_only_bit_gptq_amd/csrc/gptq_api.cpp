// extern "C" entry points of libgptq.so: argument checks, kernel choice,
// split-K workspace and launches on the caller's stream.  No exception leaves
// this file; every failure is a gptq_status code.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <map>
#include <mutex>
#include <new>
#include <utility>

#include "../../include/gptq.h"
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
  if (!aligned(qweight, 16) || !aligned(scales, 8) || !aligned(qzeros, 4) || (g_idx && !aligned(g_idx, 4)))
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

// ---- split-K workspace, one per (device, stream)
struct Workspace {
  float* partial = nullptr;
  size_t partial_elems = 0;
  int* counters = nullptr;
  size_t counter_elems = 0;
};

std::mutex g_ws_mutex;
std::map<std::pair<int, void*>, Workspace> g_ws;

int get_workspace(int device, hipStream_t stream, size_t partial_elems, size_t counter_elems, Workspace** out) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& ws = g_ws[std::make_pair(device, (void*)stream)];
  if (ws.partial_elems < partial_elems || ws.counter_elems < counter_elems) {
    if (ws.partial || ws.counters) {
      if (hipStreamSynchronize(stream) != hipSuccess) return GPTQ_ERR_DEVICE;
      (void)hipFree(ws.partial);
      (void)hipFree(ws.counters);
      ws = Workspace{};
    }
    const size_t pe = partial_elems > 0 ? partial_elems : 1;
    const size_t ce = counter_elems > 0 ? counter_elems : 1;
    if (hipMalloc(&ws.partial, pe * sizeof(float)) != hipSuccess) {
      ws = Workspace{};
      return GPTQ_ERR_NO_MEM;
    }
    if (hipMalloc(&ws.counters, ce * sizeof(int)) != hipSuccess) {
      (void)hipFree(ws.partial);
      ws = Workspace{};
      return GPTQ_ERR_NO_MEM;
    }
    // counters start at zero; every reducing workgroup puts its counter back to zero
    if (hipMemset(ws.counters, 0, ce * sizeof(int)) != hipSuccess) return GPTQ_ERR_DEVICE;
    ws.partial_elems = pe;
    ws.counter_elems = ce;
  }
  *out = &ws;
  return GPTQ_OK;
}

// Decode launch shape: 64-column tiles x K slices; aim for ~1024 workgroups.
void decode_shape(int M, int N, int K, int forced_split, bool per_elem, int* tiles, int* splits,
                  int* wg_chunks) {
  const int C = K / 32;
  const int T = (N + 63) / 64;
  constexpr int kTargetWorkgroups = 1024;
  int S = forced_split > 0 ? forced_split : (kTargetWorkgroups + T / 2) / T;
  if (S < 1) S = 1;
  if (S > C) S = C;
  int wc = (C + S - 1) / S;
  wc = (wc + 3) & ~3;
  while (wc > 4 && gptq::decode_lds_bytes(M, wc, per_elem) > 49152) wc -= 4;
  *tiles = T;
  *wg_chunks = wc;
  *splits = (C + wc - 1) / wc;
}

int gemm_impl(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
              const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
              void* out, void* stream_ptr, int path, int split_k) {
  if (path < 0 || path > 2 || split_k < 0) return GPTQ_ERR_BAD_ARG;
  int rc = check_gemm(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out);
  if (rc != GPTQ_OK) return rc;
  if (path == 1 && M > 16) return GPTQ_ERR_BAD_ARG;
  if (M == 0) return GPTQ_OK;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);

  gptq::GemmArgs a{};
  a.x = static_cast<const _Float16*>(x);
  a.qweight = qweight;
  a.qzeros = qzeros;
  a.scales = static_cast<const _Float16*>(scales);
  a.g_idx = g_idx;
  a.out = static_cast<_Float16*>(out);
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.G = (int)(K / group_size);
  a.group_size = group_size;
  a.zero_offset = is_v2 ? 0 : 1;
  a.chunks = (int)(K / 32);
  a.zrow_words = N * bits / 32;

  const bool use_decode = (path == 1) || (path == 0 && M <= 16);
  hipError_t err;
  if (use_decode) {
    const bool per_elem = (g_idx != nullptr) || (group_size % 32 != 0);
    decode_shape(a.M, a.N, a.K, split_k, per_elem, &a.tiles, &a.splits, &a.wg_chunks);
    if (a.splits > 1) {
      int device = 0;
      if (hipGetDevice(&device) != hipSuccess) return GPTQ_ERR_DEVICE;
      Workspace* ws = nullptr;
      rc = get_workspace(device, stream, (size_t)a.tiles * a.splits * a.M * 64, (size_t)a.tiles, &ws);
      if (rc != GPTQ_OK) return rc;
      a.partial = ws->partial;
      a.counters = ws->counters;
    }
    err = gptq::launch_decode(bits, per_elem, a, stream);
  } else {
    const bool per_elem = (g_idx != nullptr) || (group_size % 64 != 0);
    gptq::prefill_shape(a.M, a.N, &a.tiles_m, &a.tiles_n);
    err = gptq::launch_prefill(bits, per_elem, a, stream);
  }
  return err == hipSuccess ? GPTQ_OK : GPTQ_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int gptq_gemm_check(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                    const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K,
                    const void* out) {
  return check_gemm(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out);
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
                 void* out, void* stream, int path, int split_k) {
  try {
    return gemm_impl(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, stream, path,
                     split_k);
  } catch (const std::bad_alloc&) {
    return GPTQ_ERR_NO_MEM;
  } catch (...) {
    return GPTQ_ERR_DEVICE;
  }
}

int gptq_gemm(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales,
              const int32_t* g_idx, int bits, int group_size, int is_v2, int64_t M, int64_t N, int64_t K, void* out,
              void* stream) {
  return gptq_gemm_ex(x, qweight, qzeros, scales, g_idx, bits, group_size, is_v2, M, N, K, out, stream, 0, 0);
}

int gptq_dequant(const int32_t* qweight, const int32_t* qzeros, const void* scales, const int32_t* g_idx, int bits,
                 int group_size, int is_v2, int64_t N, int64_t K, void* w_out, void* stream) {
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
  const hipError_t err = gptq::launch_dequant(bits, a, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? GPTQ_OK : GPTQ_ERR_LAUNCH;
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

const char* gptq_strerror(int code) {
  switch (code) {
    case GPTQ_OK: return "ok";
    case GPTQ_ERR_NULL_PTR: return "a required pointer is NULL";
    case GPTQ_ERR_BAD_BITS: return "bits must be 2, 3, 4 or 8";
    case GPTQ_ERR_BAD_SHAPE: return "bad shape: need M >= 0, N and K positive multiples of 32, within size limits";
    case GPTQ_ERR_BAD_GROUP: return "group_size must be positive and divide K";
    case GPTQ_ERR_MISALIGNED: return "misaligned pointer (x, qweight, out: 16 B; scales: 8 B; qzeros, g_idx: 4 B)";
    case GPTQ_ERR_NO_MEM: return "device memory allocation failed (workspace or temporary)";
    case GPTQ_ERR_LAUNCH: return "kernel launch failed";
    case GPTQ_ERR_DEVICE: return "HIP runtime call failed";
    case GPTQ_ERR_BAD_ARG: return "option out of range (is_v2, sym, path or split_k)";
    default: return "unknown error";
  }
}

void gptq_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  for (auto& kv : g_ws) {
    (void)hipFree(kv.second.partial);
    (void)hipFree(kv.second.counters);
  }
  g_ws.clear();
}

int gptq_abi_version(void) { return 1; }

}  // extern "C"
