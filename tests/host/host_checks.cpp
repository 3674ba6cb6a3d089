// Drives the host-only entry points of libgptq (argument checks, launch
// planning, describe strings, error texts) from lines on stdin, one call per
// line, and prints each result.  Built with the host code under AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py, which feeds
// it edge and random arguments and compares every result with the library's.
// It never launches a kernel: entry points that would are only called with
// arguments their checks reject.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "gptq.h"

namespace {

const void* ptr(unsigned long long v) { return reinterpret_cast<const void*>(static_cast<uintptr_t>(v)); }
void* mptr(unsigned long long v) { return reinterpret_cast<void*>(static_cast<uintptr_t>(v)); }
const int32_t* iptr(unsigned long long v) { return reinterpret_cast<const int32_t*>(static_cast<uintptr_t>(v)); }
int32_t* miptr(unsigned long long v) { return reinterpret_cast<int32_t*>(static_cast<uintptr_t>(v)); }

}  // namespace

int main() {
  char line[1024];
  while (std::fgets(line, sizeof line, stdin)) {
    char op[64] = {0};
    if (std::sscanf(line, "%63s", op) != 1) continue;
    unsigned long long x, qw, qz, sc, gi, out;
    int bits, gs, v2, path, waves, buflen;
    long long M, N, K;
    const std::string o(op);
    if (o == "gemm" || o == "gemm_ex" || o == "describe" || o == "tiled_describe" || o == "bf16_describe" ||
        o == "tiled_bf16_describe" || o == "gemm_call" || o == "noalloc_call") {
      if (std::sscanf(line, "%*s %llx %llx %llx %llx %llx %d %d %d %lld %lld %lld %llx %d %d %d", &x, &qw, &qz, &sc,
                      &gi, &bits, &gs, &v2, &M, &N, &K, &out, &path, &waves, &buflen) != 15) {
        std::printf("parse error\n");
        continue;
      }
      int rc = 0;
      if (o == "gemm") {
        rc = gptq_gemm_check(ptr(x), iptr(qw), iptr(qz), ptr(sc), iptr(gi), bits, gs, v2, M, N, K, ptr(out));
      } else if (o == "gemm_ex") {
        rc = gptq_gemm_ex_check(ptr(x), iptr(qw), iptr(qz), ptr(sc), iptr(gi), bits, gs, v2, M, N, K, ptr(out), path,
                                waves);
      } else if (o == "gemm_call") {   // only with arguments the checks reject
        rc = gptq_gemm_ex(ptr(x), iptr(qw), iptr(qz), ptr(sc), iptr(gi), bits, gs, v2, M, N, K, mptr(out), nullptr,
                          path, waves);
      } else if (o == "noalloc_call") {
        rc = gptq_gemm_noalloc(ptr(x), iptr(qw), iptr(qz), ptr(sc), iptr(gi), bits, gs, v2, M, N, K, mptr(out),
                               nullptr);
      } else {
        char buf[512];
        std::memset(buf, 'Z', sizeof buf);
        const int64_t bl = buflen > 512 ? 512 : buflen;
        char* b = buflen < 0 ? nullptr : buf;
        if (o == "describe")
          rc = gptq_gemm_describe(ptr(x), iptr(qw), iptr(qz), ptr(sc), iptr(gi), bits, gs, v2, M, N, K, ptr(out),
                                  path, waves, b, bl);
        else if (o == "tiled_describe")
          rc = gptq_gemm_tiled_describe(ptr(x), iptr(qw), iptr(qz), ptr(sc), iptr(gi), bits, gs, v2, M, N, K,
                                        ptr(out), path, waves, b, bl);
        else if (o == "tiled_bf16_describe")
          rc = gptq_gemm_tiled_bf16_describe(ptr(x), iptr(qw), iptr(qz), ptr(sc), iptr(gi), bits, gs, v2, M, N, K,
                                             ptr(out), path, waves, b, bl);
        else
          rc = gptq_gemm_bf16_describe(ptr(x), iptr(qw), iptr(qz), ptr(sc), iptr(gi), bits, gs, v2, M, N, K,
                                       ptr(out), path, waves, b, bl);
        if (b && bl > 0) {
          std::printf("%d %s\n", rc, buf);
          continue;
        }
      }
      std::printf("%d\n", rc);
    } else if (o == "dequant_check") {
      if (std::sscanf(line, "%*s %llx %llx %llx %llx %d %d %d %lld %lld %llx", &qw, &qz, &sc, &gi, &bits, &gs, &v2, &N,
                      &K, &out) != 10) {
        std::printf("parse error\n");
        continue;
      }
      std::printf("%d\n", gptq_dequant_check(iptr(qw), iptr(qz), ptr(sc), iptr(gi), bits, gs, v2, N, K, ptr(out)));
    } else if (o == "convert_check") {
      unsigned long long in, outp, cnt;
      long long G;
      int to_v2;
      if (std::sscanf(line, "%*s %llx %llx %d %lld %lld %d %llx", &in, &outp, &bits, &G, &N, &to_v2, &cnt) != 7) {
        std::printf("parse error\n");
        continue;
      }
      std::printf("%d\n", gptq_convert_zeros_check(iptr(in), iptr(outp), bits, G, N, to_v2, iptr(cnt)));
    } else if (o == "repack_call") {   // only with arguments the checks reject
      unsigned long long in, outp;
      if (std::sscanf(line, "%*s %llx %llx %d %lld %lld", &in, &outp, &bits, &N, &K) != 5) {
        std::printf("parse error\n");
        continue;
      }
      std::printf("%d\n", gptq_repack_tiled(iptr(in), miptr(outp), bits, N, K, nullptr));
    } else if (o == "ceiling_call") {   // only with arguments the checks reject
      unsigned long long b, sink;
      long long bytes;
      if (std::sscanf(line, "%*s %llx %lld %llx", &b, &bytes, &sink) != 3) {
        std::printf("parse error\n");
        continue;
      }
      std::printf("%d\n", gptq_read_ceiling(ptr(b), bytes, mptr(sink), nullptr));
    } else if (o == "strerror") {
      int code = 0;
      std::sscanf(line, "%*s %d", &code);
      std::printf("%s\n", gptq_strerror(code));
    } else {
      std::printf("unknown op\n");
    }
    std::fflush(stdout);
  }
  return 0;
}
