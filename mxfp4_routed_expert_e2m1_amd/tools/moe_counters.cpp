// moe_counters -- a host program that runs one workload through the C ABI
// with no Python in the process, so that hardware counters (rocprofv3 --pmc
// FETCH_SIZE / WRITE_SIZE) can be collected per kernel dispatch.
//
//   moe_counters decode  ROWS ITERS [DIR]   moe_ffn_decode_step (E256 top-6 +
//                                           shared, d_model 4096, d_ff 2048)
//   moe_counters prefill ROWS ITERS [DIR]   quantiser, routing, moe_ffn_prefill
//   moe_counters matvec  ROWS ITERS         moe_matvec_mxfp4, 14336 x 4096
//
// DIR holds x.f32 [ROWS][4096] and logits.f32 [ROWS][256] (raw float32), e.g.
// written by `bench.py --dump-inputs DIR`, so the routes -- and with them the
// bytes each launch must read -- are the benchmark's; without DIR a fixed
// pattern is used.  Weight bytes are a constant pattern: which bytes a launch
// reads does not depend on their values.  Prints the experts the routes touch.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "moe_mxfp4.h"

#define CK(x)                                                                      \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                      \
      return 1;                                                                    \
    }                                                                              \
  } while (0)
#define CM(x)                                                                      \
  do {                                                                             \
    int r_ = (x);                                                                  \
    if (r_ != MOE_OK) {                                                            \
      fprintf(stderr, "%s: %d (%s)\n", #x, r_, moe_status_string(r_));             \
      return 1;                                                                    \
    }                                                                              \
  } while (0)

static bool read_f32(const std::string& path, std::vector<float>& v) {
  FILE* f = fopen(path.c_str(), "rb");
  if (!f) return false;
  const size_t n = fread(v.data(), sizeof(float), v.size(), f);
  fclose(f);
  return n == v.size();
}

static void pattern(std::vector<float>& v, uint64_t seed) {
  for (auto& x : v) {
    seed = seed * 6364136223846793005ULL + 1442695040888963407ULL;
    x = (float)((int)((seed >> 33) % 2001) - 1000) / 500.0f;
  }
}

int main(int argc, char** argv) {
  if (argc < 4) {
    fprintf(stderr, "usage: %s decode|prefill|matvec ROWS ITERS [DIR]\n", argv[0]);
    return 2;
  }
  const std::string wl = argv[1];
  const int rows = atoi(argv[2]), iters = atoi(argv[3]);
  const std::string dir = argc > 4 ? argv[4] : "";
  const int D = 4096, F = 2048, E = 256, K = 6;
  if (rows < 1 || iters < 1) return 2;

  if (wl == "matvec") {
    const int N = 14336;
    const size_t pb = moe_packed_bytes(N, D);
    uint8_t* w;
    CK(hipMalloc(&w, pb));
    CK(hipMemset(w, 0x7B, pb));
    std::vector<float> hx((size_t)rows * D);
    pattern(hx, 1);
    float *x, *qs, *y;
    int8_t* q;
    CK(hipMalloc(&x, hx.size() * 4));
    CK(hipMemcpy(x, hx.data(), hx.size() * 4, hipMemcpyHostToDevice));
    CK(hipMalloc(&q, (size_t)rows * D));
    CK(hipMalloc(&qs, (size_t)rows * D / 32 * 4));
    CK(hipMalloc(&y, (size_t)rows * N * 4));
    CM(moe_quant_act_q8(x, D, rows, D, q, D, qs, D / 32, nullptr));
    for (int i = 0; i < iters; ++i) CM(moe_matvec_mxfp4(w, N, D, q, D, qs, D / 32, rows, y, N, nullptr));
    CK(hipDeviceSynchronize());
    printf("matvec %dx%d, %d rows, %d launches; packed bytes %zu\n", N, D, rows, iters, pb);
    return 0;
  }
  if (wl != "decode" && wl != "prefill") return 2;

  const size_t gu = (moe_packed_bytes(2 * F, D) + 255) / 256 * 256;
  const size_t dn = (moe_packed_bytes(D, F) + 255) / 256 * 256;
  uint8_t *w_gu, *w_dn, *s_gu, *s_dn;
  CK(hipMalloc(&w_gu, gu * E));
  CK(hipMalloc(&w_dn, dn * E));
  CK(hipMalloc(&s_gu, gu));
  CK(hipMalloc(&s_dn, dn));
  // any byte is a valid code; 0x7B as a scale byte is 2^-4
  CK(hipMemset(w_gu, 0x7B, gu * E));
  CK(hipMemset(w_dn, 0x7B, dn * E));
  CK(hipMemset(s_gu, 0x7B, gu));
  CK(hipMemset(s_dn, 0x7B, dn));
  moe_layer_t L{};
  L.d_model = D;
  L.d_ff = F;
  L.n_experts = E;
  L.top_k = K;
  L.has_shared = 1;
  L.gate_up = w_gu;
  L.gate_up_stride = (int64_t)gu;
  L.down = w_dn;
  L.down_stride = (int64_t)dn;
  L.shared_gate_up = s_gu;
  L.shared_down = s_dn;

  std::vector<float> hx((size_t)rows * D), hl((size_t)rows * E);
  if (!dir.empty()) {
    if (!read_f32(dir + "/x.f32", hx) || !read_f32(dir + "/logits.f32", hl)) {
      fprintf(stderr, "cannot read %s/x.f32 and %s/logits.f32 for %d rows\n", dir.c_str(),
              dir.c_str(), rows);
      return 1;
    }
  } else {
    pattern(hx, 1);
    pattern(hl, 2);
  }
  float *x, *lg, *qs, *w, *y;
  int8_t* q;
  int32_t *ids, *counts, *offs, *srt;
  void* ws;
  CK(hipMalloc(&x, hx.size() * 4));
  CK(hipMalloc(&lg, hl.size() * 4));
  CK(hipMemcpy(x, hx.data(), hx.size() * 4, hipMemcpyHostToDevice));
  CK(hipMemcpy(lg, hl.data(), hl.size() * 4, hipMemcpyHostToDevice));
  CK(hipMalloc(&q, (size_t)rows * D));
  CK(hipMalloc(&qs, (size_t)rows * D / 32 * 4));
  CK(hipMalloc(&ids, (size_t)rows * K * 4));
  CK(hipMalloc(&w, (size_t)rows * K * 4));
  CK(hipMalloc(&counts, E * 4));
  CK(hipMalloc(&offs, (E + 1) * 4));
  CK(hipMalloc(&srt, (size_t)rows * K * 4));
  CK(hipMalloc(&y, (size_t)rows * D * 4));
  const size_t wsb = moe_ffn_workspace_bytes(&L, rows);
  CK(hipMalloc(&ws, wsb));
  for (int i = 0; i < iters; ++i) {
    if (wl == "decode") {
      CM(moe_ffn_decode_step(&L, x, D, lg, E, rows, q, D, qs, D / 32, ids, w, counts, offs, srt, y,
                             D, ws, wsb, nullptr));
    } else {
      CM(moe_quant_act_q8(x, D, rows, D, q, D, qs, D / 32, nullptr));
      CM(moe_route_group(lg, E, rows, E, K, ids, w, counts, offs, srt, nullptr));
      CM(moe_ffn_prefill(&L, q, D, qs, D / 32, rows, ids, w, offs, srt, y, D, ws, wsb, nullptr));
    }
  }
  CK(hipDeviceSynchronize());
  std::vector<int32_t> hc(E);
  CK(hipMemcpy(hc.data(), counts, E * 4, hipMemcpyDeviceToHost));
  int touched = 1;  // the shared expert
  for (int e = 0; e < E; ++e) touched += hc[e] > 0;
  printf("%s, %d rows, %d steps; experts touched (incl. shared) %d\n", wl.c_str(), rows, iters,
         touched);
  return 0;
}
