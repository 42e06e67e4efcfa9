// Uses libfa.so through include/fa.h alone (no Python): device buffers from hipMalloc, the
// forward, the key-split forward, the backward and the error paths. It checks facts that hold
// exactly for any correct attention (it is not a second oracle):
//   * causal row 0 attends to key 0 only: O[0] = V[0] bit for bit, LSE[0] = scale <q0, k0>;
//   * identical keys give uniform weights: every O row is the mean of the visible V rows;
//   * kv_len = 0 gives O = 0 and LSE = -inf;
//   * the split forward agrees with the plain one to rounding;
//   * with one key, dV = dO and dQ = dK = 0 (to rounding).
// Exit status 0 and a final "ok" line on success.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "fa.h"

namespace {

int failures = 0;

void check(bool ok, const char* what) {
  std::printf("%s: %s\n", ok ? "pass" : "FAIL", what);
  if (!ok) ++failures;
}

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      std::printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      return 2;                                                                \
    }                                                                          \
  } while (0)

uint16_t to_bf16(float f) {  // round to nearest even
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

float from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// A deterministic small-integer pattern, exact in bf16: values k/8 with |k| <= 16.
float pattern(int i, int salt) { return (float)(((i * 37 + salt * 101) % 33) - 16) / 8.0f; }

}  // namespace

int main() {
  std::printf("fa ABI version %d\n", fa_abi_version());
  check(fa_abi_version() >= 6, "ABI version");
  check(fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 1, 1, 8, 64, 0.125f, 1, nullptr, FA_BF16, nullptr) ==
            FA_ERR_NULL, "NULL pointers rejected");
  check(std::strlen(fa_strerror(FA_ERR_ALIGN)) > 0, "strerror text");

  const int64_t B = 2, H = 2, N = 300, D = 64;
  const int64_t elems = B * H * N * D, rows = B * H * N;
  const float scale = 0.125f;
  std::vector<uint16_t> hq(elems), hk(elems), hv(elems);
  for (int64_t i = 0; i < elems; ++i) {
    hq[i] = to_bf16(pattern((int)i, 1));
    hk[i] = to_bf16(pattern((int)i, 2));
    hv[i] = to_bf16(pattern((int)i, 3));
  }
  // Batch 1: every key row identical (uniform weights).
  for (int64_t h = 0; h < H; ++h)
    for (int64_t j = 0; j < N; ++j)
      for (int64_t d = 0; d < D; ++d) hk[((1 * H + h) * N + j) * D + d] = hk[((1 * H + h) * N + 0) * D + d];

  void *q, *k, *v, *o, *o2, *ws;
  float *lse, *lse2;
  int32_t* kvl;
  HIP_OK(hipMalloc(&q, elems * 2));
  HIP_OK(hipMalloc(&k, elems * 2));
  HIP_OK(hipMalloc(&v, elems * 2));
  HIP_OK(hipMalloc(&o, elems * 2));
  HIP_OK(hipMalloc(&o2, elems * 2));
  HIP_OK(hipMalloc(&lse, rows * 4));
  HIP_OK(hipMalloc(&lse2, rows * 4));
  HIP_OK(hipMalloc(&kvl, B * 4));
  HIP_OK(hipMemcpy(q, hq.data(), elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk.data(), elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv.data(), elems * 2, hipMemcpyHostToDevice));

  // ---- causal forward: row 0 of every (b, h)
  check(fa_fwd(q, k, v, o, lse, B, H, N, D, scale, 1, nullptr, FA_BF16, nullptr) == FA_OK, "fa_fwd causal");
  HIP_OK(hipDeviceSynchronize());
  std::vector<uint16_t> ho(elems);
  std::vector<float> hl(rows);
  HIP_OK(hipMemcpy(ho.data(), o, elems * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hl.data(), lse, rows * 4, hipMemcpyDeviceToHost));
  bool row0 = true, lse0 = true;
  for (int64_t bh = 0; bh < B * H; ++bh) {
    const int64_t r0 = bh * N * D;
    row0 = row0 && std::memcmp(&ho[r0], &hv[r0], D * 2) == 0;
    double dot = 0;
    for (int64_t d = 0; d < D; ++d) dot += (double)from_bf16(hq[r0 + d]) * from_bf16(hk[r0 + d]);
    lse0 = lse0 && std::fabs(hl[bh * N] - scale * dot) <= 1e-5 * (1 + std::fabs(scale * dot));
  }
  check(row0, "causal row 0: O = V[0] bit for bit");
  check(lse0, "causal row 0: LSE = scale <q0, k0>");

  // ---- non-causal forward, batch 1 has identical keys: O = mean of V
  check(fa_fwd(q, k, v, o, lse, B, H, N, D, scale, 0, nullptr, FA_BF16, nullptr) == FA_OK, "fa_fwd non-causal");
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(ho.data(), o, elems * 2, hipMemcpyDeviceToHost));
  double worst = 0;
  for (int64_t h = 0; h < H; ++h)
    for (int64_t d = 0; d < D; ++d) {
      double mean = 0;
      for (int64_t j = 0; j < N; ++j) mean += from_bf16(hv[((1 * H + h) * N + j) * D + d]);
      mean /= N;
      for (int64_t i = 0; i < N; ++i)
        worst = std::fmax(worst, std::fabs(from_bf16(ho[((1 * H + h) * N + i) * D + d]) - mean));
    }
  std::printf("identical keys: max |O - mean(V)| = %.3g\n", worst);
  check(worst <= 1e-2, "identical keys: every row is the mean of V");

  // ---- key-split forward against the plain one
  const int S = 3;
  const int64_t wsb = fa_fwd_split_workspace_bytes(B, H, N, D, S);
  HIP_OK(hipMalloc(&ws, wsb));
  check(fa_fwd_split(q, k, v, o2, lse2, B, H, N, D, nullptr, scale, 0, nullptr, nullptr, FA_BF16, S, ws, wsb, nullptr) ==
            FA_OK, "fa_fwd_split");
  check(fa_fwd_split(q, k, v, o2, lse2, B, H, N, D, nullptr, scale, 0, nullptr, nullptr, FA_BF16, S, ws, wsb - 1, nullptr) ==
            FA_ERR_ARG, "fa_fwd_split rejects a short workspace");
  HIP_OK(hipDeviceSynchronize());
  std::vector<uint16_t> ho2(elems);
  std::vector<float> hl2(rows);
  HIP_OK(hipMemcpy(ho2.data(), o2, elems * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hl2.data(), lse2, rows * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hl.data(), lse, rows * 4, hipMemcpyDeviceToHost));
  double dmax = 0, lmax = 0;
  for (int64_t i = 0; i < elems; ++i) dmax = std::fmax(dmax, std::fabs(from_bf16(ho2[i]) - from_bf16(ho[i])));
  for (int64_t i = 0; i < rows; ++i) lmax = std::fmax(lmax, std::fabs(hl2[i] - hl[i]));
  std::printf("split vs plain: max |dO| %.3g, max |dLSE| %.3g\n", dmax, lmax);
  check(dmax <= 2e-2 && lmax <= 1e-4, "split forward = plain forward to rounding");

  // ---- kv_len = 0 for batch 0: zeros and -inf
  const int32_t hkv[2] = {0, (int32_t)N};
  HIP_OK(hipMemcpy(kvl, hkv, sizeof(hkv), hipMemcpyHostToDevice));
  check(fa_fwd(q, k, v, o, lse, B, H, N, D, scale, 1, kvl, FA_BF16, nullptr) == FA_OK, "fa_fwd with kv_len");
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(ho.data(), o, elems * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hl.data(), lse, rows * 4, hipMemcpyDeviceToHost));
  bool empty = true;
  for (int64_t i = 0; i < H * N * D; ++i) empty = empty && ho[i] == 0;
  for (int64_t i = 0; i < H * N; ++i) empty = empty && std::isinf(hl[i]) && hl[i] < 0;
  check(empty, "kv_len = 0: O = 0, LSE = -inf");

  // ---- backward with one key: dV = dO, dQ = dK = 0
  {
    const int64_t n1 = 1, e1 = B * H * n1 * D;
    void *q1, *k1, *v1, *o1, *do1, *dq1, *dk1, *dv1, *w1;
    float* l1;
    HIP_OK(hipMalloc(&q1, e1 * 2));
    HIP_OK(hipMalloc(&k1, e1 * 2));
    HIP_OK(hipMalloc(&v1, e1 * 2));
    HIP_OK(hipMalloc(&o1, e1 * 2));
    HIP_OK(hipMalloc(&do1, e1 * 2));
    HIP_OK(hipMalloc(&dq1, e1 * 2));
    HIP_OK(hipMalloc(&dk1, e1 * 2));
    HIP_OK(hipMalloc(&dv1, e1 * 2));
    HIP_OK(hipMalloc(&l1, B * H * 4));
    const int64_t wb = fa_bwd_workspace_bytes(B, H, n1, D);
    HIP_OK(hipMalloc(&w1, wb));
    HIP_OK(hipMemcpy(q1, hq.data(), e1 * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(k1, hk.data(), e1 * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v1, hv.data(), e1 * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(do1, hq.data() + e1, e1 * 2, hipMemcpyHostToDevice));
    check(fa_fwd(q1, k1, v1, o1, l1, B, H, n1, D, scale, 0, nullptr, FA_BF16, nullptr) == FA_OK, "fa_fwd N=1");
    check(fa_bwd(q1, k1, v1, o1, l1, do1, dq1, dk1, dv1, B, H, n1, D, scale, 0, nullptr, FA_BF16, w1, wb, nullptr) ==
              FA_OK, "fa_bwd N=1");
    check(fa_bwd(q1, k1, v1, o1, l1, do1, q1, dk1, dv1, B, H, n1, D, scale, 0, nullptr, FA_BF16, w1, wb, nullptr) ==
              FA_ERR_ARG, "fa_bwd rejects dQ on Q");
    HIP_OK(hipDeviceSynchronize());
    std::vector<uint16_t> hdq(e1), hdk(e1), hdv(e1), hdo(e1);
    HIP_OK(hipMemcpy(hdq.data(), dq1, e1 * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hdk.data(), dk1, e1 * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hdv.data(), dv1, e1 * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hdo.data(), do1, e1 * 2, hipMemcpyDeviceToHost));
    double zq = 0;
    for (int64_t i = 0; i < e1; ++i)
      zq = std::fmax(zq, std::fmax(std::fabs(from_bf16(hdq[i])), std::fabs(from_bf16(hdk[i]))));
    check(std::memcmp(hdv.data(), hdo.data(), e1 * 2) == 0, "one key: dV = dO bit for bit");
    check(zq <= 1e-4, "one key: dQ = dK = 0");
    for (void* p : {q1, k1, v1, o1, do1, dq1, dk1, dv1, w1}) HIP_OK(hipFree(p));
    HIP_OK(hipFree(l1));
  }

  for (void* p : {q, k, v, o, o2, ws}) HIP_OK(hipFree(p));
  HIP_OK(hipFree(lse));
  HIP_OK(hipFree(lse2));
  HIP_OK(hipFree(kvl));
  if (failures) {
    std::printf("%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
