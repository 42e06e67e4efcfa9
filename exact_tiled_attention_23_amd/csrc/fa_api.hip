// C ABI of the attention forward (declared in include/fa.h): argument checks and
// kernel dispatch. Every check runs before any HIP call; the library keeps no state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "fa.h"
#include "fa_fwd_kernel.h"
#include "fa_fwd_mfma16.h"

namespace {

constexpr int kAbiVersion = 1;
constexpr int kWaves = 4;      // waves per workgroup: 4 x 32 = 128 query rows per tile
constexpr int kBlockKV = 64;   // keys per K/V tile
// bf16/f16 kernel shape: keys per K/V tile, and waves per workgroup (32 query rows each)
// at D = 64 and D = 128. Eight waves share each K/V tile across 256 query rows at
// D = 128, halving the copies per flop; at D = 64 (vector-bound) two 4-wave workgroups
// per CU do better. Two waves per SIMD in both cases.
#ifndef FA_BC_D64
#define FA_BC_D64 128
#endif
#ifndef FA_BC_D128
#define FA_BC_D128 64
#endif
#ifndef FA_WAVES16_D64
#define FA_WAVES16_D64 4
#endif
#ifndef FA_WAVES16_D128
#define FA_WAVES16_D128 8
#endif
constexpr int kWavesPerSimd = 2;

bool misaligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) != 0; }

template <typename T, int D>
int launch(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B, int64_t H, int64_t N,
           float scale, int causal, const int32_t* kv_len, hipStream_t stream) {
  constexpr int NW = sizeof(T) == 2 ? (D == 64 ? FA_WAVES16_D64 : FA_WAVES16_D128) : kWaves;
  constexpr int BR = 32 * NW;
  constexpr int threads = 64 * NW;
  fa::FwdParams p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = LSE;
  p.kv_len = kv_len;
  p.H = H;
  p.N = N;
  p.scale_log2 = scale * fa::kLog2e;
  p.causal = causal;
  const int64_t n_qtiles = (N + BR - 1) / BR;
  const int64_t units = B * H * n_qtiles;
  if (n_qtiles > INT32_MAX || units > INT32_MAX) return FA_ERR_SHAPE;
  p.n_qtiles = (int)n_qtiles;
  p.n_units = units;
  p.xcd_groups = (units % 8 == 0) ? 8 : 1;
  void* args[] = {&p};
  const void* fn;
  constexpr int BC = D == 64 ? FA_BC_D64 : FA_BC_D128;
  if constexpr (sizeof(T) == 2) {
    fn = reinterpret_cast<const void*>(&fa::fwd16_kernel<T, D, BC, NW, kWavesPerSimd>);
  } else {
    fn = reinterpret_cast<const void*>(&fa::fwd_kernel<T, D, kBlockKV, kWaves>);
  }
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)units), dim3(threads), args, 0, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <typename T>
int dispatch_d(int64_t D, const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B, int64_t H,
               int64_t N, float scale, int causal, const int32_t* kv_len, hipStream_t stream) {
  if (D == 64) return launch<T, 64>(Q, K, V, O, LSE, B, H, N, scale, causal, kv_len, stream);
  return launch<T, 128>(Q, K, V, O, LSE, B, H, N, scale, causal, kv_len, stream);
}

}  // namespace

extern "C" int fa_abi_version(void) { return kAbiVersion; }

extern "C" const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid sizes (negative, or too large for the kernel's indexing)";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension (64 or 128) or dtype (f32, bf16, f16)";
    case FA_ERR_ALIGN: return "misaligned pointer (Q, K, V, O need 16 bytes; LSE and kv_len 4 bytes)";
    case FA_ERR_ARG: return "invalid argument (scale must be finite and > 0, causal 0 or 1, O must not alias Q, K or V)";
    case FA_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    default: return "unknown error code";
  }
}

extern "C" int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B, int64_t H,
                      int64_t N, int64_t D, float scale, int causal, const int32_t* kv_len, int dtype,
                      void* stream) {
  if (B < 0 || H < 0 || N < 0 || D < 0) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16 && dtype != FA_F16) return FA_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (B == 0 || H == 0 || N == 0) return FA_OK;
  if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL;
  if (misaligned(Q, 16) || misaligned(K, 16) || misaligned(V, 16) || misaligned(O, 16)) return FA_ERR_ALIGN;
  if (misaligned(LSE, 4) || (kv_len && misaligned(kv_len, 4))) return FA_ERR_ALIGN;
  if (O == Q || O == K || O == V) return FA_ERR_ARG;
  // Element counts must fit in int64 with room: B*H*N*D and the byte offsets derived from it.
  const int64_t lim = INT64_MAX / 16;
  if (B > lim / H || B * H > lim / N || B * H * N > lim / D) return FA_ERR_SHAPE;
  if (N > (int64_t(1) << 30)) return FA_ERR_SHAPE;  // row indices stay in 32 bits
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (dtype) {
    case FA_BF16: return dispatch_d<__bf16>(D, Q, K, V, O, LSE, B, H, N, scale, causal, kv_len, s);
    case FA_F16: return dispatch_d<_Float16>(D, Q, K, V, O, LSE, B, H, N, scale, causal, kv_len, s);
    default: return dispatch_d<float>(D, Q, K, V, O, LSE, B, H, N, scale, causal, kv_len, s);
  }
}
