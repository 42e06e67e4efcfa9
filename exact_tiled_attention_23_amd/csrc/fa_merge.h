// Merge of partial softmax states: the associative combination of attention over disjoint
// key sets ("Paper: FlashAttention", Objectives, Math & data structures: partial softmax
// states merge associatively, with an identity element).
//
// For each row (b, h, n) and S partial states (O_s, LSE_s), each normalised over its own
// key set (O_s = 0, LSE_s = -inf for an empty set):
//
//   m   = max_s LSE_s
//   w_s = exp(LSE_s - m)            (0 for an empty set)
//   LSE = m + ln(sum_s w_s)         (-inf when every set is empty)
//   O   = sum_s w_s O_s / sum_s w_s (0 when every set is empty)
//
// Memory-bound: each row reads S*(D+1) floats and writes D elements and one float.
// Threads take 4 consecutive columns of one row (16-byte loads); a 256-thread block
// covers floor(256 / (D/4)) rows (10 at D = 96, whose last 16 threads stay idle).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct MergeParams {
  const float* part_o;    // [S][rows][D], rows = B*H*N, contiguous
  const float* part_lse;  // [S][rows]
  int n_states;
  int64_t rows;
  int64_t H, N;
  void* o;                // element (b, h, n, d) at o + b*o_sb + h*o_sh + n*o_sn + d
  int64_t o_sb, o_sh, o_sn;
  float* lse;             // [rows]
};

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 4;
  if (threadIdx.x >= RPB * TPR || row >= p.rows) return;
  float m = -INFINITY;
  for (int s = 0; s < p.n_states; ++s) m = fmaxf(m, p.part_lse[s * p.rows + row]);
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
  if (m != -INFINITY) {
    // Every state's loads are issued without a branch (so they overlap); an identity state
    // (LSE = -inf) is dropped by selection, not by a zero weight, since its O may be anything.
#pragma unroll 4
    for (int s = 0; s < p.n_states; ++s) {
      const float ls = p.part_lse[s * p.rows + row];
      const float4 x = *reinterpret_cast<const float4*>(p.part_o + (s * p.rows + row) * D + c);
      const bool live = ls != -INFINITY;
      const float w = live ? expf(ls - m) : 0.f;
      sum += w;
      acc.x = live ? acc.x + w * x.x : acc.x;
      acc.y = live ? acc.y + w * x.y : acc.y;
      acc.z = live ? acc.z + w * x.z : acc.z;
      acc.w = live ? acc.w + w * x.w : acc.w;
    }
  }
  const float inv = (sum == 0.f) ? 0.f : 1.f / sum;
  const int64_t bh = row / p.N, nn = row % p.N;
  const int64_t b = bh / p.H, h = bh % p.H;
  T* dst = reinterpret_cast<T*>(p.o) + b * p.o_sb + h * p.o_sh + nn * p.o_sn + c;
  const float v[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  if constexpr (sizeof(T) == 2) {
    T o4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o4[e] = (T)v[e];
    *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(o4);
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  }
  if (c == 0) p.lse[row] = (sum == 0.f) ? -INFINITY : m + logf(sum);
}

}  // namespace fa
