// Exact tiled attention forward, bf16/f16 kernel for gfx950.
//
// Same recurrence and work decomposition as the float32 kernel in fa_fwd_kernel.h
// ("vectorized-flash-attention-kernel", Core algorithm; Key design decisions 1 and 3),
// laid out for the CDNA4 memory path:
//
//  * K and V tiles go HBM -> LDS with direct 16-byte global_load_lds transfers (no
//    register staging), double-buffered so tile t+1 streams in while tile t is
//    computed; one barrier per tile. Both tiles stay row-major in LDS with an XOR
//    swizzle of 16-byte chunks, chosen so every LDS read below is free of bank
//    conflicts.
//  * S^T = K . Q^T on 32x32x16 MFMA: each lane owns one query (lane % 32) and half of
//    every 32-key sub-tile, so row statistics need only one swap between lane halves
//    (v_permlane32_swap).
//  * O^T = V^T . P^T on 32x32x16 MFMA: V^T fragments come straight from the row-major
//    V tile with ds_read_b64_tr_b16 (transpose on read); P^T is the S^T accumulator
//    rounded to bf16/f16, with no trip through LDS.
//  * Online softmax in base 2 with a lazily moved reference maximum: the accumulator
//    and denominator are rescaled by 2^(m_old - m_new) only when some row's maximum
//    rises more than kRescaleSlack above the reference (a wave-uniform branch). Until
//    then probabilities are formed against the stale reference and stay <= 2^slack.
//    The final O = acc / l is the same quotient whichever reference is used, so the
//    result is exact up to rounding ("Paper: FlashAttention", Objectives: the
//    online-softmax state is defined up to a common rescaling).
//  * A row whose reference is still -inf subtracts 0 instead, so exp(-inf - -inf)
//    never occurs ("js-flash-attention-tiled-online-softmax-exactness", Root causes
//    addressed 2); fully masked rows end with l = 0 and store O = 0, LSE = -inf.
//  * Padding keys (>= kv_len) in the edge tile: their V rows are zeroed in LDS after
//    the load so garbage past kv_len cannot reach O, and their scores are masked.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_kernel.h"

namespace fa {

// Reference maximum may lag the true row maximum by up to this much (base-2 units).
constexpr float kRescaleSlack = 8.0f;

typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef short s16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// XOR swizzles of the 16-byte chunk index within a row (row j of the tile).
// K is read by 16 lanes on 16 different rows at one logical chunk; V (transpose reads)
// by 16 lanes on 4 consecutive rows x 4 consecutive chunks.
template <int D> __device__ __forceinline__ int swz_k(int j) {
  if constexpr (D == 128) return j & 15;
  else return (j >> 1) & 7;
}
template <int D> __device__ __forceinline__ int swz_v(int j) {
  if constexpr (D == 128) return 4 * (j & 3);
  else return 4 * ((j >> 1) & 1);
}

template <typename T, int D, int BC, int NW, int WPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void fwd16_kernel(FwdParams p) {
  using M = Mma<T>;
  using frag = typename M::frag;
  static_assert(sizeof(T) == 2, "16-bit element types only");
  static_assert(D == 64 || D == 128, "head dimension");
  static_assert(BC % 32 == 0, "key tile");
  constexpr int BR = 32 * NW;
  constexpr int ROWB = D * 2;                   // bytes per K/V row
  constexpr int CPR = D / 8;                    // 16-byte chunks per row
  constexpr int TILEB = BC * ROWB;              // bytes per K (or V) tile
  constexpr int BLOCKS = TILEB / 1024;          // 1 KB global_load_lds blocks per tile
  constexpr int LPW = BLOCKS / NW;              // blocks per wave per tile (each for K and V)
  constexpr int RPB = 1024 / ROWB;              // rows per block
  constexpr int NSUB = BC / 32;
  constexpr int NDT = D / 32;
  constexpr int NQF = D / 16;
  static_assert(BLOCKS % NW == 0, "tile must split evenly over waves");

  __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * TILEB];  // [buf][K|V][tile]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 5;
  const int r = lane & 31;

  int64_t bid = blockIdx.x;
  int64_t unit = bid;
  if (p.xcd_groups == 8) unit = (bid % 8) * (p.n_units / 8) + bid / 8;
  const int64_t bh = unit / p.n_qtiles;
  int qt = (int)(unit % p.n_qtiles);
  if (p.causal) qt = p.n_qtiles - 1 - qt;
  const int64_t b = bh / p.H;
  const int64_t N = p.N;

  const T* __restrict__ Qh = reinterpret_cast<const T*>(p.q) + bh * N * D;
  const T* __restrict__ Kh = reinterpret_cast<const T*>(p.k) + bh * N * D;
  const T* __restrict__ Vh = reinterpret_cast<const T*>(p.v) + bh * N * D;
  T* __restrict__ Oh = reinterpret_cast<T*>(p.o) + bh * N * D;
  float* __restrict__ Lh = p.lse + bh * N;

  const int64_t q0 = (int64_t)qt * BR;
  const int64_t qw = q0 + 32 * wave;
  const int64_t qrow = qw + r;

  int64_t kvl = N;
  if (p.kv_len) {
    int64_t x = p.kv_len[b];
    kvl = x < 0 ? 0 : (x > N ? N : x);
  }
  int64_t kv_hi = kvl, wave_hi = kvl;
  if (p.causal) {
    kv_hi = kv_hi < q0 + BR ? kv_hi : q0 + BR;
    wave_hi = wave_hi < qw + 32 ? wave_hi : qw + 32;
  }
  const int ntiles = kv_hi > 0 ? (int)((kv_hi + BC - 1) / BC) : 0;

  // ---- per-lane constants of the global -> LDS copies: block blk = wave*LPW + i holds
  // rows blk*RPB .. +RPB-1; this lane fills the block's 16-byte slot `lane`, i.e. physical
  // chunk lane % CPR of row blk*RPB + lane / CPR, holding the logical chunk XOR swizzle.
  int ld_row[LPW], ld_koff[LPW], ld_voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int blk = wave * LPW + i;
    const int j = blk * RPB + lane / CPR;
    const int pc = lane % CPR;
    ld_row[i] = j;
    ld_koff[i] = j * D + (pc ^ swz_k<D>(j)) * 8;
    ld_voff[i] = j * D + (pc ^ swz_v<D>(j)) * 8;
  }

  auto issue_tile = [&](int64_t j0, int buf) {
    unsigned char* kb = lds + buf * 2 * TILEB;
    unsigned char* vb = kb + TILEB;
    const bool edge = j0 + BC > N;  // some rows past the tensor end: read row N-1 instead
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int blk = wave * LPW + i;
      int64_t ko = j0 * D + ld_koff[i];
      int64_t vo = j0 * D + ld_voff[i];
      if (edge && j0 + ld_row[i] >= N) {
        const int64_t back = (j0 + ld_row[i] - (N - 1)) * D;
        ko -= back;
        vo -= back;
      }
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(Kh + ko), (lds_void*)(kb + blk * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(Vh + vo), (lds_void*)(vb + blk * 1024), 16, 0, 0);
    }
  };

  // ---- Q^T fragments (B operand of S^T = K . Q^T), straight from global memory.
  frag qf[NQF];
#pragma unroll
  for (int s = 0; s < NQF; ++s) {
    if (qrow < N) qf[s] = *reinterpret_cast<const frag*>(Qh + qrow * D + 16 * s + 8 * g);
    else qf[s] = frag{};
  }

  // ---- per-lane LDS read offsets
  const int kr = a_row_key<8>(r);                 // K row this lane feeds as A-operand row r
  const int krow_off = kr * ROWB;
  int koff[NQF];
#pragma unroll
  for (int s = 0; s < NQF; ++s) koff[s] = krow_off + ((2 * s + g) ^ swz_k<D>(kr)) * 16;
  const int s16 = lane & 15, s4 = s16 >> 2, sm = s16 & 3, q2 = (lane >> 4) & 1;
  const int vrow_off = (8 * g + s4) * ROWB;
  int voff[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int c = 4 * dt + 2 * q2 + (sm >> 1);
    voff[dt] = vrow_off + ((c ^ swz_v<D>(s4)) * 16) + (sm & 1) * 8;
  }

  f32x16 oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) oacc[t] = f32x16{};
  float mref = -INFINITY;  // reference maximum (scaled base-2 logits)
  float lsum = 0.f;        // this lane half's share of the denominator
  const float c = p.scale_log2;

  if (ntiles > 0) issue_tile(0, 0);

  for (int t = 0; t < ntiles; ++t) {
    const int64_t j0 = (int64_t)t * BC;
    const int buf = t & 1;
    const unsigned char* kb = lds + buf * 2 * TILEB;
    const unsigned char* vb = kb + TILEB;
    wait_vmem();  // this wave's copies of tile t have landed
    if (j0 + BC > kvl) {
      // Padding rows (key >= kv_len) of V must not carry garbage into O: zero the slots
      // this lane filled itself.
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        if (j0 + ld_row[i] >= kvl) {
          const int blk = wave * LPW + i;
          *reinterpret_cast<uint4*>(lds + buf * 2 * TILEB + TILEB + blk * 1024 + lane * 16) = uint4{0, 0, 0, 0};
        }
      }
    }
    __syncthreads();  // tile t visible to all waves; all waves are done with tile t-1
    if (t + 1 < ntiles) issue_tile(j0 + BC, buf ^ 1);

    if (j0 < wave_hi) {
      // ---- S^T = K . Q^T
      f32x16 s[NSUB];
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        s[u] = f32x16{};
#pragma unroll
        for (int st = 0; st < NQF; ++st) {
          const frag a = *reinterpret_cast<const frag*>(kb + u * 32 * ROWB + koff[st]);
          s[u] = M::run(a, qf[st], s[u]);
        }
      }

      // ---- masks (edge tiles only)
      const bool need_mask = (j0 + BC > kvl) || (p.causal && j0 + BC - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int u = 0; u < NSUB; ++u)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int64_t key = j0 + 32 * u + acc_key<8>(i, g);
            if (key >= kvl || (p.causal && key > qrow)) s[u][i] = -INFINITY;
          }
      }

      // ---- online softmax with a lazily moved reference maximum
      float mx[NSUB];
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        float a0 = fmaxf(fmaxf(s[u][0], s[u][1]), fmaxf(s[u][2], s[u][3]));
        float a1 = fmaxf(fmaxf(s[u][4], s[u][5]), fmaxf(s[u][6], s[u][7]));
        float a2 = fmaxf(fmaxf(s[u][8], s[u][9]), fmaxf(s[u][10], s[u][11]));
        float a3 = fmaxf(fmaxf(s[u][12], s[u][13]), fmaxf(s[u][14], s[u][15]));
        mx[u] = fmaxf(fmaxf(a0, a1), fmaxf(a2, a3));
      }
      float m = mx[0];
#pragma unroll
      for (int u = 1; u < NSUB; ++u) m = fmaxf(m, mx[u]);
      const float mcand = pair_max(m) * c;
      if (__any(mcand > mref + kRescaleSlack)) {
        const float mnew = fmaxf(mref, mcand);
        const float alpha = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mref - mnew);
        mref = mnew;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
      }
      const float muse = (mref == -INFINITY) ? 0.f : mref;
      float part[NSUB];
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u][i], c, -muse));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u][i + 1], c, -muse));
          s[u][i] = p0;
          s[u][i + 1] = p1;
          a0 += p0;
          a1 += p1;
        }
        part[u] = a0 + a1;
      }
#pragma unroll
      for (int u = 0; u < NSUB; ++u) lsum += part[u];

      // ---- O^T += V^T . P^T
#pragma unroll
      for (int kk = 0; kk < BC / 16; ++kk) {
        const int u = kk >> 1, h = kk & 1;
        frag pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = (T)s[u][8 * h + e];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const unsigned char* va = vb + (16 * kk) * ROWB + voff[dt];
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(va));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(va + 4 * ROWB));
          const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[dt] = M::run(__builtin_bit_cast(frag, both), pf, oacc[dt]);
        }
      }
    }
  }

  // ---- epilogue
  const float ltot = pair_sum(lsum);
  if (qrow < N) {
    const float inv = (ltot == 0.f) ? 0.f : 1.f / ltot;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = 32 * dt + 8 * a4 + 4 * g;
        T o4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (T)(oacc[dt][4 * a4 + e] * inv);
        *reinterpret_cast<uint2*>(Oh + qrow * D + d) = *reinterpret_cast<const uint2*>(o4);
      }
    if (g == 0) Lh[qrow] = (ltot == 0.f) ? -INFINITY : (mref + log2f(ltot)) * kLn2;
  }
}

}  // namespace fa
