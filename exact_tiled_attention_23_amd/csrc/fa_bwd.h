// Exact attention backward by recomputation, bf16/f16 kernels for gfx950.
//
// The backward rebuilds each block of P from the forward's saved row statistics instead of
// storing P ("vectorized-flash-attention-kernel", Key design decision 4: the stored per-row
// statistics let any (query block, key block) pair of S and P be rebuilt for dQ, dK, dV;
// "Paper: FlashAttention", Objectives, Math & data structures: the backward by recomputation
// and the identity rowsum(dP o P) = rowsum(dO o O)). With LSE the natural-log statistic and
// Delta_i = rowsum(dO_i o O_i):
//
//   P_ij  = exp(scale <q_i, k_j> - LSE_i)        (0 for masked pairs and rows with no key)
//   dV_j  = sum_i P_ij dO_i
//   dS_ij = P_ij (<dO_i, v_j> - Delta_i)
//   dQ_i  = scale sum_j dS_ij k_j
//   dK_j  = scale sum_i dS_ij q_i
//
// Two kernels, each the only writer of its outputs (no atomics; the result is the same on
// every run):
//
//  * bwd_dq_kernel: one workgroup per (batch, head, query tile), each wave 32 queries; it
//    walks the key tiles like the forward. S^T = K.Q^T and dP^T = V.dO^T on the matrix
//    cores give each lane one query and 16 keys of every 32-key sub-tile, so P and dS are
//    formed per lane and feed dQ^T = K^T.dS^T straight from the accumulator registers, with
//    K^T fragments from transpose reads (ds_read_b64_tr_b16). Its prologue also forms
//    Delta = rowsum(dO o O) and stores, per 64-row block, the rows' exponent offsets
//    (LSE log2 e, +inf for a row with no key or past N) next to their negated Delta values.
//  * bwd_dkdv_kernel: one workgroup per (batch, head, key tile), each wave 32 keys held in
//    registers; it walks the query tiles. S = Q.K^T and dP = dO.V^T give each lane one key
//    and 16 queries of every 32-query sub-tile (Q and dO rows are read in a permuted order so
//    that the accumulator is exactly the next product's operand), so P and dS feed
//    dV^T = dO^T.P and dK^T = Q^T.dS directly. At D = 128, bwd_dkdv_lds_kernel keeps the
//    tile's K and V in LDS instead of registers so that two waves fit on each SIMD.
//
// Every tensor is addressed through its own batch, head and token strides (the head
// dimension contiguous). Tiles go HBM -> LDS with direct 16-byte copies, double-buffered.
// Every tile is read both row-wise and by transpose reads, so one XOR swizzle of the 16-byte
// chunks serves both without bank conflicts (swz_u below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_kernel.h"
#include "fa_fwd_mfma16.h"

namespace fa {

// Element strides of the batch, head and token dimensions of one [B][H][N][D] tensor (the head
// dimension D is contiguous): element (b, h, n, d) lives at X + b*b_ + h*h_ + n*n_ + d.
struct Strides3 {
  int64_t b, h, n;
};

struct BwdParams {
  const void* q;      // [B][H][N][D], strided as st_q, ...
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;   // contiguous [B][H][N], natural log
  void* dq;           // outputs
  void* dk;
  void* dv;
  Strides3 st_q, st_k, st_v, st_o, st_do, st_dq, st_dk, st_dv;
  float* stats;       // [B*H][ceil(N/64)][128] floats: 64 exponent offsets, then 64 values of -Delta
  const int32_t* kv_len;  // nullable: keys at or past kv_len[b] are padding
  const int32_t* q_len;   // nullable: query rows at or past q_len[b] are padding (not read, dQ = 0)
  int64_t H, N;
  float scale;
  float scale_log2;   // scale * log2(e)
  int causal;
  int n_tiles;        // query tiles (dQ kernel) or key tiles (dK/dV kernel) per head
  int64_t n_units;    // B * H * n_tiles
  int tm_group;       // heads per rank-by-rank group (unit_slot), >= 1
};

constexpr int kStatRows = 64;  // rows per block of the stats array

// Chunk swizzle for tiles read both as row fragments (16 lanes on 16 rows of one chunk) and
// by transpose reads (16 lanes on 4 consecutive rows x 2 chunks): the physical chunk is the
// logical one XOR swz_u(row).
template <int D> __device__ __forceinline__ int swz_u(int j) {
  if constexpr (D >= 128) return 4 * (j & 3) + ((j >> 2) & 3);
  else if constexpr (D == 64) return 2 * ((j >> 1) & 3) + ((j >> 3) & 1);
  else return (j >> 2) & 3;
}

__device__ __forceinline__ int decode_tile(const BwdParams& p, int bid, int* bh) {
  // a head's tiles on one XCD, longest first (fa_fwd_kernel.h)
  const int heads = (int)(p.n_units / p.n_tiles);
  int slot, rank;
  unit_slot(bid, p.n_units, heads, p.n_tiles, p.causal && !p.kv_len && !p.q_len, p.tm_group, &slot, &rank);
  *bh = slot;
  if (p.kv_len || p.q_len) *bh = head_of_slot(slot, heads / (int)p.H, (int)p.H, true);
  return rank;
}

// Per-lane copy plan of a [rows][D] tile into LDS, 1 KB per copy instruction: copy i of this
// wave fills LDS rows (wave*LPW + i)*RPB + lane/CPR, physical chunk lane%CPR. In global memory
// the rows are `stride` bytes apart (the token stride; below 2^31 / ROWS, checked by the host).
// Rows of D = 96 are padded to the LDS row of D = 128 (lds_cols); a lane whose slot is a padding
// chunk copies nothing.
template <int D, int ROWS, int NW>
struct TilePlan {
  static constexpr int DL = lds_cols<D>();
  static constexpr bool PADDED = DL != D;
  static constexpr int ROWB = DL * 2;
  static constexpr int CPR = DL / 8;
  static constexpr int TILEB = ROWS * ROWB;
  static constexpr int LPW = TILEB / 1024 / NW;
  static constexpr int RPB = 1024 / ROWB;
  static_assert(TILEB % (1024 * NW) == 0, "tile must split evenly over waves");
  int row[LPW];
  unsigned chunk[LPW];  // byte offset, within the row, of the logical chunk this lane copies
  bool data[LPW];       // that chunk holds data (not padding)
  __device__ __forceinline__ TilePlan(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int j = (wave * LPW + i) * RPB + lane / CPR;
      const int lc = (lane % CPR) ^ swz_u<DL>(j);
      row[i] = j;
      chunk[i] = lc * 16;
      data[i] = lc < D / 8;
    }
  }
  // Copy rows [r0, r0 + ROWS) of the tensor at `src` (n rows, `stride` bytes apart) into `dst`;
  // rows past n read row n-1 instead.
  __device__ __forceinline__ void issue(const unsigned char* src, unsigned stride, int r0, int n, unsigned dst,
                                        int wave) const {
    const unsigned char* t = src + (int64_t)r0 * stride;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int rr = min(row[i], n - 1 - r0);
      if (!PADDED || data[i]) lds_copy16(t, (unsigned)rr * stride + chunk[i], dst + (wave * LPW + i) * 1024);
    }
  }
  // Zero this lane's slots of rows at or past `lim` (tile-relative).
  __device__ __forceinline__ void zero_from(unsigned char* dst, int lim, int wave, int lane) const {
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      if (row[i] >= lim) *reinterpret_cast<uint4*>(dst + (wave * LPW + i) * 1024 + lane * 16) = uint4{0, 0, 0, 0};
  }
};

// Row fragment (A operand, 32 rows x 16 of the reduction) at LDS tile `t`: row 32u + a_row_key(r),
// reduction chunk 2s + g.
template <typename T, int D>
__device__ __forceinline__ typename Mma<T>::frag row_frag(const unsigned char* t, int row, int chunk) {
  constexpr int DL = lds_cols<D>();
  return *reinterpret_cast<const typename Mma<T>::frag*>(t + row * (2 * DL) + ((chunk ^ swz_u<DL>(row)) * 16));
}

// Transpose fragment: A operand whose rows are the head dimension (32 of them, block dt) and
// whose reduction runs over 16 tile rows starting at `row0` (natural order).
template <typename T, int D>
__device__ __forceinline__ typename Mma<T>::frag tr_frag(const unsigned char* t, int row0, int dt, int lane) {
  const int g = lane >> 5, s16 = lane & 15, s4 = s16 >> 2, sm = s16 & 3, q2 = (lane >> 4) & 1;
  const int c = 4 * dt + 2 * q2 + (sm >> 1);
  const int ra = row0 + 8 * g + s4, rb = ra + 4;
  constexpr int DL = lds_cols<D>();
  const unsigned char* pa = t + ra * (2 * DL) + ((c ^ swz_u<DL>(ra)) * 16) + (sm & 1) * 8;
  const unsigned char* pb = t + rb * (2 * DL) + ((c ^ swz_u<DL>(rb)) * 16) + (sm & 1) * 8;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pb));
  return __builtin_bit_cast(typename Mma<T>::frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int D> constexpr int dkdv_waves_per_eu() { return D >= 128 ? 1 : (D <= 32 ? 3 : 2); }
template <int D> constexpr int dq_waves_per_eu() { return D <= 32 ? 3 : 2; }

// ------------------------------------------------------------------------------------------
// dQ (and Delta, exponent offsets): one workgroup per (b, h, query tile of 32*NW rows).
// LPT: the key-padded launch, whose workgroups take their query tiles longest first.
template <typename T, int D, int BC, int NW, bool LPT = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(dq_waves_per_eu<D>(), dq_waves_per_eu<D>()))) void bwd_dq_kernel(BwdParams p) {
  using M = Mma<T>;
  using frag = typename M::frag;
  static_assert(sizeof(T) == 2, "16-bit element types only");
  constexpr int BR = 32 * NW;
  constexpr int NSUB = BC / 32;
  constexpr int NDT = D / 32;
  constexpr int NQF = D / 16;
  using Plan = TilePlan<D, BC, NW>;
  constexpr int TILEB = Plan::TILEB;

  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * 2 * TILEB];  // [buf][K|V][tile]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;
  const int r = lane & 31;

  int bh, qt;
  if constexpr (LPT) {
    // A head whose kv_len exceeds (t-1)*BC has n_tiles - floor((t-1)*BC/BR) query tiles with at
    // least t key tiles under the causal mask (those from that index on), and all without it.
    const int per_head = p.n_tiles;
    const bool causal = p.causal != 0;
    auto at_least = [&](int t, int kvl) {
      if (t <= 0) return per_head;
      if (kvl <= (t - 1) * BC) return 0;
      return causal ? max(0, per_head - ((t - 1) * BC) / BR) : per_head;
    };
    longest_first(blockIdx.x, (int)(p.n_units / p.n_tiles), (int)p.H, per_head, (int)((p.N + BC - 1) / BC),
                  p.kv_len, (int)p.N, true, at_least, &bh, &qt);
  } else {
    qt = decode_tile(p, blockIdx.x, &bh);
    if (p.causal) qt = p.n_tiles - 1 - qt;  // longest query tiles first
  }
  const int n = (int)p.N;
  const int64_t b_ = bh / p.H, h_ = bh % p.H;
  const T* Qh = reinterpret_cast<const T*>(p.q) + b_ * p.st_q.b + h_ * p.st_q.h;
  const T* Oh = reinterpret_cast<const T*>(p.o) + b_ * p.st_o.b + h_ * p.st_o.h;
  const T* dOh = reinterpret_cast<const T*>(p.dout) + b_ * p.st_do.b + h_ * p.st_do.h;
  const unsigned char* Kh = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.k) + b_ * p.st_k.b + h_ * p.st_k.h);
  const unsigned char* Vh = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.v) + b_ * p.st_v.b + h_ * p.st_v.h);
  T* dQh = reinterpret_cast<T*>(p.dq) + b_ * p.st_dq.b + h_ * p.st_dq.h;
  const unsigned ksn = (unsigned)(p.st_k.n * 2), vsn = (unsigned)(p.st_v.n * 2);

  const int q0 = qt * BR;
  const int qw = q0 + 32 * wave;
  const int qrow = qw + r;
  const int b = bh / (int)p.H;
  int kvl = n;
  if (p.kv_len) {
    const int x = p.kv_len[b];
    kvl = x < 0 ? 0 : (x > n ? n : x);
  }
  int nq = n;  // rows at or past nq are query padding
  if (p.q_len) {
    const int x = p.q_len[b];
    nq = x < 0 ? 0 : (x > n ? n : x);
  }
  int kv_hi = kvl, wave_hi = kvl;
  if (p.causal) {
    kv_hi = min(min(kv_hi, q0 + BR), nq);
    wave_hi = min(min(wave_hi, qw + 32), nq);
  }
  if (q0 >= nq) kv_hi = 0;
  if (qw >= nq) wave_hi = 0;
  kv_hi = __builtin_amdgcn_readfirstlane(kv_hi);    // wave-uniform: keep the tile tests scalar
  wave_hi = __builtin_amdgcn_readfirstlane(wave_hi);
  const int ntiles = kv_hi > 0 ? (kv_hi + BC - 1) / BC : 0;

  // ---- Q^T and dO^T fragments (B operands), Delta = rowsum(dO o O), exponent offset. A
  // padding row gets zero fragments, Delta 0 and an empty row's offset, which make its P, dS
  // and dQ exactly 0. At D <= 96 its loads read row min(qrow, n - 1) (in bounds) and are
  // discarded by selects, so no load sits under a branch: under a per-row branch the compiler
  // waited for each step's loads before issuing the next step's (a memory round trip per 16
  // columns). At D = 128 all of them in flight at once take registers that are not free (the
  // kernel then spilled inside its key loop), and the padding row is not read instead.
  frag qf[NQF], dof[NQF];
  float dsum = 0.f;
  if constexpr (D <= 96) {
    const bool qlive = qrow < nq;
    const int64_t qrow_ld = qrow < n ? qrow : n - 1;
#pragma unroll
    for (int s = 0; s < NQF; ++s) {
      qf[s] = *reinterpret_cast<const frag*>(Qh + qrow_ld * p.st_q.n + 16 * s + 8 * g);
      dof[s] = *reinterpret_cast<const frag*>(dOh + qrow_ld * p.st_do.n + 16 * s + 8 * g);
    }
#pragma unroll
    for (int s = 0; s < NQF; ++s) {
      const frag of = *reinterpret_cast<const frag*>(Oh + qrow_ld * p.st_o.n + 16 * s + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf((float)dof[s][e], (float)of[e], dsum);
    }
    dsum = qlive ? dsum : 0.f;
#pragma unroll
    for (int s = 0; s < NQF; ++s) {
      qf[s] = qlive ? qf[s] : frag{};
      dof[s] = qlive ? dof[s] : frag{};
    }
  } else {
#pragma unroll
    for (int s = 0; s < NQF; ++s) {
      if (qrow < nq) {
        qf[s] = *reinterpret_cast<const frag*>(Qh + (int64_t)qrow * p.st_q.n + 16 * s + 8 * g);
        dof[s] = *reinterpret_cast<const frag*>(dOh + (int64_t)qrow * p.st_do.n + 16 * s + 8 * g);
        const frag of = *reinterpret_cast<const frag*>(Oh + (int64_t)qrow * p.st_o.n + 16 * s + 8 * g);
#pragma unroll
        for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf((float)dof[s][e], (float)of[e], dsum);
      } else {
        qf[s] = frag{};
        dof[s] = frag{};
      }
    }
  }
  const float delta = pair_sum(dsum);
  constexpr bool kDeltaInAcc = D <= 64;
  f32x16 ndelta16;
#pragma unroll
  for (int i = 0; i < 16; ++i) ndelta16[i] = -delta;
  const float lse = qrow < nq ? p.lse[(int64_t)bh * n + qrow] : -INFINITY;
  // P = 2^(s*c - mo): +inf offset for a row with no valid key (its P is 0).
  const float mo = (lse == -INFINITY) ? INFINITY : lse * kLog2e;
  {
    const int n64 = (n + kStatRows - 1) / kStatRows;
    if (g == 0 && qrow < n64 * kStatRows) {
      float* st = p.stats + ((int64_t)bh * n64 + qrow / kStatRows) * (2 * kStatRows) + qrow % kStatRows;
      st[0] = mo;
      st[kStatRows] = qrow < n ? -delta : 0.f;
    }
  }

  const Plan plan(wave, lane);
  const int kr = a_row_key<8>(r);
  f32x16 acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) acc[t] = f32x16{};
  const float c = in_vgpr(p.scale_log2);  // the scaling FMAs read vector registers only (+1-2% at D <= 96)

  auto issue = [&](int t, int buf) {
    const unsigned kl = lds_address(lds + buf * 2 * TILEB);
    plan.issue(Kh, ksn, t * BC, n, kl, wave);
    plan.issue(Vh, vsn, t * BC, n, kl + TILEB, wave);
  };
  if (ntiles > 0) issue(0, 0);

  // Two tiles per iteration, one per buffer: the buffer is a compile-time constant in each copy
  // of the body, so LDS addresses are per-lane registers plus immediate offsets.
  auto tile_step = [&](const int t, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    const int j0 = t * BC;
    unsigned char* kb = lds + buf * 2 * TILEB;
    unsigned char* vb = kb + TILEB;
    wait_vmem();
    if (j0 + BC > kvl) {
      // Rows at or past kv_len may hold anything: zero them so 0 * garbage cannot reach dQ.
      plan.zero_from(kb, kvl - j0, wave, lane);
      plan.zero_from(vb, kvl - j0, wave, lane);
    }
    __syncthreads();
    if (t + 1 < ntiles) issue(t + 1, buf ^ 1);

    if (j0 < wave_hi) {
      const bool edge = j0 + BC > kvl || (p.causal && j0 + BC - 1 > qw);
      int lim = kvl - j0;
      if (p.causal) lim = min(lim, qrow - j0 + 1);
      lim -= 8 * g;
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        // S^T and dP^T for 32 keys (rows of K and V in the permuted order a_row_key), with the
        // row fragments of step st+PD and the K^T transpose fragments of the dQ product below
        // read while step st's products run (order pinned as in the dK/dV kernel).
        // At D <= 64 the dP^T accumulator starts at -Delta (this lane's query), so the products
        // leave dP - Delta in it and dS needs one multiply; at D >= 96 the 16 registers that
        // takes are not free, and Delta is subtracted per element instead.
        f32x16 s = f32x16{}, dp = kDeltaInAcc ? ndelta16 : f32x16{};
        // At D = 128 only the first half of the K^T fragments is read ahead (all of them would
        // not fit in the registers of two waves per SIMD); the second half is read while the
        // first half's products run.
        constexpr int KTH = D >= 128 ? 1 : 2;
        frag kt[2][NDT];
        {
          constexpr int PD = 2;
          static_assert(2 * 2 * NDT == 2 * NQF, "transpose reads per step");
          frag ka[PD + 1], va[PD + 1];
#pragma unroll
          for (int st = 0; st < PD; ++st) {
            ka[st] = row_frag<T, D>(kb, 32 * u + kr, 2 * st + g);
            va[st] = row_frag<T, D>(vb, 32 * u + kr, 2 * st + g);
          }
#pragma unroll
          for (int st = 0; st < NQF; ++st) {
            if (st + PD < NQF) {
              ka[(st + PD) % (PD + 1)] = row_frag<T, D>(kb, 32 * u + kr, 2 * (st + PD) + g);
              va[(st + PD) % (PD + 1)] = row_frag<T, D>(vb, 32 * u + kr, 2 * (st + PD) + g);
            }
            s = M::run(ka[st % (PD + 1)], qf[st], s);
            dp = M::run(va[st % (PD + 1)], dof[st], dp);
          }
#pragma unroll
          for (int h = 0; h < KTH; ++h)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) kt[h][dt] = tr_frag<T, D>(kb, 32 * u + 16 * h, dt, lane);
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * PD, 0);
#pragma unroll
          for (int st = 0; st < NQF; ++st) {
            if (st + PD < NQF) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // row reads of st+PD
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                    // products of st
            __builtin_amdgcn_sched_group_barrier(0x100, KTH, 0);                  // transpose reads
          }
        }
        // P and dS; register i of half g holds key 32u + 16(i/8) + 8g + i%8.
        float ds[16];
        // The key masks only on edge tiles (a wave-uniform test). At D = 128 the second copy of
        // this code costs 12 bytes of scratch per lane, and still measured 1% faster.
        if (edge) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -mo));
            x = (32 * u + 16 * (i / 8) + (i % 8) >= lim) ? 0.f : x;
            ds[i] = kDeltaInAcc ? x * dp[i] : x * (dp[i] - delta);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -mo));
            ds[i] = kDeltaInAcc ? x * dp[i] : x * (dp[i] - delta);
          }
        }
        frag dsf[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e) dsf[h][e] = (T)ds[8 * h + e];
        // dQ^T += K^T . dS^T
        if constexpr (KTH == 1) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) kt[1][dt] = tr_frag<T, D>(kb, 32 * u + 16, dt, lane);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) acc[dt] = M::run(kt[h][dt], dsf[h], acc[dt]);
      }
    }
  };
  for (int t = 0; t < ntiles; t += 2) {
    tile_step(t, Int<0>{});
    if (t + 1 >= ntiles) break;
    tile_step(t + 1, Int<1>{});
  }

  // ---- dQ = scale * acc; register i of block dt holds d = 32dt + 8(i/4) + 4g + i%4. The row's
  // 64-bit offset is formed here from its 32-bit index (an opaque copy keeps the compiler from
  // forming it before the loop and holding two more registers through it).
  int qrow_out = qrow;
  asm volatile("" : "+v"(qrow_out));
  if (qrow_out < n) {
    T* drow = dQh + (int64_t)qrow_out * p.st_dq.n + 4 * g;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        T o4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (T)(acc[dt][4 * a4 + e] * p.scale);
        *reinterpret_cast<uint2*>(drow + 32 * dt + 8 * a4) = *reinterpret_cast<const uint2*>(o4);
      }
  }
}

// Key tile of workgroup `bid` for the dK/dV kernels (BKV keys per tile, query tiles of BQ rows).
// Without LPT: decode_tile's order. With LPT (the key-padded launch): longest first. A key tile
// below kv_len is seen by ceil(N/BQ) query tiles, less floor(first key/BQ) under the causal mask,
// and one at or past kv_len by none; so a head has min(ceil(kvl/BKV), ceil((NQ-t+1)*BQ/BKV)) key
// tiles with at least t query tiles under the mask (ceil(kvl/BKV) for t <= NQ without it), its
// tiles with the most work being the first.
template <int BKV, int BQ, bool LPT>
__device__ __forceinline__ int decode_key_tile(const BwdParams& p, int bid, int* bh) {
  if constexpr (LPT) {
    const int per_head = p.n_tiles;
    const int n = (int)p.N;
    const int nq = (n + BQ - 1) / BQ;
    const bool causal = p.causal != 0;
    auto at_least = [&](int t, int kvl) {
      if (t <= 0) return per_head;
      const int live = (kvl + BKV - 1) / BKV;  // key tiles below kv_len
      if (!causal) return t <= nq ? live : 0;
      const int lim = nq - t + 1;
      return lim <= 0 ? 0 : min(live, (lim * BQ + BKV - 1) / BKV);
    };
    int kt;
    longest_first(bid, (int)(p.n_units / p.n_tiles), (int)p.H, per_head, nq, p.kv_len, n, false, at_least, bh, &kt);
    return kt;
  } else {
    return decode_tile(p, bid, bh);  // causal: key tile 0 has the most work
  }
}

// ------------------------------------------------------------------------------------------
// dK, dV: one workgroup per (b, h, key tile of 32*NW keys); query tiles of BQ rows.
// Two waves per SIMD where the registers allow it; at D = 128 the K, V fragments and the dK, dV
// accumulators alone take 192 registers, so one.

template <typename T, int D, int BQ, int NW, bool LPT = false>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(dkdv_waves_per_eu<D>(), dkdv_waves_per_eu<D>())))
void bwd_dkdv_kernel(BwdParams p) {
  using M = Mma<T>;
  using frag = typename M::frag;
  static_assert(sizeof(T) == 2, "16-bit element types only");
  static_assert(BQ == kStatRows, "one stats block per query tile");
  constexpr int BKV = 32 * NW;
  constexpr int NSUB = BQ / 32;
  constexpr int NDT = D / 32;
  constexpr int NQF = D / 16;
  using Plan = TilePlan<D, BQ, NW>;
  constexpr int TILEB = Plan::TILEB;
  constexpr int STATB = 1024;                 // one copy instruction: the 512-byte stats block, twice
  constexpr int BUFB = 2 * TILEB + STATB;

  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * BUFB];  // [buf][Q|dO|stats]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;
  const int r = lane & 31;

  int bh;
  const int kt = decode_key_tile<BKV, BQ, LPT>(p, blockIdx.x, &bh);
  const int n = (int)p.N;
  const int64_t b_ = bh / p.H, h_ = bh % p.H;
  const unsigned char* Qh = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.q) + b_ * p.st_q.b + h_ * p.st_q.h);
  const unsigned char* dOh = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.dout) + b_ * p.st_do.b + h_ * p.st_do.h);
  const T* Kh = reinterpret_cast<const T*>(p.k) + b_ * p.st_k.b + h_ * p.st_k.h;
  const T* Vh = reinterpret_cast<const T*>(p.v) + b_ * p.st_v.b + h_ * p.st_v.h;
  T* dKh = reinterpret_cast<T*>(p.dk) + b_ * p.st_dk.b + h_ * p.st_dk.h;
  T* dVh = reinterpret_cast<T*>(p.dv) + b_ * p.st_dv.b + h_ * p.st_dv.h;
  const unsigned qsn = (unsigned)(p.st_q.n * 2), osn = (unsigned)(p.st_do.n * 2);
  const int n64 = (n + kStatRows - 1) / kStatRows;
  const unsigned char* Sh = reinterpret_cast<const unsigned char*>(p.stats + (int64_t)bh * n64 * (2 * kStatRows));

  const int k0 = kt * BKV;
  const int kw = k0 + 32 * wave;
  const int key = kw + r;
  const int b = bh / (int)p.H;
  int kvl = n;
  if (p.kv_len) {
    const int x = p.kv_len[b];
    kvl = x < 0 ? 0 : (x > n ? n : x);
  }
  int nq = n;  // rows at or past nq are query padding
  if (p.q_len) {
    const int x = p.q_len[b];
    nq = x < 0 ? 0 : (x > n ? n : x);
  }
  // Query tiles that can see some key of this tile: all of them up to the last present row,
  // or from the diagonal on.
  const int nqt = k0 < kvl ? (nq + BQ - 1) / BQ : 0;
  const int t0 = p.causal ? k0 / BQ : 0;

  // ---- K^T and V^T fragments (B operands) of this lane's key; zero past kv_len, where
  // P is forced to 0 as well.
  const bool key_dead = key >= kvl;
  const bool any_key_dead = __any(key_dead);  // wave-uniform
  frag kf[NQF], vf[NQF];
#pragma unroll
  for (int s = 0; s < NQF; ++s) {
    if (key < kvl) {
      kf[s] = *reinterpret_cast<const frag*>(Kh + (int64_t)key * p.st_k.n + 16 * s + 8 * g);
      vf[s] = *reinterpret_cast<const frag*>(Vh + (int64_t)key * p.st_v.n + 16 * s + 8 * g);
    } else {
      kf[s] = frag{};
      vf[s] = frag{};
    }
  }

  const Plan plan(wave, lane);
  const int qr = a_row_key<8>(r);
  f32x16 dka[NDT], dva[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    dka[t] = f32x16{};
    dva[t] = f32x16{};
  }
  const float c = in_vgpr(p.scale_log2);  // the scaling FMAs read vector registers only (+1-2% at D <= 96)
  // Stats copy: lanes 0-31 bring the 512-byte block of 64 offsets and 64 values of -Delta,
  // lanes 32-63 the same bytes again (the copy instruction always moves 1 KB).
  const unsigned stat_off = (unsigned)(lane & 31) * 16;

  auto issue = [&](int t, int buf) {
    const unsigned ql = lds_address(lds + buf * BUFB);
    plan.issue(Qh, qsn, t * BQ, n, ql, wave);
    plan.issue(dOh, osn, t * BQ, n, ql + TILEB, wave);
    if (wave == 0) lds_copy16(Sh + (int64_t)t * (2 * kStatRows) * 4, stat_off, ql + 2 * TILEB);
  };
  if (t0 < nqt) issue(t0, 0);

  // Two query tiles per iteration, one per buffer (compile-time buffer offsets, as in the dQ
  // kernel).
  auto tile_step = [&](const int t, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    const int i0 = t * BQ;
    const unsigned char* qb = lds + buf * BUFB;
    const unsigned char* ob = qb + TILEB;
    const float* sb = reinterpret_cast<const float*>(qb + 2 * TILEB);
    wait_vmem();
    if (i0 + BQ > nq) {
      // Padding query rows may hold anything: zero them so 0 * garbage cannot reach dK, dV.
      plan.zero_from(lds + buf * BUFB, nq - i0, wave, lane);
      plan.zero_from(lds + buf * BUFB + TILEB, nq - i0, wave, lane);
    }
    __syncthreads();
    if (t + 1 < nqt) issue(t + 1, buf ^ 1);

#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
      const int qs = i0 + 32 * u;
      if (p.causal && qs + 31 < kw) continue;  // every query of this sub-tile precedes every key of the wave
      // S and dP for 32 queries (rows of Q and dO in the permuted order a_row_key). The row
      // fragments of step st+PD are read while step st's products run, and the transpose
      // fragments of the dV/dK products below are read in the same stretch, so no product
      // waits on a read issued just before it. The order is pinned with scheduling-group
      // barriers (the scheduler otherwise places each read right before its product).
      // Register i of half g holds query qs + 16(i/8) + 8g + i%8 of this lane's key. The dP
      // accumulator starts at those queries' -Delta, so the products leave dP - Delta in it.
      float mo[16];
      f32x16 dp;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4* pm = reinterpret_cast<const float4*>(sb + 32 * u + 16 * h + 8 * g);
        const float4* pd = reinterpret_cast<const float4*>(sb + kStatRows + 32 * u + 16 * h + 8 * g);
        const float4 m0 = pm[0], m1 = pm[1], d0 = pd[0], d1 = pd[1];
        mo[8 * h + 0] = m0.x; mo[8 * h + 1] = m0.y; mo[8 * h + 2] = m0.z; mo[8 * h + 3] = m0.w;
        mo[8 * h + 4] = m1.x; mo[8 * h + 5] = m1.y; mo[8 * h + 6] = m1.z; mo[8 * h + 7] = m1.w;
        dp[8 * h + 0] = d0.x; dp[8 * h + 1] = d0.y; dp[8 * h + 2] = d0.z; dp[8 * h + 3] = d0.w;
        dp[8 * h + 4] = d1.x; dp[8 * h + 5] = d1.y; dp[8 * h + 6] = d1.z; dp[8 * h + 7] = d1.w;
      }
      f32x16 s = f32x16{};
      frag tq[2][NDT], to[2][NDT];
      {
        constexpr int PD = 2;
        // 16 transpose fragments of two reads each: 4 reads per reduction step at every D.
        static_assert(4 * 2 * NDT == 4 * NQF, "transpose reads per step");
        frag qa[PD + 1], oa[PD + 1];
#pragma unroll
        for (int st = 0; st < PD; ++st) {
          qa[st] = row_frag<T, D>(qb, 32 * u + qr, 2 * st + g);
          oa[st] = row_frag<T, D>(ob, 32 * u + qr, 2 * st + g);
        }
#pragma unroll
        for (int st = 0; st < NQF; ++st) {
          if (st + PD < NQF) {
            qa[(st + PD) % (PD + 1)] = row_frag<T, D>(qb, 32 * u + qr, 2 * (st + PD) + g);
            oa[(st + PD) % (PD + 1)] = row_frag<T, D>(ob, 32 * u + qr, 2 * (st + PD) + g);
          }
          s = M::run(qa[st % (PD + 1)], kf[st], s);
          dp = M::run(oa[st % (PD + 1)], vf[st], dp);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            to[h][dt] = tr_frag<T, D>(ob, 32 * u + 16 * h, dt, lane);
            tq[h][dt] = tr_frag<T, D>(qb, 32 * u + 16 * h, dt, lane);
          }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PD, 0);
#pragma unroll
        for (int st = 0; st < NQF; ++st) {
          if (st + PD < NQF) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // row reads of st+PD
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                    // products of st
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                    // transpose reads
        }
      }
      const bool diag = p.causal && qs < kw + 31;
      float pr[16], ds[16];
      // Masks only where a key of the wave is padding or the tile meets the diagonal (a
      // wave-uniform test); elsewhere every (query, key) pair is live.
      if (diag || any_key_dead) {
        // Element i (query qs + 16(i/8) + 8g + i%8) is dead when its offset 16(i/8) + i%8 is
        // below lim: always for a padding key, never off the diagonal.
        const int lim = key_dead ? INT_MAX : (diag ? key - qs - 8 * g : INT_MIN);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -mo[i]));
          x = (16 * (i / 8) + (i % 8) < lim) ? 0.f : x;
          pr[i] = x;
          ds[i] = x * dp[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -mo[i]));
          ds[i] = pr[i] * dp[i];
        }
      }
      frag pf[2], dsf[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pf[h][e] = (T)pr[8 * h + e];
          dsf[h][e] = (T)ds[8 * h + e];
        }
      // dV^T += dO^T . P and dK^T += Q^T . dS
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          dva[dt] = M::run(to[h][dt], pf[h], dva[dt]);
          dka[dt] = M::run(tq[h][dt], dsf[h], dka[dt]);
        }
    }
  };
  for (int t = t0; t < nqt; t += 2) {
    tile_step(t, Int<0>{});
    if (t + 1 >= nqt) break;
    tile_step(t + 1, Int<1>{});
  }

  // ---- dK = scale * dka, dV = dva; register i of block dt holds d = 32dt + 8(i/4) + 4g + i%4.
  // Keys past kv_len have zero P and dS, so they store exact zeros.
  if (key < n) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        T k4[4], v4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = (T)(dka[dt][4 * a4 + e] * p.scale);
          v4[e] = (T)dva[dt][4 * a4 + e];
        }
        const int dd = 32 * dt + 8 * a4 + 4 * g;
        *reinterpret_cast<uint2*>(dKh + (int64_t)key * p.st_dk.n + dd) = *reinterpret_cast<const uint2*>(k4);
        *reinterpret_cast<uint2*>(dVh + (int64_t)key * p.st_dv.n + dd) = *reinterpret_cast<const uint2*>(v4);
      }
  }
}

// ------------------------------------------------------------------------------------------
// dK, dV at D = 128 with two waves per SIMD: the registers cannot hold each wave's K and V
// fragments next to its dK and dV accumulators (192 registers), so the workgroup's 128 keys of K
// and V live in LDS (64 KB, loaded once) and are read as B operands at each use. Eight waves: a
// pair of waves shares each 32-key group, and wave w takes the 32-query half w / 4 of every
// 64-row query tile; at the end the pair's partial dK and dV are added through LDS.
template <typename T, int D, int BQ, int NW, bool LPT = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_lds_kernel(BwdParams p) {
  using M = Mma<T>;
  using frag = typename M::frag;
  static_assert(sizeof(T) == 2, "16-bit element types only");
  static_assert(BQ == kStatRows && BQ == 64, "one stats block per query tile, two halves of 32");
  static_assert(NW == 8, "four key groups x two query halves");
  constexpr int BKV = 128;
  constexpr int NDT = D / 32;
  constexpr int NQF = D / 16;
  constexpr int PD = 1;  // fragments read one reduction step ahead (two would spill)
  using KPlan = TilePlan<D, BKV, NW>;
  using QPlan = TilePlan<D, BQ, NW>;
  constexpr int KTB = KPlan::TILEB;            // K (or V) tile bytes
  constexpr int QTB = QPlan::TILEB;            // Q (or dO) tile bytes
  constexpr int STATB = 1024;
  constexpr int BUFB = 2 * QTB + STATB;
  constexpr int LDSB = 2 * KTB + 2 * BUFB;
  static_assert(4 * 64 * 2 * NDT * 16 * 4 <= LDSB, "the partner partials fit in LDS");
  static_assert(4 * 2 * NDT == 4 * NQF, "transpose reads per step");

  __shared__ __attribute__((aligned(1024))) unsigned char lds[LDSB];  // [K|V][buf][Q|dO|stats]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;
  const int r = lane & 31;
  const int kg = wave & 3;   // key group
  const int qh = wave >> 2;  // query half of each tile

  int bh;
  const int kt = decode_key_tile<BKV, BQ, LPT>(p, blockIdx.x, &bh);
  const int n = (int)p.N;
  const int64_t b_ = bh / p.H, h_ = bh % p.H;
  const unsigned char* Qh = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.q) + b_ * p.st_q.b + h_ * p.st_q.h);
  const unsigned char* dOh = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.dout) + b_ * p.st_do.b + h_ * p.st_do.h);
  const unsigned char* Kh = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.k) + b_ * p.st_k.b + h_ * p.st_k.h);
  const unsigned char* Vh = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.v) + b_ * p.st_v.b + h_ * p.st_v.h);
  T* dKh = reinterpret_cast<T*>(p.dk) + b_ * p.st_dk.b + h_ * p.st_dk.h;
  T* dVh = reinterpret_cast<T*>(p.dv) + b_ * p.st_dv.b + h_ * p.st_dv.h;
  const unsigned qsn = (unsigned)(p.st_q.n * 2), osn = (unsigned)(p.st_do.n * 2);
  const unsigned ksn = (unsigned)(p.st_k.n * 2), vsn = (unsigned)(p.st_v.n * 2);
  const int n64 = (n + kStatRows - 1) / kStatRows;
  const unsigned char* Sh = reinterpret_cast<const unsigned char*>(p.stats + (int64_t)bh * n64 * (2 * kStatRows));

  const int k0 = kt * BKV;
  const int kw = k0 + 32 * kg;
  const int key = kw + r;
  const int b = bh / (int)p.H;
  int kvl = n;
  if (p.kv_len) {
    const int x = p.kv_len[b];
    kvl = x < 0 ? 0 : (x > n ? n : x);
  }
  int nq = n;  // rows at or past nq are query padding
  if (p.q_len) {
    const int x = p.q_len[b];
    nq = x < 0 ? 0 : (x > n ? n : x);
  }
  const int nqt = k0 < kvl ? (nq + BQ - 1) / BQ : 0;
  const int t0 = p.causal ? k0 / BQ : 0;
  const bool key_dead = key >= kvl;
  const bool any_key_dead = __any(key_dead);  // wave-uniform

  unsigned char* kb = lds;
  unsigned char* vb = lds + KTB;
  unsigned char* qbuf = lds + 2 * KTB;
  const KPlan kplan(wave, lane);
  const QPlan qplan(wave, lane);
  const unsigned stat_off = (unsigned)(lane & 31) * 16;
  auto issue = [&](int t, int buf) {
    const unsigned ql = lds_address(qbuf + buf * BUFB);
    qplan.issue(Qh, qsn, t * BQ, n, ql, wave);
    qplan.issue(dOh, osn, t * BQ, n, ql + QTB, wave);
    if (wave == 0) lds_copy16(Sh + (int64_t)t * (2 * kStatRows) * 4, stat_off, ql + 2 * QTB);
  };
  if (t0 < nqt) {
    kplan.issue(Kh, ksn, k0, n, lds_address(kb), wave);
    kplan.issue(Vh, vsn, k0, n, lds_address(vb), wave);
    issue(t0, 0);
    wait_vmem();
    // Keys at or past kv_len may hold anything: zero them so 0 * garbage cannot reach dK, dV.
    if (k0 + BKV > kvl) {
      kplan.zero_from(kb, kvl - k0, wave, lane);
      kplan.zero_from(vb, kvl - k0, wave, lane);
    }
  }

  const int qr = a_row_key<8>(r);
  f32x16 dka[NDT], dva[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    dka[t] = f32x16{};
    dva[t] = f32x16{};
  }
  const float c = in_vgpr(p.scale_log2);  // the scaling FMAs read vector registers only (+1-2% at D <= 96)

  for (int t = t0; t < nqt; ++t) {
    const int i0 = t * BQ;
    const int buf = (t - t0) & 1;
    const unsigned char* qb = qbuf + buf * BUFB;
    const unsigned char* ob = qb + QTB;
    const float* sb = reinterpret_cast<const float*>(qb + 2 * QTB);
    if (t > t0) wait_vmem();
    if (i0 + BQ > nq) {
      // Padding query rows may hold anything: zero them so 0 * garbage cannot reach dK, dV.
      qplan.zero_from(qbuf + buf * BUFB, nq - i0, wave, lane);
      qplan.zero_from(qbuf + buf * BUFB + QTB, nq - i0, wave, lane);
    }
    __syncthreads();
    if (t + 1 < nqt) issue(t + 1, buf ^ 1);

    const int qs = i0 + 32 * qh;
    if (p.causal && qs + 31 < kw) continue;  // every query of this half precedes every key of the group
    // S = Q K^T and dP = dO V^T for this wave's 32 queries (rows in the permuted order a_row_key)
    // and 32 keys (B operands read from the K and V tiles), each step's fragments read PD steps
    // ahead of its products.
    f32x16 s = f32x16{}, dp = f32x16{};
    {
      frag qa[PD + 1], oa[PD + 1], ka[PD + 1], va[PD + 1];
      auto rd = [&](int st, int slot) {
        qa[slot] = row_frag<T, D>(qb, 32 * qh + qr, 2 * st + g);
        oa[slot] = row_frag<T, D>(ob, 32 * qh + qr, 2 * st + g);
        ka[slot] = row_frag<T, D>(kb, 32 * kg + r, 2 * st + g);
        va[slot] = row_frag<T, D>(vb, 32 * kg + r, 2 * st + g);
      };
#pragma unroll
      for (int st = 0; st < PD; ++st) rd(st, st);
#pragma unroll
      for (int st = 0; st < NQF; ++st) {
        if (st + PD < NQF) rd(st + PD, (st + PD) % (PD + 1));
        s = M::run(qa[st % (PD + 1)], ka[st % (PD + 1)], s);
        dp = M::run(oa[st % (PD + 1)], va[st % (PD + 1)], dp);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * PD, 0);
#pragma unroll
      for (int st = 0; st < NQF; ++st) {
        if (st + PD < NQF) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // fragments of st+PD
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                    // products of st
      }
    }
    // Transpose fragments of the dV/dK products come two at a time (pair j = h*NDT + dt: dO^T and
    // Q^T for 16 queries and 32 dims); pair 0 is read here, under the arithmetic below.
    constexpr int NPAIR = 2 * NDT;
    frag tto[2], ttq[2];
    ttq[0] = tr_frag<T, D>(qb, 32 * qh, 0, lane);
    tto[0] = tr_frag<T, D>(ob, 32 * qh, 0, lane);
    // Register i of half g holds query qs + 16(i/8) + 8g + i%8 of this lane's key. The queries'
    // exponent offsets and -Delta come from LDS 8 at a time (per 16-query half), as needed.
    auto stats8 = [&](int hh, float* mo8, float* dl8) __attribute__((always_inline)) {
      const float4* pm = reinterpret_cast<const float4*>(sb + 32 * qh + 16 * hh + 8 * g);
      const float4* pd = reinterpret_cast<const float4*>(sb + kStatRows + 32 * qh + 16 * hh + 8 * g);
      const float4 m0 = pm[0], m1 = pm[1], d0 = pd[0], d1 = pd[1];
      mo8[0] = m0.x; mo8[1] = m0.y; mo8[2] = m0.z; mo8[3] = m0.w;
      mo8[4] = m1.x; mo8[5] = m1.y; mo8[6] = m1.z; mo8[7] = m1.w;
      dl8[0] = d0.x; dl8[1] = d0.y; dl8[2] = d0.z; dl8[3] = d0.w;
      dl8[4] = d1.x; dl8[5] = d1.y; dl8[6] = d1.z; dl8[7] = d1.w;
    };
    const bool diag = p.causal && qs < kw + 31;
    frag pf[2], dsf[2];
    // Masks only where a key of the wave is padding or the tile meets the diagonal (a
    // wave-uniform test); elsewhere every (query, key) pair is live. At D = 128 the second
    // copy of this code pushes the kernel past its registers (spills measured 3% slower), so
    // there the masked form runs on every tile.
    if (D >= 128 || diag || any_key_dead) {
      // Element i (query qs + 16(i/8) + 8g + i%8) is dead when its offset 16(i/8) + i%8 is below
      // lim: always for a padding key, never off the diagonal.
      const int lim = key_dead ? INT_MAX : (diag ? key - qs - 8 * g : INT_MIN);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float mo[8], dl[8];
        stats8(hh, mo, dl);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * hh + e;
          float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -mo[e]));
          x = (16 * hh + e < lim) ? 0.f : x;
          pf[hh][e] = (T)x;
          dsf[hh][e] = (T)(x * (dp[i] + dl[e]));  // dl holds -Delta
        }
      }
    } else {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float mo[8], dl[8];
        stats8(hh, mo, dl);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * hh + e;
          const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -mo[e]));
          pf[hh][e] = (T)x;
          dsf[hh][e] = (T)(x * (dp[i] + dl[e]));  // dl holds -Delta
        }
      }
    }
    // dV^T += dO^T . P and dK^T += Q^T . dS, reading pair j+1 while pair j's products run.
#pragma unroll
    for (int j = 0; j < NPAIR; ++j) {
      if (j + 1 < NPAIR) {
        ttq[(j + 1) & 1] = tr_frag<T, D>(qb, 32 * qh + 16 * ((j + 1) / NDT), (j + 1) % NDT, lane);
        tto[(j + 1) & 1] = tr_frag<T, D>(ob, 32 * qh + 16 * ((j + 1) / NDT), (j + 1) % NDT, lane);
      }
      dva[j % NDT] = M::run(tto[j & 1], pf[j / NDT], dva[j % NDT]);
      dka[j % NDT] = M::run(ttq[j & 1], dsf[j / NDT], dka[j % NDT]);
    }
  }

  // ---- add the pair's partials: waves of the second query half hand theirs over through LDS.
  __syncthreads();  // every wave is done with the tiles
  float4* part = reinterpret_cast<float4*>(lds) + (kg * 2 * NDT * 4) * 64 + lane;
  if (qh == 1) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        part[((2 * dt) * 4 + a4) * 64] = make_float4(dka[dt][4 * a4], dka[dt][4 * a4 + 1], dka[dt][4 * a4 + 2], dka[dt][4 * a4 + 3]);
        part[((2 * dt + 1) * 4 + a4) * 64] = make_float4(dva[dt][4 * a4], dva[dt][4 * a4 + 1], dva[dt][4 * a4 + 2], dva[dt][4 * a4 + 3]);
      }
  }
  __syncthreads();
  if (qh == 1 || key >= n) return;
  // dK = scale * dka, dV = dva; register i of block dt holds d = 32dt + 8(i/4) + 4g + i%4.
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const float4 pk = part[((2 * dt) * 4 + a4) * 64];
      const float4 pv = part[((2 * dt + 1) * 4 + a4) * 64];
      const float ks[4] = {pk.x, pk.y, pk.z, pk.w}, vs[4] = {pv.x, pv.y, pv.z, pv.w};
      T k4[4], v4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k4[e] = (T)((dka[dt][4 * a4 + e] + ks[e]) * p.scale);
        v4[e] = (T)(dva[dt][4 * a4 + e] + vs[e]);
      }
      const int dd = 32 * dt + 8 * a4 + 4 * g;
      *reinterpret_cast<uint2*>(dKh + (int64_t)key * p.st_dk.n + dd) = *reinterpret_cast<const uint2*>(k4);
      *reinterpret_cast<uint2*>(dVh + (int64_t)key * p.st_dv.n + dd) = *reinterpret_cast<const uint2*>(v4);
    }
}

}  // namespace fa
