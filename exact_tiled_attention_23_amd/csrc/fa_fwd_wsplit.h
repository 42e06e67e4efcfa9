// Exact tiled attention forward for problems far smaller than the GPU: the key axis of each query
// block split over the waves of one workgroup.
//
// With few query tiles (a short sequence, one head), the regular kernels leave most compute
// units idle and their time is one wave's walk over all the keys of its rows. Here a workgroup
// owns 32 query rows, and its NW waves take the key tiles of those rows in turn (wave w takes
// tiles w, w + NW, ...), each with its own running state (reference maximum m, denominator l,
// unnormalised accumulator O). The partial states are then combined with the associative merge
// of online-softmax states ("Paper: FlashAttention", Objectives, Math & data structures: partial
// results over disjoint key sets merge exactly, and the empty state (m = -inf, l = 0, O = 0) is
// the identity):
//
//     m = max_w m_w,   a_w = 2^(m_w - m) (0 for an empty part),   l = sum_w a_w l_w,
//     O = (sum_w a_w O_w) / l,   LSE = (m + log2 l) ln 2,
//
// through LDS inside the workgroup, so the call needs no workspace. A wave's tile is 32 keys,
// staged global -> registers -> the wave's own LDS region (K and V row-major), with the
// next tile's loads in flight while the current one is computed; the waves touch only their own
// LDS until the merge, so they need no barrier before it. The arithmetic per tile is that of
// fwd_kernel in fa_fwd_kernel.h (S^T = K . Q^T, masks, base-2 online softmax, O^T += V^T . P^T).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_kernel.h"

namespace fa {

template <typename T, int D, int NW>
__global__ __launch_bounds__(NW * 64) void fwd_wsplit_kernel(FwdParams p) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int KPER = M::KPER;
  constexpr int KSTEP = 2 * KPER;
  constexpr int BC = 32;                          // keys per wave tile
  constexpr int CH = 16 / (int)sizeof(T);         // elements per 16-byte chunk
  constexpr int CPR = D / CH;                     // chunks per row
  constexpr int KLD = D + CH;                     // K row stride in LDS (padded by 16 bytes)
  constexpr int VLD = BC + CH;                    // V^T row stride in LDS (16-bit types)
  constexpr int NDT = D / 32;
  constexpr int NQF = D / KSTEP;
  constexpr int WAVE_ELEMS = BC * KLD + D * VLD;  // one wave's K and V tiles (V row-major for float32)
  static_assert(BC * KLD <= D * VLD, "a row-major V tile fits in the V area");
  constexpr int K_UNITS = BC * CPR / 64;          // 16-byte K chunks per lane per tile
  constexpr int V_ROWS = (sizeof(T) == 2) ? 2 : 1;
  constexpr int V_UNITS = (BC / V_ROWS) * CPR / 64;
  constexpr int OLD = D + 4;                      // row stride of the merge's O rows (floats)
  constexpr int STAGE_BYTES = NW * WAVE_ELEMS * (int)sizeof(T);
  constexpr int MERGE_BYTES = NW * 32 * (OLD + 2) * 4;
  constexpr int LDS_BYTES = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
  static_assert(BC * CPR % 64 == 0 && (BC / V_ROWS) * CPR % 64 == 0, "staging must divide evenly");

  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int r = lane & 31;
  T* k_lds = reinterpret_cast<T*>(lds) + wave * WAVE_ELEMS;
  T* vt_lds = k_lds + BC * KLD;

  const Unit wu = decode_unit<false>(p, blockIdx.x);
  const int64_t bh = wu.bh;
  const int64_t b = bh / p.H;
  const int64_t h = bh % p.H;
  const int64_t N = p.N;
  const T* __restrict__ Qh = reinterpret_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh;
  const T* __restrict__ Kh = reinterpret_cast<const T*>(p.k) + b * p.k_sb + h * p.k_sh;
  const T* __restrict__ Vh = reinterpret_cast<const T*>(p.v) + b * p.v_sb + h * p.v_sh;
  T* __restrict__ Oh = reinterpret_cast<T*>(p.o) + b * p.o_sb + h * p.o_sh;
  float* __restrict__ Lh = p.lse + bh * N;
  const int64_t qsn = p.q_sn, ksn = p.k_sn, vsn = p.v_sn, osn = p.o_sn;

  const int64_t q0 = (int64_t)wu.qt * 32;  // first query row of the block
  const int64_t qrow = q0 + r;             // this lane's query row

  int64_t kvl = N;
  if (p.kv_len) {
    const int64_t x = p.kv_len[b];
    kvl = x < 0 ? 0 : (x > N ? N : x);
  }
  int64_t nq = N;  // rows at or past nq are query padding: no key, O = 0, LSE = -inf
  if (p.q_len) {
    const int64_t x = p.q_len[b];
    nq = x < 0 ? 0 : (x > N ? N : x);
  }
  // Keys any row of the block may see; the block's key tiles, of which this wave takes every NW-th.
  int64_t kv_hi = kvl;
  if (p.causal) kv_hi = kv_hi < q0 + 32 ? kv_hi : q0 + 32;
  if (kv_hi > nq && p.causal) kv_hi = nq;
  if (q0 >= nq) kv_hi = 0;
  const int n_tiles = kv_hi > 0 ? (int)((kv_hi + BC - 1) / BC) : 0;

  // ---- the block's 32 Q rows, loaded with 16-byte row chunks (coalesced; a float32 fragment is
  // one element per lane, so loading fragments directly would touch 32 rows per instruction)
  // and read back from this wave's K staging region in the B-operand layout below.
  uint4 qreg[K_UNITS];
#pragma unroll
  for (int n = 0; n < K_UNITS; ++n) {
    const int cidx = lane + n * 64;
    const int64_t qr = q0 + cidx / CPR;
    qreg[n] = qr < nq ? *reinterpret_cast<const uint4*>(Qh + qr * qsn + (cidx % CPR) * CH) : uint4{0, 0, 0, 0};
  }
  frag qf[NQF];

  f32x16 oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) oacc[t] = f32x16{};
  float m2 = -INFINITY;  // running maximum of this wave's scaled base-2 logits, this lane's query
  float lsum = 0.f;      // this lane half's share of the wave's denominator
  const float c = p.scale_log2;
  const int krow_a = a_row_key<KPER>(r);

  // A tile's rows at or past kv_hi are loaded from row kv_hi - 1 (in bounds: a tile is loaded
  // only when the block has a key) and stored to LDS as zeros. The loads themselves take no
  // branch: a load under a per-row branch made the compiler wait for it inside the branch, one
  // memory round trip for every second row of the first tile.
  uint4 kreg[K_UNITS];
  uint4 vreg[V_UNITS][V_ROWS];
  auto load_tile = [&](int64_t j0) {
#pragma unroll
    for (int n = 0; n < K_UNITS; ++n) {
      const int cidx = lane + n * 64;
      const int row = cidx / CPR;
      const int col = (cidx % CPR) * CH;
      const int64_t key = j0 + row < kv_hi ? j0 + row : kv_hi - 1;
      kreg[n] = *reinterpret_cast<const uint4*>(Kh + key * ksn + col);
    }
#pragma unroll
    for (int n = 0; n < V_UNITS; ++n) {
      const int cidx = lane + n * 64;
      const int row0 = (cidx / CPR) * V_ROWS;
      const int col = (cidx % CPR) * CH;
#pragma unroll
      for (int e = 0; e < V_ROWS; ++e) {
        const int64_t key = j0 + row0 + e < kv_hi ? j0 + row0 + e : kv_hi - 1;
        vreg[n][e] = *reinterpret_cast<const uint4*>(Vh + key * vsn + col);
      }
    }
  };
  // Zero the words of a row at or past kv_hi (component selects: a select of the vector type
  // as a whole went through scratch memory).
  auto live4 = [](uint4 x, bool live) __attribute__((always_inline)) {
    return uint4{live ? x.x : 0u, live ? x.y : 0u, live ? x.z : 0u, live ? x.w : 0u};
  };
  auto store_tile = [&](int64_t j0) {
#pragma unroll
    for (int n = 0; n < K_UNITS; ++n) {
      const int cidx = lane + n * 64;
      *reinterpret_cast<uint4*>(&k_lds[(cidx / CPR) * KLD + (cidx % CPR) * CH]) = live4(kreg[n], j0 + cidx / CPR < kv_hi);
    }
#pragma unroll
    for (int n = 0; n < V_UNITS; ++n) {
      const int cidx = lane + n * 64;
      const int row0 = (cidx / CPR) * V_ROWS;
      const int col = (cidx % CPR) * CH;
#pragma unroll
      for (int e = 0; e < V_ROWS; ++e) vreg[n][e] = live4(vreg[n][e], j0 + row0 + e < kv_hi);
      if constexpr (sizeof(T) == 2) {
        // Two consecutive keys per 32-bit word of V^T.
        const uint32_t a[4] = {vreg[n][0].x, vreg[n][0].y, vreg[n][0].z, vreg[n][0].w};
        const uint32_t bb[4] = {vreg[n][1].x, vreg[n][1].y, vreg[n][1].z, vreg[n][1].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          *reinterpret_cast<uint32_t*>(&vt_lds[(col + 2 * w) * VLD + row0]) = (a[w] & 0xffffu) | (bb[w] << 16);
          *reinterpret_cast<uint32_t*>(&vt_lds[(col + 2 * w + 1) * VLD + row0]) = (a[w] >> 16) | (bb[w] & 0xffff0000u);
        }
      } else {
        // float32: V stays row-major (one 16-byte write per chunk, like K). A float32 A-operand
        // fragment of the P.V product is one element per lane, V[key][d] with d along the lanes,
        // which a row-major tile serves directly; a transposed copy took 32 single-word writes
        // per lane and tile, with bank conflicts, and its LDS traffic held up the other waves.
        *reinterpret_cast<uint4*>(&vt_lds[row0 * KLD + col]) = vreg[n][0];
      }
    }
  };

  int t = wave;
  if (t < n_tiles) load_tile((int64_t)t * BC);  // in flight with the Q rows, and while the fragments are read
#pragma unroll
  for (int n = 0; n < K_UNITS; ++n) {
    const int cidx = lane + n * 64;
    *reinterpret_cast<uint4*>(&k_lds[(cidx / CPR) * KLD + (cidx % CPR) * CH]) = qreg[n];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int s = 0; s < NQF; ++s)  // padding rows read zeros (their rows were not loaded)
    qf[s] = *reinterpret_cast<const frag*>(&k_lds[r * KLD + KSTEP * s + KPER * g]);
  for (; t < n_tiles; t += NW) {
    const int64_t j0 = (int64_t)t * BC;
    // Only this wave touches its LDS region, and the LDS serves one wave's accesses in order;
    // the fences keep the compiler from moving this tile's stores above the previous tile's
    // reads, or this tile's reads above its stores.
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    store_tile(j0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (t + NW < n_tiles) load_tile(j0 + (int64_t)NW * BC);

    // ---- S^T = K . Q^T for the tile's 32 keys
    f32x16 s = f32x16{};
    {
      // The K fragments are read PF steps ahead of their products, so an LDS read's latency
      // passes under earlier products instead of stalling the chain at every step.
      constexpr int PF = NQF < 8 ? NQF : 8;
      const T* arow = &k_lds[krow_a * KLD + KPER * g];
      frag kf[NQF];
#pragma unroll
      for (int st = 0; st < PF; ++st) kf[st] = *reinterpret_cast<const frag*>(arow + KSTEP * st);
#pragma unroll
      for (int st = 0; st < NQF; ++st) {
        if (st + PF < NQF) kf[st + PF] = *reinterpret_cast<const frag*>(arow + KSTEP * (st + PF));
        s = M::run(kf[st], qf[st], s);
      }
      // Pin that order (left alone, the scheduler moves each read back next to its product).
      // Two consecutive float fragments merge into one ds_read2_b32.
      constexpr int RD = KPER == 1 ? 2 : 1;  // fragments per LDS read instruction
      __builtin_amdgcn_sched_group_barrier(0x100, PF / RD, 0);
#pragma unroll
      for (int st = 0; st < NQF; st += RD) {
        __builtin_amdgcn_sched_group_barrier(0x008, RD, 0);
        if (st + PF < NQF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    // ---- masks (edge tiles; rows at or past N are never stored and need none)
    const bool need_mask = (j0 + BC > kvl) || (p.causal && j0 + BC - 1 > q0) || (nq < N && q0 + 32 > nq);
    auto dead = [&](int i) __attribute__((always_inline)) {
      const int64_t key = j0 + acc_key<KPER>(i, g);
      return key >= kvl || (p.causal && key > qrow) || qrow >= nq;
    };
    // ---- online softmax (base 2): running max of the scaled logits s*c
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, (need_mask && dead(i)) ? -INFINITY : s[i] * c);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m2, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m2 - m_use);
    m2 = m_new;
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -m_use));
      if (need_mask && dead(i)) pv = 0.f;
      s[i] = pv;
      lsum += pv;
    }
    // ---- O^T += V^T . P^T
#pragma unroll
    for (int kk = 0; kk < BC / KSTEP; ++kk) {
      frag pf;
      if constexpr (KPER == 1) {
        pf = s[kk];
      } else {
#pragma unroll
        for (int e = 0; e < KPER; ++e) pf[e] = (T)s[kk * KPER + e];
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const frag a = sizeof(T) == 4 ? *reinterpret_cast<const frag*>(&vt_lds[(KSTEP * kk + g) * KLD + 32 * dt + r])
                                      : *reinterpret_cast<const frag*>(&vt_lds[(32 * dt + r) * VLD + KSTEP * kk + KPER * g]);
        oacc[dt] = M::run(a, pf, oacc[dt]);
      }
    }
  }

  // ---- merge of the waves' partial states through LDS
  __syncthreads();  // every wave is done with its staging region
  float* mo = reinterpret_cast<float*>(lds);  // [NW][32][OLD] unnormalised O
  float* mm = mo + NW * 32 * OLD;             // [NW][32] reference maxima
  float* ml = mm + NW * 32;                   // [NW][32] denominators
  {
    const float ltot = lsum + __shfl_xor(lsum, 32);
    if (g == 0) {
      mm[wave * 32 + r] = m2;
      ml[wave * 32 + r] = ltot;
    }
    float* orow = mo + (wave * 32 + r) * OLD;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        float4 o4;
        o4.x = oacc[dt][4 * a4 + 0];
        o4.y = oacc[dt][4 * a4 + 1];
        o4.z = oacc[dt][4 * a4 + 2];
        o4.w = oacc[dt][4 * a4 + 3];
        *reinterpret_cast<float4*>(orow + 32 * dt + 8 * a4 + 4 * g) = o4;
      }
  }
  __syncthreads();
  constexpr int CHUNKS = 32 * D / 4;  // float4 chunks of the block's output
  for (int cidx = tid; cidx < CHUNKS; cidx += NW * 64) {
    const int row = cidx / (D / 4);
    const int col = (cidx % (D / 4)) * 4;
    const int64_t qr = q0 + row;
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = fmaxf(m, mm[w * 32 + row]);
    float l = 0.f;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    if (m != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = mm[w * 32 + row];
        const float aw = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - m);
        l += aw * ml[w * 32 + row];
        const float4 ow = *reinterpret_cast<const float4*>(mo + (w * 32 + row) * OLD + col);
        acc.x += aw * ow.x;
        acc.y += aw * ow.y;
        acc.z += aw * ow.z;
        acc.w += aw * ow.w;
      }
    }
    if (qr < N) {
      const float inv = (l == 0.f) ? 0.f : 1.f / l;
      if constexpr (sizeof(T) == 2) {
        T o4[4] = {(T)(acc.x * inv), (T)(acc.y * inv), (T)(acc.z * inv), (T)(acc.w * inv)};
        *reinterpret_cast<uint2*>(Oh + qr * osn + col) = *reinterpret_cast<const uint2*>(o4);
      } else {
        *reinterpret_cast<float4*>(Oh + qr * osn + col) = float4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
      }
      if (col == 0) Lh[qr] = (l == 0.f) ? -INFINITY : (m + log2f(l)) * kLn2;
    }
  }
}

}  // namespace fa
