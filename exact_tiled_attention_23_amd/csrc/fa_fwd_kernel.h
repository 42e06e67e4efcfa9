// Exact tiled attention forward with online softmax: the gfx950 kernel.
//
// One workgroup owns one (batch, head, query tile) ("vectorized-flash-attention-kernel",
// Core algorithm: for each batch, head and query block, loop over key/value blocks).
// NW waves of 64 lanes each own 32 consecutive query rows. Per key/value tile:
//
//   stage   K tile -> LDS row-major, V tile -> LDS transposed (V^T; row-major for float32),
//           from 16-byte coalesced global loads that were issued one tile ahead into registers;
//   S^T     = K . Q^T on 32x32 MFMA (fp32 accumulate). With this orientation the
//           accumulator layout puts one query per lane (lane % 32) and half of the
//           tile's keys in each 32-lane half, so row statistics stay in registers;
//   mask    causal (key > query) and padding (key >= kv_len) to -inf, only on tiles
//           that straddle the diagonal or the kv_len edge;
//   softmax running max m (base-2, scaled), alpha = 2^(m_old - m_new), p = 2^(s*c - m),
//           with c = scale*log2(e); a row whose max is still -inf subtracts 0 instead,
//           so no exp(-inf - -inf) ever happens ("js-flash-attention-tiled-online-
//           softmax-exactness", Root causes addressed 1 and 2);
//   O^T    = alpha*O^T + V^T . P^T on 32x32 MFMA, P taken straight from the S^T
//           accumulator registers (K rows are loaded in a permuted order so that the
//           accumulator layout is exactly the B-operand layout of this product).
//
// Tiles wholly above the causal diagonal or past kv_len are never loaded
// ("vectorized-flash-attention-kernel", Key design decision 3). The epilogue writes
// O = acc / l (exact zeros when l == 0) and LSE = m + ln l.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// A wave-uniform value moved into a vector register once. A VOP3 instruction that reads a
// scalar register (v_fma_f32 with the softmax scale, a kernel argument) issues about one cycle
// slower per SIMD than the same instruction on vector registers alone once two or more waves
// share the SIMD: measured on gfx950 with register-only loops, 3.56 against 2.56 cycles per
// v_fma_f32 at two waves per SIMD and 3.03 against 2.04 at three.
__device__ __forceinline__ float in_vgpr(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Per-element-type matrix-core step. KPER: reduction elements a lane holds per
// operand per instruction; one instruction reduces over KSTEP = 2*KPER elements
// (lanes 0-31 hold the first KPER, lanes 32-63 the next KPER).
template <typename T> struct Mma;

template <> struct Mma<__bf16> {
  static constexpr int KPER = 8;
  typedef __bf16 frag __attribute__((__vector_size__(8 * sizeof(__bf16))));
  static __device__ __forceinline__ f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<_Float16> {
  static constexpr int KPER = 8;
  typedef _Float16 frag __attribute__((__vector_size__(8 * sizeof(_Float16))));
  static __device__ __forceinline__ f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int KPER = 1;
  typedef float frag;
  static __device__ __forceinline__ f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;             // contiguous [B][H][N]
  const int32_t* kv_len;  // nullable: keys at or past kv_len[b] are padding
  const int32_t* q_len;   // nullable: query rows at or past q_len[b] are padding (O = 0, LSE = -inf)
  // Element strides of the batch, head and token dimensions (the head dimension D is
  // contiguous): tensor X element (b, h, n, d) lives at X + b*x_sb + h*x_sh + n*x_sn + d.
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t H;
  int64_t N;
  float scale_log2;       // scale * log2(e), any finite value
  int causal;
  int n_qtiles;           // ceil(N / BR)
  int64_t n_units;        // B * H * n_qtiles * n_splits (the grid size)
  int tm_group;           // heads per rank-by-rank group (unit_slot), >= 1
  // Key-axis split: with n_splits > 1 the work unit also names a split s. A query tile
  // with T visible key tiles gives split s the tiles [s*c, min(T, (s+1)*c)), c = ceil(T/S),
  // and the epilogue stores that split's normalised partial state (O_s in float32, LSE_s)
  // to part_o [S][B*H][N][D] and part_lse [S][B*H][N] instead of O and LSE.
  int n_splits;
  int64_t BH;
  float* part_o;
  float* part_lse;
};

// Work unit of workgroup `bid`. The dispatcher hands workgroups to the 8 XCDs in turn (bid mod
// 8), and each XCD has its own L2. Numbering each XCD's workgroups as one contiguous run of units
// keeps consecutive units (the query tiles of one head) on one XCD, so a head's K/V tiles come
// from HBM once. With n_units = 8q + r, XCD x takes units [xq + min(x, r), ... + q + (x < r)):
// a bijection of [0, n_units) for any unit count (only locality depends on the dispatch order).
__device__ __forceinline__ int xcd_unit(int bid, int64_t n_units) {
  const int q = (int)(n_units / 8), r = (int)(n_units % 8);
  const int x = bid % 8;
  return x * q + min(x, r) + bid / 8;
}

// (b, h) of head slot `slot` (slots are the consecutive runs of units that one head's tiles
// occupy). With per-batch padding (`mixed`) the work of a batch element varies, and slots in
// (b, h) order would give whole elements, and so unequal work, to single XCDs; the slots then
// run over the batch fastest, so the run of slots an XCD takes holds heads of every element.
// Without padding they keep the (b, h) order, which reads K and V from fewer memory regions.
__device__ __forceinline__ int head_of_slot(int slot, int B, int H, bool mixed) {
  return mixed ? (slot % B) * H + slot / B : slot;
}

// Work unit -> (bh, query tile, split); causal runs the longest query tiles first.
struct Unit {
  int bh, qt, split;
};
// SPLIT = false compiles the unsplit case (n_splits == 1) without the split arithmetic.
// Head slot and rank within the head (0 first) of workgroup `bid`, for `heads` heads of
// `per_head` units each. Each XCD takes a contiguous run of heads (xcd_unit). Within an XCD the
// units go head by head, or, with `tile_major` and whole heads on every XCD (heads % 8 == 0),
// rank by rank over groups of `group` of the XCD's heads. Under the causal mask a head's units
// shrink from the first rank to the last. Head by head, the next head's long units start behind
// the previous head's short ones, and with few units per head the XCD's last long unit ends
// late; rank by rank is the longest-first order. The group bounds how many heads' K/V the XCD
// reads at once: the host sizes it so that a group's K and V fit in the XCD's L2 (rank by rank
// over all of the XCD's heads would otherwise stream them from HBM when there are many heads).
// It is used only when every head has the same work (no per-batch padding, since with padding
// the ranks of different heads are not comparable) and heads are short (at most
// kTileMajorUnits units: with longer heads head by head is already balanced).
constexpr int kTileMajorUnits = 32;
__device__ __forceinline__ void unit_slot(int bid, int64_t n_units, int heads, int per_head, bool tile_major,
                                          int group, int* slot, int* rank) {
  if (tile_major && heads % 8 == 0 && per_head <= kTileMajorUnits) {
    const int hx = heads / 8, i = bid / 8;      // heads of this XCD, index of the unit in it
    const int G = min(hx, max(group, 1));
    const int gi = i / (G * per_head);          // group of the unit
    const int h0 = gi * G;                      // its first head
    const int gh = min(G, hx - h0);             // heads in the group (the last may hold fewer)
    const int w = i - gi * G * per_head;        // index within the group
    *slot = (bid % 8) * hx + h0 + w % gh;
    *rank = w / gh;
  } else {
    const int unit = xcd_unit(bid, n_units);
    *slot = unit / per_head;
    *rank = unit % per_head;
  }
}

template <bool SPLIT>
__device__ __forceinline__ Unit decode_unit(const FwdParams& p, int bid) {
  Unit u;
  const int ns = SPLIT ? p.n_splits : 1;
  const int per_head = p.n_qtiles * ns;
  int slot, rem;
  unit_slot(bid, p.n_units, (int)p.BH, per_head, p.causal && !p.kv_len && !p.q_len, p.tm_group, &slot, &rem);
  u.bh = slot;
  if (p.kv_len || p.q_len) u.bh = head_of_slot(slot, (int)p.BH / (int)p.H, (int)p.H, true);  // B*H < 2^31
  u.qt = rem / ns;
  u.split = rem % ns;
  if (p.causal) u.qt = p.n_qtiles - 1 - u.qt;
  return u;
}

// Longest-first order of the units of a key-padded problem (kv_len given, no q_len, no split,
// whole heads on every XCD and at most 64 of them: the host checks all of this and then launches
// the kernel instantiation that calls this). The work of a unit is its number of key tiles (or,
// for a dK/dV unit, of query tiles), which under key padding differs between batch elements, and
// each XCD runs its units in the order of decreasing work (ties in head-slot order), so that its
// longest units start first and the short ones fill the end. The host cannot sort the units
// (kv_len lives on the device), so every wave finds its workgroup's place in that order itself:
//  * The XCD holds head slots [x*hx, (x+1)*hx) (slots run over the batch fastest, as in
//    head_of_slot); lane s holds the kv_len of slot x*hx + s.
//  * at_least(t, kvl) gives the number of a head's units with at least t units of work, in closed
//    form (per_head at t = 0, non-increasing in t); a wave sum gives the XCD's count.
//  * A binary search over t finds the work ts of the i-th unit (the largest t whose count
//    exceeds i). The units of work exactly ts, taken head by head (a prefix sum over the lanes),
//    give the head and the unit's place among them; within a head the units of more work sit at
//    the high end of the unit index (more_work_last: query tiles under the causal mask) or at the
//    low end (key tiles of the dK/dV kernels), and the unit is counted from there.
// All of it is wave-uniform: every wave of the workgroup finds the same unit.
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}
template <class AtLeast>
__device__ __forceinline__ void longest_first(int bid, int heads, int H, int per_head, int max_work,
                                              const int32_t* kv_len, int n, bool more_work_last,
                                              AtLeast at_least, int* bh, int* unit) {
  const int B = heads / H, hx = heads / 8;
  const int x = bid % 8, i = bid / 8;
  const int lane = threadIdx.x & 63;
  int kv = -1;  // kv_len of this lane's head slot (lanes past hx hold none)
  if (lane < hx) {
    const int v = kv_len[(x * hx + lane) % B];
    kv = v < 0 ? 0 : (v > n ? n : v);
  }
  auto mine = [&](int t) { return kv < 0 ? 0 : at_least(t, kv); };
  int lo = 0, hi = max_work + 1;  // count(lo) > i >= count(hi) = 0
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (wave_sum(mine(mid)) > i) lo = mid;
    else hi = mid;
  }
  const int ts = lo;
  const int above = mine(ts + 1);
  const int j = i - wave_sum(above);  // place among the XCD's units of work exactly ts
  const int e = mine(ts) - above;     // this head's units of work exactly ts
  int pre = e;                        // inclusive prefix sum over the lanes
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(pre, d);
    if (lane >= d) pre += y;
  }
  const unsigned long long m = __ballot(pre > j);
  int sl = m ? (int)__builtin_ctzll(m) : hx - 1;
  sl = min(sl, hx - 1);
  const int jj = j - (__shfl(pre, sl) - __shfl(e, sl));
  const int above_s = __shfl(above, sl);
  int u = more_work_last ? per_head - 1 - above_s - jj : above_s + jj;
  u = max(0, min(u, per_head - 1));
  const int slot = x * hx + sl;
  // Wave-uniform values that came through lane moves: say so, so that the addresses formed from
  // them stay in scalar registers.
  *bh = __builtin_amdgcn_readfirstlane((slot % B) * H + slot / B);
  *unit = __builtin_amdgcn_readfirstlane(u);
}

// Forward units (query tiles of BR rows, key tiles of BC) in the longest-first order. A head whose
// kv_len exceeds (t-1)*BC has per_head - floor((t-1)*BC/BR) units with at least t key tiles under
// the causal mask (its query tiles from that index on), and all of them without it.
template <int BR, int BC>
__device__ __forceinline__ Unit decode_unit_lpt(const FwdParams& p, int bid) {
  const int per_head = p.n_qtiles;
  const bool causal = p.causal != 0;
  auto at_least = [&](int t, int kvl) {
    if (t <= 0) return per_head;
    if (kvl <= (t - 1) * BC) return 0;
    return causal ? max(0, per_head - ((t - 1) * BC) / BR) : per_head;
  };
  Unit u;
  longest_first(bid, (int)p.BH, (int)p.H, per_head, (int)((p.N + BC - 1) / BC), p.kv_len, (int)p.N, true,
                at_least, &u.bh, &u.qt);
  u.split = 0;
  return u;
}

// Key index (within a 32-key sub-tile) held by accumulator register i of lane half g.
// The 32x32 accumulator gives register i of half g the row 8*(i/4) + 4*g + i%4; the
// K rows are loaded permuted so that this row holds key KSTEP*(i/KPER) + KPER*g + i%KPER,
// which makes registers [KPER*h, KPER*h + KPER) of half g exactly the P^T operand
// (keys KSTEP*h + KPER*g + 0..KPER-1) of the h-th reduction step of P.V.
template <int KPER>
__device__ __forceinline__ int acc_key(int i, int g) {
  return (2 * KPER) * (i / KPER) + KPER * g + (i % KPER);
}

// The K row that A-operand row r must hold so that the accumulator row layout above holds.
template <int KPER>
__device__ __forceinline__ int a_row_key(int r) {
  return acc_key<KPER>(4 * (r / 8) + (r % 4), (r / 4) % 2);
}

template <typename T, int D, int BC, int NW>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(FwdParams p) {
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int KPER = M::KPER;
  constexpr int KSTEP = 2 * KPER;
  constexpr int NT = NW * 64;
  constexpr int BR = 32 * NW;
  constexpr int CH = 16 / (int)sizeof(T);        // elements per 16-byte chunk
  constexpr int CPR = D / CH;                    // chunks per row
  constexpr int KLD = D + CH;                    // K row stride in LDS (padded by 16 bytes)
  constexpr int VLD = BC + CH;                   // V^T row stride in LDS
  constexpr int NSUB = BC / 32;                  // 32-key sub-tiles per tile
  constexpr int NDT = D / 32;                    // 32-wide output column tiles
  constexpr int NQF = D / KSTEP;                 // Q fragments (reduction steps over D)
  constexpr int K_UNITS = BC * CPR / NT;         // 16-byte K chunks per thread per tile
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert((BC * CPR) % NT == 0, "K staging must divide evenly");

  __shared__ __attribute__((aligned(16))) T k_lds[BC * KLD];
  // V^T for 16-bit types; for float32, V row-major (stride KLD, like K): a float32 A-operand
  // fragment of the P.V product is one element per lane, V[key][d] with d along the lanes, which
  // a row-major tile serves directly, and 16-byte writes replace a transposed copy's
  // bank-conflicted single-word writes.
  constexpr int VELEMS = sizeof(T) == 4 && BC * KLD > D * VLD ? BC * KLD : D * VLD;
  __shared__ __attribute__((aligned(16))) T vt_lds[VELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;       // lane half
  const int r = lane & 31;       // query column of this lane / A-operand row

  const Unit wu = decode_unit<true>(p, blockIdx.x);
  const int64_t bh = wu.bh;
  const int qt = wu.qt;
  const int64_t b = bh / p.H;
  const int64_t h = bh % p.H;
  const int64_t N = p.N;

  const T* __restrict__ Qh = reinterpret_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh;
  const T* __restrict__ Kh = reinterpret_cast<const T*>(p.k) + b * p.k_sb + h * p.k_sh;
  const T* __restrict__ Vh = reinterpret_cast<const T*>(p.v) + b * p.v_sb + h * p.v_sh;
  T* __restrict__ Oh = reinterpret_cast<T*>(p.o) + b * p.o_sb + h * p.o_sh;
  float* __restrict__ Lh = p.lse + bh * N;
  const int64_t qsn = p.q_sn, ksn = p.k_sn, vsn = p.v_sn, osn = p.o_sn;

  const int64_t q0 = (int64_t)qt * BR;
  const int64_t qw = q0 + 32 * wave;       // first query row of this wave
  const int64_t qrow = qw + r;             // this lane's query row

  int64_t kvl = N;
  if (p.kv_len) {
    int64_t x = p.kv_len[b];
    kvl = x < 0 ? 0 : (x > N ? N : x);
  }
  int64_t nq = N;  // rows at or past nq are query padding: no key, O = 0, LSE = -inf
  if (p.q_len) {
    int64_t x = p.q_len[b];
    nq = x < 0 ? 0 : (x > N ? N : x);
  }
  // Keys any row of this tile may see, and keys any row of this wave may see.
  int64_t kv_hi = kvl;
  int64_t wave_hi = kvl;
  if (p.causal) {
    kv_hi = kv_hi < q0 + BR ? kv_hi : q0 + BR;
    wave_hi = wave_hi < qw + 32 ? wave_hi : qw + 32;
    kv_hi = kv_hi < nq ? kv_hi : nq;
    wave_hi = wave_hi < nq ? wave_hi : nq;
  }
  if (q0 >= nq) kv_hi = 0;
  if (qw >= nq) wave_hi = 0;
  // Key tiles [t_lo, t_hi) of this unit's split.
  const int all_tiles = kv_hi > 0 ? (int)((kv_hi + BC - 1) / BC) : 0;
  const int chunk = (all_tiles + p.n_splits - 1) / p.n_splits;
  const int t_lo = min(all_tiles, wu.split * chunk);
  const int t_hi = min(all_tiles, t_lo + chunk);

  // Q^T as the B operand of S^T = K . Q^T: lane holds Q[qrow][KSTEP*s + KPER*g + 0..KPER-1].
  frag qf[NQF];
#pragma unroll
  for (int s = 0; s < NQF; ++s) {
    if (qrow < nq) {  // padding rows are not read (they may hold anything)
      qf[s] = *reinterpret_cast<const frag*>(Qh + qrow * qsn + KSTEP * s + KPER * g);
    } else {
      qf[s] = frag{};
    }
  }

  f32x16 oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) oacc[t] = f32x16{};
  float m2 = -INFINITY;  // running max of scaled base-2 logits for this lane's query
  float lsum = 0.f;      // this lane half's share of the running denominator

  const float c = p.scale_log2;
  const int krow_a = a_row_key<KPER>(r);

  // ---- register staging of the next K/V tile
  uint4 kreg[K_UNITS];
  constexpr int V_UNITS = (sizeof(T) == 2) ? (BC / 2) * CPR / NT : BC * CPR / NT;
  constexpr int V_ROWS = (sizeof(T) == 2) ? 2 : 1;
  static_assert(((sizeof(T) == 2) ? (BC / 2) * CPR : BC * CPR) % NT == 0, "V staging must divide evenly");
  uint4 vreg[V_UNITS][V_ROWS];

  auto load_tile = [&](int64_t j0) {
#pragma unroll
    for (int n = 0; n < K_UNITS; ++n) {
      const int cidx = tid + n * NT;
      const int row = cidx / CPR;
      const int col = (cidx % CPR) * CH;
      const int64_t key = j0 + row;
      kreg[n] = key < kv_hi ? *reinterpret_cast<const uint4*>(Kh + key * ksn + col) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int n = 0; n < V_UNITS; ++n) {
      const int cidx = tid + n * NT;
      const int row0 = (cidx / CPR) * V_ROWS;
      const int col = (cidx % CPR) * CH;
#pragma unroll
      for (int e = 0; e < V_ROWS; ++e) {
        const int64_t key = j0 + row0 + e;
        vreg[n][e] = key < kv_hi ? *reinterpret_cast<const uint4*>(Vh + key * vsn + col) : uint4{0, 0, 0, 0};
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int n = 0; n < K_UNITS; ++n) {
      const int cidx = tid + n * NT;
      const int row = cidx / CPR;
      const int col = (cidx % CPR) * CH;
      *reinterpret_cast<uint4*>(&k_lds[row * KLD + col]) = kreg[n];
    }
#pragma unroll
    for (int n = 0; n < V_UNITS; ++n) {
      const int cidx = tid + n * NT;
      const int row0 = (cidx / CPR) * V_ROWS;
      const int col = (cidx % CPR) * CH;
      if constexpr (sizeof(T) == 2) {
        // Two consecutive keys per 32-bit word of V^T: word (d, row0/2) = V[row0][d] | V[row0+1][d] << 16.
        const uint32_t a[4] = {vreg[n][0].x, vreg[n][0].y, vreg[n][0].z, vreg[n][0].w};
        const uint32_t bb[4] = {vreg[n][1].x, vreg[n][1].y, vreg[n][1].z, vreg[n][1].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo = (a[w] & 0xffffu) | (bb[w] << 16);
          const uint32_t hi = (a[w] >> 16) | (bb[w] & 0xffff0000u);
          *reinterpret_cast<uint32_t*>(&vt_lds[(col + 2 * w) * VLD + row0]) = lo;
          *reinterpret_cast<uint32_t*>(&vt_lds[(col + 2 * w + 1) * VLD + row0]) = hi;
        }
      } else {
        *reinterpret_cast<uint4*>(&vt_lds[row0 * KLD + col]) = vreg[n][0];
      }
    }
  };

  if (t_lo < t_hi) load_tile((int64_t)t_lo * BC);

  for (int t = t_lo; t < t_hi; ++t) {
    const int64_t j0 = (int64_t)t * BC;
    __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();  // the tile is in LDS
    if (t + 1 < t_hi) load_tile(j0 + BC);

    if (j0 < wave_hi) {  // wave-uniform: some row of this wave sees a key of this tile
      // ---- S^T = K . Q^T
      f32x16 s[NSUB];
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        s[u] = f32x16{};
        const T* arow = &k_lds[(32 * u + krow_a) * KLD + KPER * g];
#pragma unroll
        for (int st = 0; st < NQF; ++st) {
          const frag a = *reinterpret_cast<const frag*>(arow + KSTEP * st);
          s[u] = M::run(a, qf[st], s[u]);
        }
      }

      // ---- masks: only where the tile crosses the kv_len edge or this wave's diagonal. A dead
      // key's scaled logit is -inf and its probability 0, for a scale of either sign (or zero).
      // (Rows at or past N are never stored: only rows of query padding below N need the mask.)
      const bool need_mask = (j0 + BC > kvl) || (p.causal && j0 + BC - 1 > qw) || (nq < N && qw + 32 > nq);
      auto dead = [&](int u, int i) __attribute__((always_inline)) {
        const int64_t key = j0 + 32 * u + acc_key<KPER>(i, g);
        return key >= kvl || (p.causal && key > qrow) || qrow >= nq;
      };

      // ---- online softmax (base 2): running max of the scaled logits s*c
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < NSUB; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = (need_mask && dead(u, i)) ? -INFINITY : s[u][i] * c;
          mx = fmaxf(mx, x);
        }
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
      for (int u = 0; u < NSUB; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u][i], c, -m_use));
          if (need_mask && dead(u, i)) pv = 0.f;
          s[u][i] = pv;
          lsum += pv;
        }

      // ---- O^T += V^T . P^T
#pragma unroll
      for (int kk = 0; kk < BC / KSTEP; ++kk) {
        constexpr int STEPS_PER_SUB = 32 / KSTEP;
        const int u = kk / STEPS_PER_SUB;
        const int h = kk % STEPS_PER_SUB;
        frag pf;
        if constexpr (KPER == 1) {
          pf = s[u][h];
        } else {
#pragma unroll
          for (int e = 0; e < KPER; ++e) pf[e] = (T)s[u][h * KPER + e];
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const frag a = sizeof(T) == 4 ? *reinterpret_cast<const frag*>(&vt_lds[(KSTEP * kk + g) * KLD + 32 * dt + r])
                                        : *reinterpret_cast<const frag*>(&vt_lds[(32 * dt + r) * VLD + KSTEP * kk + KPER * g]);
          oacc[dt] = M::run(a, pf, oacc[dt]);
        }
      }
    }
  }

  // ---- epilogue: O = acc / l (0 when l == 0), LSE = (m + log2 l) * ln 2
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (p.n_splits > 1) {
    if (qrow < N) {
      const float inv = (ltot == 0.f) ? 0.f : 1.f / ltot;
      const int64_t prow = ((int64_t)wu.split * p.BH + bh) * N + qrow;
      float* po = p.part_o + prow * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          float4 o4;
          o4.x = oacc[dt][4 * a4 + 0] * inv;
          o4.y = oacc[dt][4 * a4 + 1] * inv;
          o4.z = oacc[dt][4 * a4 + 2] * inv;
          o4.w = oacc[dt][4 * a4 + 3] * inv;
          *reinterpret_cast<float4*>(po + 32 * dt + 8 * a4 + 4 * g) = o4;
        }
      if (g == 0) p.part_lse[prow] = (ltot == 0.f) ? -INFINITY : (m2 + log2f(ltot)) * kLn2;
    }
    return;
  }
  if (qrow < N) {
    const float inv = (ltot == 0.f) ? 0.f : 1.f / ltot;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = 32 * dt + 8 * a4 + 4 * g;
        if constexpr (sizeof(T) == 2) {
          T o4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = (T)(oacc[dt][4 * a4 + e] * inv);
          *reinterpret_cast<uint2*>(Oh + qrow * osn + d) = *reinterpret_cast<const uint2*>(o4);
        } else {
          float4 o4;
          o4.x = oacc[dt][4 * a4 + 0] * inv;
          o4.y = oacc[dt][4 * a4 + 1] * inv;
          o4.z = oacc[dt][4 * a4 + 2] * inv;
          o4.w = oacc[dt][4 * a4 + 3] * inv;
          *reinterpret_cast<float4*>(Oh + qrow * osn + d) = o4;
        }
      }
    }
    if (g == 0) Lh[qrow] = (ltot == 0.f) ? -INFINITY : (m2 + log2f(ltot)) * kLn2;
  }
}

}  // namespace fa
