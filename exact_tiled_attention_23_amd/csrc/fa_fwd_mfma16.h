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
//    The exponent s*c - m is formed first and its row maximum over the whole key tile
//    taken afterwards (one decision per tile), so the usual case costs one FMA, half a
//    max and one exp2 per score.
//    The final O = acc / l is the same quotient whichever reference is used, so the
//    result is exact up to rounding ("Paper: FlashAttention", Objectives: the
//    online-softmax state is defined up to a common rescaling).
//  * A row whose reference is still -inf subtracts 0 instead, so exp(-inf - -inf)
//    never occurs ("js-flash-attention-tiled-online-softmax-exactness", Root causes
//    addressed 2); fully masked rows end with l = 0 and store O = 0, LSE = -inf.
//  * Padding keys (>= kv_len) in the edge tile: their V rows are zeroed in LDS after
//    the load so garbage past kv_len cannot reach O, and their scores are masked.
//  * Padding queries (>= q_len): their Q rows are not read and every score of theirs is
//    masked, so they end as fully masked rows; tiles and waves made only of padding rows
//    skip the key loop.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_kernel.h"

namespace fa {

// A compile-time integer passed as a value (selects an unrolled copy of a loop body).
template <int V> struct Int { static constexpr int value = V; };

// Reference maximum may lag the true row maximum by up to this much (base-2 units).
constexpr float kRescaleSlack = 8.0f;
constexpr float kSlackSum = 256.0f;      // 2^kRescaleSlack
// A tile whose reference was not tested first must keep every probability at most this large
// (through each lane's sum of them); beyond it the workgroup computes again with every tile tested.
// Below float16's largest finite value, so no probability that passes rounds to infinity when it
// is converted for the product with V.
constexpr float kUntestedSumBound = 32768.0f;
// Tiles at the start, and after each move of the reference, that test it first.
constexpr int kCalmTiles = 2;

typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef short s16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Maximum of x over the lane pair (i, i ^ 32). The two swapped values are plain lane moves of
// a maximum already formed in this kernel, so they need no canonicalisation: the final max is
// written as one instruction (fmaxf would first quiet each operand with a max of itself).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float m;
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
  return m;
}

// IEEE maximum of three values (NaN-propagating): one v_maximum3_f32.
__device__ __forceinline__ float fmax3_ieee(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One 16-byte-per-lane copy HBM -> LDS: lane i's 16 bytes at base + off land at LDS
// address lds_addr + 16*i. Issued as inline assembly so the compiler does not treat
// every later LDS read as a possible reader of this copy (it would otherwise wait for
// the copy's completion before the transpose reads); the kernel orders the copies
// itself with an explicit vmcnt wait and a workgroup barrier before any wave reads
// the destination. Vector-memory operations retire in order, so copies the compiler
// does not know about only make its own waits for earlier loads stricter.
// M0 is reserved to the compiler, which (re)loads it before each of its own uses; no
// compiler-generated instruction in this library reads M0, so writing it here is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(const void* base, unsigned off, unsigned lds_addr) {
  // The destination is wave-uniform; readfirstlane keeps it in a scalar register even where the
  // compiler has a copy of the value in a vector register (it may otherwise pick that one).
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"
               :: "v"(off), "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ unsigned lds_address(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// XOR swizzles of the 16-byte chunk index within a row (row j of the tile).
// K is read by 16 lanes on 16 different rows at one logical chunk; V (transpose reads)
// by 16 lanes on 4 consecutive rows x 4 consecutive chunks.
// Bank of chunk p of row j: (j * 2D + 16 p) / 4 mod 64, so rows of 64 B (D = 32) shift by
// 16 banks, rows of 128 B (D = 64) by 32, and rows of 256 B or more do not shift at all.
template <int D> __device__ __forceinline__ int swz_k(int j) {
  if constexpr (D >= 128) return j & 15;
  else if constexpr (D == 64) return (j >> 1) & 7;
  else return (j >> 2) & 3;
}
template <int D> __device__ __forceinline__ int swz_v(int j) {
  if constexpr (D >= 128) return 4 * (j & 3);
  else if constexpr (D == 64) return 4 * ((j >> 1) & 1);
  else return 0;  // D = 32: four consecutive rows already sit in four different bank quarters
}

// LDS row width, in elements, of a tile of head dimension D. Rows of D = 96 (192 bytes) do not
// tile the 1 KB copy blocks, so they take the 256-byte row of D = 128 and its swizzles; their
// last four 16-byte chunks are never copied nor read.
template <int D> constexpr int lds_cols() { return D == 96 ? 128 : D; }

// LPT: the key-padded launch, whose workgroups take their units longest first (decode_unit_lpt).
template <typename T, int D, int BC, int NW, int WPE, bool SPLIT, int KG = 1, bool LPT = false>
__global__ __launch_bounds__(NW * KG * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void fwd16_kernel(FwdParams p) {
  using M = Mma<T>;
  using frag = typename M::frag;
  static_assert(sizeof(T) == 2, "16-bit element types only");
  static_assert(D == 32 || D == 64 || D == 96 || D == 128 || D == 256, "head dimension");
  static_assert(BC % 32 == 0, "key tile");
  constexpr int BR = 32 * NW;
  constexpr int DL = lds_cols<D>();
  constexpr bool PADDED = DL != D;
  constexpr int ROWB = DL * 2;                  // bytes per K/V row in LDS
  constexpr int CPR = DL / 8;                   // 16-byte chunks per LDS row
  constexpr int VCH = D / 8;                    // chunks of a row that hold data
  constexpr int TILEB = BC * ROWB;              // bytes per K (or V) tile
  constexpr int BLOCKS = TILEB / 1024;          // 1 KB global_load_lds blocks per tile
  constexpr int LPW = BLOCKS / NW;              // blocks per wave per tile (each for K and V)
  constexpr int RPB = 1024 / ROWB;              // rows per block
  constexpr int NSUB = BC / 32;
  constexpr int NDT = D / 32;
  constexpr int NQF = D / 16;
  static_assert(BLOCKS % NW == 0, "tile must split evenly over waves");
  static_assert(KG >= 1 && KG <= 4, "key groups");
  constexpr int GROUPB = 2 * 2 * TILEB;          // LDS bytes of one key group's two buffers
  // Partial states of key groups 1..KG-1 for the merge: per wave, NDT*16 accumulators and the
  // reference and sum, element-major over the 64 lanes.
  constexpr int STATEF = NDT * 16 + 2;
  static_assert(KG == 1 || (KG - 1) * NW * 64 * STATEF * 4 <= KG * GROUPB, "merge area fits in LDS");

  __shared__ __attribute__((aligned(1024))) unsigned char lds[KG * GROUPB];  // [group][buf][K|V][tile]

  const int lane = threadIdx.x & 63;
  // Waves NW*k .. NW*k + NW-1 form key group k: group k takes the k-th of KG equal runs of
  // the unit's key tiles, each wave of it the same 32 query rows as wave w % NW of every group.
  const int kgrp = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6) / NW);   // wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6) % NW);   // wave-uniform
  const unsigned gbase = (unsigned)kgrp * GROUPB;  // this group's buffers
  const int g = lane >> 5;
  const int r = lane & 31;

  static_assert(!(LPT && SPLIT), "the longest-first order is for unsplit launches");
  Unit wu;
  if constexpr (LPT) wu = decode_unit_lpt<BR, BC>(p, blockIdx.x);
  else wu = decode_unit<SPLIT>(p, blockIdx.x);
  const int bh = wu.bh;
  const int qt = wu.qt;
  const int b = bh / (int)p.H;
  const int h = bh % (int)p.H;
  const int n = (int)p.N;

  const T* __restrict__ Qh = reinterpret_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh;
  const unsigned char* __restrict__ Kh =
      reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.k) + b * p.k_sb + h * p.k_sh);
  const unsigned char* __restrict__ Vh =
      reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.v) + b * p.v_sb + h * p.v_sh);
  T* __restrict__ Oh = reinterpret_cast<T*>(p.o) + b * p.o_sb + h * p.o_sh;
  float* __restrict__ Lh = p.lse + (int64_t)bh * n;
  // Token strides in bytes for K and V (per-lane copy offsets stay below 2^31: checked by
  // the host), in elements for Q and O.
  const unsigned ksnb = (unsigned)(p.k_sn * 2), vsnb = (unsigned)(p.v_sn * 2);
  const int64_t qsn = p.q_sn, osn = p.o_sn;

  const int q0 = qt * BR;
  const int qw = q0 + 32 * wave;
  const int qrow = qw + r;

  int kvl = n;
  if (p.kv_len) {
    const int x = p.kv_len[b];
    kvl = x < 0 ? 0 : (x > n ? n : x);
  }
  int nq = n;  // rows at or past nq are query padding: no key, O = 0, LSE = -inf
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
  // This wave holds rows before q_len and rows of query padding that are stored (O = 0).
  const bool qpad_wave = nq < n && qw + 32 > nq;
  // Both bounds are wave-uniform; saying so keeps the per-tile tests on them scalar branches
  // (the compiler otherwise forms the three-way minimum in a vector register).
  kv_hi = __builtin_amdgcn_readfirstlane(kv_hi);
  wave_hi = __builtin_amdgcn_readfirstlane(wave_hi);
  // Key tiles [t_lo, t_hi) of this unit's split (all of them without a split).
  const int all_tiles = kv_hi > 0 ? (kv_hi + BC - 1) / BC : 0;
  const int ns = SPLIT ? p.n_splits : 1;
  const int chunk = (all_tiles + ns - 1) / ns;
  const int u_lo = min(all_tiles, wu.split * chunk);
  const int u_hi = min(all_tiles, u_lo + chunk);
  // This key group's run [t_lo, t_hi) of them. Every group passes the barriers of `steps`
  // tiles (a group with a shorter run idles through its last ones).
  const int steps = (u_hi - u_lo + KG - 1) / KG;
  const int t_lo = min(u_hi, u_lo + kgrp * steps);
  const int t_hi = min(u_hi, t_lo + steps);

  // ---- per-lane constants of the global -> LDS copies: block blk = wave*LPW + i holds
  // rows blk*RPB .. +RPB-1; this lane fills the block's 16-byte slot `lane`, i.e. physical
  // chunk lane % CPR of row blk*RPB + lane / CPR, holding the logical chunk XOR swizzle.
  // With padded rows, a lane whose slot holds a padding chunk copies nothing (ld_kok/ld_vok).
  int ld_row[LPW];
  unsigned ld_kb[LPW], ld_vb[LPW];  // byte offsets within a tile
  bool ld_kok[LPW], ld_vok[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int j = (wave * LPW + i) * RPB + lane / CPR;
    const int pc = lane % CPR;
    const int ck = pc ^ swz_k<DL>(j), cv = pc ^ swz_v<DL>(j);
    ld_row[i] = j;
    ld_kb[i] = j * ksnb + ck * 16;
    ld_vb[i] = j * vsnb + cv * 16;
    ld_kok[i] = ck < VCH;
    ld_vok[i] = cv < VCH;
  }

  auto issue_tile = [&](int j0, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    const unsigned char* kt = Kh + (int64_t)j0 * ksnb;
    const unsigned char* vt = Vh + (int64_t)j0 * vsnb;
    unsigned char* kb = lds + gbase + buf * 2 * TILEB;
    unsigned char* vb = kb + TILEB;
    const unsigned kl = lds_address(kb), vl = lds_address(vb);
    if (j0 + BC <= n) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int blk = wave * LPW + i;
        if (!PADDED || ld_kok[i]) lds_copy16(kt, ld_kb[i], kl + blk * 1024);
        if (!PADDED || ld_vok[i]) lds_copy16(vt, ld_vb[i], vl + blk * 1024);
      }
    } else {
      // Rows past the tensor end read row n-1 instead (their scores are masked and their
      // V rows zeroed after the copy lands).
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int blk = wave * LPW + i;
        const int over = j0 + ld_row[i] - (n - 1);
        const unsigned rows_back = over > 0 ? (unsigned)over : 0u;
        if (!PADDED || ld_kok[i]) lds_copy16(kt, ld_kb[i] - rows_back * ksnb, kl + blk * 1024);
        if (!PADDED || ld_vok[i]) lds_copy16(vt, ld_vb[i] - rows_back * vsnb, vl + blk * 1024);
      }
    }
  };

  // ---- Q^T fragments (B operand of S^T = K . Q^T), straight from global memory.
  frag qf[NQF];
#pragma unroll
  for (int s = 0; s < NQF; ++s) {
    if (qrow < nq) qf[s] = *reinterpret_cast<const frag*>(Qh + qrow * qsn + 16 * s + 8 * g);
    else qf[s] = frag{};  // padding rows are not read (they may hold anything)
  }

  // ---- per-lane LDS read offsets
  const int kr = a_row_key<8>(r);                 // K row this lane feeds as A-operand row r
  int koff[NQF];
#pragma unroll
  for (int s = 0; s < NQF; ++s) koff[s] = gbase + kr * ROWB + ((2 * s + g) ^ swz_k<DL>(kr)) * 16;
  const int s16 = lane & 15, s4 = s16 >> 2, sm = s16 & 3, q2 = (lane >> 4) & 1;
  int voff[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int c = 4 * dt + 2 * q2 + (sm >> 1);
    voff[dt] = gbase + (8 * g + s4) * ROWB + ((c ^ swz_v<DL>(s4)) * 16) + (sm & 1) * 8;
  }

  f32x16 oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) oacc[t] = f32x16{};
  float mref = -INFINITY;  // reference maximum (scaled base-2 logits)
  float nmuse = 0.f;       // -mref, or 0 while mref is -inf (no valid key seen yet): the FMA addend
  float lsum = 0.f;        // this lane half's share of the denominator
  // At D <= 64, where the softmax's vector work sets the pace, the scaling FMAs read the scale
  // from a vector register (+1.5% at B4 H16 N2048 D64 causal); at D >= 96 that measured level to
  // 0.5% slower (two more registers), and the scale stays a scalar operand.
  const float c = D <= 64 ? in_vgpr(p.scale_log2) : p.scale_log2;

  // Testing the reference. Edge tiles, the first tiles of a unit and the tiles right after a
  // move of the reference take the row maximum of their exponents first (the decision below).
  // Elsewhere the reference rarely moves, and the tile skips the maximum: its probabilities are
  // formed against the current reference and each lane's sum of them is checked afterwards. A sum
  // above 2^slack only makes the next tile test again (the probabilities are exact for any
  // reference while nothing overflows); a sum above kUntestedSumBound (or infinite, or NaN) is an
  // overflow, and the whole workgroup then computes its unit again with every tile tested.
  // A wave whose reference moves a second time (a row's maximum rising past the slack after its
  // first valid key) tests every later tile of the unit: rows whose logits spread that widely
  // (queries of very different norms, say) would keep overflowing untested tiles.
  // The last key tile of the unit is always tested, so every wave has reported an overflow
  // (one LDS word, cleared before the first tile's barrier) before the barrier of that tile, and
  // after the loop every wave reads the same word without another barrier.
  int calm = 0;              // wave-uniform: tiles since the reference last moved
  bool test_all = false;     // wave-uniform: the second pass, or a reference that moved twice
  __shared__ int overflow_flag;
  if (threadIdx.x == 0) overflow_flag = 0;

  // Tile t lives in buffer (t - t_lo) & 1 and is copied one tile ahead. The loop below runs
  // two tiles per iteration, one per buffer, so the buffer is a compile-time constant in each
  // copy of the body and every LDS address is a per-lane register plus an immediate offset.

  auto tile_step = [&](const int t, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    const int j0 = t * BC;
    const unsigned char* kb = lds + buf * 2 * TILEB;
    const unsigned char* vb = kb + TILEB;
    wait_vmem();  // this wave's copies of tile t have landed
    if ((KG == 1 || t < t_hi) && j0 + BC > kvl) {
      // Padding rows (key >= kv_len) of V must not carry garbage into O: zero the slots
      // this lane filled itself.
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        if (j0 + ld_row[i] >= kvl) {
          const int blk = wave * LPW + i;
          *reinterpret_cast<uint4*>(lds + gbase + buf * 2 * TILEB + TILEB + blk * 1024 + lane * 16) = uint4{0, 0, 0, 0};
        }
      }
    }
    __syncthreads();  // tile t visible to all waves; all waves are done with tile t-1
    if (t + 1 < t_hi) issue_tile(j0 + BC, Int<buf ^ 1>{});

    if ((KG == 1 || t < t_hi) && j0 < wave_hi) {
      // ---- S^T = K . Q^T. The sub-tiles' products advance together, one reduction step
      // at a time, and the K fragments of step st+PD are read while step st's products run,
      // so each LDS read has about four products' time (~128 cycles) to land. The order is
      // pinned with scheduling-group barriers: left to itself the scheduler reuses one
      // fragment register and waits on every read.
      f32x16 s[NSUB];
      {
        constexpr int PD = NSUB >= 4 ? 1 : 2;
        frag ka[PD + 1][NSUB];
#pragma unroll
        for (int u = 0; u < NSUB; ++u) s[u] = f32x16{};
#pragma unroll
        for (int st = 0; st < PD; ++st)
#pragma unroll
          for (int u = 0; u < NSUB; ++u) ka[st][u] = *reinterpret_cast<const frag*>(kb + u * 32 * ROWB + koff[st]);
#pragma unroll
        for (int st = 0; st < NQF; ++st) {
          if (st + PD < NQF) {
#pragma unroll
            for (int u = 0; u < NSUB; ++u)
              ka[(st + PD) % (PD + 1)][u] = *reinterpret_cast<const frag*>(kb + u * 32 * ROWB + koff[st + PD]);
          }
#pragma unroll
          for (int u = 0; u < NSUB; ++u) s[u] = M::run(ka[st % (PD + 1)][u], qf[st], s[u]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, PD * NSUB, 0);  // DS reads of the first PD steps
#pragma unroll
        for (int st = 0; st < NQF; ++st) {
          if (st + PD < NQF) __builtin_amdgcn_sched_group_barrier(0x100, NSUB, 0);  // reads for st+PD
          __builtin_amdgcn_sched_group_barrier(0x008, NSUB, 0);                    // products of st
        }
      }

      // ---- V^T fragments (transpose reads). At D = 64..128 those of the whole tile are read
      // here, so their latency passes under the vector work below; at D = 32 (128-key tiles)
      // and D = 256 they would not fit in registers beside the rest, and each sub-tile reads
      // its own just before its products.
      constexpr bool kHoistV = D >= 64 && D <= 128;
      frag vall[kHoistV ? NSUB : 1][2][NDT];
      auto read_v = [&](int u, frag (&dst)[2][NDT]) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const unsigned char* vp = vb + (32 * u + 16 * h) * ROWB + voff[dt];
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 4 * ROWB));
            dst[h][dt] = __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
      };
      if constexpr (kHoistV) {
#pragma unroll
        for (int u = 0; u < NSUB; ++u) read_v(u, vall[u]);
      }

      // ---- online softmax: the exponents x = s*c - mref of the whole tile (s*c while mref is
      // -inf), and one decision per tile on moving the reference, from the row maximum over
      // all of the tile's keys.
      float x[NSUB][16];
#pragma unroll
      for (int u = 0; u < NSUB; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) x[u][i] = __builtin_fmaf(s[u][i], c, nmuse);

      // ---- masks (edge tiles, and every tile of the wave that holds the last query rows
      // before query padding): key j0 + 32u + acc_key(i, g) is dead when it is at or past
      // kv_len, or (causal) after this lane's query, or this lane's query is padding. The
      // exponent is set to -inf after the scaling, so the mask holds for a scale of either sign
      // (or zero) and whatever a padding key's score holds. Rows at or past N are never stored,
      // so the wave that holds the tensor's last rows needs no mask of its own.
      const bool edge = j0 + BC > kvl || (p.causal && j0 + BC - 1 > qw) || qpad_wave;
      if (edge) {
        int lim = qrow < nq ? kvl - j0 : 0;
        if (p.causal) lim = min(lim, qrow - j0 + 1);
        lim -= 8 * g;
#pragma unroll
        for (int u = 0; u < NSUB; ++u)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * u + 16 * (i / 8) + (i % 8) >= lim) x[u][i] = -INFINITY;
      }
      const bool tested = edge || calm < kCalmTiles || test_all || t + 1 == t_hi;
      if (tested) {
      float mx;
      {
        // 16*NSUB values in three-input maxima (each nested pair below becomes one
        // v_maximum3_f32). The IEEE maximum propagates NaN instead of quieting its operands, so
        // the masked exponents (a select) need no canonicalising max of their own.
        constexpr int NV = 16 * NSUB;
        float m[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) m[i] = x[i / 16][i % 16];
        int cnt = NV;
#pragma unroll
        for (int lvl = 0; lvl < 6; ++lvl) {
          if (cnt > 1) {
            int o = 0, i = 0;
#pragma unroll
            for (; i + 2 < cnt; i += 3) m[o++] = fmax3_ieee(m[i], m[i + 1], m[i + 2]);
            if (cnt - i == 2) m[o++] = __builtin_elementwise_maximum(m[i], m[i + 1]);
            else if (cnt - i == 1) m[o++] = m[i];
            cnt = o;
          }
        }
        mx = pair_max(m[0]);
      }
      // Move the reference when some row's maximum rose more than the slack above it, or when
      // a row sees its first valid key (its reference is still -inf).
      calm = calm + 1;
      if (__any((mx > kRescaleSlack) & (mref != -INFINITY))) test_all = true;
      if (__any((mx > kRescaleSlack) | ((mref == -INFINITY) & (mx != -INFINITY)))) {
        calm = 0;
        const float mnew = fmaxf(mref, mx - nmuse);
        if (mnew != mref) {
          const float alpha = __builtin_amdgcn_exp2f(mref - mnew);  // 0 when mref = -inf
          lsum *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
          const float delta = mnew + nmuse;
#pragma unroll
          for (int u = 0; u < NSUB; ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) x[u][i] -= delta;
          mref = mnew;
          nmuse = -mnew;
        }
      }
      }
      // ---- probabilities and O^T += V^T . P^T, one 32-key sub-tile at a time, so the
      // vector work on one sub-tile can run while the matrix core works on another.
      float tsum = 0.f;  // this lane's sum of the tile's probabilities
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        if constexpr (!kHoistV) read_v(u, vall[0]);
        frag (&va)[2][NDT] = vall[kHoistV ? u : 0];
        x[u][0] = __builtin_amdgcn_exp2f(x[u][0]);
        x[u][1] = __builtin_amdgcn_exp2f(x[u][1]);
        float a0 = x[u][0], a1 = x[u][1];
#pragma unroll
        for (int i = 2; i < 16; i += 2) {
          x[u][i] = __builtin_amdgcn_exp2f(x[u][i]);
          x[u][i + 1] = __builtin_amdgcn_exp2f(x[u][i + 1]);
          a0 += x[u][i];
          a1 += x[u][i + 1];
        }
        const float part = a0 + a1;
        lsum += part;
        tsum += part;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          frag pf;
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[e] = (T)x[u][8 * h + e];
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) oacc[dt] = M::run(va[h][dt], pf, oacc[dt]);
        }
        if constexpr (!kHoistV) {
          __builtin_amdgcn_sched_group_barrier(0x100, 4 * NDT, 0);  // the V^T transpose reads
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * NDT, 0);  // then this sub-tile's products
        }
      }
      if (!tested) {
        calm = __any(tsum > kSlackSum) ? 0 : calm + 1;
        if (__any(!(tsum <= kUntestedSumBound)) && lane == 0) overflow_flag = 1;
      }
    }
  };
  auto tile_loop = [&]() __attribute__((always_inline)) {
    if (t_lo < t_hi) issue_tile(t_lo * BC, Int<0>{});
    // Consume the Q fragments here: the compiler's wait for them is then placed before the loop
    // rather than re-issued (as a full vmcnt wait) in every iteration, and it comes after the
    // first tile's copies are issued, so the two loads' latencies overlap.
#pragma unroll
    for (int s = 0; s < NQF; ++s) asm volatile("" ::"v"(qf[s]));
    for (int i = 0; i < steps; i += 2) {
      tile_step(t_lo + i, Int<0>{});
      if (i + 1 >= steps) break;
      tile_step(t_lo + i + 1, Int<1>{});
    }
  };
  tile_loop();
  if (steps > 0 && *static_cast<volatile int*>(&overflow_flag)) {
    __syncthreads();  // every wave is done with the tiles, so the buffers can be refilled
    test_all = true;
    calm = 0;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
    mref = -INFINITY;
    nmuse = 0.f;
    lsum = 0.f;
    tile_loop();
  }

  // ---- merge of the key groups' partial states into group 0 (the monoid of (m, l, O) pairs:
  // the larger reference, and each state's sum and accumulators brought to it).
  if constexpr (KG > 1) {
    __syncthreads();  // every wave is done with the tiles; the merge area overlays them
    float* area = reinterpret_cast<float*>(lds);
    if (kgrp > 0) {
      float* st = area + ((kgrp - 1) * NW + wave) * (64 * STATEF);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) st[(dt * 16 + i) * 64 + lane] = oacc[dt][i];
      st[(NDT * 16) * 64 + lane] = mref;
      st[(NDT * 16 + 1) * 64 + lane] = lsum;
    }
    __syncthreads();
    if (kgrp > 0) return;
#pragma unroll
    for (int k = 1; k < KG; ++k) {
      const float* st = area + ((k - 1) * NW + wave) * (64 * STATEF);
      const float mk = st[(NDT * 16) * 64 + lane];
      const float lk = st[(NDT * 16 + 1) * 64 + lane];
      const float m = fmaxf(mref, mk);
      // A state that has seen no key (reference -inf, sum and accumulators 0) weighs nothing.
      const float a = mref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mref - m);
      const float bk = mk == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mk - m);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] = oacc[dt][i] * a + st[(dt * 16 + i) * 64 + lane] * bk;
      lsum = lsum * a + lk * bk;
      mref = m;
    }
  }

  // ---- epilogue
  const float ltot = pair_sum(lsum);
  if constexpr (SPLIT) {
    // Normalised partial state of this split, in float32, for the merge kernel.
    if (qrow < n) {
      const float inv = (ltot == 0.f) ? 0.f : 1.f / ltot;
      const int64_t prow = ((int64_t)wu.split * p.BH + bh) * n + qrow;
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
      if (g == 0) p.part_lse[prow] = (ltot == 0.f) ? -INFINITY : (mref + log2f(ltot)) * kLn2;
    }
    return;
  }
  if (qrow < n) {
    const float inv = (ltot == 0.f) ? 0.f : 1.f / ltot;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = 32 * dt + 8 * a4 + 4 * g;
        T o4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (T)(oacc[dt][4 * a4 + e] * inv);
        *reinterpret_cast<uint2*>(Oh + qrow * osn + d) = *reinterpret_cast<const uint2*>(o4);
      }
    if (g == 0) Lh[qrow] = (ltot == 0.f) ? -INFINITY : (mref + log2f(ltot)) * kLn2;
  }
}

}  // namespace fa
