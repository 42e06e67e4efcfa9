// C ABI of the attention forward, key-split forward, partial-state merge and backward
// (declared in include/fa.h): argument checks and kernel dispatch. Every check runs before
// any kernel launch; the library allocates nothing. Its only state is the per-device address
// of the static scratch array that fa_bwd_noalloc uses.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

#include "fa.h"
#include "fa_fwd_kernel.h"
#include "fa_fwd_mfma16.h"
#include "fa_fwd_wsplit.h"
#include "fa_merge.h"
#include "fa_bwd.h"

namespace {

constexpr int kAbiVersion = 7;
constexpr int kWaves = 4;      // waves per workgroup: 4 x 32 = 128 query rows per tile
constexpr int kBlockKV = 64;   // keys per K/V tile
// bf16/f16 kernel shape per head dimension: keys per K/V tile, waves per workgroup (32
// query rows each) and waves per SIMD. Eight waves share each K/V tile across 256 query
// rows at D = 128, halving the copies per flop. At D <= 64 (vector-bound) 4-wave workgroups
// run three waves per SIMD (three workgroups per CU) to hide the softmax's latencies: 128-key
// tiles fit in the registers of three waves at D = 32, 64-key tiles at D = 64 (measured
// +5-15% at D = 32 and +2-10% at D = 64 against two waves per SIMD with 128-key tiles, -1.5%
// on the padded, row-scaled f16 workload). D = 256 needs one wave per SIMD for its registers.
template <int D> struct Shape16;
template <> struct Shape16<32> { static constexpr int BC = 128, NW = 4, WPE = 3, KG = 1; };
template <> struct Shape16<64> { static constexpr int BC = 64, NW = 4, WPE = 3, KG = 1; };
template <> struct Shape16<96> { static constexpr int BC = 64, NW = 8, WPE = 2, KG = 1; };
template <> struct Shape16<128> { static constexpr int BC = 64, NW = 8, WPE = 2, KG = 1; };
template <> struct Shape16<256> { static constexpr int BC = 64, NW = 4, WPE = 1, KG = 1; };
constexpr int kMaxBC = 128;  // largest key tile: bounds the per-lane 32-bit copy offsets
// Narrower workgroups for small causal problems at D = 96 and 128: four waves (128 query rows)
// instead of eight. Causal query tiles differ in length, and smaller ones balance better over
// the CUs; measured +7-17% below 2048 tiles of 256 rows, -3% at 2048, and slower without the
// causal mask at every size tried.
struct Shape16Narrow { static constexpr int BC = 64, NW = 4, WPE = 2, KG = 1; };
constexpr int64_t kNarrowBelowUnits = 2048;
// Key groups at D = 64: three groups of four waves share each 128-row query tile, each group
// walking a third of its key tiles, and merge their partial states through LDS at the end. A
// 12-wave workgroup fills its CU, so tiles run about 7% slower than in three 4-wave workgroups,
// but the longest query tile finishes three times sooner. That pays only where the longest
// tile decides the run time: causal problems without padding (whose tiles' lengths the host
// knows) whose longest query tile has between kGroupsMinTiles and kGroupsMaxTiles key tiles and
// exceeds the average work per workgroup slot by kGroupsTailRatio. Measured: B1 H16 N8192
// causal +10..14%; B4 H16 N2048 causal -23% (tiles too short for the merge to pay); B1 H8
// N16384 causal -1% (the same tail ratio, but the longer tiles already balance).
struct Shape16Groups { static constexpr int BC = 64, NW = 4, WPE = 3, KG = 3; };
constexpr int64_t kGroupsMinTiles = 96;
constexpr int64_t kGroupsMaxTiles = 160;
constexpr double kGroupsTailRatio = 1.3;
struct ShapeF32 { static constexpr int BC = kBlockKV, NW = kWaves, KG = 1; };
template <typename T, int D> struct DefaultShape { using type = Shape16<D>; };
template <int D> struct DefaultShape<float, D> { using type = ShapeF32; };

template <typename T, int D, typename S, bool SPLIT, bool LPT = false> const void* fwd_kernel_ptr() {
  if constexpr (sizeof(T) == 2) {
    return reinterpret_cast<const void*>(&fa::fwd16_kernel<T, D, S::BC, S::NW, S::WPE, SPLIT, S::KG, LPT>);
  } else {
    return reinterpret_cast<const void*>(&fa::fwd_kernel<T, D, S::BC, S::NW>);  // decodes splits itself
  }
}

bool misaligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) != 0; }

struct Strides {
  int64_t q[3], k[3], v[3], o[3];  // (batch, head, token) in elements
};

// Key-axis split of the forward: n partial states written to part_o / part_lse.
struct Split {
  int n = 1;
  float* part_o = nullptr;
  float* part_lse = nullptr;
};

// Workgroups of kernel `fn` (launched with `threads` threads) that one XCD of the stream's GPU
// holds at once: its compute units (the GPU's, over 8 XCDs) times the kernel's occupancy. Both
// are queried once and kept.
constexpr int kXcds = 8;
constexpr int kMaxDevicesCached = 64;
int slots_per_xcd(hipStream_t stream, const void* fn, int threads) {
  static std::atomic<int> cus_of[kMaxDevicesCached];
  struct Occ { const void* fn; int threads, blocks; };
  static Occ occ[64];
  static int n_occ = 0;
  static std::mutex mu;
  int dev = 0;
  int cus = 256;
  if (hipStreamGetDevice(stream, &dev) == hipSuccess && dev >= 0 && dev < kMaxDevicesCached) {
    cus = cus_of[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
      cus_of[dev].store(cus, std::memory_order_relaxed);
    }
  }
  int blocks = 1;
  {
    std::lock_guard<std::mutex> lock(mu);
    int i = 0;
    while (i < n_occ && !(occ[i].fn == fn && occ[i].threads == threads)) ++i;
    if (i < n_occ) {
      blocks = occ[i].blocks;
    } else {
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, threads, 0) != hipSuccess || blocks <= 0) blocks = 1;
      if (n_occ < 64) occ[n_occ++] = Occ{fn, threads, blocks};
    }
  }
  return std::max(1, cus / kXcds) * blocks;
}

// Heads per rank-by-rank group of the causal work order (unit_slot). At least as many as keep
// two [N, D] operands per head (K and V for the forward and dQ kernels, Q and dO for the dK/dV
// kernel) within the 4 MB L2 of an XCD, and at least as many as give the last group of an XCD
// about twice its workgroup slots in units (a head's units average half its longest, so the
// last group's longest unit, which starts when that group does, still ends with the rest).
// The XCD's `hx` heads then go in groups of near-equal size, none below that.
constexpr int64_t kL2BytesPerXcd = 4 << 20;
int rank_group(int64_t heads, int64_t N, int64_t D, int64_t elt, int64_t per_head, int slots) {
  const int64_t hx = std::max<int64_t>(1, heads / kXcds);
  const int64_t head_bytes = 2 * N * D * elt;
  const int64_t g_l2 = head_bytes > 0 ? kL2BytesPerXcd / head_bytes : hx;
  const int64_t g_tail = (2 * (int64_t)slots + per_head - 1) / std::max<int64_t>(1, per_head);
  const int64_t g_min = std::max<int64_t>(1, std::max(g_l2, g_tail));
  const int64_t groups = std::max<int64_t>(1, hx / g_min);
  return (int)std::min<int64_t>(hx, (hx + groups - 1) / groups);
}

template <typename T, int D, typename S>
int launch_shape(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B, int64_t H, int64_t N,
                 const Strides& st, float scale, int causal, const int32_t* q_len, const int32_t* kv_len,
                 hipStream_t stream, const Split& sp) {
  constexpr int NW = S::NW;
  constexpr int BR = 32 * NW;
  constexpr int threads = 64 * NW * S::KG;
  fa::FwdParams p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = LSE;
  p.q_len = q_len;
  p.kv_len = kv_len;
  p.q_sb = st.q[0]; p.q_sh = st.q[1]; p.q_sn = st.q[2];
  p.k_sb = st.k[0]; p.k_sh = st.k[1]; p.k_sn = st.k[2];
  p.v_sb = st.v[0]; p.v_sh = st.v[1]; p.v_sn = st.v[2];
  p.o_sb = st.o[0]; p.o_sh = st.o[1]; p.o_sn = st.o[2];
  p.H = H;
  p.N = N;
  p.scale_log2 = scale * fa::kLog2e;
  p.causal = causal;
  const int64_t n_qtiles = (N + BR - 1) / BR;
  const int64_t units = B * H * n_qtiles * sp.n;
  if (n_qtiles > INT32_MAX || units > INT32_MAX) return FA_ERR_SHAPE;
  p.n_qtiles = (int)n_qtiles;
  p.n_units = units;
  p.n_splits = sp.n;
  p.BH = B * H;
  p.part_o = sp.part_o;
  p.part_lse = sp.part_lse;
  void* args[] = {&p};
  // Key padding: each XCD runs its units longest first (decode_unit_lpt) when it holds whole
  // heads, at most one per lane of a wave. Measured on B8 H8 N4096 D64 f16 causal with three
  // kv_len draws: +17% to +35% against the head-by-head order.
  const bool lpt = sizeof(T) == 2 && S::KG == 1 && kv_len && !q_len && sp.n == 1 && (B * H) % kXcds == 0 &&
                   B * H / kXcds <= 64;
  const void* fn = fwd_kernel_ptr<T, D, S, false>();
  if (sp.n > 1) {
    fn = fwd_kernel_ptr<T, D, S, true>();
  } else if constexpr (sizeof(T) == 2 && S::KG == 1) {
    if (lpt) fn = fwd_kernel_ptr<T, D, S, false, true>();
  }
  p.tm_group = causal ? rank_group(B * H, N, D, sizeof(T), n_qtiles * sp.n, slots_per_xcd(stream, fn, threads)) : 1;
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)units), dim3(threads), args, 0, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Problems of at most this many 128-row query tiles fill a small part of the GPU; the float32
// forward then runs 32-row query blocks whose key tiles are split over the waves of each
// workgroup (fwd_wsplit_kernel), which shortens the longest chain of key tiles a wave walks.
constexpr int64_t kWaveSplitMaxTiles = 64;
template <int D> struct WSplitWaves { static constexpr int NW = D <= 64 ? 8 : 4; };

template <typename T, int D>
int launch_wsplit(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B, int64_t H,
                  int64_t N, const Strides& st, float scale, int causal, const int32_t* q_len,
                  const int32_t* kv_len, hipStream_t stream) {
  constexpr int NW = WSplitWaves<D>::NW;
  fa::FwdParams p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = LSE;
  p.q_len = q_len;
  p.kv_len = kv_len;
  p.q_sb = st.q[0]; p.q_sh = st.q[1]; p.q_sn = st.q[2];
  p.k_sb = st.k[0]; p.k_sh = st.k[1]; p.k_sn = st.k[2];
  p.v_sb = st.v[0]; p.v_sh = st.v[1]; p.v_sn = st.v[2];
  p.o_sb = st.o[0]; p.o_sh = st.o[1]; p.o_sn = st.o[2];
  p.H = H;
  p.N = N;
  p.scale_log2 = scale * fa::kLog2e;
  p.causal = causal;
  const int64_t n_blocks = (N + 31) / 32;
  const int64_t units = B * H * n_blocks;
  if (units > INT32_MAX) return FA_ERR_SHAPE;
  p.n_qtiles = (int)n_blocks;
  p.n_units = units;
  p.tm_group = 1;  // (never more than 64 units here: one group whatever the order)
  p.n_splits = 1;
  p.BH = B * H;
  p.part_o = nullptr;
  p.part_lse = nullptr;
  void* args[] = {&p};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa::fwd_wsplit_kernel<T, D, NW>), dim3((unsigned)units),
                                 dim3(64 * NW), args, 0, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Whether the longest causal query tile (128 rows, 64-key tiles) outlasts the average work per
// workgroup slot enough for the key-group kernel (Shape16Groups) to win.
bool use_key_groups(int64_t B, int64_t H, int64_t N, hipStream_t stream) {
  const int64_t longest = (N + 63) / 64;
  if (longest < kGroupsMinTiles || longest > kGroupsMaxTiles) return false;
  const int64_t qtiles = (N + 127) / 128;
  int64_t tiles = 0;  // key tiles of one head's query tiles
  for (int64_t i = 0; i < qtiles; ++i) tiles += (std::min<int64_t>(N, 128 * (i + 1)) + 63) / 64;
  const void* fn = reinterpret_cast<const void*>(&fa::fwd16_kernel<__bf16, 64, 64, 4, 3, false, 1>);
  const double slots = (double)slots_per_xcd(stream, fn, 64 * 4) * kXcds;
  return (double)longest >= kGroupsTailRatio * (double)(B * H * tiles) / slots;
}

template <typename T, int D>
int launch(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B, int64_t H, int64_t N,
           const Strides& st, float scale, int causal, const int32_t* q_len, const int32_t* kv_len,
           hipStream_t stream, const Split& sp = Split()) {
  if constexpr (sizeof(T) == 4) {
    if (sp.n == 1 && B * H * ((N + 127) / 128) <= kWaveSplitMaxTiles)
      return launch_wsplit<T, D>(Q, K, V, O, LSE, B, H, N, st, scale, causal, q_len, kv_len, stream);
  }
  if constexpr (sizeof(T) == 2 && D == 64) {
    if (sp.n == 1 && causal && !kv_len && !q_len && use_key_groups(B, H, N, stream)) {
      return launch_shape<T, D, Shape16Groups>(Q, K, V, O, LSE, B, H, N, st, scale, causal, q_len, kv_len, stream,
                                                sp);
    }
  }
  if constexpr (sizeof(T) == 2 && (D == 96 || D == 128)) {
    static_assert(Shape16<D>::NW == 8, "the narrow shape halves an 8-wave workgroup");
    if (sp.n == 1 && causal && B * H * ((N + 255) / 256) < kNarrowBelowUnits)
      return launch_shape<T, D, Shape16Narrow>(Q, K, V, O, LSE, B, H, N, st, scale, causal, q_len, kv_len, stream,
                                                sp);
  }
  return launch_shape<T, D, typename DefaultShape<T, D>::type>(Q, K, V, O, LSE, B, H, N, st, scale, causal, q_len,
                                                               kv_len, stream, sp);
}

template <typename T>
int dispatch_d(int64_t D, const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B, int64_t H,
               int64_t N, const Strides& st, float scale, int causal, const int32_t* q_len, const int32_t* kv_len,
               hipStream_t stream, const Split& sp = Split()) {
  switch (D) {
    case 32: return launch<T, 32>(Q, K, V, O, LSE, B, H, N, st, scale, causal, q_len, kv_len, stream, sp);
    case 64: return launch<T, 64>(Q, K, V, O, LSE, B, H, N, st, scale, causal, q_len, kv_len, stream, sp);
    case 96: return launch<T, 96>(Q, K, V, O, LSE, B, H, N, st, scale, causal, q_len, kv_len, stream, sp);
    case 128: return launch<T, 128>(Q, K, V, O, LSE, B, H, N, st, scale, causal, q_len, kv_len, stream, sp);
    default:
      if constexpr (sizeof(T) == 2) return launch<T, 256>(Q, K, V, O, LSE, B, H, N, st, scale, causal, q_len, kv_len, stream, sp);
      return FA_ERR_UNSUPPORTED;
  }
}

template <typename T, int D>
int launch_merge(const float* part_o, const float* part_lse, int S, int64_t B, int64_t H, int64_t N, void* O,
                 const int64_t o_st[3], float* LSE, hipStream_t stream) {
  fa::MergeParams m;
  m.part_o = part_o;
  m.part_lse = part_lse;
  m.n_states = S;
  m.rows = B * H * N;
  m.H = H;
  m.N = N;
  m.o = O;
  m.o_sb = o_st[0];
  m.o_sh = o_st[1];
  m.o_sn = o_st[2];
  m.lse = LSE;
  constexpr int rows_per_block = 256 / (D / 4);
  const int64_t blocks = (m.rows + rows_per_block - 1) / rows_per_block;
  if (blocks > INT32_MAX) return FA_ERR_SHAPE;
  void* args[] = {&m};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa::merge_kernel<T, D>), dim3((unsigned)blocks),
                                 dim3(256), args, 0, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <typename T>
int dispatch_merge(int64_t D, const float* part_o, const float* part_lse, int S, int64_t B, int64_t H, int64_t N,
                   void* O, const int64_t o_st[3], float* LSE, hipStream_t stream) {
  switch (D) {
    case 32: return launch_merge<T, 32>(part_o, part_lse, S, B, H, N, O, o_st, LSE, stream);
    case 64: return launch_merge<T, 64>(part_o, part_lse, S, B, H, N, O, o_st, LSE, stream);
    case 96: return launch_merge<T, 96>(part_o, part_lse, S, B, H, N, O, o_st, LSE, stream);
    case 128: return launch_merge<T, 128>(part_o, part_lse, S, B, H, N, O, o_st, LSE, stream);
    default: return launch_merge<T, 256>(part_o, part_lse, S, B, H, N, O, o_st, LSE, stream);
  }
}

constexpr int kMaxSplits = 256;
constexpr int kAutoSplitCap = 16;     // suggested part counts stay at or below this
constexpr int kMinTilesPerPart = 4;   // and give every part at least this many key tiles

// Suggested part count: enough work units to fill every workgroup slot of the GPU once
// (twice for causal, whose query tiles differ in length), without parts shorter than
// kMinTilesPerPart key tiles.
template <typename T, int D>
int suggest_splits(int64_t B, int64_t H, int64_t N, int causal, int* n_splits) {
  using S = typename DefaultShape<T, D>::type;
  constexpr int NW = S::NW;
  constexpr int BR = 32 * NW;
  constexpr int BC = S::BC;
  const void* fn = fwd_kernel_ptr<T, D, S, true>();
  int dev = 0, n_cu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return FA_ERR_HIP;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64 * NW, 0) != hipSuccess) return FA_ERR_HIP;
  const int64_t units = B * H * ((N + BR - 1) / BR);
  const int64_t target = (int64_t)n_cu * (per_cu > 0 ? per_cu : 1) * (causal ? 2 : 1);
  int64_t s = (target + units - 1) / units;
  const int64_t key_tiles = (N + BC - 1) / BC;
  s = std::min<int64_t>(s, std::max<int64_t>(1, key_tiles / kMinTilesPerPart));
  s = std::max<int64_t>(1, std::min<int64_t>(s, kAutoSplitCap));
  *n_splits = (int)s;
  return FA_OK;
}

template <typename T>
int suggest_splits_d(int64_t D, int64_t B, int64_t H, int64_t N, int causal, int* n_splits) {
  switch (D) {
    case 32: return suggest_splits<T, 32>(B, H, N, causal, n_splits);
    case 64: return suggest_splits<T, 64>(B, H, N, causal, n_splits);
    case 96: return suggest_splits<T, 96>(B, H, N, causal, n_splits);
    case 128: return suggest_splits<T, 128>(B, H, N, causal, n_splits);
    default:
      if constexpr (sizeof(T) == 2) return suggest_splits<T, 256>(B, H, N, causal, n_splits);
      return FA_ERR_UNSUPPORTED;
  }
}

// Workspace of a split forward: S*B*H*N*D floats of partial O, then (256-byte aligned)
// S*B*H*N floats of partial LSE.
int64_t part_o_bytes(int64_t S, int64_t BHN, int64_t D) { return ((S * BHN * D * 4 + 255) / 256) * 256; }
int64_t split_workspace(int64_t S, int64_t BHN, int64_t D) { return part_o_bytes(S, BHN, D) + S * BHN * 4; }

bool supported(int dtype, int64_t D) {
  if (D == 32 || D == 64 || D == 96 || D == 128) return true;
  return D == 256 && dtype != FA_F32;
}

// Largest element offset (b, h, n, d) of a strided tensor, or -1 on overflow.
int64_t max_offset(int64_t B, int64_t H, int64_t N, int64_t D, const int64_t s[3]) {
  __int128 m = (__int128)(B - 1) * s[0] + (__int128)(H - 1) * s[1] + (__int128)(N - 1) * s[2] + (D - 1);
  return m > (__int128)(INT64_MAX / 16) ? -1 : (int64_t)m;
}

// True when no two (b, h, n, d) index the same element: sorted by stride, every dimension
// of extent > 1 must step past everything the finer dimensions span.
bool non_overlapping(int64_t B, int64_t H, int64_t N, int64_t D, const int64_t s[3]) {
  int64_t ext[3] = {B, H, N}, str[3] = {s[0], s[1], s[2]};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (str[j] < str[i]) {
        int64_t t = str[i]; str[i] = str[j]; str[j] = t;
        t = ext[i]; ext[i] = ext[j]; ext[j] = t;
      }
  __int128 span = D;
  for (int i = 0; i < 3; ++i) {
    if (ext[i] <= 1) continue;
    if ((__int128)str[i] < span) return false;
    span += (__int128)str[i] * (ext[i] - 1);
  }
  return true;
}

}  // namespace

extern "C" int fa_abi_version(void) { return kAbiVersion; }

extern "C" const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid sizes (negative, or too large for the kernel's indexing)";
    case FA_ERR_UNSUPPORTED: return "unsupported dtype or head dimension (forward: f32, bf16, f16 with D 32, 64, 96, 128, and 256 for bf16/f16; backward: bf16, f16 with D 32, 64, 96, 128)";
    case FA_ERR_ALIGN: return "misaligned pointer or stride (Q, K, V, O and their strides need 16 bytes; LSE, q_len and kv_len 4 bytes)";
    case FA_ERR_ARG: return "invalid argument (scale finite, causal 0 or 1, strides >= 0, outputs not aliasing inputs nor themselves, part count in range, workspace large enough)";
    case FA_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    case FA_ERR_TOO_LARGE: return "the problem needs more than the static scratch of fa_bwd_noalloc (FA_NOALLOC_SCRATCH_BYTES); call fa_bwd with a workspace";
    default: return "unknown error code";
  }
}

namespace {

// Checks shared by every forward entry point. Returns FA_OK and fills st, or an error;
// *empty is set when there is nothing to compute (then nothing else is inspected).
int validate_forward(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B, int64_t H,
                     int64_t N, int64_t D, const int64_t* strides, float scale, int causal, const int32_t* q_len,
                     const int32_t* kv_len, int dtype, Strides& st, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || N < 0 || D < 0) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16 && dtype != FA_F16) return FA_ERR_UNSUPPORTED;
  if (!supported(dtype, D)) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return FA_OK;
  }
  const int64_t lim = INT64_MAX / 16;
  if (B > lim / H || B * H > lim / N || B * H * N > lim / D) return FA_ERR_SHAPE;
  if (N > (int64_t(1) << 30)) return FA_ERR_SHAPE;  // row indices stay in 32 bits
  // The layout is checked before the pointers (it does not depend on them).
  if (strides) {
    for (int i = 0; i < 12; ++i)
      if (strides[i] < 0) return FA_ERR_ARG;
    for (int i = 0; i < 3; ++i) {
      st.q[i] = strides[i];
      st.k[i] = strides[3 + i];
      st.v[i] = strides[6 + i];
      st.o[i] = strides[9 + i];
    }
  } else {
    const int64_t c[3] = {H * N * D, N * D, D};
    for (int i = 0; i < 3; ++i) st.q[i] = st.k[i] = st.v[i] = st.o[i] = c[i];
  }
  const int64_t elt = dtype == FA_F32 ? 4 : 2;
  for (const int64_t* t : {st.q, st.k, st.v, st.o}) {
    for (int i = 0; i < 3; ++i)
      if ((t[i] * elt) % 16 != 0) return FA_ERR_ALIGN;
    if (max_offset(B, H, N, D, t) < 0) return FA_ERR_SHAPE;
  }
  if (!non_overlapping(B, H, N, D, st.o)) return FA_ERR_ARG;
  // Per-lane copy offsets within a key tile are 32-bit: kMaxBC rows of K or V.
  if (st.k[2] * elt > (int64_t(1) << 31) / kMaxBC || st.v[2] * elt > (int64_t(1) << 31) / kMaxBC) return FA_ERR_SHAPE;
  if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL;
  if (misaligned(Q, 16) || misaligned(K, 16) || misaligned(V, 16) || misaligned(O, 16)) return FA_ERR_ALIGN;
  if (misaligned(LSE, 4) || (kv_len && misaligned(kv_len, 4)) || (q_len && misaligned(q_len, 4))) return FA_ERR_ALIGN;
  if (O == Q || O == K || O == V) return FA_ERR_ARG;
  return FA_OK;
}

int run_forward(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B, int64_t H, int64_t N,
                int64_t D, const Strides& st, float scale, int causal, const int32_t* q_len, const int32_t* kv_len,
                int dtype, hipStream_t s, const Split& sp) {
  switch (dtype) {
    case FA_BF16: return dispatch_d<__bf16>(D, Q, K, V, O, LSE, B, H, N, st, scale, causal, q_len, kv_len, s, sp);
    case FA_F16: return dispatch_d<_Float16>(D, Q, K, V, O, LSE, B, H, N, st, scale, causal, q_len, kv_len, s, sp);
    default: return dispatch_d<float>(D, Q, K, V, O, LSE, B, H, N, st, scale, causal, q_len, kv_len, s, sp);
  }
}

int run_merge(const float* part_o, const float* part_lse, int S, int64_t B, int64_t H, int64_t N, int64_t D,
              void* O, const int64_t o_st[3], float* LSE, int dtype, hipStream_t s) {
  switch (dtype) {
    case FA_BF16: return dispatch_merge<__bf16>(D, part_o, part_lse, S, B, H, N, O, o_st, LSE, s);
    case FA_F16: return dispatch_merge<_Float16>(D, part_o, part_lse, S, B, H, N, O, o_st, LSE, s);
    default: return dispatch_merge<float>(D, part_o, part_lse, S, B, H, N, O, o_st, LSE, s);
  }
}

// ---- backward
constexpr int kBwdWaves = 4;   // 128 query rows (dQ kernel) or 128 keys (dK/dV kernel) per workgroup
constexpr int kBwdKeyTile = 64;

bool bwd_supported(int dtype, int64_t D) {
  return (dtype == FA_BF16 || dtype == FA_F16) && (D == 32 || D == 64 || D == 96 || D == 128);
}

int64_t bwd_stats_bytes(int64_t BH, int64_t N) {
  return BH * ((N + fa::kStatRows - 1) / fa::kStatRows) * (2 * fa::kStatRows) * 4;
}

bool ranges_overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

template <typename T, int D>
int launch_bwd(const fa::BwdParams& base, int64_t B, int64_t H, int64_t N, hipStream_t stream) {
  constexpr int R = 32 * kBwdWaves;
  const int64_t tiles = (N + R - 1) / R;
  const int64_t units = B * H * tiles;
  if (tiles > INT32_MAX || units > INT32_MAX) return FA_ERR_SHAPE;
  fa::BwdParams p = base;
  p.n_tiles = (int)tiles;
  p.n_units = units;
  void* args[] = {&p};
  // Key padding: both kernels take their units longest first (as the forward does).
  const bool lpt = p.kv_len && !p.q_len && (B * H) % kXcds == 0 && B * H / kXcds <= 64;
  const void* dq_fn = lpt ? reinterpret_cast<const void*>(&fa::bwd_dq_kernel<T, D, kBwdKeyTile, kBwdWaves, true>)
                          : reinterpret_cast<const void*>(&fa::bwd_dq_kernel<T, D, kBwdKeyTile, kBwdWaves>);
  p.tm_group = p.causal ? rank_group(B * H, N, D, sizeof(T), tiles, slots_per_xcd(stream, dq_fn, 64 * kBwdWaves)) : 1;
  hipError_t e = hipLaunchKernel(dq_fn, dim3((unsigned)units), dim3(64 * kBwdWaves), args, 0, stream);
  if (e != hipSuccess) return FA_ERR_HIP;
  // K/V in LDS, eight waves (two per key group) at D >= 96: two waves per SIMD there.
  constexpr int kv_threads = D >= 96 ? 64 * 8 : 64 * kBwdWaves;
  const void* kv_fn;
  if constexpr (D >= 96) {
    kv_fn = lpt ? reinterpret_cast<const void*>(&fa::bwd_dkdv_lds_kernel<T, D, fa::kStatRows, 8, true>)
                : reinterpret_cast<const void*>(&fa::bwd_dkdv_lds_kernel<T, D, fa::kStatRows, 8>);
  } else {
    kv_fn = lpt ? reinterpret_cast<const void*>(&fa::bwd_dkdv_kernel<T, D, fa::kStatRows, kBwdWaves, true>)
                : reinterpret_cast<const void*>(&fa::bwd_dkdv_kernel<T, D, fa::kStatRows, kBwdWaves>);
  }
  p.tm_group = p.causal ? rank_group(B * H, N, D, sizeof(T), tiles, slots_per_xcd(stream, kv_fn, kv_threads)) : 1;
  e = hipLaunchKernel(kv_fn, dim3((unsigned)units), dim3(kv_threads), args, 0, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

template <typename T>
int dispatch_bwd(int64_t D, const fa::BwdParams& p, int64_t B, int64_t H, int64_t N, hipStream_t s) {
  switch (D) {
    case 32: return launch_bwd<T, 32>(p, B, H, N, s);
    case 64: return launch_bwd<T, 64>(p, B, H, N, s);
    case 96: return launch_bwd<T, 96>(p, B, H, N, s);
    default: return launch_bwd<T, 128>(p, B, H, N, s);
  }
}

}  // namespace

extern "C" int64_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D) {
  if (B < 0 || H < 0 || N < 0 || D < 0) return -1;
  if (B == 0 || H == 0 || N == 0) return 0;
  const int64_t lim = INT64_MAX / 1024;
  if (B > lim / H || B * H > lim / (N + fa::kStatRows)) return -1;
  return bwd_stats_bytes(B * H, N);
}

namespace {

// Checks and launch shared by fa_bwd and fa_bwd_strided. `st` holds the 8 tensors' strides in
// the order Q, K, V, O, dO, dQ, dK, dV.
int bwd_common(const void* Q, const void* K, const void* V, const void* O, const float* LSE, const void* dO,
               void* dQ, void* dK, void* dV, int64_t B, int64_t H, int64_t N, int64_t D, const int64_t st[8][3],
               float scale, int causal, const int32_t* q_len, const int32_t* kv_len, int dtype, void* workspace,
               int64_t workspace_bytes, void* stream, bool contiguous) {
  const int64_t need = fa_bwd_workspace_bytes(B, H, N, D);
  if (need < 0) return FA_ERR_SHAPE;
  // The layout is checked before the pointers (it does not depend on them).
  for (int t = 0; t < 8; ++t) {
    for (int i = 0; i < 3; ++i) {
      if (st[t][i] < 0) return FA_ERR_ARG;
      if ((st[t][i] * 2) % 16 != 0) return FA_ERR_ALIGN;
    }
    if (max_offset(B, H, N, D, st[t]) < 0) return FA_ERR_SHAPE;
  }
  for (int t = 5; t < 8; ++t)
    if (!non_overlapping(B, H, N, D, st[t])) return FA_ERR_ARG;
  // Tiles of Q, dO, K and V are copied with 32-bit per-lane offsets over up to 128 rows.
  for (int t : {0, 1, 2, 4})
    if (st[t][2] * 2 > (int64_t(1) << 31) / 128) return FA_ERR_SHAPE;
  if (!Q || !K || !V || !O || !LSE || !dO || !dQ || !dK || !dV || !workspace) return FA_ERR_NULL;
  for (const void* ptr : {Q, K, V, O, dO, (const void*)dQ, (const void*)dK, (const void*)dV})
    if (misaligned(ptr, 16)) return FA_ERR_ALIGN;
  if (misaligned(LSE, 4) || (kv_len && misaligned(kv_len, 4)) || (q_len && misaligned(q_len, 4)) ||
      misaligned(workspace, 256))
    return FA_ERR_ALIGN;
  if (workspace_bytes < need) return FA_ERR_ARG;
  const int64_t tb = B * H * N * D * 2;
  if (contiguous) {
    // Outputs (and the workspace, which is written) must not overlap each other or any input.
    const void* outs[4] = {dQ, dK, dV, workspace};
    const int64_t out_b[4] = {tb, tb, tb, need};
    const void* ins[6] = {Q, K, V, O, dO, LSE};
    const int64_t in_b[6] = {tb, tb, tb, tb, tb, B * H * N * 4};
    for (int i = 0; i < 4; ++i) {
      for (int j = 0; j < 6; ++j)
        if (ranges_overlap(outs[i], out_b[i], ins[j], in_b[j])) return FA_ERR_ARG;
      for (int j = i + 1; j < 4; ++j)
        if (ranges_overlap(outs[i], out_b[i], outs[j], out_b[j])) return FA_ERR_ARG;
    }
  } else {
    // Strided views may interleave (e.g. dQ, dK, dV as slices of one packed tensor), so only
    // an output that starts at an input, another output or the workspace is rejected here.
    const void* outs[3] = {dQ, dK, dV};
    for (int i = 0; i < 3; ++i) {
      for (const void* in : {Q, K, V, O, dO, (const void*)LSE, (const void*)workspace})
        if (outs[i] == in) return FA_ERR_ARG;
      for (int j = i + 1; j < 3; ++j)
        if (outs[i] == outs[j]) return FA_ERR_ARG;
    }
  }
  fa::BwdParams p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.dout = dO;
  p.lse = LSE;
  p.dq = dQ;
  p.dk = dK;
  p.dv = dV;
  fa::Strides3* ps[8] = {&p.st_q, &p.st_k, &p.st_v, &p.st_o, &p.st_do, &p.st_dq, &p.st_dk, &p.st_dv};
  for (int t = 0; t < 8; ++t) *ps[t] = fa::Strides3{st[t][0], st[t][1], st[t][2]};
  p.stats = static_cast<float*>(workspace);
  p.q_len = q_len;
  p.kv_len = kv_len;
  p.H = H;
  p.N = N;
  p.scale = scale;
  p.scale_log2 = scale * fa::kLog2e;
  p.causal = causal;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return dtype == FA_BF16 ? dispatch_bwd<__bf16>(D, p, B, H, N, s) : dispatch_bwd<_Float16>(D, p, B, H, N, s);
}

int bwd_precheck(int64_t B, int64_t H, int64_t N, int64_t D, float scale, int causal, int dtype, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || N < 0 || D < 0) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16 && dtype != FA_F16) return FA_ERR_UNSUPPORTED;
  if (!bwd_supported(dtype, D)) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return FA_OK;
  }
  const int64_t lim = INT64_MAX / 16;
  if (B > lim / H || B * H > lim / N || B * H * N > lim / D) return FA_ERR_SHAPE;
  if (N > (int64_t(1) << 30)) return FA_ERR_SHAPE;
  return FA_OK;
}

}  // namespace

extern "C" int fa_bwd_strided(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                              const void* dO, void* dQ, void* dK, void* dV, int64_t B, int64_t H, int64_t N,
                              int64_t D, const int64_t* strides, float scale, int causal, const int32_t* q_len,
                              const int32_t* kv_len, int dtype, void* workspace, int64_t workspace_bytes,
                              void* stream) {
  bool empty;
  const int rc = bwd_precheck(B, H, N, D, scale, causal, dtype, &empty);
  if (rc != FA_OK || empty) return rc;
  int64_t st[8][3];
  for (int t = 0; t < 8; ++t) {
    for (int i = 0; i < 3; ++i) {
      const int64_t contiguous_stride[3] = {H * N * D, N * D, D};
      st[t][i] = strides ? strides[3 * t + i] : contiguous_stride[i];
    }
  }
  return bwd_common(Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, N, D, st, scale, causal, q_len, kv_len, dtype, workspace,
                    workspace_bytes, stream, strides == nullptr);
}

extern "C" int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const float* LSE, const void* dO,
                      void* dQ, void* dK, void* dV, int64_t B, int64_t H, int64_t N, int64_t D, float scale,
                      int causal, const int32_t* kv_len, int dtype, void* workspace, int64_t workspace_bytes,
                      void* stream) {
  return fa_bwd_strided(Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, N, D, nullptr, scale, causal, nullptr, kv_len, dtype,
                        workspace, workspace_bytes, stream);
}

// ---- fa_bwd_noalloc: fa_bwd with its workspace in a file-scope device array, for callers that
// cannot allocate. In host code `scratch` names a host-side stand-in, never the device memory:
// host code uses only the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mutex;
void* scratch_address[kMaxScratchDevices];  // device address of `scratch` per device, once looked up

// The device address of `scratch` on the device of `stream` (the current device for the null
// stream), looked up once per device with that device current.
int scratch_on(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_HIP;
  int dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_address[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return FA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return FA_ERR_HIP;
    if (e != hipSuccess || !p) return FA_ERR_HIP;
    scratch_address[dev] = p;
  }
  *out = scratch_address[dev];
  return FA_OK;
}

}  // namespace

extern "C" int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                              const void* dO, void* dQ, void* dK, void* dV, int64_t B, int64_t H, int64_t N,
                              int64_t D, float scale, int causal, const int32_t* kv_len, int dtype, void* stream) {
  bool empty;
  int rc = bwd_precheck(B, H, N, D, scale, causal, dtype, &empty);
  if (rc != FA_OK || empty) return rc;
  const int64_t need = fa_bwd_workspace_bytes(B, H, N, D);
  if (need < 0) return FA_ERR_SHAPE;
  if (need > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_TOO_LARGE;
  // The caller's pointers are checked before the first HIP call; fa_bwd checks everything again.
  if (!Q || !K || !V || !O || !LSE || !dO || !dQ || !dK || !dV) return FA_ERR_NULL;
  for (const void* ptr : {Q, K, V, O, dO, (const void*)dQ, (const void*)dK, (const void*)dV})
    if (misaligned(ptr, 16)) return FA_ERR_ALIGN;
  if (misaligned(LSE, 4) || (kv_len && misaligned(kv_len, 4))) return FA_ERR_ALIGN;
  void* ws = nullptr;
  rc = scratch_on(reinterpret_cast<hipStream_t>(stream), &ws);
  if (rc != FA_OK) return rc;
  return fa_bwd(Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, N, D, scale, causal, kv_len, dtype, ws,
                FA_NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" int fa_fwd_strided(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B,
                              int64_t H, int64_t N, int64_t D, const int64_t* strides, float scale, int causal,
                              const int32_t* q_len, const int32_t* kv_len, int dtype, void* stream) {
  Strides st;
  bool empty;
  const int rc =
      validate_forward(Q, K, V, O, LSE, B, H, N, D, strides, scale, causal, q_len, kv_len, dtype, st, &empty);
  if (rc != FA_OK || empty) return rc;
  return run_forward(Q, K, V, O, LSE, B, H, N, D, st, scale, causal, q_len, kv_len, dtype,
                     reinterpret_cast<hipStream_t>(stream), Split());
}

extern "C" int64_t fa_fwd_split_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int n_splits) {
  if (B < 0 || H < 0 || N < 0 || D < 0 || n_splits < 1 || n_splits > kMaxSplits) return -1;
  if (n_splits == 1) return 0;
  const int64_t lim = INT64_MAX / 1024;
  if ((H && B > lim / H) || (N && B * H > lim / N) || (D && B * H * N > lim / D / kMaxSplits)) return -1;
  return split_workspace(n_splits, B * H * N, D);
}

extern "C" int fa_fwd_split(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B,
                            int64_t H, int64_t N, int64_t D, const int64_t* strides, float scale, int causal,
                            const int32_t* q_len, const int32_t* kv_len, int dtype, int n_splits, void* workspace,
                            int64_t workspace_bytes, void* stream) {
  if (n_splits < 1 || n_splits > kMaxSplits) return FA_ERR_ARG;
  Strides st;
  bool empty;
  int rc = validate_forward(Q, K, V, O, LSE, B, H, N, D, strides, scale, causal, q_len, kv_len, dtype, st, &empty);
  if (rc != FA_OK || empty) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (n_splits == 1)
    return run_forward(Q, K, V, O, LSE, B, H, N, D, st, scale, causal, q_len, kv_len, dtype, s, Split());
  const int64_t need = fa_fwd_split_workspace_bytes(B, H, N, D, n_splits);
  if (need < 0) return FA_ERR_SHAPE;
  if (!workspace) return FA_ERR_NULL;
  if (misaligned(workspace, 256)) return FA_ERR_ALIGN;
  if (workspace_bytes < need) return FA_ERR_ARG;
  Split sp;
  sp.n = n_splits;
  sp.part_o = static_cast<float*>(workspace);
  sp.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + part_o_bytes(n_splits, B * H * N, D));
  rc = run_forward(Q, K, V, O, LSE, B, H, N, D, st, scale, causal, q_len, kv_len, dtype, s, sp);
  if (rc != FA_OK) return rc;
  return run_merge(sp.part_o, sp.part_lse, n_splits, B, H, N, D, O, st.o, LSE, dtype, s);
}

extern "C" int fa_fwd_split_count(int64_t B, int64_t H, int64_t N, int64_t D, int causal, int dtype,
                                  int* n_splits) {
  if (B < 0 || H < 0 || N < 0 || D < 0) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16 && dtype != FA_F16) return FA_ERR_UNSUPPORTED;
  if (!supported(dtype, D)) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (!n_splits) return FA_ERR_NULL;
  if (B == 0 || H == 0 || N == 0) {
    *n_splits = 1;
    return FA_OK;
  }
  const int64_t lim = INT64_MAX / 16;
  if (B > lim / H || B * H > lim / N || N > (int64_t(1) << 30)) return FA_ERR_SHAPE;
  switch (dtype) {
    case FA_BF16: return suggest_splits_d<__bf16>(D, B, H, N, causal, n_splits);
    case FA_F16: return suggest_splits_d<_Float16>(D, B, H, N, causal, n_splits);
    default: return suggest_splits_d<float>(D, B, H, N, causal, n_splits);
  }
}

extern "C" int fa_merge_states(const float* part_o, const float* part_lse, int n_states, int64_t B, int64_t H,
                               int64_t N, int64_t D, void* O, const int64_t* o_strides, float* LSE, int dtype,
                               void* stream) {
  if (B < 0 || H < 0 || N < 0 || D < 0) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16 && dtype != FA_F16) return FA_ERR_UNSUPPORTED;
  if (D != 32 && D != 64 && D != 96 && D != 128 && D != 256) return FA_ERR_UNSUPPORTED;
  if (n_states < 1 || n_states > kMaxSplits) return FA_ERR_ARG;
  if (B == 0 || H == 0 || N == 0) return FA_OK;
  const int64_t lim = INT64_MAX / 1024;
  if (B > lim / H || B * H > lim / N || B * H * N > lim / D / kMaxSplits) return FA_ERR_SHAPE;
  int64_t o_st[3] = {H * N * D, N * D, D};
  if (o_strides) {
    for (int i = 0; i < 3; ++i) {
      if (o_strides[i] < 0) return FA_ERR_ARG;
      o_st[i] = o_strides[i];
    }
  }
  const int64_t elt = dtype == FA_F32 ? 4 : 2;
  for (int i = 0; i < 3; ++i)
    if ((o_st[i] * elt) % 16 != 0) return FA_ERR_ALIGN;
  if (max_offset(B, H, N, D, o_st) < 0) return FA_ERR_SHAPE;
  if (!non_overlapping(B, H, N, D, o_st)) return FA_ERR_ARG;
  if (!part_o || !part_lse || !O || !LSE) return FA_ERR_NULL;
  if (misaligned(part_o, 16) || misaligned(part_lse, 4) || misaligned(O, 16) || misaligned(LSE, 4)) return FA_ERR_ALIGN;
  return run_merge(part_o, part_lse, n_states, B, H, N, D, O, o_st, LSE, dtype, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B, int64_t H,
                      int64_t N, int64_t D, float scale, int causal, const int32_t* kv_len, int dtype,
                      void* stream) {
  return fa_fwd_strided(Q, K, V, O, LSE, B, H, N, D, nullptr, scale, causal, nullptr, kv_len, dtype, stream);
}
