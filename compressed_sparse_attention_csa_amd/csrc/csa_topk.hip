// Top-k selection of indexer scores.
//
// Contract: pypto-lib "DeepSeek V4.1 Flash", section "Decode composition"
// (eligible positions only, unique, ascending logical positions, trailing -1);
// gitcode hyper-parallel issue #2, section 7.4 (the selection width is capped
// by the number of visible keys).  Ranking is score descending, ties to the
// lower position, NaN last (scores map to order-preserving 32-bit keys).
//
// Selection core (one work-group over keys held in registers): refine a
// histogram whose bins are linear in score VALUE over the range [min, max] of
// the keys still in play, so the bins spread the keys whatever the shape of
// the score distribution (bit-prefix bins pile a bell-shaped row into a few
// exponent bins and serialise the LDS atomics).  Each pass finds the bin that
// holds the m-th best key; keys above it are chosen, keys below it drop out,
// and the pass repeats inside that bin until its count is exactly what is
// still needed or all of its keys are equal (then the lowest positions win).
// NaN, -inf and +inf get bins of their own at the ends, and a pass whose value
// bins would not separate its min from its max bins the keys' integer codes
// instead, so every pass shrinks the set in play.  Each thread holds a
// contiguous run of positions, so a block scan writes the chosen positions
// already ascending -- no sort.
//
// Rows with span <= 32,768: one work-group per row, keys straight from the
// score row.  Longer rows (up to the 1,048,576-position context): three
// kernels over the row, which the indexer has just left in L2 / MALL:
//   sample: one work-group per row reads 8,192 scores spread over the row and
//           takes as threshold tau the key of sampled rank r = e + 3 sqrt(e)
//           + 4, e = m * samples / span (three standard deviations above the
//           expected rank of the m-th best), which leaves about
//           r * span / samples keys >= tau (4,096 for m = 2,048 over a
//           1,048,576-position row); for r <= 64 the r-th best 16-lane
//           maximum bounds it from below and the few samples above that
//           bound are ranked directly, else the selection core;
//   filter: work-groups over 4,096-score chunks keep every key >= tau, each
//           wave writing its (key, position) pairs in position order into the
//           workspace slots of its own positions, with its count;
//   final:  one work-group per row gathers the segments in position order
//           into LDS and runs the selection core on them.  When the sample
//           misled it (fewer than m keys >= tau, or more candidates than LDS
//           holds), it selects exactly over the whole row instead.
// All three map work-group L to XCD L mod 8 with a contiguous block of rows
// per XCD, so a row's three kernels meet its data in one L2.  The sample and
// final kernels fetch their first data together with the row's position,
// laid out for a row that fills the stride, and fetch again only when the
// row is shorter.
// No work-group waits on another inside a kernel and no counter is shared
// between work-groups, so the kernels need no device-scope fences or atomics
// in global memory, and the workspace keeps nothing between calls.
#include "csa_common.h"

namespace csa {

namespace {

constexpr int kMaxK = 4096;
constexpr int kSmallMax = 32768;     // spans up to this use the one-group kernel
constexpr int kSBins = 2048;         // selection-core histogram bins
constexpr int kChunk = 4096;         // scores per work-group in the long-row kernels
constexpr int kLThreads = 256;
constexpr int kLWaves = kLThreads / 64;
constexpr int kSub = kChunk / kLWaves;   // contiguous positions per wave
constexpr int kLLoads = kSub / 256;      // 16-byte loads per lane
constexpr int kLCap = 2048;          // threshold-bin keys compacted into LDS
constexpr int kRankMax = 256;        // up to this many are ranked directly
constexpr int kCap = 8192;           // candidates the final kernel selects among
constexpr int kFThreads = 1024;      // sample and final kernels
constexpr int kFPer = kCap / kFThreads;
constexpr int kSampleGroups = 2048;  // float4 groups a row's sample reads (2 per thread)
constexpr long long kMaxStride = 1ll << 24;
constexpr int kMaxSeg = static_cast<int>(kMaxStride / kChunk) * kLWaves;   // segments per row
constexpr int kMetaWords = 8;        // [0]: the row's sampled threshold key
constexpr uint32_t kKeyNegInf = 0x007fffffu;
constexpr uint32_t kKeyPosInf = 0xff800000u;

// Long-row workspace (no state survives a call: a word is used only after
// this call wrote it; the final kernel may fetch counts and slots before it
// knows which of them this call wrote, and drops the others): per row a
// threshold word, one candidate count per wave segment, and one (score bits,
// position) slot per score (a segment owns the slots of its own positions,
// so no counter is shared between work-groups).
struct Workspace {
  uint32_t* meta;   // [T][kMetaWords]
  uint32_t* seg;    // [T][nseg]
  uint2* cand;      // [T][stride]
  int nseg;         // segments per row: chunks * waves
};

inline int segs_for(long long stride) {
  return static_cast<int>(((stride + kChunk - 1) / kChunk) * kLWaves);
}

inline size_t ws_bytes(int T, long long stride) {
  const size_t words = static_cast<size_t>(T) * kMetaWords + static_cast<size_t>(T) * segs_for(stride);
  return ((words * sizeof(uint32_t) + 15) & ~size_t(15)) +
         static_cast<size_t>(T) * stride * sizeof(uint2);
}

inline Workspace ws_layout(void* base, int T, long long stride) {
  Workspace w;
  w.nseg = segs_for(stride);
  w.meta = static_cast<uint32_t*>(base);
  w.seg = w.meta + static_cast<size_t>(T) * kMetaWords;
  const size_t words = static_cast<size_t>(T) * kMetaWords + static_cast<size_t>(T) * w.nseg;
  w.cand = reinterpret_cast<uint2*>(static_cast<char*>(base) +
                                    ((words * sizeof(uint32_t) + 15) & ~size_t(15)));
  return w;
}

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: below everything
  if (u == 0x80000000u) u = 0u;                      // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ bool key_finite(uint32_t k) { return k > kKeyNegInf && k < kKeyPosInf; }

// Monotone map from keys to nb bins: NaN -> 0, -inf -> 1, +inf -> nb - 1,
// finite keys -> 2 .. nb - 2, linear in value over [lo, hi] (or, when that
// does not separate lo from hi in float arithmetic, linear in key code).
struct Binner {
  bool by_value;
  float lo_h;      // lo / 2 (halved so hi - lo cannot overflow)
  float scale;
  uint32_t klo;
  float kscale;
  int nb;
  __device__ __forceinline__ int operator()(uint32_t key) const {
    // branch-free: non-finite keys produce a finite d (clamped) and are then
    // overridden by their own bins
    const float dv = fmaf(key_value(key), 0.5f, -lo_h) * scale;
    const float dk = static_cast<float>(key - klo) * kscale;
    const float d = fminf(fmaxf(by_value ? dv : dk, 0.0f), static_cast<float>(nb - 4));
    int b = 2 + static_cast<int>(d);
    b = key == kKeyPosInf ? nb - 1 : b;
    b = key == kKeyNegInf ? 1 : b;
    b = key == 0u ? 0 : b;
    return b;
  }
};

// kfmin / kfmax: smallest and largest finite key in play (kfmin > kfmax when
// there is none).
__device__ __forceinline__ Binner make_binner(uint32_t kfmin, uint32_t kfmax, int nb) {
  Binner b;
  b.nb = nb;
  b.by_value = false;
  b.lo_h = 0.0f;
  b.scale = 0.0f;
  b.klo = kfmin;
  b.kscale = 0.0f;
  if (kfmin >= kfmax) return b;   // at most one finite value: one finite bin
  // any positive scale keeps the map monotone, so approximate reciprocals do
  const float top = static_cast<float>(nb - 4);
  b.kscale = top * __builtin_amdgcn_rcpf(static_cast<float>(kfmax - kfmin));
  const float lo = key_value(kfmin), hi = key_value(kfmax);
  b.lo_h = lo * 0.5f;
  const float range_h = fmaf(hi, 0.5f, -b.lo_h);
  const float sc = top * __builtin_amdgcn_rcpf(range_h);
  if (range_h > 0.0f && sc < 3.0e38f) {
    b.scale = sc;
    b.by_value = true;
    if (b(kfmin) == b(kfmax)) b.by_value = false;
  }
  return b;
}

// Wave-wide primitives on DPP row shifts and row broadcasts (gfx9 family):
// a few dependent VALU ops instead of a chain of LDS permutes.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xa, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xc, 0xf, false)));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
  v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(-1, static_cast<int>(v), 0x111, 0xf, 0xf, false)));
  v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(-1, static_cast<int>(v), 0x112, 0xf, 0xf, false)));
  v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(-1, static_cast<int>(v), 0x114, 0xf, 0xf, false)));
  v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(-1, static_cast<int>(v), 0x118, 0xf, 0xf, false)));
  v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(-1, static_cast<int>(v), 0x142, 0xa, 0xf, false)));
  v = min(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(-1, static_cast<int>(v), 0x143, 0xc, 0xf, false)));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// Exclusive scan over a work-group of NW waves.  `wsum` holds 2 * NW + 1
// ints; wave 0 scans the wave totals, so every thread reads one prefix.
// Back-to-back calls are safe: a call's writes to wsum are ordered after the
// previous call's reads by its own barriers.
template <int NW>
__device__ int block_excl_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int tw = lane < NW ? wsum[lane] : 0;
    const int pw = wave_incl_scan(tw);
    if (lane < NW) wsum[NW + lane] = pw - tw;
    if (lane == NW - 1) wsum[2 * NW] = pw;
  }
  __syncthreads();
  if (total) *total = wsum[2 * NW];
  return wsum[NW + wave] + incl - v;
}

// The work-group scans an NB-bin histogram from the top: thread t sums bins
// [NB - (t+1)*PER, NB - t*PER) (consecutive threads, consecutive words), a
// block scan orders the sums, and the one thread whose range holds the
// need-th key writes that bin and the count strictly above it.
template <int NB, int THREADS>
__device__ void find_bin(const uint32_t* hist, int need, int* wsum, int* bin_out,
                         int* above_out) {
  constexpr int PER = NB / THREADS;
  static_assert(PER >= 1 && NB % THREADS == 0, "bins per thread");
  const int lo = NB - (static_cast<int>(threadIdx.x) + 1) * PER;
  int h[PER];
  int s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    h[i] = static_cast<int>(hist[lo + i]);
    s += h[i];
  }
  int run = block_excl_scan<THREADS / 64>(s, wsum, nullptr);
  if (run < need && run + s >= need) {
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (run < need && run + h[i] >= need) {
        *bin_out = lo + i;
        *above_out = run;
      }
      run += h[i];
    }
  }
  __syncthreads();
}

template <int THREADS>
struct SelShared {
  alignas(16) uint32_t hist[kSBins + 64];   // + one dummy bin per lane
  // threshold-bin keys then their positions (position order); the whole-row
  // path uses it as its selection buffer (kMaxK entries)
  uint32_t list[2 * kLCap];
  uint32_t red[4][THREADS / 64];
  int wsum[2 * (THREADS / 64) + 1];
  int bsel[2];
  uint32_t cut[2];                          // key and position of the m-th best
  int sel_count;
};
static_assert(2 * kLCap >= kMaxK, "whole-row selection buffer");

__device__ __forceinline__ uint32_t uniform_u(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}

// Block min / max of one u32 per thread (result uniform in every thread):
// wave partials go to red[0..1], and after one barrier every thread combines
// the NW partials itself (same-address LDS reads broadcast).  A later call
// that writes the same red rows must be separated from this one's reads by a
// barrier; back-to-back calls use different rows.
template <int NW>
__device__ __forceinline__ void block_minmax(uint32_t& lo, uint32_t& hi, uint32_t (*red)[NW]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  lo = wave_min_u(lo);
  hi = wave_max_u(hi);
  if (lane == 0) {
    red[0][wave] = lo;
    red[1][wave] = hi;
  }
  __syncthreads();
  uint32_t a = 0xffffffffu, b = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    a = min(a, red[0][w]);
    b = max(b, red[1][w]);
  }
  lo = uniform_u(a);
  hi = uniform_u(b);
}

// Refinement select (the path for a threshold bin too large for the LDS
// list).  Thread-local keys key[0..nmine), positions ascending within the
// thread and threads in position order; the m best over the work-group are
// the `chosen` bits plus, of the `tie` bits (equal keys), the thread's first
// `take`.
template <int THREADS, int KPT>
__device__ void block_select(const uint32_t (&key)[KPT], int nmine, int m, SelShared<THREADS>& sh,
                             uint32_t& chosen, uint32_t& tie, int& take) {
  static_assert(KPT <= 32, "one bit per key");
  constexpr int NW = THREADS / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  uint32_t live = nmine >= 32 ? 0xffffffffu : ((1u << nmine) - 1u);
  chosen = 0u;
  tie = 0u;
  take = 0;
  int rem = m;
  for (;;) {
    uint32_t kmin = 0xffffffffu, kmax = 0u, fmin = 0xffffffffu, fmax = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool lv = (live >> j) & 1u;
      const uint32_t kk = key[j];
      kmin = min(kmin, lv ? kk : 0xffffffffu);
      kmax = max(kmax, lv ? kk : 0u);
      const bool fin = lv && key_finite(kk);
      fmin = min(fmin, fin ? kk : 0xffffffffu);
      fmax = max(fmax, fin ? kk : 0u);
    }
    for (int i = tid; i < kSBins + 64; i += THREADS) sh.hist[i] = 0u;
    block_minmax<NW>(kmin, kmax, sh.red);
    block_minmax<NW>(fmin, fmax, sh.red + 2);
    if (kmin == kmax) {
      // every key in play is equal: the rem lowest positions among them
      const int eq = __popc(live);
      const int eq_before = block_excl_scan<NW>(eq, sh.wsum, nullptr);
      take = max(0, min(eq, rem - eq_before));
      tie = live;
      return;
    }
    const Binner bn = make_binner(fmin, fmax, kSBins);
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      atomicAdd(&sh.hist[((live >> j) & 1u) ? bn(key[j]) : kSBins + lane], 1u);
    __syncthreads();
    find_bin<kSBins, THREADS>(sh.hist, rem, sh.wsum, &sh.bsel[0], &sh.bsel[1]);
    const int b = sh.bsel[0];
    rem -= sh.bsel[1];
    const int cnt = static_cast<int>(sh.hist[b]);
    uint32_t in_b = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int bb = bn(key[j]);
      const bool lv = (live >> j) & 1u;
      chosen |= (lv && bb > b) ? (1u << j) : 0u;
      in_b |= (lv && bb == b) ? (1u << j) : 0u;
    }
    live = in_b;
    if (cnt == rem) {
      chosen |= live;
      return;
    }
    __syncthreads();   // hist, bsel and red are rewritten by the next pass
  }
}

// The cut of a refinement select: key and position of its worst winner.
template <int THREADS, int KPT, typename PosFn>
__device__ void cut_of_selection(const uint32_t (&key)[KPT], uint32_t chosen, uint32_t tie,
                                 int take, SelShared<THREADS>& sh, PosFn pos) {
  constexpr int NW = THREADS / 64;
  uint32_t kmin = 0xffffffffu, dummy = 0u;
  uint32_t win = chosen;
  int taken = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (((tie >> j) & 1u) && taken < take) {
      win |= 1u << j;
      ++taken;
    }
    kmin = min(kmin, ((win >> j) & 1u) ? key[j] : 0xffffffffu);
  }
  block_minmax<NW>(kmin, dummy, sh.red);
  uint32_t pmin = 0xffffffffu, pmax = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (((win >> j) & 1u) && key[j] == kmin) pmax = max(pmax, static_cast<uint32_t>(pos(j)));
  __syncthreads();   // red is reused
  block_minmax<NW>(pmin, pmax, sh.red + 2);
  if (threadIdx.x == 0) {
    sh.cut[0] = kmin;
    sh.cut[1] = pmax;
  }
  __syncthreads();
}

// Selection core: leaves in sh.cut the key and position of the m-th best
// (score descending, position ascending) of the work-group's keys
// key[0..nmine), whose positions pos(j) ascend within a thread and across
// threads.  One value-histogram pass over every key finds the bin holding the
// m-th best; that bin's keys are compacted into LDS in position order and,
// when few, ranked directly, else refined as a list.  HOLD keeps each key's
// bin in registers between the histogram, the count and the compaction
// instead of recomputing it (callers short of registers leave it off).
template <int THREADS, int KPT, bool HOLD, typename PosFn>
__device__ bool find_cut(const uint32_t (&key)[KPT], int nmine, int m, SelShared<THREADS>& sh,
                         PosFn pos) {
  constexpr int NW = THREADS / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  uint32_t fmin = 0xffffffffu, fmax = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool fin = j < nmine && key_finite(key[j]);
    fmin = min(fmin, fin ? key[j] : 0xffffffffu);
    fmax = max(fmax, fin ? key[j] : 0u);
  }
  for (int i = tid; i < kSBins + 64; i += THREADS) sh.hist[i] = 0u;
  block_minmax<NW>(fmin, fmax, sh.red);
  const Binner bn = make_binner(fmin, fmax, kSBins);
  // a key's bin, -1 past nmine
  constexpr bool kHold = HOLD;
  int bj[kHold ? KPT : 1];
  auto bin_of = [&](int j) {
    if constexpr (kHold) return bj[j];
    else return j < nmine ? bn(key[j]) : -1;
  };
  if constexpr (kHold) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) bj[j] = j < nmine ? bn(key[j]) : -1;
  }
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int bb = bin_of(j);
    atomicAdd(&sh.hist[bb >= 0 ? bb : kSBins + lane], 1u);
  }
  __syncthreads();
  find_bin<kSBins, THREADS>(sh.hist, m, sh.wsum, &sh.bsel[0], &sh.bsel[1]);
  const int b0 = sh.bsel[0];
  const int rem = m - sh.bsel[1];
  const int cnt = static_cast<int>(sh.hist[b0]);
  if (cnt > kLCap) return false;   // massive ties: the caller selects on the whole row
  int c = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) c += bin_of(j) == b0 ? 1 : 0;
  int o = block_excl_scan<NW>(c, sh.wsum, nullptr);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (bin_of(j) == b0) {
      sh.list[o] = key[j];
      sh.list[kLCap + o] = static_cast<uint32_t>(pos(j));
      ++o;
    }
  }
  __syncthreads();
  if (cnt <= kRankMax) {
    // rank of element i among the bin: how many are better (larger key, or
    // the same key at a lower position); the one of rank rem - 1 is the cut
    if (tid < cnt) {
      const uint32_t ki = sh.list[tid], pi = sh.list[kLCap + tid];
      int r = 0;
      for (int q = 0; q < cnt; ++q) {
        const uint32_t kq = sh.list[q], pq = sh.list[kLCap + q];
        r += (kq > ki || (kq == ki && pq < pi)) ? 1 : 0;
      }
      if (r == rem - 1) {
        sh.cut[0] = ki;
        sh.cut[1] = pi;
      }
    }
    __syncthreads();
    return true;
  }
  // a larger bin: refine on the list, LPT elements per thread in order
  constexpr int LPT = kLCap / THREADS;
  const int lbase = tid * LPT;
  uint32_t lk[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) lk[j] = lbase + j < cnt ? sh.list[lbase + j] : 0u;
  const int nl = max(0, min(LPT, cnt - lbase));
  uint32_t chosen, tie;
  int take;
  block_select<THREADS, LPT>(lk, nl, rem, sh, chosen, tie, take);
  cut_of_selection<THREADS, LPT>(lk, chosen, tie, take, sh,
                                 [&](int j) { return static_cast<int>(sh.list[kLCap + lbase + j]); });
  return true;
}

// Which entries of a score row take part, and how a chosen entry is reported.
// The span of row t is its visible count (p + 1) / ratio, grouped into
// ceil(count / group) entries (group 8: the blocks of a candidate mask), or
// counts[t] when counts is given.  A chosen entry i is reported as i, or with
// remap as remap[t][i / rgroup] * rgroup + i % rgroup (the position of
// candidate slot i).
// (The fields are handed on as scalars: a helper that took the struct by
// address would make the compiler keep it in scratch memory.)
struct RowSpec {
  const int32_t* positions;
  int ratio;
  int group;
  const int32_t* counts;
  const int32_t* remap;
  int rgroup;
  int rstride;
};

__device__ __forceinline__ int row_span(const RowSpec rs, int t, long long stride, int32_t* err,
                                        bool report) {
  long long nv;
  if (rs.counts) {
    nv = max(0, rs.counts[t]);
  } else {
    nv = visible_count(rs.positions[t], rs.ratio);
    if (rs.group > 1) nv = (nv + rs.group - 1) / rs.group;
  }
  if (nv > stride) {
    if (report) flag_error(err, CSA_EFLAG_POS_RANGE);
    nv = stride;
  }
  return static_cast<int>(nv);
}

// How a chosen entry i of row t is reported (see RowSpec).
struct Remap {
  const int32_t* remap;
  int rgroup;
  int rstride;
  int t;
  __device__ __forceinline__ int operator()(int i) const {
    if (!remap) return i;
    const int q = i / rgroup;
    return remap[static_cast<long long>(t) * rstride + q] * rgroup + (i - q * rgroup);
  }
};

// Writes, in position order, every key better than or equal to the cut
// (exactly m of them), then the -1 / -inf padding; val(j) is key j's score.
template <int THREADS, int KPT, typename PosFn, typename ValFn>
__device__ void emit_cut(const uint32_t (&key)[KPT], int nmine, int m, int k, ValFn val_of,
                         int32_t* out_i, float* out_v, SelShared<THREADS>& sh, PosFn pos,
                         Remap rm) {
  const uint32_t ck = sh.cut[0], cp = sh.cut[1];
  uint32_t pick = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool in = j < nmine &&
                    (key[j] > ck || (key[j] == ck && static_cast<uint32_t>(pos(j)) <= cp));
    pick |= in ? (1u << j) : 0u;
  }
  // the chosen scores are fetched before any is stored, so a thread's picks
  // share one latency
  float val[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) val[j] = (out_v && ((pick >> j) & 1u)) ? val_of(j) : 0.0f;
  int o = block_excl_scan<THREADS / 64>(__popc(pick), sh.wsum, nullptr);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if ((pick >> j) & 1u) {
      out_i[o] = rm(pos(j));
      if (out_v) out_v[o] = val[j];
      ++o;
    }
  }
  const float neg_inf = -__builtin_huge_valf();
  for (int i = m + static_cast<int>(threadIdx.x); i < k; i += THREADS) {
    out_i[i] = -1;
    if (out_v) out_v[i] = neg_inf;
  }
}

// Every visible position is chosen: 0 .. n-1 ascending, then padding.
template <int THREADS>
__device__ void write_all(int n, int k, const float* row, int32_t* out_i, float* out_v,
                          Remap rm) {
  const float neg_inf = -__builtin_huge_valf();
  for (int i = threadIdx.x; i < k; i += THREADS) {
    out_i[i] = i < n ? rm(i) : -1;
    if (out_v) out_v[i] = i < n ? row[i] : neg_inf;
  }
}

// Exact radix select over a whole row from global memory (8-bit digits on the
// key, then on the position for ties) and a bitonic sort of the chosen
// positions: the path for rows whose threshold bin held too many keys.
template <int THREADS>
__device__ void select_whole_row(const float* row, int n, int m, int k, int32_t* out_i,
                                 float* out_v, SelShared<THREADS>& sh, Remap rm) {
  const int tid = threadIdx.x;
  int* sel = reinterpret_cast<int*>(sh.list);
  int* sel_count = &sh.sel_count;
  __syncthreads();   // the caller's last reads of the shared state are done
  uint32_t* hist = sh.hist;   // first 256 bins
  // wave 0: the digit where the running count from the top (or the bottom)
  // first reaches need, and the count before it
  auto digit = [&](bool descending, int need) {
    if (tid < 64) {
      const int lane = tid;
      const int b0 = descending ? (255 - 4 * lane) : (4 * lane);
      const int step = descending ? -1 : 1;
      int hh[4];
      int s = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hh[i] = static_cast<int>(hist[b0 + step * i]);
        s += hh[i];
      }
      const int incl = wave_incl_scan(s);
      int run = incl - s;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (run < need && run + hh[i] >= need) {
          sh.bsel[0] = b0 + step * i;
          sh.bsel[1] = run;
        }
        run += hh[i];
      }
    }
  };
  uint32_t prefix = 0u, mask = 0u;
  int rem = m;
  bool exact = false;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += THREADS) {
      const uint32_t kk = order_key(row[i]);
      if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & 255], 1u);
    }
    __syncthreads();
    digit(true, rem);
    __syncthreads();
    const int d = sh.bsel[0];
    rem -= sh.bsel[1];
    const int cnt = static_cast<int>(hist[d]);
    prefix |= static_cast<uint32_t>(d) << shift;
    mask |= 0xffu << shift;
    __syncthreads();
    if (cnt == rem) {
      exact = true;
      break;
    }
  }
  uint32_t pos_limit = 0xffffffffu;
  if (!exact) {
    uint32_t pprefix = 0u, pmask = 0u;
    int prem = rem;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0u;
      __syncthreads();
      for (int i = tid; i < n; i += THREADS) {
        const uint32_t p = static_cast<uint32_t>(i);
        if ((order_key(row[i]) & mask) == prefix && (p & pmask) == pprefix)
          atomicAdd(&hist[(p >> shift) & 255], 1u);
      }
      __syncthreads();
      digit(false, prem);
      __syncthreads();
      prem -= sh.bsel[1];
      pprefix |= static_cast<uint32_t>(sh.bsel[0]) << shift;
      pmask |= 0xffu << shift;
      __syncthreads();
    }
    pos_limit = pprefix;
  }
  if (tid == 0) *sel_count = 0;
  __syncthreads();
  for (int i = tid; i < n; i += THREADS) {
    const uint32_t km = order_key(row[i]) & mask;
    if (km > prefix || (km == prefix && static_cast<uint32_t>(i) <= pos_limit)) {
      const int slot = atomicAdd(sel_count, 1);
      if (slot < kMaxK) sel[slot] = i;
    }
  }
  __syncthreads();
  int P = 1;
  while (P < m) P <<= 1;
  for (int i = m + tid; i < P; i += THREADS) sel[i] = 0x7fffffff;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int j = size >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < (P >> 1); i += THREADS) {
        const int lo = 2 * i - (i & (j - 1));
        const int hi = lo + j;
        const bool up = ((lo & size) == 0);
        const int a = sel[lo], b = sel[hi];
        if ((a > b) == up) {
          sel[lo] = b;
          sel[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  const float neg_inf = -__builtin_huge_valf();
  for (int i = tid; i < k; i += THREADS) {
    const int c = i < m ? sel[i] : -1;
    out_i[i] = c >= 0 ? rm(c) : -1;
    if (out_v) out_v[i] = c >= 0 ? row[c] : neg_inf;
  }
}

// ----------------------------------------------------------------------------
// short rows: one work-group, keys in registers
// ----------------------------------------------------------------------------
template <int THREADS, int KPT>
__global__ void __launch_bounds__(THREADS) topk_small_kernel(
    const float* __restrict__ scores, long long stride, RowSpec rs,
    int num_tokens, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_val, int32_t* err) {
  constexpr int kSmallCand = THREADS >= 1024 ? 4096 : 8 * THREADS;
  __shared__ SelShared<THREADS> sh;
  __shared__ uint32_t cand_k[kSmallCand];
  __shared__ uint32_t cand_p[kSmallCand];
  // rows in reverse launch order: a causal prefill's later rows span more
  // keys, so they are dispatched first and the short rows fill in behind
  const int t = static_cast<int>(gridDim.x) - 1 - static_cast<int>(blockIdx.x);
  const int tid = threadIdx.x;
  if (t >= num_tokens) return;
  const float* row = scores + static_cast<long long>(t) * stride;
  // the whole allocated row is loaded before the span is known (one memory
  // latency instead of two); per is a multiple of 4 and stride is too, so a
  // 16-byte load starting below stride stays inside the row
  const int span = static_cast<int>(stride);
  const int per = 4 * ((span + 4 * THREADS - 1) / (4 * THREADS));
  const int base = tid * per;
  float4 v[KPT / 4];
#pragma unroll
  for (int i = 0; i < KPT / 4; ++i) {
    v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (4 * i < per && base + 4 * i < span)
      v[i] = *reinterpret_cast<const float4*>(row + base + 4 * i);
  }
  const int n = row_span(rs, t, stride, err, tid == 0);
  int32_t* out_i = topk_idx + static_cast<long long>(t) * k;
  float* out_v = topk_val ? topk_val + static_cast<long long>(t) * k : nullptr;
  const int m = min(k, n);
  if (m == n) {
    write_all<THREADS>(n, k, row, out_i, out_v, Remap{rs.remap, rs.rgroup, rs.rstride, t});
    return;
  }
  uint32_t key[KPT];
#pragma unroll
  for (int i = 0; i < KPT / 4; ++i) {
    key[4 * i] = order_key(v[i].x);
    key[4 * i + 1] = order_key(v[i].y);
    key[4 * i + 2] = order_key(v[i].z);
    key[4 * i + 3] = order_key(v[i].w);
  }
  const int nmine = max(0, min(per, n - base));
  auto pos = [&](int j) { return base + j; };
  constexpr int NW = THREADS / 64;
  constexpr int CPT = kSmallCand / THREADS;
  bool done = false;
  // Sampled threshold: every thread's first key is a sample (S of them,
  // evenly spaced); the key tau of the r-th best sample, with r a little above
  // m * S / n, leaves in expectation slightly more than m keys >= tau.  Those
  // candidates are compacted in position order and selected exactly; when the
  // sample misleads (fewer than m or too many candidates) the row takes the
  // full path below.
  const int S = (n + per - 1) / per;
  const float expect = static_cast<float>(m) * static_cast<float>(S) / static_cast<float>(n);
  const int r = static_cast<int>(ceilf(expect + 2.0f * sqrtf(expect) + 2.0f));
  if (S >= 64 && r < S) {
    {
      // histogram of the samples' top 11 key bits; tau is the lower edge of
      // the bin holding the r-th best sample
      for (int i = tid; i < kSBins + 64; i += THREADS) sh.hist[i] = 0u;
      __syncthreads();
      atomicAdd(&sh.hist[nmine > 0 ? (key[0] >> 21) : kSBins + (tid & 63)], 1u);
      __syncthreads();
      find_bin<kSBins, THREADS>(sh.hist, r, sh.wsum, &sh.bsel[0], &sh.bsel[1]);
      const uint32_t tau = static_cast<uint32_t>(sh.bsel[0]) << 21;
      int c = 0;
#pragma unroll
      for (int j = 0; j < KPT; ++j) c += (j < nmine && key[j] >= tau) ? 1 : 0;
      int total = 0;
      int o = block_excl_scan<NW>(c, sh.wsum, &total);
      if (total >= m && total <= kSmallCand) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          if (j < nmine && key[j] >= tau) {
            cand_k[o] = key[j];
            cand_p[o] = static_cast<uint32_t>(base + j);
            ++o;
          }
        }
        __syncthreads();
        const int cper = (total + THREADS - 1) / THREADS;
        const int cbase = tid * cper;
        uint32_t ck[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) ck[j] = (j < cper && cbase + j < total) ? cand_k[cbase + j] : 0u;
        const int cn = max(0, min(cper, total - cbase));
        auto cpos = [&](int j) { return static_cast<int>(cand_p[cbase + j]); };
        if (find_cut<THREADS, CPT, (KPT <= 16)>(ck, cn, m, sh, cpos)) {
          emit_cut<THREADS, CPT>(ck, cn, m, k, [&](int j) { return row[cpos(j)]; }, out_i, out_v,
                                 sh, cpos, Remap{rs.remap, rs.rgroup, rs.rstride, t});
          done = true;
        }
      }
    }
    __syncthreads();
  }
  if (done) return;
  if (find_cut<THREADS, KPT, false>(key, nmine, m, sh, pos))
    emit_cut<THREADS, KPT>(key, nmine, m, k, [&](int j) { return row[pos(j)]; }, out_i, out_v, sh,
                           pos, Remap{rs.remap, rs.rgroup, rs.rstride, t});
  else
    select_whole_row<THREADS>(row, n, m, k, out_i, out_v, sh, Remap{rs.remap, rs.rgroup, rs.rstride, t});
}

// ----------------------------------------------------------------------------
// long rows
// ----------------------------------------------------------------------------
// Long-row work is split over the XCDs in contiguous runs of rows (work-group
// L runs on XCD L % 8): a row's sample, filter chunks and final selection
// share one XCD's L2, so the final kernel reads its candidates (and the
// filter its threshold) where they were written.
__device__ __forceinline__ int xcd_item(int per_xcd) {
  const int L = blockIdx.x;
  return (L & 7) * per_xcd + (L >> 3);
}

// Largest u32 of a row of 16 lanes, in every lane of the row (DPP quad swaps
// and row mirrors: each step compares symmetric pairs).
__device__ __forceinline__ uint32_t row16_max_u(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xb1, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4e, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xf, 0xf, false)));
  return v;
}

// The r-th largest of the work-group's keys for a small r (r <= kRows16, the
// number of 16-lane rows of the work-group): the r-th largest row maximum is
// a lower bound lo for it (r rows hold a key >= lo), so it is the r-th
// largest of the keys >= lo -- for a sample of a row's scores a few dozen --
// which are compacted into LDS and ranked directly.  Returns false when more
// than kSmallRCap keys reach lo (then the caller runs the selection core).
constexpr int kSmallRCap = 1024;
template <int THREADS, int KPT>
__device__ bool small_r_threshold(const uint32_t (&key)[KPT], int r, SelShared<THREADS>& sh,
                                  uint32_t* tau) {
  constexpr int NW = THREADS / 64;
  constexpr int kRows16 = THREADS / 16;
  static_assert(kRows16 + kSmallRCap <= 2 * kLCap, "LDS list");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint32_t mx = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) mx = max(mx, key[j]);
  mx = row16_max_u(mx);
  if ((lane & 15) == 0) sh.list[wave * 4 + (lane >> 4)] = mx;
  __syncthreads();
  // rank the row maxima (larger first, ties by row index); the one of rank
  // r - 1 is the bound
  for (int g = tid; g < kRows16; g += THREADS) {
    const uint32_t v = sh.list[g];
    int rank = 0;
    for (int u = 0; u < kRows16; ++u) {
      const uint32_t o = sh.list[u];
      rank += (o > v || (o == v && u < g)) ? 1 : 0;
    }
    if (rank == r - 1) sh.cut[0] = v;
  }
  __syncthreads();
  const uint32_t lo = sh.cut[0];
  int c = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) c += key[j] >= lo ? 1 : 0;
  int total = 0;
  int o = block_excl_scan<NW>(c, sh.wsum, &total);
  if (total > kSmallRCap) return false;
  uint32_t* list = sh.list + kRows16;
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (key[j] >= lo) list[o++] = key[j];
  __syncthreads();
  for (int i = tid; i < total; i += THREADS) {
    const uint32_t v = list[i];
    int rank = 0;
    for (int u = 0; u < total; ++u) {
      const uint32_t w = list[u];
      rank += (w > v || (w == v && u < i)) ? 1 : 0;
    }
    if (rank == r - 1) sh.cut[1] = v;
  }
  __syncthreads();
  *tau = sh.cut[1];
  return true;
}

// Sampled threshold of a long row: one float4 group every `span` positions
// (span a multiple of 256 that keeps the groups within kSampleGroups), S
// samples in all.  The key tau of the r-th best sample, with r a few standard
// deviations above m * S / n, leaves in expectation about 1.6 m keys >= tau
// and fewer than m only with a probability of order 1e-4 for random data;
// the final kernel checks the count and falls back to an exact whole-row
// select when the sample misled it.
__global__ void __launch_bounds__(kFThreads) topk_sample_kernel(
    const float* __restrict__ scores, long long stride, RowSpec rs,
    int num_tokens, int k, Workspace ws, int rows_per_xcd) {
  __shared__ SelShared<kFThreads> sh;
  const int t = xcd_item(rows_per_xcd);
  const int tid = threadIdx.x;
  if (t >= num_tokens) return;
  const float* row = scores + static_cast<long long>(t) * stride;
  // groups of 4 scores, one every `span` positions (a multiple of 256)
  auto span_of = [](long long len) {
    return 256ll * ((len + 256ll * kSampleGroups - 1) / (256ll * kSampleGroups));
  };
  constexpr int KPT = 4 * (kSampleGroups / kFThreads);
  // The groups are read with the row's position, spaced for a row that fills
  // the stride (the usual case), and read again only when the row's own span
  // spaces them differently.
  float4 v[KPT / 4];
  const long long span_g = span_of(stride);
#pragma unroll
  for (int i = 0; i < KPT / 4; ++i) {
    const long long p0 = static_cast<long long>(tid + i * kFThreads) * span_g;
    v[i] = p0 < stride ? *reinterpret_cast<const float4*>(row + p0)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int n = row_span(rs, t, stride, nullptr, false);
  if (n <= kCap) return;
  const long long span = span_of(n);
  const int G = static_cast<int>((n + span - 1) / span);   // groups, <= kSampleGroups
  if (span != span_g) {
#pragma unroll
    for (int i = 0; i < KPT / 4; ++i) {
      const int g = tid + i * kFThreads;
      v[i] = g < G ? *reinterpret_cast<const float4*>(row + g * span)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  // thread tid reads groups tid, tid + 1024, ...: its valid groups are a
  // prefix, so its keys [0, nmine) are the samples it holds (components past
  // the span take the lowest key, which never moves the r-th best)
  uint32_t key[KPT];
  int ng = 0;
#pragma unroll
  for (int i = 0; i < KPT / 4; ++i) {
    const int g = tid + i * kFThreads;
    const long long p0 = g * span;
    key[4 * i] = g < G ? order_key(v[i].x) : 0u;
    key[4 * i + 1] = (g < G && p0 + 1 < n) ? order_key(v[i].y) : 0u;
    key[4 * i + 2] = (g < G && p0 + 2 < n) ? order_key(v[i].z) : 0u;
    key[4 * i + 3] = (g < G && p0 + 3 < n) ? order_key(v[i].w) : 0u;
    ng += g < G ? 1 : 0;
  }
  const int nmine = 4 * ng;
  int S = 0;
  block_excl_scan<kFThreads / 64>(nmine, sh.wsum, &S);
  const int m = min(k, n);
  const float expect = static_cast<float>(m) * static_cast<float>(S) / static_cast<float>(n);
  const int r = static_cast<int>(ceilf(expect + 3.0f * sqrtf(expect) + 4.0f));
  // keys past nmine are 0, the lowest key: with r < S they never move the
  // r-th best, so the small-r path may take every slot.  It needs r rows of
  // 16 lanes holding samples (threads below G hold at least one group).
  uint32_t tau = 0u;   // every key is a candidate
  if (r < S) {
    const bool small_r = r <= min(G, kFThreads) / 16;
    if (!(small_r && small_r_threshold<kFThreads, KPT>(key, r, sh, &tau)) &&
        find_cut<kFThreads, KPT, true>(key, nmine, r, sh, [&](int j) { return tid * KPT + j; }))
      tau = sh.cut[0];
  }
  if (tid == 0) ws.meta[static_cast<size_t>(t) * kMetaWords] = tau;
}

// Lane `lane` of wave `wave` loads kLLoads 16-byte groups of the chunk at c0:
// positions c0 + wave*kSub + 256*i + 4*lane, so each wave owns a contiguous
// kSub-position run and position order is (i, lane, component).
struct ChunkKeys {
  uint32_t key[4 * kLLoads];
  uint32_t raw[4 * kLLoads];   // the scores' bits
  int first;                   // position of key[0]
};

__device__ __forceinline__ void load_chunk(const float* row, long long stride, int n, int c0,
                                           ChunkKeys& ck) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  ck.first = c0 + wave * kSub + 4 * lane;
  float4 v[kLLoads];
#pragma unroll
  for (int i = 0; i < kLLoads; ++i) {
    const int c = ck.first + 256 * i;
    v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < stride) v[i] = *reinterpret_cast<const float4*>(row + c);
  }
#pragma unroll
  for (int i = 0; i < kLLoads; ++i) {
    ck.raw[4 * i] = __float_as_uint(v[i].x);
    ck.raw[4 * i + 1] = __float_as_uint(v[i].y);
    ck.raw[4 * i + 2] = __float_as_uint(v[i].z);
    ck.raw[4 * i + 3] = __float_as_uint(v[i].w);
  }
#pragma unroll
  for (int j = 0; j < 4 * kLLoads; ++j) ck.key[j] = order_key(__uint_as_float(ck.raw[j]));
}

__device__ __forceinline__ bool in_span(const ChunkKeys& ck, int j, int n) {
  return ck.first + 256 * (j >> 2) + (j & 3) < n;
}

// Keep every key >= tau: each wave writes its kept (score bits, position)
// pairs, in position order, into the slots of its own segment and its count
// into seg[].
__global__ void __launch_bounds__(kLThreads) topk_filter_kernel(
    const float* __restrict__ scores, long long stride, RowSpec rs,
    int num_tokens, Workspace ws, int nchunks, int chunks_per_xcd) {
  const int item = xcd_item(chunks_per_xcd);   // row-major (row, chunk)
  const int t = item / nchunks;
  const int chunk = item - t * nchunks;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (t >= num_tokens) return;
  const int n = row_span(rs, t, stride, nullptr, false);
  const int c0 = chunk * kChunk;
  if (n <= kCap || c0 >= n) return;
  ChunkKeys ck;
  load_chunk(scores + static_cast<long long>(t) * stride, stride, n, c0, ck);
  const uint32_t tau = ws.meta[static_cast<size_t>(t) * kMetaWords];
  int cnt[kLLoads];
  int off[kLLoads];
  int wave_total = 0;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int i = 0; i < kLLoads; ++i) {
    int c = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) c += (in_span(ck, 4 * i + q, n) && ck.key[4 * i + q] >= tau) ? 1 : 0;
    cnt[i] = c;
    const uint64_t b0 = __ballot(c & 1), b1 = __ballot(c & 2), b2 = __ballot(c & 4);
    off[i] = wave_total + __popcll(b0 & below) + 2 * __popcll(b1 & below) +
             4 * __popcll(b2 & below);
    wave_total += __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
  }
  const int sidx = chunk * kLWaves + wave;
  if (lane == 0) ws.seg[static_cast<size_t>(t) * ws.nseg + sidx] = static_cast<uint32_t>(wave_total);
  uint2* slots = ws.cand + static_cast<size_t>(t) * stride + static_cast<size_t>(c0) + wave * kSub;
#pragma unroll
  for (int i = 0; i < kLLoads; ++i) {
    if (cnt[i] == 0) continue;
    int o = off[i];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (in_span(ck, 4 * i + q, n) && ck.key[4 * i + q] >= tau) {
        slots[o] = make_uint2(ck.raw[4 * i + q], static_cast<uint32_t>(ck.first + 256 * i + q));
        ++o;
      }
    }
  }
}

__global__ void __launch_bounds__(kFThreads) topk_final_kernel(
    const float* __restrict__ scores, long long stride, RowSpec rs,
    int num_tokens, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_val, Workspace ws, int32_t* err, int rows_per_xcd) {
  __shared__ SelShared<kFThreads> sh;
  __shared__ uint32_t craw[kCap];   // candidate score bits
  __shared__ uint32_t cpos[kCap];
  __shared__ uint32_t segstart[kMaxSeg + 1];   // first candidate slot of each segment, then total
  const int t = xcd_item(rows_per_xcd);
  const int tid = threadIdx.x;
  if (t >= num_tokens) return;
  // Segment s of a row is copied by tps threads (kFThreads / nseg rounded
  // down to a power of two, at least 1), each taking every tps-th entry in
  // batches of kBatch loads before any is stored.  The row's span is not
  // known until its position is read, so the counts of the first kFThreads
  // segments and the first batch of each thread's first segment are fetched
  // with it, laid out for a row that fills the stride (the usual case); they
  // are used when the row's layout turns out the same, else fetched again.
  // Slots and counts past the row's own are dropped.
  constexpr int kBatch = 8;
  const uint32_t* seg = ws.seg + static_cast<size_t>(t) * ws.nseg;
  const uint2* cand = ws.cand + static_cast<size_t>(t) * stride;
  int tps_g = 1;
  while (tps_g * 2 * ws.nseg <= kFThreads) tps_g *= 2;
  uint2 pre[kBatch];
  {
    const int s0 = tid / tps_g;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const long long slot = static_cast<long long>(s0) * kSub + tid % tps_g + u * tps_g;
      pre[u] = (s0 < ws.nseg && slot < stride) ? cand[slot] : make_uint2(0u, 0u);
    }
  }
  const uint32_t seg_g = tid < ws.nseg ? seg[tid] : 0u;
  const int n = row_span(rs, t, stride, err, tid == 0);
  const float* row = scores + static_cast<long long>(t) * stride;
  int32_t* out_i = topk_idx + static_cast<long long>(t) * k;
  float* out_v = topk_val ? topk_val + static_cast<long long>(t) * k : nullptr;
  const int m = min(k, n);
  if (m == n) {
    write_all<kFThreads>(n, k, row, out_i, out_v, Remap{rs.remap, rs.rgroup, rs.rstride, t});
  } else {
    int total = 0;
    bool whole_row = false;
    if (n <= kCap) {
      // short row: the row itself is the candidate list
      for (int i = tid; i < n; i += kFThreads) {
        craw[i] = __float_as_uint(row[i]);
        cpos[i] = static_cast<uint32_t>(i);
      }
      total = n;
    } else {
      // candidates: the positions of the keys >= tau, each wave segment's in
      // position order in the slots of its own positions
      const int nseg = ((n + kChunk - 1) / kChunk) * kLWaves;   // <= ws.nseg
      const int spt = (nseg + kFThreads - 1) / kFThreads;
      int tps = 1;
      while (tps * 2 * nseg <= kFThreads) tps *= 2;
      const int s0 = tid / tps;
      if (tps != tps_g) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const long long slot = static_cast<long long>(s0) * kSub + tid % tps + u * tps;
          pre[u] = (s0 < nseg && slot < stride) ? cand[slot] : make_uint2(0u, 0u);
        }
      }
      int mine = 0;
      if (spt == 1) {
        mine = tid < nseg ? static_cast<int>(seg_g) : 0;
      } else {
        for (int i = 0; i < spt; ++i) {
          const int sidx = tid * spt + i;
          if (sidx < nseg) mine += static_cast<int>(seg[sidx]);
        }
      }
      int dst = block_excl_scan<kFThreads / 64>(mine, sh.wsum, &total);
      if (total < m || total > kCap) {
        whole_row = true;   // the sample misled: exact select over the row
      } else {
        if (spt == 1) {
          if (tid < nseg) segstart[tid] = static_cast<uint32_t>(dst);
        } else {
          for (int i = 0; i < spt; ++i) {
            const int sidx = tid * spt + i;
            if (sidx < nseg) {
              segstart[sidx] = static_cast<uint32_t>(dst);
              dst += static_cast<int>(seg[sidx]);
            }
          }
        }
        if (tid == 0) segstart[nseg] = static_cast<uint32_t>(total);
        __syncthreads();
        for (int sidx = s0; sidx < nseg; sidx += kFThreads / tps) {
          const int d0 = static_cast<int>(segstart[sidx]);
          const int c = static_cast<int>(segstart[sidx + 1]) - d0;
          const uint2* src = cand + static_cast<size_t>(sidx) * kSub;
          int q0 = tid % tps;
          if (sidx == s0) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
              const int q = q0 + u * tps;
              if (q < c) {
                craw[d0 + q] = pre[u].x;
                cpos[d0 + q] = pre[u].y;
              }
            }
            q0 += kBatch * tps;
          }
          for (; q0 < c; q0 += kBatch * tps) {
            uint2 e[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
              const int q = q0 + u * tps;
              e[u] = q < c ? src[q] : make_uint2(0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
              const int q = q0 + u * tps;
              if (q < c) {
                craw[d0 + q] = e[u].x;
                cpos[d0 + q] = e[u].y;
              }
            }
          }
        }
      }
    }
    __syncthreads();
    if (whole_row) {
      select_whole_row<kFThreads>(row, n, m, k, out_i, out_v, sh, Remap{rs.remap, rs.rgroup, rs.rstride, t});
    } else {
      const int per = (total + kFThreads - 1) / kFThreads;   // <= kFPer
      const int base = tid * per;
      uint32_t key[kFPer];
#pragma unroll
      for (int j = 0; j < kFPer; ++j)
        key[j] = (j < per && base + j < total) ? order_key(__uint_as_float(craw[base + j])) : 0u;
      const int nmine = max(0, min(per, total - base));
      auto pos = [&](int j) { return static_cast<int>(cpos[base + j]); };
      // the chosen scores come from the candidates' own bits, not the row
      auto val = [&](int j) { return __uint_as_float(craw[base + j]); };
      if (find_cut<kFThreads, kFPer, true>(key, nmine, m, sh, pos))
        emit_cut<kFThreads, kFPer>(key, nmine, m, k, val, out_i, out_v, sh, pos,
                                   Remap{rs.remap, rs.rgroup, rs.rstride, t});
      else
        select_whole_row<kFThreads>(row, n, m, k, out_i, out_v, sh, Remap{rs.remap, rs.rgroup, rs.rstride, t});
    }
  }
}

// Block score of a candidate mask: the best visible score of each group of
// `block` consecutive positions (NaN only when every visible score of the
// block is NaN).  Writes the row's block count for the selection.
__global__ void __launch_bounds__(256) block_max_kernel(
    const float* __restrict__ scores, long long stride, const int32_t* __restrict__ positions,
    int ratio, int block, int num_tokens, float* __restrict__ bs, long long bstride,
    int32_t* __restrict__ counts, int32_t* err) {
  const int t = blockIdx.y;
  if (t >= num_tokens) return;
  long long nv = visible_count(positions[t], ratio);
  if (nv > stride) {
    if (blockIdx.x == 0 && threadIdx.x == 0) flag_error(err, CSA_EFLAG_POS_RANGE);
    nv = stride;
  }
  const long long nb = (nv + block - 1) / block;
  if (blockIdx.x == 0 && threadIdx.x == 0) counts[t] = static_cast<int32_t>(nb);
  const long long j = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= nb) return;
  const long long c0 = j * block;
  const int cnt = static_cast<int>(min(static_cast<long long>(block), nv - c0));
  const float* row = scores + static_cast<long long>(t) * stride + c0;
  float m = __builtin_nanf("");
  if (cnt == block && (block & 3) == 0) {
    for (int i = 0; i < block; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(row + i);
      m = fmaxf(fmaxf(m, v.x), fmaxf(v.y, fmaxf(v.z, v.w)));
    }
  } else {
    for (int i = 0; i < cnt; ++i) m = fmaxf(m, row[i]);
  }
  bs[static_cast<long long>(t) * bstride + j] = m;
}

size_t topk_ws_bytes(int T, long long stride) {
  return (T <= 0 || stride <= kSmallMax) ? 0 : ws_bytes(T, stride);
}

// Launches the selection of the k best entries of each row of `scores`
// (row length `stride`, a multiple of 4, 16-byte aligned).
int launch_topk(const float* scores, long long stride, const RowSpec& rs, int T, int num_tokens,
                int k, int32_t* topk_idx, float* topk_val, void* workspace,
                size_t workspace_bytes, int32_t* err, hipStream_t st) {
  if (reinterpret_cast<uintptr_t>(scores) & 15 || (stride & 3)) return CSA_ERR_UNSUPPORTED;
  if (stride <= 4096) {
    hipLaunchKernelGGL((topk_small_kernel<256, 16>), dim3(num_tokens), dim3(256), 0, st,
                       scores, stride, rs, num_tokens, k, topk_idx, topk_val, err);
  } else if (stride <= 16384) {
    hipLaunchKernelGGL((topk_small_kernel<1024, 16>), dim3(num_tokens), dim3(1024), 0, st,
                       scores, stride, rs, num_tokens, k, topk_idx, topk_val, err);
  } else if (stride <= kSmallMax) {
    hipLaunchKernelGGL((topk_small_kernel<1024, 32>), dim3(num_tokens), dim3(1024), 0, st,
                       scores, stride, rs, num_tokens, k, topk_idx, topk_val, err);
  } else {
    if (stride > kMaxStride || num_tokens > 65535) return CSA_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < ws_bytes(T, stride)) return CSA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 15) return CSA_ERR_UNSUPPORTED;
    const Workspace ws = ws_layout(workspace, T, stride);
    // rows in contiguous runs per XCD: rpx rows, their chunks cpx = rpx * nch
    const long long nch = (stride + kChunk - 1) / kChunk;
    const long long rpx = (num_tokens + 7) / 8;
    const long long cpx = rpx * nch;
    if (8 * cpx > 0x7fffffffll) return CSA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(topk_sample_kernel, dim3(static_cast<unsigned>(8 * rpx)), dim3(kFThreads),
                       0, st, scores, stride, rs, num_tokens, k, ws, static_cast<int>(rpx));
    hipLaunchKernelGGL(topk_filter_kernel, dim3(static_cast<unsigned>(8 * cpx)), dim3(kLThreads),
                       0, st, scores, stride, rs, num_tokens, ws, static_cast<int>(nch),
                       static_cast<int>(cpx));
    hipLaunchKernelGGL(topk_final_kernel, dim3(static_cast<unsigned>(8 * rpx)), dim3(kFThreads),
                       0, st, scores, stride, rs, num_tokens, k, topk_idx, topk_val, ws, err,
                       static_cast<int>(rpx));
  }
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}

// Candidate-mask workspace: block scores [T][bstride], block counts [T]
// (16-byte aligned), then the selection's own workspace.
long long block_stride(long long stride, int block) {
  return ((stride + block - 1) / block + 3) / 4 * 4;
}
size_t cand_ws_head(int T, long long bstride) {
  return (static_cast<size_t>(T) * bstride * 4 + static_cast<size_t>(T) * 4 + 15) / 16 * 16;
}

}  // namespace

}  // namespace csa

extern "C" size_t csa_topk_workspace_bytes(int32_t T, int64_t score_stride, int32_t k) {
  (void)k;
  if (score_stride < 0) return 0;
  return csa::topk_ws_bytes(T, score_stride);
}

extern "C" int csa_topk(const float* scores, int64_t score_stride, const int32_t* positions,
                        int32_t ratio, int32_t T, int32_t num_tokens, int32_t k,
                        int32_t* topk_idx, float* topk_val, void* workspace,
                        size_t workspace_bytes, int32_t* err, void* stream) {
  if (T < 0 || score_stride < 0) return CSA_ERR_SHAPE;
  if (num_tokens < 0 || num_tokens > T || ratio < 1 || k < 1 || k > csa::kMaxK)
    return CSA_ERR_RANGE;
  if (num_tokens == 0) return CSA_OK;
  if (!scores || !positions || !topk_idx) return CSA_ERR_NULL;
  const csa::RowSpec rs{positions, ratio, 1, nullptr, nullptr, 1, 0};
  return csa::launch_topk(scores, score_stride, rs, T, num_tokens, k, topk_idx, topk_val,
                          workspace, workspace_bytes, err, static_cast<hipStream_t>(stream));
}

extern "C" size_t csa_candidate_blocks_workspace_bytes(int32_t T, int64_t score_stride,
                                                       int32_t block, int32_t kb) {
  (void)kb;
  if (T <= 0 || score_stride < 0 || block < 1) return 0;
  const long long bstride = csa::block_stride(score_stride, block);
  return csa::cand_ws_head(T, bstride) + csa::topk_ws_bytes(T, bstride);
}

extern "C" int csa_candidate_blocks(const float* scores, int64_t score_stride,
                                    const int32_t* positions, int32_t ratio, int32_t T,
                                    int32_t num_tokens, int32_t block, int32_t kb,
                                    int32_t* cand_blocks, void* workspace, size_t workspace_bytes,
                                    int32_t* err, void* stream) {
  if (T < 0 || score_stride < 0) return CSA_ERR_SHAPE;
  if (num_tokens < 0 || num_tokens > T || ratio < 1 || block < 1 || block > 128 ||
      (csa::kPage % block) != 0 || kb < 1 || kb > csa::kMaxK)
    return CSA_ERR_RANGE;
  if (num_tokens == 0) return CSA_OK;
  if (!scores || !positions || !cand_blocks) return CSA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(scores) & 15 || (score_stride & 3)) return CSA_ERR_UNSUPPORTED;
  const long long bstride = csa::block_stride(score_stride, block);
  const size_t head = csa::cand_ws_head(T, bstride);
  if (!workspace || workspace_bytes < head + csa::topk_ws_bytes(T, bstride))
    return CSA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return CSA_ERR_UNSUPPORTED;
  float* bs = static_cast<float*>(workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(bs + static_cast<size_t>(T) * bstride);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const long long nb_max = (score_stride + block - 1) / block;
  const dim3 grid(static_cast<unsigned>(std::max<long long>(1, (nb_max + 255) / 256)),
                  static_cast<unsigned>(num_tokens));
  hipLaunchKernelGGL(csa::block_max_kernel, grid, dim3(256), 0, st, scores,
                     static_cast<long long>(score_stride), positions, ratio, block, num_tokens,
                     bs, bstride, counts, err);
  const csa::RowSpec rs{nullptr, 1, 1, counts, nullptr, 1, 0};
  return csa::launch_topk(bs, bstride, rs, T, num_tokens, kb, cand_blocks, nullptr,
                          static_cast<uint8_t*>(workspace) + head, workspace_bytes - head, err,
                          st);
}

extern "C" size_t csa_topk_candidates_workspace_bytes(int32_t T, int64_t cand_stride, int32_t k) {
  (void)k;
  if (cand_stride < 0) return 0;
  return csa::topk_ws_bytes(T, cand_stride);
}

extern "C" int csa_topk_candidates(const float* cand_scores, int64_t cand_stride,
                                   const int32_t* cand_count, const int32_t* cand_blocks,
                                   int32_t kb, int32_t block, int32_t T, int32_t num_tokens,
                                   int32_t k, int32_t* topk_idx, float* topk_val, void* workspace,
                                   size_t workspace_bytes, int32_t* err, void* stream) {
  if (T < 0 || cand_stride < 0) return CSA_ERR_SHAPE;
  if (num_tokens < 0 || num_tokens > T || block < 1 || kb < 1 || k < 1 || k > csa::kMaxK ||
      cand_stride < static_cast<int64_t>(kb) * block)
    return CSA_ERR_RANGE;
  if (num_tokens == 0) return CSA_OK;
  if (!cand_scores || !cand_count || !cand_blocks || !topk_idx) return CSA_ERR_NULL;
  const csa::RowSpec rs{nullptr, 1, 1, cand_count, cand_blocks, block, kb};
  return csa::launch_topk(cand_scores, cand_stride, rs, T, num_tokens, k, topk_idx, topk_val,
                          workspace, workspace_bytes, err, static_cast<hipStream_t>(stream));
}
