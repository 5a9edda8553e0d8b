// Top-k selection of indexer scores.
//
// Contract: pypto-lib "DeepSeek V4.1 Flash", section "Decode composition"
// (eligible positions only, unique, ascending logical positions, trailing -1);
// gitcode hyper-parallel issue #2, section 7.4 (the selection width is capped
// by the number of visible keys).  Ranking is score descending, ties to the
// lower position, NaN last (scores map to order-preserving 32-bit keys).
//
// Short rows (visible span <= 32,768): one work-group of 1024 threads per row.
// Each thread holds a contiguous run of up to 32 keys in registers; an
// MSB-first radix select (8-bit digits, per-wave LDS histograms, stopping as
// soon as the threshold digit holds exactly the count still needed) finds the
// cut; a block scan in position order then writes the chosen positions
// already ascending -- no sort.
//
// Long rows (up to the 1,048,576-position context): three kernels over the
// row, which the indexer has just left in L2 / Infinity Cache.
//   hist:   work-groups over 8,192-score chunks add a 4,096-bin histogram of
//           the top 12 key bits into the row's global histogram; the last
//           work-group of a row (device-scope counter) finds the 12-bit bin
//           that holds the k-th key, records it, and clears the histogram.
//   filter: work-groups over chunks append every key in or above that bin
//           (typically ~k + a few hundred) to the row's candidate list.
//   final:  one work-group per row loads the candidates into LDS, radix
//           selects the exact cut (ties by position), bitonic-sorts the chosen
//           positions and clears the row's counters.
// The histogram and counters of the workspace are zero on first use and every
// call leaves them zero again; candidate slots are always written before read.
#include "csa_common.h"

namespace csa {

namespace {

constexpr int kMaxK = 4096;
constexpr int kSmallMax = 32768;     // rows up to this span take the one-group path
constexpr int kSThreads = 1024;
constexpr int kSPer = kSmallMax / kSThreads;  // keys per thread
constexpr int kBins = 4096;          // 12-bit first-level histogram
constexpr int kChunk = 8192;         // scores per work-group in hist / filter
constexpr int kLThreads = 256;
constexpr int kCap = 8192;           // candidate slots per row
constexpr int kMetaWords = 8;        // done counter, candidate count, bin, above, ...
constexpr int kPerThread4 = kChunk / (4 * kLThreads);  // float4 loads per thread

struct Workspace {
  uint32_t* hist;   // [T][kBins]
  uint32_t* meta;   // [T][kMetaWords]
  uint2* cand;      // [T][kCap] (key, position)
};

__host__ __device__ inline size_t ws_bytes(int T) {
  return static_cast<size_t>(T) * (kBins + kMetaWords) * sizeof(uint32_t) +
         static_cast<size_t>(T) * kCap * sizeof(uint2);
}

__host__ __device__ inline Workspace ws_layout(void* base, int T) {
  Workspace w;
  w.hist = static_cast<uint32_t*>(base);
  w.meta = w.hist + static_cast<size_t>(T) * kBins;
  w.cand = reinterpret_cast<uint2*>(w.meta + static_cast<size_t>(T) * kMetaWords);
  return w;
}

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: below everything
  if (u == 0x80000000u) u = 0u;                      // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int row_span(const int32_t* positions, int t, int ratio,
                                        long long stride, int32_t* err, bool report) {
  long long nv = visible_count(positions[t], ratio);
  if (nv > stride) {
    if (report) flag_error(err, CSA_EFLAG_POS_RANGE);
    nv = stride;
  }
  return static_cast<int>(nv);
}

// Wave 0 finds the digit d such that, scanning `nb` bins (4 per lane) from the
// top (descending) or bottom, the running count first reaches `need`; writes
// d and the count strictly before it.
__device__ void find_digit(const uint32_t* hist, int need, bool descending, int* d_out,
                           int* before_out) {
  const int lane = threadIdx.x & 63;
  const int b0 = descending ? (255 - 4 * lane) : (4 * lane);
  const int step = descending ? -1 : 1;
  int h[4];
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = static_cast<int>(hist[b0 + step * i]);
    s += h[i];
  }
  int incl = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  int run = incl - s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (run < need && run + h[i] >= need) {
      *d_out = b0 + step * i;
      *before_out = run;
    }
    run += h[i];
  }
}

// Exclusive scan over a work-group of nwaves*64 threads; `wsum` holds nwaves ints.
__device__ int block_excl_scan(int v, int* wsum, int nwaves, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < nwaves; ++w) {
    const int s = wsum[w];
    if (w < wave) before += s;
    tot += s;
  }
  if (total) *total = tot;
  return before + incl - v;
}

// ----------------------------------------------------------------------------
// short rows: one work-group, keys in registers
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(kSThreads) topk_small_kernel(
    const float* __restrict__ scores, long long stride, const int32_t* __restrict__ positions,
    int ratio, int num_tokens, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_val, int32_t* err, int skip_long) {
  __shared__ uint32_t hist[kSThreads / 64][256];
  __shared__ uint32_t total[256];
  __shared__ int wsum[kSThreads / 64];
  __shared__ int dig_s, before_s;

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  if (t >= num_tokens) return;
  const int n = row_span(positions, t, ratio, stride, err, tid == 0);
  if (skip_long && n > kSmallMax) return;
  const float* row = scores + static_cast<long long>(t) * stride;
  int32_t* out_i = topk_idx + static_cast<long long>(t) * k;
  float* out_v = topk_val ? topk_val + static_cast<long long>(t) * k : nullptr;
  const int m = min(k, n);
  const float neg_inf = -__builtin_huge_valf();
  if (m == n) {  // every visible position is chosen, already ascending
    for (int i = tid; i < k; i += kSThreads) {
      out_i[i] = i < n ? i : -1;
      if (out_v) out_v[i] = i < n ? row[i] : neg_inf;
    }
    return;
  }

  // contiguous run per thread, a multiple of 4 keys so loads are 16 bytes
  const int per = 4 * ((n + 4 * kSThreads - 1) / (4 * kSThreads));
  const int base = tid * per;
  uint32_t key[kSPer];
#pragma unroll
  for (int j = 0; j < kSPer; j += 4) {
    if (j < per) {
      const int c = base + j;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c + 3 < n) {
        v = *reinterpret_cast<const float4*>(row + c);
      } else {
        if (c < n) v.x = row[c];
        if (c + 1 < n) v.y = row[c + 1];
        if (c + 2 < n) v.z = row[c + 2];
      }
      key[j] = order_key(v.x);
      key[j + 1] = order_key(v.y);
      key[j + 2] = order_key(v.z);
      key[j + 3] = order_key(v.w);
    }
  }
  const int nmine = max(0, min(per, n - base));

  for (int i = tid; i < (kSThreads / 64) * 256; i += kSThreads) (&hist[0][0])[i] = 0;
  __syncthreads();

  uint32_t prefix = 0, mask = 0;
  int rem = m;
  bool exact = false;   // threshold digit holds exactly the needed count
  int cnt_d = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int j = 0; j < kSPer; ++j)
      if (j < nmine && (key[j] & mask) == prefix) atomicAdd(&hist[wave][(key[j] >> shift) & 255], 1u);
    __syncthreads();
    if (tid < 256) {
      uint32_t s = 0;
#pragma unroll
      for (int w = 0; w < kSThreads / 64; ++w) {
        s += hist[w][tid];
        hist[w][tid] = 0;
      }
      total[tid] = s;
    }
    __syncthreads();
    if (tid < 64) find_digit(total, rem, true, &dig_s, &before_s);
    __syncthreads();
    const int d = dig_s;
    rem -= before_s;
    cnt_d = static_cast<int>(total[d]);
    prefix |= static_cast<uint32_t>(d) << shift;
    mask |= 0xffu << shift;
    if (cnt_d == rem) {
      exact = true;
      break;
    }
  }
  // chosen: (key & mask) > prefix, plus keys equal to the threshold -- all of
  // them when exact, else the rem lowest positions among them
  int gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < kSPer; ++j) {
    if (j < nmine) {
      const uint32_t km = key[j] & mask;
      gt += km > prefix;
      eq += km == prefix;
    }
  }
  int take = eq;
  if (!exact) {
    const int eq_before = block_excl_scan(eq, wsum, kSThreads / 64, nullptr);
    take = max(0, min(eq, rem - eq_before));
  }
  const int off = block_excl_scan(gt + take, wsum, kSThreads / 64, nullptr);
  int o = off, taken = 0;
#pragma unroll
  for (int j = 0; j < kSPer; ++j) {
    if (j < nmine) {
      const uint32_t km = key[j] & mask;
      bool pick = km > prefix;
      if (km == prefix && taken < take) {
        pick = true;
        ++taken;
      }
      if (pick) {
        const int c = base + j;
        out_i[o] = c;
        if (out_v) out_v[o] = row[c];
        ++o;
      }
    }
  }
  for (int i = m + tid; i < k; i += kSThreads) {
    out_i[i] = -1;
    if (out_v) out_v[i] = neg_inf;
  }
}

// ----------------------------------------------------------------------------
// long rows: histogram + threshold bin
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(kLThreads) topk_hist_kernel(
    const float* __restrict__ scores, long long stride, const int32_t* __restrict__ positions,
    int ratio, int num_tokens, int k, Workspace ws, int32_t* err) {
  __shared__ uint32_t hist[kBins];
  __shared__ int last_s;
  __shared__ int wsum[kLThreads / 64];
  const int t = blockIdx.y;
  const int tid = threadIdx.x;
  if (t >= num_tokens) return;
  const int n = row_span(positions, t, ratio, stride, err, blockIdx.x == 0 && tid == 0);
  if (n <= kSmallMax) return;
  const float* row = scores + static_cast<long long>(t) * stride;
  for (int i = tid; i < kBins; i += kLThreads) hist[i] = 0;
  // issue all of this thread's loads before touching the histogram
  const int c0 = blockIdx.x * kChunk;
  const int c1 = min(n, c0 + kChunk);
  float4 v[kPerThread4];
#pragma unroll
  for (int i = 0; i < kPerThread4; ++i) {
    const int c = c0 + 4 * (tid + kLThreads * i);
    if (c + 3 < c1) {
      v[i] = *reinterpret_cast<const float4*>(row + c);
    } else {
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < c1) v[i].x = row[c];
      if (c + 1 < c1) v[i].y = row[c + 1];
      if (c + 2 < c1) v[i].z = row[c + 2];
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPerThread4; ++i) {
    const int c = c0 + 4 * (tid + kLThreads * i);
    if (c < c1) atomicAdd(&hist[order_key(v[i].x) >> 20], 1u);
    if (c + 1 < c1) atomicAdd(&hist[order_key(v[i].y) >> 20], 1u);
    if (c + 2 < c1) atomicAdd(&hist[order_key(v[i].z) >> 20], 1u);
    if (c + 3 < c1) atomicAdd(&hist[order_key(v[i].w) >> 20], 1u);
  }
  __syncthreads();
  uint32_t* gh = ws.hist + static_cast<size_t>(t) * kBins;
  uint32_t* meta = ws.meta + static_cast<size_t>(t) * kMetaWords;
  for (int i = tid; i < kBins; i += kLThreads)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
  __threadfence();
  __syncthreads();
  if (tid == 0) last_s = (atomicAdd(&meta[0], 1u) == gridDim.x - 1);
  __syncthreads();
  if (!last_s) return;
  __threadfence();
  // this work-group is the row's last: find the bin holding the m-th key
  const int m = min(k, n);
  constexpr int kPerT = kBins / kLThreads;  // 16 bins per thread, from the top
  uint32_t h[kPerT];
  int s = 0;
#pragma unroll
  for (int i = 0; i < kPerT; ++i) {
    const int b = kBins - 1 - (tid * kPerT + i);
    h[i] = __hip_atomic_load(&gh[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s += static_cast<int>(h[i]);
  }
  const int before = block_excl_scan(s, wsum, kLThreads / 64, nullptr);
  int run = before;
#pragma unroll
  for (int i = 0; i < kPerT; ++i) {
    if (run < m && run + static_cast<int>(h[i]) >= m) {
      meta[2] = static_cast<uint32_t>(kBins - 1 - (tid * kPerT + i));  // threshold bin
      meta[3] = static_cast<uint32_t>(run);                            // keys above it
    }
    run += static_cast<int>(h[i]);
  }
  for (int i = tid; i < kBins; i += kLThreads) gh[i] = 0;
  if (tid == 0) meta[0] = 0;
}

// ----------------------------------------------------------------------------
// long rows: keep every key in or above the threshold bin
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(kLThreads) topk_filter_kernel(
    const float* __restrict__ scores, long long stride, const int32_t* __restrict__ positions,
    int ratio, int num_tokens, Workspace ws) {
  const int t = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  if (t >= num_tokens) return;
  const int n = row_span(positions, t, ratio, stride, nullptr, false);
  if (n <= kSmallMax) return;
  const int c0 = blockIdx.x * kChunk;
  if (c0 >= n) return;
  const int c1 = min(n, c0 + kChunk);
  const float* row = scores + static_cast<long long>(t) * stride;
  uint32_t* meta = ws.meta + static_cast<size_t>(t) * kMetaWords;
  uint2* cand = ws.cand + static_cast<size_t>(t) * kCap;
  const uint32_t bin = meta[2];
  uint32_t key[4 * kPerThread4];
  int keep = 0;
#pragma unroll
  for (int i = 0; i < kPerThread4; ++i) {
    const int c = c0 + 4 * (tid + kLThreads * i);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c + 3 < c1) {
      v = *reinterpret_cast<const float4*>(row + c);
    } else {
      if (c < c1) v.x = row[c];
      if (c + 1 < c1) v.y = row[c + 1];
      if (c + 2 < c1) v.z = row[c + 2];
    }
    key[4 * i] = order_key(v.x);
    key[4 * i + 1] = order_key(v.y);
    key[4 * i + 2] = order_key(v.z);
    key[4 * i + 3] = order_key(v.w);
  }
#pragma unroll
  for (int j = 0; j < 4 * kPerThread4; ++j) {
    const int c = c0 + 4 * (tid + kLThreads * (j >> 2)) + (j & 3);
    keep += (c < c1 && (key[j] >> 20) >= bin) ? 1 : 0;
  }
  // one device atomic per wave: in-wave exclusive prefix of the keep counts
  int incl = keep;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  const int wave_total = __shfl(incl, 63, 64);
  if (wave_total == 0) return;
  uint32_t base = 0;
  if (lane == 63) base = atomicAdd(&meta[1], static_cast<uint32_t>(wave_total));
  base = __shfl(base, 63, 64);
  uint32_t slot = base + static_cast<uint32_t>(incl - keep);
#pragma unroll
  for (int j = 0; j < 4 * kPerThread4; ++j) {
    const int c = c0 + 4 * (tid + kLThreads * (j >> 2)) + (j & 3);
    if (c < c1 && (key[j] >> 20) >= bin) {
      if (slot < static_cast<uint32_t>(kCap)) cand[slot] = make_uint2(key[j], static_cast<uint32_t>(c));
      ++slot;
    }
  }
}

// ----------------------------------------------------------------------------
// long rows: exact cut among the candidates (or the whole row if they overflowed)
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(kSThreads) topk_final_kernel(
    const float* __restrict__ scores, long long stride, const int32_t* __restrict__ positions,
    int ratio, int num_tokens, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_val, Workspace ws) {
  __shared__ uint32_t ckey[kCap];
  __shared__ uint32_t cpos[kCap];
  __shared__ uint32_t hist[256];
  __shared__ int sel[kMaxK];
  __shared__ int sel_count;
  __shared__ int dig_s, before_s;

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  if (t >= num_tokens) return;
  const int n = row_span(positions, t, ratio, stride, nullptr, false);
  if (n <= kSmallMax) return;
  const float* row = scores + static_cast<long long>(t) * stride;
  int32_t* out_i = topk_idx + static_cast<long long>(t) * k;
  float* out_v = topk_val ? topk_val + static_cast<long long>(t) * k : nullptr;
  uint32_t* meta = ws.meta + static_cast<size_t>(t) * kMetaWords;
  const uint2* cand = ws.cand + static_cast<size_t>(t) * kCap;
  const int m = min(k, n);
  const int ncand = static_cast<int>(meta[1]);
  const bool in_lds = ncand <= kCap;
  const int nc = in_lds ? ncand : n;   // candidates, or the whole row on overflow
  if (in_lds) {
    for (int i = tid; i < nc; i += kSThreads) {
      const uint2 e = cand[i];
      ckey[i] = e.x;
      cpos[i] = e.y;
    }
  }
  __syncthreads();
  auto key_at = [&](int i) -> uint32_t { return in_lds ? ckey[i] : order_key(row[i]); };
  auto pos_at = [&](int i) -> uint32_t { return in_lds ? cpos[i] : static_cast<uint32_t>(i); };

  uint32_t prefix = 0, mask = 0;
  int rem = m, cnt_d = 0;
  bool exact = false;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < nc; i += kSThreads) {
      const uint32_t kk = key_at(i);
      if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & 255], 1u);
    }
    __syncthreads();
    if (tid < 64) find_digit(hist, rem, true, &dig_s, &before_s);
    __syncthreads();
    const int d = dig_s;
    rem -= before_s;
    cnt_d = static_cast<int>(hist[d]);
    prefix |= static_cast<uint32_t>(d) << shift;
    mask |= 0xffu << shift;
    __syncthreads();
    if (cnt_d == rem) {
      exact = true;
      break;
    }
  }
  // ties beyond the need: keep the rem lowest positions among them
  uint32_t pos_limit = 0xffffffffu;
  if (!exact) {
    uint32_t pprefix = 0, pmask = 0;
    int prem = rem;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < nc; i += kSThreads) {
        const uint32_t p = pos_at(i);
        if ((key_at(i) & mask) == prefix && (p & pmask) == pprefix)
          atomicAdd(&hist[(p >> shift) & 255], 1u);
      }
      __syncthreads();
      if (tid < 64) find_digit(hist, prem, false, &dig_s, &before_s);
      __syncthreads();
      prem -= before_s;
      pprefix |= static_cast<uint32_t>(dig_s) << shift;
      pmask |= 0xffu << shift;
      __syncthreads();
    }
    pos_limit = pprefix;
  }
  if (tid == 0) sel_count = 0;
  __syncthreads();
  for (int i = tid; i < nc; i += kSThreads) {
    const uint32_t km = key_at(i) & mask;
    if (km > prefix || (km == prefix && pos_at(i) <= pos_limit)) {
      const int slot = atomicAdd(&sel_count, 1);
      if (slot < kMaxK) sel[slot] = static_cast<int>(pos_at(i));
    }
  }
  __syncthreads();
  int P = 1;
  while (P < m) P <<= 1;
  for (int i = m + tid; i < P; i += kSThreads) sel[i] = 0x7fffffff;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int j = size >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < (P >> 1); i += kSThreads) {
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
  for (int i = tid; i < k; i += kSThreads) {
    const int c = i < m ? sel[i] : -1;
    out_i[i] = c;
    if (out_v) out_v[i] = c >= 0 ? row[c] : neg_inf;
  }
  if (tid == 0) {
    meta[1] = 0;
    meta[2] = 0;
    meta[3] = 0;
  }
}

}  // namespace

}  // namespace csa

extern "C" size_t csa_topk_workspace_bytes(int32_t T, int64_t score_stride, int32_t k) {
  (void)k;
  if (T <= 0 || score_stride <= csa::kSmallMax) return 0;
  return csa::ws_bytes(T);
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
  if (reinterpret_cast<uintptr_t>(scores) & 15 || (score_stride & 3)) return CSA_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool long_rows = score_stride > csa::kSmallMax;
  if (long_rows) {
    if (!workspace || workspace_bytes < csa::ws_bytes(T)) return CSA_ERR_WORKSPACE;
    const csa::Workspace ws = csa::ws_layout(workspace, T);
    const long long chunks = (score_stride + csa::kChunk - 1) / csa::kChunk;
    if (chunks > 0x7fffffffll || num_tokens > 65535) return CSA_ERR_UNSUPPORTED;
    const dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(num_tokens));
    hipLaunchKernelGGL(csa::topk_hist_kernel, grid, dim3(csa::kLThreads), 0, st, scores,
                       static_cast<long long>(score_stride), positions, ratio, num_tokens, k, ws,
                       err);
    hipLaunchKernelGGL(csa::topk_filter_kernel, grid, dim3(csa::kLThreads), 0, st, scores,
                       static_cast<long long>(score_stride), positions, ratio, num_tokens, ws);
    hipLaunchKernelGGL(csa::topk_final_kernel, dim3(num_tokens), dim3(csa::kSThreads), 0, st,
                       scores, static_cast<long long>(score_stride), positions, ratio,
                       num_tokens, k, topk_idx, topk_val, ws);
  }
  hipLaunchKernelGGL(csa::topk_small_kernel, dim3(num_tokens), dim3(csa::kSThreads), 0, st,
                     scores, static_cast<long long>(score_stride), positions, ratio, num_tokens,
                     k, topk_idx, topk_val, long_rows ? nullptr : err, long_rows ? 1 : 0);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}
