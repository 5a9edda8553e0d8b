// Top-k selection of indexer scores.
//
// Contract: pypto-lib "DeepSeek V4.1 Flash", section "Decode composition"
// (eligible positions only, unique, ascending logical positions, trailing -1);
// gitcode hyper-parallel issue #2, section 7.4 (the selection width is capped
// by the number of visible keys).  Ranking is score descending, ties to the
// lower position, NaN last.
//
// Method (one work-group of 1024 threads per query row):
//   1. map each visible score to an order-preserving 32-bit key (the row is
//      held in LDS when it fits, else re-read from L2/HBM per pass);
//   2. radix-select the m-th largest key with four 8-bit digit passes whose
//      256-bin histograms live in LDS; a wave-parallel suffix scan finds the
//      digit holding the m-th key;
//   3. if more keys equal the threshold than are still needed, radix-select
//      the needed count of smallest positions among those ties;
//   4. collect the m chosen positions into LDS and bitonic-sort them ascending.
#include "csa_common.h"

namespace csa {

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kLdsKeysMax = 32768;  // rows up to this width are held in LDS
constexpr int kMaxK = 4096;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: below everything
  if (u == 0x80000000u) u = 0u;                      // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave 0 finds the digit d such that, scanning bins from 255 downward
// (descending=true) or from 0 upward, the running count first reaches `need`.
// Writes d and the count of keys strictly before it in scan order.
__device__ void find_digit(const int* hist, int need, bool descending, int* d_out,
                           int* before_out) {
  const int lane = threadIdx.x & 63;
  int b0 = descending ? (255 - 4 * lane) : (4 * lane);
  int step = descending ? -1 : 1;
  int h[4];
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = hist[b0 + step * i];
    s += h[i];
  }
  // inclusive prefix over lanes in scan order
  int incl = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(incl, off, 64);
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

template <bool kInLds>
__global__ void __launch_bounds__(kTopkThreads) topk_kernel(
    const float* __restrict__ scores, long long stride, const int32_t* __restrict__ positions,
    int ratio, int num_tokens, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_val, int32_t* err) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  __shared__ int hist[256];
  __shared__ int sel_count;
  __shared__ int dig_s, before_s;
  int* sel = reinterpret_cast<int*>(smem);               // [kMaxK]
  uint32_t* keys = smem + kMaxK;                           // [stride] when kInLds

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  if (t >= num_tokens) return;
  const float* row = scores + static_cast<long long>(t) * stride;
  int32_t* out_i = topk_idx + static_cast<long long>(t) * k;
  float* out_v = topk_val ? topk_val + static_cast<long long>(t) * k : nullptr;

  long long nv = visible_count(positions[t], ratio);
  if (nv > stride) {
    if (tid == 0) flag_error(err, CSA_EFLAG_POS_RANGE);
    nv = stride;
  }
  const int n = static_cast<int>(nv);
  const int m = min(k, n);
  const float neg_inf = -__builtin_huge_valf();

  if (m == n) {  // every visible position is chosen, already ascending
    for (int i = tid; i < k; i += kTopkThreads) {
      out_i[i] = i < n ? i : -1;
      if (out_v) out_v[i] = i < n ? row[i] : neg_inf;
    }
    return;
  }

  if (kInLds) {
    for (int c = tid; c < n; c += kTopkThreads) keys[c] = order_key(row[c]);
  }
  auto key_at = [&](int c) -> uint32_t { return kInLds ? keys[c] : order_key(row[c]); };

  // ---- radix select of the m-th largest key
  uint32_t prefix = 0, mask = 0;
  int rem = m;
  int ties = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int c = tid; c < n; c += kTopkThreads) {
      uint32_t kk = key_at(c);
      if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid < 64) find_digit(hist, rem, true, &dig_s, &before_s);
    __syncthreads();
    const int d = dig_s;
    rem -= before_s;
    ties = hist[d];
    prefix |= static_cast<uint32_t>(d) << shift;
    mask |= 0xffu << shift;
    __syncthreads();
  }
  const uint32_t tau = prefix;  // key of the m-th largest; rem ties of it are taken

  // ---- among keys equal to tau take the rem lowest positions
  uint32_t pos_limit = 0xffffffffu;
  if (ties > rem) {
    uint32_t pprefix = 0, pmask = 0;
    int prem = rem;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int c = tid; c < n; c += kTopkThreads) {
        uint32_t uc = static_cast<uint32_t>(c);
        if (key_at(c) == tau && (uc & pmask) == pprefix) atomicAdd(&hist[(uc >> shift) & 255], 1);
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

  // ---- collect the m chosen positions
  if (tid == 0) sel_count = 0;
  __syncthreads();
  for (int c = tid; c < n; c += kTopkThreads) {
    uint32_t kk = key_at(c);
    if (kk > tau || (kk == tau && static_cast<uint32_t>(c) <= pos_limit)) {
      int slot = atomicAdd(&sel_count, 1);
      if (slot < kMaxK) sel[slot] = c;
    }
  }
  __syncthreads();
  // ---- bitonic sort ascending over the next power of two
  int P = 1;
  while (P < m) P <<= 1;
  for (int i = m + tid; i < P; i += kTopkThreads) sel[i] = 0x7fffffff;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int j = size >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < (P >> 1); i += kTopkThreads) {
        int lo = 2 * i - (i & (j - 1));
        int hi = lo + j;
        bool up = ((lo & size) == 0);
        int a = sel[lo], b = sel[hi];
        if ((a > b) == up) {
          sel[lo] = b;
          sel[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < k; i += kTopkThreads) {
    int c = i < m ? sel[i] : -1;
    out_i[i] = c;
    if (out_v) out_v[i] = c >= 0 ? row[c] : neg_inf;
  }
}

}  // namespace

}  // namespace csa

extern "C" size_t csa_topk_workspace_bytes(int32_t T, int64_t score_stride, int32_t k) {
  (void)T;
  (void)score_stride;
  (void)k;
  return 0;
}

extern "C" int csa_topk(const float* scores, int64_t score_stride, const int32_t* positions,
                        int32_t ratio, int32_t T, int32_t num_tokens, int32_t k,
                        int32_t* topk_idx, float* topk_val, void* workspace,
                        size_t workspace_bytes, int32_t* err, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (T < 0 || score_stride < 0) return CSA_ERR_SHAPE;
  if (num_tokens < 0 || num_tokens > T || ratio < 1 || k < 1 || k > csa::kMaxK)
    return CSA_ERR_RANGE;
  if (num_tokens == 0) return CSA_OK;
  if (!scores || !positions || !topk_idx) return CSA_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (score_stride <= csa::kLdsKeysMax) {
    size_t lds = (csa::kMaxK + static_cast<size_t>(score_stride)) * sizeof(uint32_t);
    static bool attr_set = false;
    if (!attr_set) {
      hipFuncSetAttribute(reinterpret_cast<const void*>(&csa::topk_kernel<true>),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>((csa::kMaxK + csa::kLdsKeysMax) * sizeof(uint32_t)));
      attr_set = true;
    }
    hipLaunchKernelGGL(csa::topk_kernel<true>, dim3(num_tokens), dim3(csa::kTopkThreads), lds,
                       st, scores, static_cast<long long>(score_stride), positions, ratio,
                       num_tokens, k, topk_idx, topk_val, err);
  } else {
    size_t lds = csa::kMaxK * sizeof(uint32_t);
    hipLaunchKernelGGL(csa::topk_kernel<false>, dim3(num_tokens), dim3(csa::kTopkThreads), lds,
                       st, scores, static_cast<long long>(score_stride), positions, ratio,
                       num_tokens, k, topk_idx, topk_val, err);
  }
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}
