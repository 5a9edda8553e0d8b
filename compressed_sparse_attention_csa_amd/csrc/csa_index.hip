// Lightning-indexer scores on CDNA4 INT8 MFMA.
//
// Method: gitcode hyper-parallel issue #2 (DeepSeek V4 CP notes), sections
// 10.2 / 10.3 -- per query row, score every causally visible compressed slot
// c < (p+1)/ratio with the indexer; pypto-lib "DeepSeek V4-Flash, MTP point",
// section "What is quantized" -- index keys are INT8 with an FP32 per-row
// scale.  Score = sum_h w[t,h] * relu(qs[t,h] * ks[c] * <q8[t,h], k8[c]>).
//
// Mapping.  Work-groups are (request, up to 4 of its rows) x (a run of
// 128-key pages); wave w owns one query row and computes its heads as 16-row
// MFMA tiles (M = heads, N = keys, K = Di), so a key page staged once in LDS
// feeds every row of the group.  The block ids of the run's pages are read up
// front, and while a page is scored from LDS the next page is already on its
// way into registers (software pipelining), so HBM latency overlaps the MFMA
// and epilogue work.  LDS rows are 128 bytes with XOR-swizzled 16-byte chunks
// (conflict-free MFMA operand reads).  INT32 accumulators stay in registers:
// the epilogue applies ReLU, the folded weight w*qs, reduces the heads (16 in
// lane, then across the four 16-lane groups) and scales by ks.  Pages past
// every row's visible span only receive -inf.
#include "csa_common.h"

namespace csa {

namespace {

constexpr int kRowsPerWG = 4;
constexpr int kThreads = 256;
constexpr int kRowBytes = 128;   // LDS bytes per key (Di <= 128, zero padded)
constexpr int kMaxPPW = 16;      // pages per work-group
constexpr int kChunksPerThread = (kPage * 8) / kThreads;  // 16-byte chunks staged per thread

__device__ __forceinline__ int swz_chunk(int key, int chunk) {
  return chunk ^ ((key >> 1) & 7);
}

// Work-group y -> (request, first row) with groups of up to 4 rows that never
// straddle two requests.  Returns the request or -1 (past the last group).
__device__ int locate_group(const int32_t* __restrict__ qsl, int B, int num_tokens, int g,
                            int* row0, int* nrows, int* scratch /*[kThreads/64 + 2]*/) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int carry = 0;
  for (int base = 0; base < B; base += kThreads) {
    const int b = base + tid;
    int groups = 0;
    if (b < B) {
      const int lo = min(max(qsl[b], 0), num_tokens);
      const int hi = min(max(qsl[b + 1], 0), num_tokens);
      groups = hi > lo ? (hi - lo + kRowsPerWG - 1) / kRowsPerWG : 0;
    }
    int incl = groups;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    __syncthreads();
    if (lane == 63) scratch[wave] = incl;
    if (tid == 0) scratch[kThreads / 64] = -1;
    __syncthreads();
    int before = carry, total = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      if (w < wave) before += scratch[w];
      total += scratch[w];
    }
    const int first = before + incl - groups;  // this request's first group id
    if (b < B && groups > 0 && g >= first && g < first + groups) {
      scratch[kThreads / 64] = b;
      scratch[kThreads / 64 + 1] = min(max(qsl[b], 0), num_tokens) + (g - first) * kRowsPerWG;
    }
    __syncthreads();
    const int found = scratch[kThreads / 64];
    if (found >= 0) {
      *row0 = scratch[kThreads / 64 + 1];
      *nrows = min(kRowsPerWG, min(max(qsl[found + 1], 0), num_tokens) - *row0);
      return found;
    }
    carry += total;
  }
  return -1;
}

template <int KK>
__global__ void __launch_bounds__(kThreads) index_score_kernel(
    const int8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ head_w, const int8_t* __restrict__ idx_kv,
    const float* __restrict__ idx_scale, int num_blocks, const int32_t* __restrict__ bt,
    int max_blocks, const int32_t* __restrict__ qsl, const int32_t* __restrict__ positions,
    int B, int num_tokens, int Hi, int Di, int ratio, float* __restrict__ scores,
    long long stride, int pages_per_wg, int32_t* err) {
  __shared__ __attribute__((aligned(16))) int8_t keys_s[2][kPage * kRowBytes];
  __shared__ float ks_s[2][kPage];
  __shared__ int blk_s[kMaxPPW];
  __shared__ int nvis_s[kRowsPerWG];
  __shared__ int scratch[kThreads / 64 + 2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const long long stride_pages = (stride + kPage - 1) / kPage;
  const int page0 = blockIdx.x * pages_per_wg;
  const int npages = static_cast<int>(min(static_cast<long long>(pages_per_wg),
                                          stride_pages - page0));
  if (npages <= 0) return;

  int row0 = 0, nrows = 0;
  const int b = locate_group(qsl, B, num_tokens, blockIdx.y, &row0, &nrows, scratch);
  if (b < 0) {
    // rows that no request owns: the first groups past the owned ones cover them
    const int owned_end = (B > 0) ? min(max(qsl[B], 0), num_tokens) : 0;
    const int owned_begin = (B > 0) ? min(max(qsl[0], 0), num_tokens) : 0;
    // enumerate unowned rows in blocks of 4 after the owned groups
    int gfirst = 0;
    for (int bb = 0; bb < B; ++bb) {
      const int lo = min(max(qsl[bb], 0), num_tokens);
      const int hi = min(max(qsl[bb + 1], 0), num_tokens);
      gfirst += hi > lo ? (hi - lo + kRowsPerWG - 1) / kRowsPerWG : 0;
    }
    const int u = blockIdx.y - gfirst;  // index among unowned 4-row blocks
    const int n_unowned = owned_begin + (num_tokens - owned_end);
    if (u < 0 || u * kRowsPerWG >= n_unowned) return;
    const float neg_inf = -__builtin_huge_valf();
    for (int r = 0; r < kRowsPerWG; ++r) {
      const int j = u * kRowsPerWG + r;
      if (j >= n_unowned) break;
      const int t = j < owned_begin ? j : owned_end + (j - owned_begin);
      if (blockIdx.x == 0 && tid == 0) flag_error(err, CSA_EFLAG_META);
      float* out_row = scores + static_cast<long long>(t) * stride;
      for (int c = page0 * kPage + tid; c < (page0 + npages) * kPage; c += kThreads)
        if (c < stride) out_row[c] = neg_inf;
    }
    return;
  }

  if (tid < kRowsPerWG) {
    int n = 0;
    if (tid < nrows) {
      n = visible_count(positions[row0 + tid], ratio);
      const long long cap = static_cast<long long>(max_blocks) * kPage;
      if (static_cast<long long>(n) > stride || static_cast<long long>(n) > cap) {
        if (blockIdx.x == 0) flag_error(err, CSA_EFLAG_POS_RANGE);
        const long long m = stride < cap ? stride : cap;
        if (static_cast<long long>(n) > m) n = static_cast<int>(m);
      }
    }
    nvis_s[tid] = n;
  }
  __syncthreads();
  int nmax = 0;
  for (int r = 0; r < nrows; ++r) nmax = max(nmax, nvis_s[r]);
  // block ids of this run's pages (-1: nothing to stage)
  if (tid < npages) {
    const int page = page0 + tid;
    int blk = -1;
    if (page * kPage < nmax) {
      blk = (page < max_blocks) ? bt[static_cast<long long>(b) * max_blocks + page] : -1;
      if (blk < 0 || blk >= num_blocks) {
        flag_error(err, CSA_EFLAG_BLOCK_RANGE);
        blk = -1;
      }
    }
    blk_s[tid] = blk;
  }

  const bool active = wave < nrows;
  const int my_t = row0 + wave;
  const int my_n = nvis_s[wave];
  const int col = lane & 15;
  const int grp = lane >> 4;

  // A operand (this wave's query row) and folded head weights, loaded once
  constexpr int MT = 4;
  v4i qa[MT][KK];
  float ww[MT][4];
  if (active) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = mt * 16 + col;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int off = kk * 64 + grp * 16;
        qa[mt][kk] = (h < Hi && off < Di)
                         ? *reinterpret_cast<const v4i*>(
                               q_idx + (static_cast<long long>(my_t) * Hi + h) * Di + off)
                         : v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hh = mt * 16 + grp * 4 + r;
        ww[mt][r] = (hh < Hi) ? head_w[static_cast<long long>(my_t) * Hi + hh] *
                                    q_scale[static_cast<long long>(my_t) * Hi + hh]
                              : 0.0f;
      }
    }
  }
  __syncthreads();  // blk_s ready

  // staging helpers: thread -> (key, chunk) pairs of one page
  v4i pre[kChunksPerThread];
  float pre_ks = 0.0f;
  auto fetch = [&](int pi) {
    const int blk = blk_s[pi];
    if (blk < 0) return;
    const int8_t* src = idx_kv + static_cast<long long>(blk) * kPage * Di;
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
      const int ch = tid + u * kThreads;
      const int key = ch >> 3, c = ch & 7;
      pre[u] = (c * 16 < Di) ? *reinterpret_cast<const v4i*>(src + key * Di + c * 16)
                             : v4i{0, 0, 0, 0};
    }
    if (tid < kPage) pre_ks = idx_scale[static_cast<long long>(blk) * kPage + tid];
  };
  auto store = [&](int pi, int buf) {
    if (blk_s[pi] < 0) return;
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
      const int ch = tid + u * kThreads;
      const int key = ch >> 3, c = ch & 7;
      *reinterpret_cast<v4i*>(&keys_s[buf][key * kRowBytes + swz_chunk(key, c) * 16]) = pre[u];
    }
    if (tid < kPage) ks_s[buf][tid] = pre_ks;
  };

  const float neg_inf = -__builtin_huge_valf();
  fetch(0);
  store(0, 0);
  if (npages > 1) fetch(1);
  __syncthreads();
  for (int pi = 0; pi < npages; ++pi) {
    const int buf = pi & 1;
    const int c0 = (page0 + pi) * kPage;
    const bool staged = blk_s[pi] >= 0;
    if (active) {
      float* out_row = scores + static_cast<long long>(my_t) * stride;
#pragma unroll 2
      for (int s = 0; s < kPage / 16; ++s) {
        const int kj = s * 16 + col;
        const int c = c0 + kj;
        float sc = neg_inf;
        if (staged && c0 + s * 16 < my_n) {
          v4i bk[KK];
#pragma unroll
          for (int kk = 0; kk < KK; ++kk)
            bk[kk] = *reinterpret_cast<const v4i*>(
                &keys_s[buf][kj * kRowBytes + swz_chunk(kj, kk * 4 + grp) * 16]);
          float x = 0.0f;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            v4i acc = v4i{0, 0, 0, 0};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
              acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[mt][kk], bk[kk], acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              x = fmaf(ww[mt][r], static_cast<float>(max(acc[r], 0)), x);
          }
          x += shfl_xor_f(x, 16);
          x += shfl_xor_f(x, 32);
          if (c < my_n) {
            sc = ks_s[buf][kj] * x;
            if (sc == 0.0f) sc = 0.0f;  // one zero: +0.0
          }
        }
        if (grp == 0 && c < stride) out_row[c] = sc;
      }
    }
    // next page: registers -> other LDS buffer, then start the one after
    if (pi + 1 < npages) {
      store(pi + 1, buf ^ 1);
      if (pi + 2 < npages) fetch(pi + 2);
    }
    __syncthreads();
  }
}

}  // namespace

}  // namespace csa

extern "C" int csa_index_score(const int8_t* q_idx, const float* q_scale, const float* head_w,
                               const int8_t* idx_kv, const float* idx_scale, int32_t num_blocks,
                               const int32_t* block_table, int32_t max_blocks,
                               const int32_t* query_start_loc, const int32_t* positions,
                               int32_t B, int32_t T, int32_t num_tokens, int32_t Hi, int32_t Di,
                               int32_t ratio, float* scores, int64_t score_stride, int32_t* err,
                               void* stream) {
  if (T < 0 || B < 0 || num_blocks < 0 || max_blocks < 0 || score_stride < 0) return CSA_ERR_SHAPE;
  if (num_tokens < 0 || num_tokens > T || ratio < 1) return CSA_ERR_RANGE;
  if (num_tokens == 0 || score_stride == 0) return CSA_OK;
  if (!q_idx || !q_scale || !head_w || !query_start_loc || !positions || !scores)
    return CSA_ERR_NULL;
  if (num_blocks > 0 && max_blocks > 0 && B > 0 && (!idx_kv || !idx_scale || !block_table))
    return CSA_ERR_NULL;
  if (Hi < 1 || Hi > 64 || Di < 16 || Di > 128 || (Di % 16) != 0) return CSA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(q_idx) | reinterpret_cast<uintptr_t>(idx_kv)) & 15)
    return CSA_ERR_UNSUPPORTED;
  if (static_cast<long long>(num_blocks) * csa::kPage * Di >= (1ll << 40)) return CSA_ERR_SHAPE;

  const long long pages = (score_stride + csa::kPage - 1) / csa::kPage;
  // groups of <= 4 rows never straddle requests: at most ceil(T/4) + B of them
  const long long groups = (num_tokens + 3) / 4 + B;
  // enough work-groups to fill 256 CUs several times over, few enough that
  // each amortises loading its query rows over several pages
  long long ppw = (pages * ((num_tokens + 3) / 4)) / 2048;
  if (ppw < 1) ppw = 1;
  if (ppw > csa::kMaxPPW) ppw = csa::kMaxPPW;
  const long long gx = (pages + ppw - 1) / ppw;
  if (gx > 0x7fffffffll || groups > 65535) return CSA_ERR_UNSUPPORTED;
  dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(groups));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (Di <= 64) {
    hipLaunchKernelGGL(csa::index_score_kernel<1>, grid, dim3(csa::kThreads), 0, st, q_idx,
                       q_scale, head_w, idx_kv, idx_scale, num_blocks, block_table, max_blocks,
                       query_start_loc, positions, B, num_tokens, Hi, Di, ratio, scores,
                       static_cast<long long>(score_stride), static_cast<int>(ppw), err);
  } else {
    hipLaunchKernelGGL(csa::index_score_kernel<2>, grid, dim3(csa::kThreads), 0, st, q_idx,
                       q_scale, head_w, idx_kv, idx_scale, num_blocks, block_table, max_blocks,
                       query_start_loc, positions, B, num_tokens, Hi, Di, ratio, scores,
                       static_cast<long long>(score_stride), static_cast<int>(ppw), err);
  }
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}
