// Lightning-indexer scores on CDNA4 INT8 MFMA.
//
// Method: gitcode hyper-parallel issue #2 (DeepSeek V4 CP notes), sections
// 10.2 / 10.3 -- per query row, score every causally visible compressed slot
// c < (p+1)/ratio with the indexer; pypto-lib "DeepSeek V4-Flash, MTP point",
// section "What is quantized" -- index keys are INT8 with an FP32 per-row
// scale.  Score = sum_h w[t,h] * relu(qs[t,h] * ks[c] * <q8[t,h], k8[c]>).
//
// Mapping.  A work-group is 4 waves; wave w owns query row 4*blockIdx.y + w
// and computes its 64 heads as four 16-row MFMA tiles (M = heads, N = keys,
// K = Di), so one key tile staged in LDS feeds every row of the request that
// sits in the group.  Each work-group walks `pages_per_wg` consecutive
// 128-key pages of the request (request-local positions), staging one page
// (128 x Di bytes, rows padded to 128 B, 16-byte chunks XOR-swizzled against
// LDS bank conflicts) per step.  The INT32 accumulators never leave
// registers: the epilogue applies ReLU, the folded weight w*qs, reduces the 64
// heads (16 in-lane, then across the four 16-lane groups) and scales by ks.
// Work scales with the visible context: pages past every row's visible span
// only receive -inf.
#include "csa_common.h"

namespace csa {

namespace {

constexpr int kRowsPerWG = 4;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowBytes = 128;  // LDS bytes per key (Di <= 128, zero padded)

__device__ __forceinline__ int swz_chunk(int key, int chunk) {
  return chunk ^ ((key >> 1) & 7);
}

template <int KK>
__global__ void __launch_bounds__(kThreads) index_score_kernel(
    const int8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ head_w, const int8_t* __restrict__ idx_kv,
    const float* __restrict__ idx_scale, int num_blocks, const int32_t* __restrict__ bt,
    int max_blocks, const int32_t* __restrict__ qsl, const int32_t* __restrict__ positions,
    int B, int num_tokens, int Hi, int Di, int ratio, float* __restrict__ scores,
    long long stride, int pages_per_wg, int32_t* err) {
  __shared__ __attribute__((aligned(16))) int8_t keys_s[kPage * kRowBytes];
  __shared__ float ks_s[kPage];
  __shared__ int req_s[kRowsPerWG];
  __shared__ int nvis_s[kRowsPerWG];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int t0 = blockIdx.y * kRowsPerWG;
  const int page0 = blockIdx.x * pages_per_wg;
  const long long stride_pages = (stride + kPage - 1) / kPage;

  if (tid < kRowsPerWG) {
    int t = t0 + tid;
    int b = -2, n = 0;
    if (t < num_tokens) {
      b = owner_request(qsl, B, t);
      if (b < 0) {
        if (blockIdx.x == 0) flag_error(err, CSA_EFLAG_META);
      } else {
        n = visible_count(positions[t], ratio);
        long long cap = static_cast<long long>(max_blocks) * kPage;
        if (static_cast<long long>(n) > stride || static_cast<long long>(n) > cap) {
          if (blockIdx.x == 0) flag_error(err, CSA_EFLAG_POS_RANGE);
          long long m = stride < cap ? stride : cap;
          if (static_cast<long long>(n) > m) n = static_cast<int>(m);
        }
      }
    }
    req_s[tid] = b;
    nvis_s[tid] = n;
  }
  __syncthreads();

  const int my_t = t0 + wave;
  const int my_req = req_s[wave];
  const int my_n = nvis_s[wave];
  const int col = lane & 15;   // key within a 16-key tile / head within an M tile
  const int grp = lane >> 4;   // 16-byte K chunk group

  // A operand (this wave's query row) and folded head weights, loaded once.
  v4i qa[4][KK];
  float ww[4][4];
  if (my_req >= 0) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      int h = mt * 16 + col;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        int off = kk * 64 + grp * 16;
        if (h < Hi && off < Di) {
          qa[mt][kk] = *reinterpret_cast<const v4i*>(
              q_idx + (static_cast<long long>(my_t) * Hi + h) * Di + off);
        } else {
          qa[mt][kk] = v4i{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int hh = mt * 16 + grp * 4 + r;
        ww[mt][r] = (hh < Hi) ? head_w[static_cast<long long>(my_t) * Hi + hh] *
                                    q_scale[static_cast<long long>(my_t) * Hi + hh]
                              : 0.0f;
      }
    }
  }

  const float neg_inf = -__builtin_huge_valf();
  int cur = 0;
  while (cur < kRowsPerWG) {
    const int b = req_s[cur];
    int end = cur + 1;
    while (end < kRowsPerWG && req_s[end] == b) ++end;
    const bool mine = (wave >= cur && wave < end);
    if (b == -2) break;  // rows past num_tokens: nothing to write
    int nmax = 0;
    for (int r = cur; r < end; ++r) nmax = max(nmax, nvis_s[r]);

    for (int pi = 0; pi < pages_per_wg; ++pi) {
      const int page = page0 + pi;
      if (page >= stride_pages) break;
      const int c0 = page * kPage;
      bool need = (b >= 0) && (c0 < nmax);
      int blk = -1;
      if (need) {
        blk = (page < max_blocks) ? bt[static_cast<long long>(b) * max_blocks + page] : -1;
        if (blk < 0 || blk >= num_blocks) {
          if (tid == 0) flag_error(err, CSA_EFLAG_BLOCK_RANGE);
          need = false;  // visible positions of this page score -inf
        }
      }
      if (need) {
        const int8_t* src = idx_kv + static_cast<long long>(blk) * kPage * Di;
#pragma unroll
        for (int u = 0; u < (kPage * 8) / kThreads; ++u) {
          int ch = tid + u * kThreads;
          int key = ch >> 3, c = ch & 7;
          v4i v = v4i{0, 0, 0, 0};
          if (c * 16 < Di) v = *reinterpret_cast<const v4i*>(src + key * Di + c * 16);
          *reinterpret_cast<v4i*>(keys_s + key * kRowBytes + swz_chunk(key, c) * 16) = v;
        }
        if (tid < kPage) ks_s[tid] = idx_scale[static_cast<long long>(blk) * kPage + tid];
      }
      __syncthreads();
      if (mine && my_req >= 0) {
        float* out_row = scores + static_cast<long long>(my_t) * stride;
#pragma unroll 2
        for (int s = 0; s < kPage / 16; ++s) {
          const int kj = s * 16 + col;
          const int c = c0 + kj;
          float sc = neg_inf;
          if (need && c0 + s * 16 < my_n) {
            v4i bk[KK];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
              bk[kk] = *reinterpret_cast<const v4i*>(keys_s + kj * kRowBytes +
                                                     swz_chunk(kj, kk * 4 + grp) * 16);
            float x = 0.0f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
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
              sc = ks_s[kj] * x;
              if (sc == 0.0f) sc = 0.0f;  // one zero: +0.0
            }
          }
          if (grp == 0 && c < stride) out_row[c] = sc;
        }
      } else if (mine && my_req == -1) {
        float* out_row = scores + static_cast<long long>(my_t) * stride;
        for (int j = lane; j < kPage; j += 64)
          if (c0 + j < stride) out_row[c0 + j] = neg_inf;
      }
      __syncthreads();
    }
    cur = end;
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
  const long long groups = (num_tokens + 3) / 4;
  // enough work-groups to fill 256 CUs several times over, few enough that
  // each amortises loading its query rows over several pages
  long long ppw = (pages * groups) / 4096;
  if (ppw < 1) ppw = 1;
  if (ppw > 16) ppw = 16;
  const long long gx = (pages + ppw - 1) / ppw;
  if (gx > 0x7fffffffll || groups > 65535) return CSA_ERR_UNSUPPORTED;
  dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(groups));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (Di <= 64) {
    hipLaunchKernelGGL(csa::index_score_kernel<1>, grid, dim3(256), 0, st, q_idx, q_scale,
                       head_w, idx_kv, idx_scale, num_blocks, block_table, max_blocks,
                       query_start_loc, positions, B, num_tokens, Hi, Di, ratio, scores,
                       static_cast<long long>(score_stride), static_cast<int>(ppw), err);
  } else {
    hipLaunchKernelGGL(csa::index_score_kernel<2>, grid, dim3(256), 0, st, q_idx, q_scale,
                       head_w, idx_kv, idx_scale, num_blocks, block_table, max_blocks,
                       query_start_loc, positions, B, num_tokens, Hi, Di, ratio, scores,
                       static_cast<long long>(score_stride), static_cast<int>(ppw), err);
  }
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}
