// Ratio-2 compressor publication with its FP32 state ring: pypto-lib
// "DeepSeek V4.1 Flash", section "Compressor state ownership" (ring slot
// block * CAP + p % CAP, odd positions close pairs, a chunk's first token
// reads its predecessor from the ring, every read before any write, only the
// last min(chunk, CAP) rows of a chunk written, negative positions and
// disabled requests touch nothing) and the paragraph on the production cache
// ABI (a ring row is the token's KV projection followed by its gate score).
// The pooling, the BF16 rounding before RMSNorm and the group-start RoPE rows
// are only named there; the arithmetic below is the plain reading:
//   pooled[c] = sum_j e^{g_j[c]} kv_j[c] / sum_j e^{g_j[c]} over the pair,
//   x = bf16(pooled), y = x * rsqrt(mean(x^2) + eps) * gamma, the rope span
//   of y rotated by the pair's start row, bf16(y) published at p / 2.
//
// Two launches on the stream: the publication kernel reads the ring, the
// state kernel then writes it, so every read precedes every write.
#include "csa_common.h"

namespace csa {

namespace {

constexpr int kCmpThreads = 256;

struct CompressArgs {
  const float* kv;      // [T][D]
  const float* gate;    // [T][D]
  int D;
  const int32_t* qsl;
  const int32_t* pos;
  int B;
  int num_tokens;
  const int32_t* sbt;   // [B]
  float* state;         // [nsb][cap][2D]
  int nsb;
  int cap;
  const float* gamma;   // [D]
  float eps;
  const float* rcos;    // [T][half]: the rope row of each token's pair start
  const float* rsin;
  int half;
  int rope_offset;
  uint16_t* cmp;        // [ncb][128][D] BF16
  int ncb;
  const int32_t* cbt;   // [B][max_cb]
  int max_cb;
  int32_t* err;
};

// One work-group per token; the tokens at odd positions publish.  Thread i
// owns channel pairs (2i + 2 * kCmpThreads * m, + 1), so a rope pair is
// always one thread's.
__global__ void __launch_bounds__(kCmpThreads) compress_publish_kernel(CompressArgs a) {
  __shared__ float red_s[kCmpThreads / 64];
  const int t = blockIdx.x;
  if (t >= a.num_tokens) return;
  const int tid = threadIdx.x;
  const int b = owner_request_wave(a.qsl, a.B, t);
  if (b < 0) {
    if (tid == 0) flag_error(a.err, CSA_EFLAG_META);
    return;
  }
  const int p = a.pos[t];
  const int blk = a.sbt[b];
  if (blk < 0) return;            // compressor disabled for the request
  // a state block outside the pool skips only the ring accesses
  const bool ring_ok = blk < a.nsb;
  if (!ring_ok && tid == 0) flag_error(a.err, CSA_EFLAG_BLOCK_RANGE);
  if (p < 0 || (p & 1) == 0) return;   // no publication; an even position opens a pair
  const int lo = min(max(a.qsl[b], 0), a.num_tokens);
  // predecessor: the preceding input row inside the chunk, else the ring
  const float* pk;
  const float* pg;
  if (t > lo) {
    pk = a.kv + static_cast<long long>(t - 1) * a.D;
    pg = a.gate + static_cast<long long>(t - 1) * a.D;
  } else {
    if (!ring_ok) return;
    pk = a.state + (static_cast<long long>(blk) * a.cap + (p - 1) % a.cap) * 2 * a.D;
    pg = pk + a.D;
  }
  const float* ck = a.kv + static_cast<long long>(t) * a.D;
  const float* cg = a.gate + static_cast<long long>(t) * a.D;
  // the publication row (checked before anything is computed)
  const int cp = p >> 1;
  const long long crow = page_row(a.cbt + static_cast<long long>(b) * a.max_cb, a.max_cb, a.ncb, cp);
  if (crow < 0) {
    if (tid == 0) flag_error(a.err, CSA_EFLAG_BLOCK_RANGE);
    return;
  }
  constexpr int kMaxPairs = 4;    // D <= 2 * kCmpThreads * kMaxPairs
  float x[kMaxPairs][2];
  float ss = 0.0f;
#pragma unroll
  for (int m = 0; m < kMaxPairs; ++m) {
    const int c = 2 * tid + 2 * kCmpThreads * m;
    x[m][0] = x[m][1] = 0.0f;
    if (c < a.D) {
      const float2 k0 = *reinterpret_cast<const float2*>(pk + c);
      const float2 g0 = *reinterpret_cast<const float2*>(pg + c);
      const float2 k1 = *reinterpret_cast<const float2*>(ck + c);
      const float2 g1 = *reinterpret_cast<const float2*>(cg + c);
      const float kk0[2] = {k0.x, k0.y}, gg0[2] = {g0.x, g0.y};
      const float kk1[2] = {k1.x, k1.y}, gg1[2] = {g1.x, g1.y};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float mg = fmaxf(gg0[e], gg1[e]);
        const float w0 = expf(gg0[e] - mg), w1 = expf(gg1[e] - mg);
        const float pooled = (w0 * kk0[e] + w1 * kk1[e]) / (w0 + w1);
        x[m][e] = bf16_to_f32(f32_to_bf16(pooled));   // BF16 before the norm
        ss += x[m][e] * x[m][e];
      }
    }
  }
  // sum of squares over the row
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((tid & 63) == 0) red_s[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < kCmpThreads / 64; ++w) tot += red_s[w];
  const float r = rsqrtf(tot / static_cast<float>(a.D) + a.eps);
  uint16_t* dst = a.cmp + crow * a.D;
#pragma unroll
  for (int m = 0; m < kMaxPairs; ++m) {
    const int c = 2 * tid + 2 * kCmpThreads * m;
    if (c >= a.D) continue;
    const float2 gm = *reinterpret_cast<const float2*>(a.gamma + c);
    float y0 = x[m][0] * r * gm.x, y1 = x[m][1] * r * gm.y;
    const int rr = c - a.rope_offset;
    if (rr >= 0 && rr < 2 * a.half) {
      const float co = a.rcos[static_cast<long long>(t) * a.half + (rr >> 1)];
      const float si = a.rsin[static_cast<long long>(t) * a.half + (rr >> 1)];
      const float z0 = y0 * co - y1 * si, z1 = y0 * si + y1 * co;
      y0 = z0;
      y1 = z1;
    }
    *reinterpret_cast<uint32_t*>(dst + c) = pack_bf16x2(y0, y1);
  }
}

// One work-group per token: the last min(chunk, CAP) rows of each request's
// chunk go to their ring slots.
__global__ void __launch_bounds__(kCmpThreads) compress_state_kernel(CompressArgs a) {
  const int t = blockIdx.x;
  if (t >= a.num_tokens) return;
  const int b = owner_request_wave(a.qsl, a.B, t);
  if (b < 0) return;
  const int p = a.pos[t];
  const int blk = a.sbt[b];
  if (p < 0 || blk < 0 || blk >= a.nsb) return;
  const int lo = min(max(a.qsl[b], 0), a.num_tokens);
  const int hi = min(max(a.qsl[b + 1], 0), a.num_tokens);
  if (t < max(lo, hi - a.cap)) return;
  float* row = a.state + (static_cast<long long>(blk) * a.cap + p % a.cap) * 2 * a.D;
  const float* k = a.kv + static_cast<long long>(t) * a.D;
  const float* g = a.gate + static_cast<long long>(t) * a.D;
  for (int c = threadIdx.x; c < a.D; c += kCmpThreads) {
    row[c] = k[c];
    row[a.D + c] = g[c];
  }
}

}  // namespace

}  // namespace csa

extern "C" int csa_compress_pairs(const float* kv_proj, const float* gate, int32_t D,
                                  const int32_t* query_start_loc, const int32_t* positions,
                                  int32_t B, int32_t T, int32_t num_tokens,
                                  const int32_t* state_block_table, float* state_cache,
                                  int32_t num_state_blocks, int32_t state_capacity,
                                  const float* rms_gamma, float rms_eps, const float* rope_cos,
                                  const float* rope_sin, int32_t rope_dim, int32_t rope_offset,
                                  uint16_t* cmp_kv, int32_t num_cmp_blocks,
                                  const int32_t* cmp_block_table, int32_t max_cmp_blocks,
                                  int32_t* err, void* stream) {
  if (T < 0 || B < 0 || D < 0 || num_state_blocks < 0 || num_cmp_blocks < 0 ||
      max_cmp_blocks < 0 || rope_dim < 0 || rope_offset < 0)
    return CSA_ERR_SHAPE;
  if (num_tokens < 0 || num_tokens > T || state_capacity < 1) return CSA_ERR_RANGE;
  if ((D & 1) || D > 2 * 256 * 4 || (rope_dim & 1) || (rope_offset & 1) ||
      rope_offset + rope_dim > D || !(rms_eps >= 0.0f))
    return CSA_ERR_UNSUPPORTED;
  if (num_tokens == 0 || D == 0) return CSA_OK;
  if (!kv_proj || !gate || !query_start_loc || !positions || !state_block_table ||
      !rms_gamma || !cmp_block_table || (rope_dim > 0 && (!rope_cos || !rope_sin)))
    return CSA_ERR_NULL;
  if ((num_state_blocks > 0 && !state_cache) || (num_cmp_blocks > 0 && !cmp_kv))
    return CSA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(kv_proj) | reinterpret_cast<uintptr_t>(gate) |
       reinterpret_cast<uintptr_t>(state_cache) | reinterpret_cast<uintptr_t>(rms_gamma) |
       reinterpret_cast<uintptr_t>(cmp_kv)) & 7)
    return CSA_ERR_UNSUPPORTED;
  if (static_cast<long long>(num_cmp_blocks) * csa::kPage >= (1ll << 31)) return CSA_ERR_SHAPE;
  csa::CompressArgs a{};
  a.kv = kv_proj;
  a.gate = gate;
  a.D = D;
  a.qsl = query_start_loc;
  a.pos = positions;
  a.B = B;
  a.num_tokens = num_tokens;
  a.sbt = state_block_table;
  a.state = state_cache;
  a.nsb = num_state_blocks;
  a.cap = state_capacity;
  a.gamma = rms_gamma;
  a.eps = rms_eps;
  a.rcos = rope_cos;
  a.rsin = rope_sin;
  a.half = rope_dim / 2;
  a.rope_offset = rope_offset;
  a.cmp = cmp_kv;
  a.ncb = num_cmp_blocks;
  a.cbt = cmp_block_table;
  a.max_cb = max_cmp_blocks;
  a.err = err;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(csa::compress_publish_kernel, dim3(static_cast<unsigned>(num_tokens)),
                     dim3(csa::kCmpThreads), 0, st, a);
  if (hipGetLastError() != hipSuccess) return CSA_ERR_LAUNCH;
  hipLaunchKernelGGL(csa::compress_state_kernel, dim3(static_cast<unsigned>(num_tokens)),
                     dim3(csa::kCmpThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}
