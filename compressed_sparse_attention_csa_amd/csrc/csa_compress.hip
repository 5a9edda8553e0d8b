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
// One launch: only a request's first row reads the ring, and its wave writes
// the request's ring rows after that read.  Requests must not share a state
// block.
#include "csa_common.h"

namespace csa {

namespace {

constexpr int kCmpLanes = 64;   // one wave per token

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
  // or the full tables [tab_cap][half] (rcos NULL): row rope_pos[t], the
  // identity rotation for a negative position, and for one past the tables
  // (flagged)
  const int32_t* rope_pos;
  const float* tab_cos;
  const float* tab_sin;
  int tab_cap;
  int half;
  int rope_offset;
  uint16_t* cmp;        // [ncb][128][D] BF16
  int ncb;
  const int32_t* cbt;   // [B][max_cb]
  int max_cb;
  int32_t* err;
};

// One wave per token; the tokens at odd positions publish.  Lane l owns the
// channel pairs (2l + 128 m, + 1), m < NCH, so a rope pair is always one
// lane's.  The row loads (this row, the input row before it, the RMSNorm
// weights and the rope row) are issued before the request lookup; a chunk's
// first row replaces the predecessor by its ring slot.  Only that first row
// reads the ring, and its wave writes every ring row of the request after
// the read (each lane rewrites the channels it read), so every read precedes
// every write within one launch.
template <int NCH>
__global__ void __launch_bounds__(kCmpLanes) compress_pairs_kernel(CompressArgs a) {
  const int t = blockIdx.x;
  if (t >= a.num_tokens) return;
  const int lane = threadIdx.x;
  const int D = a.D;
  const int qv = qsl_lane_load(a.qsl, a.B);
  const int p = a.pos[t];
  const bool odd = p >= 0 && (p & 1) == 1;
  // the rope row of the pair start: row t of the rope rows, or row rp of the
  // full tables (negative: identity; past the tables: flagged as the
  // materialisation flags it, identity here)
  const int rp = a.tab_cos ? a.rope_pos[t] : -1;
  if (a.tab_cos && a.half > 0 && rp >= a.tab_cap && lane == 0)
    flag_error(a.err, CSA_EFLAG_POS_RANGE);
  const bool tab_row = a.tab_cos && rp >= 0 && rp < a.tab_cap;
  float2 k0[NCH], g0[NCH], k1[NCH], g1[NCH], gm[NCH], rot[NCH];
  uint32_t in_rope = 0;           // bit m: chunk m's pair lies in the rope span
  if (odd) {
    const float* ck = a.kv + static_cast<long long>(t) * D;
    const float* cg = a.gate + static_cast<long long>(t) * D;
    const long long prev = static_cast<long long>(t > 0 ? t - 1 : 0) * D;
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = 2 * lane + 2 * kCmpLanes * m;
      k0[m] = g0[m] = k1[m] = g1[m] = gm[m] = make_float2(0.0f, 0.0f);
      rot[m] = make_float2(0.0f, 0.0f);
      if (c < D) {
        k1[m] = *reinterpret_cast<const float2*>(ck + c);
        g1[m] = *reinterpret_cast<const float2*>(cg + c);
        k0[m] = *reinterpret_cast<const float2*>(a.kv + prev + c);
        g0[m] = *reinterpret_cast<const float2*>(a.gate + prev + c);
        gm[m] = *reinterpret_cast<const float2*>(a.gamma + c);
        const int rr = c - a.rope_offset;
        if (rr >= 0 && rr < 2 * a.half) {
          if (!a.tab_cos) {
            const long long ri = static_cast<long long>(t) * a.half + (rr >> 1);
            rot[m] = make_float2(a.rcos[ri], a.rsin[ri]);
          } else if (tab_row) {
            const long long ri = static_cast<long long>(rp) * a.half + (rr >> 1);
            rot[m] = make_float2(a.tab_cos[ri], a.tab_sin[ri]);
          } else {
            rot[m] = make_float2(1.0f, 0.0f);
          }
          in_rope |= 1u << m;
        }
      }
    }
  }
  const int b = owner_from_lanes(qv, a.qsl, a.B, t);
  if (b < 0) {
    if (lane == 0) flag_error(a.err, CSA_EFLAG_META);
    return;
  }
  const int blk = a.sbt[b];
  if (blk < 0) return;            // compressor disabled for the request
  // a state block outside the pool skips only the ring accesses
  const bool ring_ok = blk < a.nsb;
  if (!ring_ok && lane == 0) flag_error(a.err, CSA_EFLAG_BLOCK_RANGE);
  const int lo = min(max(a.qsl[b], 0), a.num_tokens);
  const int hi = min(max(a.qsl[b + 1], 0), a.num_tokens);
  // an odd position closes a pair; its predecessor is the preceding input
  // row inside the chunk, else the ring
  bool publish = odd && (t > lo || ring_ok);
  long long crow = -1;
  if (publish) {
    crow = page_row(a.cbt + static_cast<long long>(b) * a.max_cb, a.max_cb, a.ncb, p >> 1);
    if (crow < 0) {
      if (lane == 0) flag_error(a.err, CSA_EFLAG_BLOCK_RANGE);
      publish = false;
    }
  }
  if (publish) {
    if (t == lo) {
      const float* pk = a.state + (static_cast<long long>(blk) * a.cap + (p - 1) % a.cap) * 2 * D;
#pragma unroll
      for (int m = 0; m < NCH; ++m) {
        const int c = 2 * lane + 2 * kCmpLanes * m;
        if (c < D) {
          k0[m] = *reinterpret_cast<const float2*>(pk + c);
          g0[m] = *reinterpret_cast<const float2*>(pk + D + c);
        }
      }
    }
    float x[NCH][2];
    float ss = 0.0f;
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const float kk0[2] = {k0[m].x, k0[m].y}, gg0[2] = {g0[m].x, g0[m].y};
      const float kk1[2] = {k1[m].x, k1[m].y}, gg1[2] = {g1[m].x, g1[m].y};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float mg = fmaxf(gg0[e], gg1[e]);
        const float w0 = expf(gg0[e] - mg), w1 = expf(gg1[e] - mg);
        const float pooled = (w0 * kk0[e] + w1 * kk1[e]) / (w0 + w1);
        x[m][e] = bf16_to_f32(f32_to_bf16(pooled));   // BF16 before the norm
        ss += x[m][e] * x[m][e];                      // lanes past D hold zeros
      }
    }
    const float r = rsqrtf(wave_sum(ss) / static_cast<float>(D) + a.eps);
    uint16_t* dst = a.cmp + crow * D;
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = 2 * lane + 2 * kCmpLanes * m;
      if (c >= D) continue;
      float y0 = x[m][0] * r * gm[m].x, y1 = x[m][1] * r * gm[m].y;
      if (in_rope & (1u << m)) {
        const float co = rot[m].x, si = rot[m].y;
        const float z0 = y0 * co - y1 * si, z1 = y0 * si + y1 * co;
        y0 = z0;
        y1 = z1;
      }
      *reinterpret_cast<uint32_t*>(dst + c) = pack_bf16x2(y0, y1);
    }
  }
  if (t != lo || !ring_ok) return;
  // the request's ring rows: the last min(chunk, CAP) of its chunk, in row
  // order (a later row with the same slot wins, channel by channel in the
  // same lane)
  for (int tt = max(lo, hi - a.cap); tt < hi; ++tt) {
    const int q = a.pos[tt];
    if (q < 0) continue;
    float* row = a.state + (static_cast<long long>(blk) * a.cap + q % a.cap) * 2 * D;
    const float* k = a.kv + static_cast<long long>(tt) * D;
    const float* g = a.gate + static_cast<long long>(tt) * D;
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = 2 * lane + 2 * kCmpLanes * m;
      if (c < D) {
        *reinterpret_cast<float2*>(row + c) = *reinterpret_cast<const float2*>(k + c);
        *reinterpret_cast<float2*>(row + D + c) = *reinterpret_cast<const float2*>(g + c);
      }
    }
  }
}

int compress_entry(const float* kv_proj, const float* gate, int32_t D,
                   const int32_t* query_start_loc, const int32_t* positions, int32_t B, int32_t T,
                   int32_t num_tokens, const int32_t* state_block_table, float* state_cache,
                   int32_t num_state_blocks, int32_t state_capacity, const float* rms_gamma,
                   float rms_eps, const float* rope_cos, const float* rope_sin,
                   const float* tab_cos, const float* tab_sin, int32_t tab_cap,
                   const int32_t* rope_pos, int32_t rope_dim, int32_t rope_offset,
                   uint16_t* cmp_kv, int32_t num_cmp_blocks, const int32_t* cmp_block_table,
                   int32_t max_cmp_blocks, int32_t* err, void* stream) {
  const bool tables = tab_cos || tab_sin || rope_pos;
  if (T < 0 || B < 0 || D < 0 || num_state_blocks < 0 || num_cmp_blocks < 0 ||
      max_cmp_blocks < 0 || rope_dim < 0 || rope_offset < 0 || tab_cap < 0)
    return CSA_ERR_SHAPE;
  if (num_tokens < 0 || num_tokens > T || state_capacity < 1) return CSA_ERR_RANGE;
  if ((D & 1) || D > 2048 || (rope_dim & 1) || (rope_offset & 1) ||
      rope_offset + rope_dim > D || !(rms_eps >= 0.0f))
    return CSA_ERR_UNSUPPORTED;
  if (num_tokens == 0 || D == 0) return CSA_OK;
  if (!kv_proj || !gate || !query_start_loc || !positions || !state_block_table ||
      !rms_gamma || !cmp_block_table)
    return CSA_ERR_NULL;
  if (rope_dim > 0 && (tables ? (!tab_cos || !tab_sin || !rope_pos) : (!rope_cos || !rope_sin)))
    return CSA_ERR_NULL;
  if ((num_state_blocks > 0 && !state_cache) || (num_cmp_blocks > 0 && !cmp_kv))
    return CSA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(kv_proj) | reinterpret_cast<uintptr_t>(gate) |
       reinterpret_cast<uintptr_t>(state_cache) | reinterpret_cast<uintptr_t>(rms_gamma) |
       reinterpret_cast<uintptr_t>(cmp_kv)) & 7)
    return CSA_ERR_UNSUPPORTED;
  if (static_cast<long long>(num_cmp_blocks) * kPage >= (1ll << 31)) return CSA_ERR_SHAPE;
  CompressArgs a{};
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
  if (tables && rope_dim > 0) {
    a.rope_pos = rope_pos;
    a.tab_cos = tab_cos;
    a.tab_sin = tab_sin;
    a.tab_cap = tab_cap;
  } else if (!tables) {
    a.rcos = rope_cos;
    a.rsin = rope_sin;
  }
  a.half = rope_dim / 2;
  a.rope_offset = rope_offset;
  a.cmp = cmp_kv;
  a.ncb = num_cmp_blocks;
  a.cbt = cmp_block_table;
  a.max_cb = max_cmp_blocks;
  a.err = err;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(num_tokens)), block(kCmpLanes);
  if (D <= 128)
    hipLaunchKernelGGL(compress_pairs_kernel<1>, grid, block, 0, st, a);
  else if (D <= 256)
    hipLaunchKernelGGL(compress_pairs_kernel<2>, grid, block, 0, st, a);
  else if (D <= 512)
    hipLaunchKernelGGL(compress_pairs_kernel<4>, grid, block, 0, st, a);
  else if (D <= 1024)
    hipLaunchKernelGGL(compress_pairs_kernel<8>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(compress_pairs_kernel<16>, grid, block, 0, st, a);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
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
  return csa::compress_entry(kv_proj, gate, D, query_start_loc, positions, B, T, num_tokens,
                             state_block_table, state_cache, num_state_blocks, state_capacity,
                             rms_gamma, rms_eps, rope_cos, rope_sin, nullptr, nullptr, 0, nullptr,
                             rope_dim, rope_offset, cmp_kv, num_cmp_blocks, cmp_block_table,
                             max_cmp_blocks, err, stream);
}

extern "C" int csa_compress_pairs_rope(const float* kv_proj, const float* gate, int32_t D,
                                       const int32_t* query_start_loc, const int32_t* positions,
                                       int32_t B, int32_t T, int32_t num_tokens,
                                       const int32_t* state_block_table, float* state_cache,
                                       int32_t num_state_blocks, int32_t state_capacity,
                                       const float* rms_gamma, float rms_eps,
                                       const float* freqs_cos, const float* freqs_sin,
                                       int32_t table_capacity, const int32_t* rope_position_ids,
                                       int32_t rope_dim, int32_t rope_offset, uint16_t* cmp_kv,
                                       int32_t num_cmp_blocks, const int32_t* cmp_block_table,
                                       int32_t max_cmp_blocks, int32_t* err, void* stream) {
  if (rope_dim > 0 && (!freqs_cos || !freqs_sin || !rope_position_ids)) {
    // checked here: without a table the shared entry would read rope rows
    if (T < 0 || B < 0 || D < 0 || table_capacity < 0) return CSA_ERR_SHAPE;
    return CSA_ERR_NULL;
  }
  return csa::compress_entry(kv_proj, gate, D, query_start_loc, positions, B, T, num_tokens,
                             state_block_table, state_cache, num_state_blocks, state_capacity,
                             rms_gamma, rms_eps, nullptr, nullptr, freqs_cos, freqs_sin,
                             table_capacity, rope_position_ids, rope_dim, rope_offset, cmp_kv,
                             num_cmp_blocks, cmp_block_table, max_cmp_blocks, err, stream);
}
