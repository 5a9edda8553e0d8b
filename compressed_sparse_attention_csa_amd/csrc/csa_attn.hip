// Shared-KV sparse attention with sink on CDNA4 BF16 MFMA.
//
// Method: gitcode hyper-parallel issue #2 (DeepSeek V4 CP notes), Stage-2
// operator calls (sinks = attn_sink, softmax_scale, ori_win_left = 127,
// ori_win_right = 0) and section 9.1: each query attends, with every head,
// over its window rows followed by its selected compressed rows, one shared
// row serving as key and value.  pypto-lib "DeepSeek V4.1 Flash", section
// "Serving-owned full RoPE tables": the query is rotated with FP32 half-width
// rows in adjacent pairs.
//
// Mapping.  A work-group (4 waves) owns one query row and one contiguous span
// (a "split") of its key list; wave w owns heads 16w..16w+15.  The key list is
// virtual -- entry i < W_len is window position w_lo + i, later entries are
// topk_idx[t][i - W_len] -- and is resolved through the block tables one
// 32-row tile at a time.  Each tile is gathered (1 KiB rows, coalesced) into
// LDS twice: row-major K (MFMA A operand of S^T = K Q^T) and transposed V
// (A operand of O^T = V^T P^T).  S^T puts one head per lane, so the online
// softmax needs only two cross-lane steps per tile, and P^T leaves the MFMA
// already laid out as the B operand of the P*V product (the key order inside
// the MFMA is permuted identically on both operands).  The rotated query
// stays in registers as the B operand of S^T for the whole walk.
//
// With one split per row the kernel writes BF16 output and lse directly
// (prefill, many rows); with several it writes FP32 partials (unnormalised O,
// running max and sum, base-2 domain) that a merge kernel combines with the
// sink.
#include "csa_common.h"

namespace csa {

namespace {

constexpr int kTile = 32;       // key rows per LDS tile
constexpr int kAttnWaves = 4;   // 16 heads per wave
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kVtStride = 36;   // bf16 elements per transposed row (32 + pad)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const uint16_t* q;
  const float* rope_cos;
  const float* rope_sin;
  int half_rope;
  int rope_offset;
  const uint16_t* cmp_kv;
  int num_cmp_blocks;
  const int32_t* cmp_bt;
  int max_cmp_blocks;
  const int32_t* topk;
  int k;
  int ratio;
  const uint16_t* win_kv;
  int num_win_blocks;
  const int32_t* win_bt;
  int max_win_blocks;
  int window;
  const float* sink;
  float scale_log2;  // softmax_scale * log2(e)
  const int32_t* qsl;
  const int32_t* positions;
  int B;
  int num_tokens;
  int H;
  uint16_t* out;
  float* lse;
  float* part_o;     // [T][splits][H][D]
  float2* part_ml;   // [T][splits][H]
  int splits;
  int split_len;
  int items_per_xcd;
  int32_t* err;
};

__device__ __forceinline__ v8bf as_v8bf(v4i x) { return __builtin_bit_cast(v8bf, x); }

template <int D>
__global__ void __launch_bounds__(kAttnThreads, 2) attn_kernel(AttnArgs a) {
  constexpr int KS = D / 32;   // K steps of S^T
  constexpr int DT = D / 16;   // d tiles of O^T
  constexpr int KROW = D + 8;  // padded bf16 elements per K row
  __shared__ __attribute__((aligned(16))) uint16_t k_s[kTile * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t vt_s[D * kVtStride];
  __shared__ const uint16_t* rowptr_s[kTile];
  __shared__ int err_s;

  // XCD-aware work mapping: consecutive items (row, split) land on one XCD.
  const int L = blockIdx.x;
  const int item = (L & 7) * a.items_per_xcd + (L >> 3);
  const int t = item / a.splits;
  const int split = item % a.splits;
  if (t >= a.num_tokens) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;  // head within the wave's 16 (B/C column index)
  const int grp = lane >> 4;  // lane group
  const int h0 = wave * 16;
  const bool wave_active = h0 < a.H;

  if (tid == 0) err_s = 0;

  const int b = owner_request(a.qsl, a.B, t);
  const int p = a.positions[t];
  const int nv = visible_count(p, a.ratio);
  int w_len = 0, w_lo = 0;
  if (b >= 0 && p >= 0 && a.window > 0) {
    w_lo = max(0, p - a.window + 1);
    w_len = p - w_lo + 1;
  }
  const int list_len = (b >= 0) ? (w_len + a.k) : 0;
  const int i_begin = split * a.split_len;
  const int i_end = min(list_len, i_begin + a.split_len);

  // ---- query fragments (B operand of S^T): lane (head col, group grp) holds
  //      channels ks*32 + grp*8 .. +8, rotated where they fall in the rope span.
  v8bf qf[KS];
  {
    const int h = h0 + col;
    const bool hv = wave_active && h < a.H;
    const uint16_t* qrow = a.q + (static_cast<long long>(t) * a.H + (hv ? h : 0)) * D;
    const float* rc = a.rope_cos + static_cast<long long>(t) * a.half_rope;
    const float* rs = a.rope_sin + static_cast<long long>(t) * a.half_rope;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = ks * 32 + grp * 8;
      v4i raw = hv ? *reinterpret_cast<const v4i*>(qrow + d0) : v4i{0, 0, 0, 0};
      const int r0 = d0 - a.rope_offset;
      if (hv && r0 + 8 > 0 && r0 < 2 * a.half_rope) {
        uint16_t e[8];
        *reinterpret_cast<v4i*>(e) = raw;
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
          const int rr = r0 + 2 * pr;
          if (rr >= 0 && rr < 2 * a.half_rope) {
            const float c = rc[rr >> 1], s = rs[rr >> 1];
            const float x = bf16_to_f32(e[2 * pr]), y = bf16_to_f32(e[2 * pr + 1]);
            e[2 * pr] = f32_to_bf16(x * c - y * s);
            e[2 * pr + 1] = f32_to_bf16(x * s + y * c);
          }
        }
        raw = *reinterpret_cast<v4i*>(e);
      }
      qf[ks] = as_v8bf(raw);
    }
  }

  const float neg_inf = -__builtin_huge_valf();
  float m_run = neg_inf;  // running max of this lane's head (base-2 logits)
  float l_run = 0.0f;     // running sum
  v4f o_acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o_acc[i] = v4f{0.f, 0.f, 0.f, 0.f};

  const int32_t* topk_row = a.topk + static_cast<long long>(t) * a.k;
  for (int i0 = i_begin; i0 < i_end; i0 += kTile) {
    // resolve this tile's rows through the block tables
    if (tid < kTile) {
      const int i = i0 + tid;
      const uint16_t* ptr = nullptr;
      int ebits = 0;
      if (i < i_end) {
        if (i < w_len) {
          const long long r = page_row(a.win_bt + static_cast<long long>(b) * a.max_win_blocks,
                                       a.max_win_blocks, a.num_win_blocks, w_lo + i);
          if (r >= 0) ptr = a.win_kv + r * D; else ebits |= CSA_EFLAG_BLOCK_RANGE;
        } else {
          const int c = topk_row[i - w_len];
          if (c >= 0) {
            if (c >= nv) {
              ebits |= CSA_EFLAG_TOPK_RANGE;
            } else {
              const long long r = page_row(a.cmp_bt + static_cast<long long>(b) * a.max_cmp_blocks,
                                           a.max_cmp_blocks, a.num_cmp_blocks, c);
              if (r >= 0) ptr = a.cmp_kv + r * D; else ebits |= CSA_EFLAG_BLOCK_RANGE;
            }
          }
        }
      }
      rowptr_s[tid] = ptr;
      if (ebits) atomicOr(&err_s, ebits);
    }
    __syncthreads();
    // gather: lane (c4 = lane&3, rp = lane>>2) moves two rows' 16-byte chunk
    {
      const int c4 = lane & 3;
      const int rp = lane >> 2;
      const int r0 = 2 * rp, r1 = r0 + 1;
      const uint16_t* p0 = rowptr_s[r0];
      const uint16_t* p1 = rowptr_s[r1];
      for (int cg = wave; cg < D / 32; cg += kAttnWaves) {
        const int cc = cg * 4 + c4;  // 16-byte chunk index within the row
        v4i x0 = p0 ? *reinterpret_cast<const v4i*>(p0 + cc * 8) : v4i{0, 0, 0, 0};
        v4i x1 = p1 ? *reinterpret_cast<const v4i*>(p1 + cc * 8) : v4i{0, 0, 0, 0};
        *reinterpret_cast<v4i*>(k_s + r0 * KROW + cc * 8) = x0;
        *reinterpret_cast<v4i*>(k_s + r1 * KROW + cc * 8) = x1;
        const uint16_t* e0 = reinterpret_cast<const uint16_t*>(&x0);
        const uint16_t* e1 = reinterpret_cast<const uint16_t*>(&x1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t pair = static_cast<uint32_t>(e0[e]) | (static_cast<uint32_t>(e1[e]) << 16);
          *reinterpret_cast<uint32_t*>(vt_s + (cc * 8 + e) * kVtStride + r0) = pair;
        }
      }
    }
    __syncthreads();

    if (wave_active) {
      // S^T tile: rows = 32 keys (two 16-row M tiles), columns = 16 heads
      v4f s0 = v4f{0.f, 0.f, 0.f, 0.f}, s1 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const v8bf a0 = as_v8bf(*reinterpret_cast<const v4i*>(k_s + col * KROW + ks * 32 + grp * 8));
        const v8bf a1 = as_v8bf(*reinterpret_cast<const v4i*>(k_s + (16 + col) * KROW + ks * 32 + grp * 8));
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], s1, 0, 0, 0);
      }
      // lane holds keys grp*4 + r (s0) and 16 + grp*4 + r (s1) of head col
      float lg[8];
      float tmax = neg_inf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool v0 = rowptr_s[grp * 4 + r] != nullptr;
        const bool v1 = rowptr_s[16 + grp * 4 + r] != nullptr;
        lg[r] = v0 ? s0[r] * a.scale_log2 : neg_inf;
        lg[4 + r] = v1 ? s1[r] * a.scale_log2 : neg_inf;
        tmax = fmaxf(tmax, fmaxf(lg[r], lg[4 + r]));
      }
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = (m_new == neg_inf) ? 0.0f : m_new;
      const float alpha = exp2f(m_run - m_use);
      float psum = 0.0f;
      uint16_t pb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pj = exp2f(lg[j] - m_use);
        psum += pj;
        pb[j] = f32_to_bf16(pj);
      }
      psum += shfl_xor_f(psum, 16);
      psum += shfl_xor_f(psum, 32);
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const v8bf pf = as_v8bf(*reinterpret_cast<v4i*>(pb));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o_acc[dt] *= alpha;
        const uint16_t* vrow = vt_s + (dt * 16 + col) * kVtStride + grp * 4;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
        const v4i va = v4i{static_cast<int>(lo.x), static_cast<int>(lo.y),
                           static_cast<int>(hi.x), static_cast<int>(hi.y)};
        o_acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(va), pf, o_acc[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  if (tid == 0 && err_s) flag_error(a.err, err_s);
  if (b < 0 && split == 0 && tid == 0) flag_error(a.err, CSA_EFLAG_META);
  if (!wave_active) return;
  const int h = h0 + col;
  if (h >= a.H) return;

  if (a.splits == 1) {
    const float sink2 = a.sink[h] * kLog2e;
    const float M = fmaxf(m_run, sink2);
    const float corr = (m_run == neg_inf) ? 0.0f : exp2f(m_run - M);
    const float Z = l_run * corr + exp2f(sink2 - M);
    const float f = corr / Z;
    uint16_t* orow = a.out + (static_cast<long long>(t) * a.H + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      // o_acc[dt][r] is channel dt*16 + grp*4 + r of head h
      const int d = dt * 16 + grp * 4;
      uint2 w;
      w.x = static_cast<uint32_t>(f32_to_bf16(o_acc[dt][0] * f)) |
            (static_cast<uint32_t>(f32_to_bf16(o_acc[dt][1] * f)) << 16);
      w.y = static_cast<uint32_t>(f32_to_bf16(o_acc[dt][2] * f)) |
            (static_cast<uint32_t>(f32_to_bf16(o_acc[dt][3] * f)) << 16);
      *reinterpret_cast<uint2*>(orow + d) = w;
    }
    if (a.lse && grp == 0) a.lse[static_cast<long long>(t) * a.H + h] = (M + log2f(Z)) * kLn2;
  } else {
    const long long slot = (static_cast<long long>(t) * a.splits + split) * a.H + h;
    float* po = a.part_o + slot * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<v4f*>(po + dt * 16 + grp * 4) = o_acc[dt];
    if (grp == 0) a.part_ml[slot] = make_float2(m_run, l_run);
  }
}

// Combine split partials with the sink: one work-group per (row, head).
template <int D>
__global__ void __launch_bounds__(128) attn_merge_kernel(
    const float* __restrict__ part_o, const float2* __restrict__ part_ml,
    const float* __restrict__ sink, int splits, int H, int num_tokens,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int t = blockIdx.x / H;
  const int h = blockIdx.x % H;
  if (t >= num_tokens) return;
  const float neg_inf = -__builtin_huge_valf();
  const long long base = static_cast<long long>(t) * splits * H + h;
  float M = sink[h] * kLog2e;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, part_ml[base + static_cast<long long>(s) * H].x);
  float Z = exp2f(sink[h] * kLog2e - M);
  for (int s = 0; s < splits; ++s) {
    const float2 ml = part_ml[base + static_cast<long long>(s) * H];
    if (ml.x != neg_inf) Z += ml.y * exp2f(ml.x - M);
  }
  const float invZ = 1.0f / Z;
  for (int d = threadIdx.x * 4; d < D; d += 128 * 4) {
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) {
      const long long slot = base + static_cast<long long>(s) * H;
      const float mx = part_ml[slot].x;
      if (mx == neg_inf) continue;
      const float w = exp2f(mx - M) * invZ;
      const v4f v = *reinterpret_cast<const v4f*>(part_o + slot * D + d);
      acc += v * w;
    }
    uint2 pk;
    pk.x = static_cast<uint32_t>(f32_to_bf16(acc[0])) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    pk.y = static_cast<uint32_t>(f32_to_bf16(acc[2])) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    *reinterpret_cast<uint2*>(out + (static_cast<long long>(t) * H + h) * D + d) = pk;
  }
  if (lse && threadIdx.x == 0) lse[static_cast<long long>(t) * H + h] = (M + log2f(Z)) * kLn2;
}

// Split plan shared by the launcher and the workspace helper: enough
// work-groups to spread a small decode batch over the chip, spans long enough
// (>= 128 rows) that FP32 partials stay smaller than the rows they replace.
struct SplitPlan {
  int splits;
  int split_len;
};

SplitPlan plan_splits(int T, int k, int window, bool prefill) {
  const int lmax = max(1, window + k);
  if (prefill || T >= 256) return SplitPlan{1, ((lmax + kTile - 1) / kTile) * kTile};
  int by_len = (lmax + 127) / 128;
  int want = (512 + T - 1) / max(T, 1);
  int splits = max(1, min(by_len, want));
  int len = (lmax + splits - 1) / splits;
  len = ((len + kTile - 1) / kTile) * kTile;
  splits = (lmax + len - 1) / len;
  return SplitPlan{splits, len};
}

template <int D>
int launch_attn(const AttnArgs& in, hipStream_t st) {
  AttnArgs a = in;
  const long long items = static_cast<long long>(a.num_tokens) * a.splits;
  a.items_per_xcd = static_cast<int>((items + 7) / 8);
  const long long grid = static_cast<long long>(a.items_per_xcd) * 8;
  if (grid > 0x7fffffffll) return CSA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(attn_kernel<D>, dim3(static_cast<unsigned>(grid)), dim3(kAttnThreads), 0, st,
                     a);
  if (hipGetLastError() != hipSuccess) return CSA_ERR_LAUNCH;
  if (a.splits > 1) {
    hipLaunchKernelGGL(attn_merge_kernel<D>, dim3(static_cast<unsigned>(a.num_tokens * a.H)),
                       dim3(128), 0, st, a.part_o, a.part_ml, a.sink, a.splits, a.H, a.num_tokens,
                       a.out, a.lse);
    if (hipGetLastError() != hipSuccess) return CSA_ERR_LAUNCH;
  }
  return CSA_OK;
}

int attn_entry(bool prefill, const uint16_t* q, const float* rope_cos, const float* rope_sin,
               int32_t rope_dim, int32_t rope_offset, const uint16_t* cmp_kv,
               int32_t num_cmp_blocks, const int32_t* cmp_block_table, int32_t max_cmp_blocks,
               const int32_t* topk_idx, int32_t k, int32_t ratio, const uint16_t* win_kv,
               int32_t num_win_blocks, const int32_t* win_block_table, int32_t max_win_blocks,
               int32_t window, const float* attn_sink, float softmax_scale,
               const int32_t* query_start_loc, const int32_t* positions, int32_t B, int32_t T,
               int32_t num_tokens, int32_t H, int32_t D, uint16_t* out, float* lse,
               void* workspace, size_t workspace_bytes, int32_t* err, void* stream) {
  if (T < 0 || B < 0 || num_cmp_blocks < 0 || num_win_blocks < 0 || max_cmp_blocks < 0 ||
      max_win_blocks < 0 || window < 0 || k < 0)
    return CSA_ERR_SHAPE;
  if (num_tokens < 0 || num_tokens > T || ratio < 1 || k > 4096) return CSA_ERR_RANGE;
  if (num_tokens == 0) return CSA_OK;
  if (!q || !attn_sink || !query_start_loc || !positions || !out) return CSA_ERR_NULL;
  if (k > 0 && !topk_idx) return CSA_ERR_NULL;
  if (rope_dim > 0 && (!rope_cos || !rope_sin)) return CSA_ERR_NULL;
  if (H < 1 || H > 64) return CSA_ERR_UNSUPPORTED;
  if (D != 64 && D != 128 && D != 256 && D != 512) return CSA_ERR_UNSUPPORTED;
  if (rope_dim < 0 || (rope_dim & 1) || rope_offset < 0 || (rope_offset & 1) ||
      rope_offset + rope_dim > D)
    return CSA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) |
       reinterpret_cast<uintptr_t>(cmp_kv) | reinterpret_cast<uintptr_t>(win_kv)) & 15)
    return CSA_ERR_UNSUPPORTED;
  const SplitPlan plan = plan_splits(num_tokens, k, window, prefill);
  AttnArgs a{};
  a.q = q;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.half_rope = rope_dim / 2;
  a.rope_offset = rope_offset;
  a.cmp_kv = cmp_kv;
  a.num_cmp_blocks = cmp_kv ? num_cmp_blocks : 0;
  a.cmp_bt = cmp_block_table;
  a.max_cmp_blocks = cmp_block_table ? max_cmp_blocks : 0;
  a.topk = topk_idx;
  a.k = k;
  a.ratio = ratio;
  a.win_kv = win_kv;
  a.num_win_blocks = win_kv ? num_win_blocks : 0;
  a.win_bt = win_block_table;
  a.max_win_blocks = win_block_table ? max_win_blocks : 0;
  a.window = window;
  a.sink = attn_sink;
  a.scale_log2 = softmax_scale * kLog2e;
  a.qsl = query_start_loc;
  a.positions = positions;
  a.B = B;
  a.num_tokens = num_tokens;
  a.H = H;
  a.out = out;
  a.lse = lse;
  a.splits = plan.splits;
  a.split_len = plan.split_len;
  a.err = err;
  if (plan.splits > 1) {
    const size_t need = static_cast<size_t>(num_tokens) * plan.splits * H * (D + 2) * sizeof(float);
    if (!workspace || workspace_bytes < need) return CSA_ERR_WORKSPACE;
    a.part_o = static_cast<float*>(workspace);
    a.part_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) +
                                          static_cast<size_t>(num_tokens) * plan.splits * H * D *
                                              sizeof(float));
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (D) {
    case 64: return launch_attn<64>(a, st);
    case 128: return launch_attn<128>(a, st);
    case 256: return launch_attn<256>(a, st);
    default: return launch_attn<512>(a, st);
  }
}

}  // namespace

}  // namespace csa

extern "C" size_t csa_sparse_attn_workspace_bytes(int32_t T, int32_t H, int32_t D, int32_t k,
                                                  int32_t window) {
  if (T <= 0 || H <= 0 || D <= 0 || k < 0 || window < 0) return 0;
  const csa::SplitPlan plan = csa::plan_splits(T, k, window, false);
  if (plan.splits <= 1) return 0;
  return static_cast<size_t>(T) * plan.splits * H * (D + 2) * sizeof(float);
}

extern "C" int csa_sparse_attn_decode(
    const uint16_t* q, const float* rope_cos, const float* rope_sin, int32_t rope_dim,
    int32_t rope_offset, const uint16_t* cmp_kv, int32_t num_cmp_blocks,
    const int32_t* cmp_block_table, int32_t max_cmp_blocks, const int32_t* topk_idx, int32_t k,
    int32_t ratio, const uint16_t* win_kv, int32_t num_win_blocks,
    const int32_t* win_block_table, int32_t max_win_blocks, int32_t window,
    const float* attn_sink, float softmax_scale, const int32_t* query_start_loc,
    const int32_t* positions, int32_t B, int32_t T, int32_t num_tokens, int32_t H, int32_t D,
    uint16_t* out, float* lse, void* workspace, size_t workspace_bytes, int32_t* err,
    void* stream) {
  return csa::attn_entry(false, q, rope_cos, rope_sin, rope_dim, rope_offset, cmp_kv,
                         num_cmp_blocks, cmp_block_table, max_cmp_blocks, topk_idx, k, ratio,
                         win_kv, num_win_blocks, win_block_table, max_win_blocks, window,
                         attn_sink, softmax_scale, query_start_loc, positions, B, T, num_tokens,
                         H, D, out, lse, workspace, workspace_bytes, err, stream);
}

extern "C" int csa_sparse_attn_prefill(
    const uint16_t* q, const float* rope_cos, const float* rope_sin, int32_t rope_dim,
    int32_t rope_offset, const uint16_t* cmp_kv, int32_t num_cmp_blocks,
    const int32_t* cmp_block_table, int32_t max_cmp_blocks, const int32_t* topk_idx, int32_t k,
    int32_t ratio, const uint16_t* win_kv, int32_t num_win_blocks,
    const int32_t* win_block_table, int32_t max_win_blocks, int32_t window,
    const float* attn_sink, float softmax_scale, const int32_t* query_start_loc,
    const int32_t* positions, int32_t B, int32_t T, int32_t num_tokens, int32_t H, int32_t D,
    uint16_t* out, float* lse, void* workspace, size_t workspace_bytes, int32_t* err,
    void* stream) {
  return csa::attn_entry(true, q, rope_cos, rope_sin, rope_dim, rope_offset, cmp_kv,
                         num_cmp_blocks, cmp_block_table, max_cmp_blocks, topk_idx, k, ratio,
                         win_kv, num_win_blocks, win_block_table, max_win_blocks, window,
                         attn_sink, softmax_scale, query_start_loc, positions, B, T, num_tokens,
                         H, D, out, lse, workspace, workspace_bytes, err, stream);
}

extern "C" const char* csa_status_string(int status) {
  switch (status) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_NULL: return "CSA_ERR_NULL: a required pointer is NULL";
    case CSA_ERR_SHAPE: return "CSA_ERR_SHAPE: a size is negative or inconsistent";
    case CSA_ERR_RANGE: return "CSA_ERR_RANGE: num_tokens, k or ratio out of range";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED: shape or alignment without a kernel";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE: workspace missing or too small";
    case CSA_ERR_LAUNCH: return "CSA_ERR_LAUNCH: the HIP runtime refused a launch";
    default: return "unknown csa_status";
  }
}
