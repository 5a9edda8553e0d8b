// Lightning-indexer scores on CDNA4 INT8 MFMA.
//
// Method: gitcode hyper-parallel issue #2 (DeepSeek V4 CP notes), sections
// 10.2 / 10.3 -- per query row, score every causally visible compressed slot
// c < (p+1)/ratio with the indexer; pypto-lib "DeepSeek V4-Flash, MTP point",
// section "What is quantized" -- index keys are INT8 with an FP32 per-row
// scale.  Score = sum_h w[t,h] * relu(qs[t,h] * ks[c] * <q8[t,h], k8[c]>).
//
// Mapping.  Work-groups are (request, up to 4 of its rows) x (a run of
// 128-key pages); wave w owns one query row and computes its 64 heads as
// 32x32x32 INT8 MFMA tiles (M = 32 heads, N = 32 keys, K = Di in 32-byte
// steps), so a key page staged once in LDS feeds every row of the group.
// Pages stream through a 3-stage LDS ring filled by direct-to-LDS loads (two
// pages in flight behind the one being scored, three work-groups per CU);
// the barriers between pages order LDS only, so the loads stay in flight
// across them.  LDS rows are 128 bytes with XOR-swizzled 16-byte chunks
// (conflict-free operand reads), the swizzle applied by choosing each lane's
// source chunk.  INT32 accumulators stay in registers and start from a bias
// that makes ReLU one clamped float add (see the page loop); the folded
// weight w*qs of each head follows in one FMA, a cross-lane swap (gfx950
// permlane32) finishes the head sum of each key, and each lane scales its
// two keys by ks and stores them.  Pages past every row's visible span only
// receive -inf.
#include <algorithm>
#include <type_traits>

#include "csa_common.h"

namespace csa {

namespace {

constexpr int kRowsPerWG = 4;
constexpr int kThreads = 256;
constexpr int kRowBytes = 128;   // LDS bytes per key (Di <= 128, padded)
constexpr int kMaxPPW = 64;      // pages per work-group
constexpr int kStages = 3;       // key pages resident in LDS (in flight or in use)
constexpr int kLoadsPerWave = kPage * kRowBytes / (64 * 16) / (kThreads / 64);  // per page
constexpr int kVmPerPage = kLoadsPerWave + 1;   // + one load of 32 key scales
#ifndef CSA_IDX_WPE
#define CSA_IDX_WPE 3
#endif
#ifndef CSA_IDX_DB
#define CSA_IDX_DB 0
#endif
constexpr int kIdxWaves = CSA_IDX_WPE;       // waves per SIMD (work-groups per CU)
constexpr bool kIdxDB = CSA_IDX_DB != 0;     // key operands double-buffered by key tile

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

// s_waitcnt for "at most n vector-memory operations outstanding", n known at
// run time (small): one case per immediate.
__device__ __forceinline__ void wait_vm_rt(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break;
    case 16: wait_vmcnt<16>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// LDS address of a __shared__ object, and LDS reads the compiler does not
// track (the caller waits with an explicit lgkmcnt that names the result).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}
__device__ __forceinline__ void lds_read_b128(v4i& d, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1" : "=v"(d) : "v"(addr));
}
__device__ __forceinline__ void lds_read_b32(uint32_t& d, uint32_t addr) {
  asm volatile("ds_read_b32 %0, %1" : "=v"(d) : "v"(addr));
}
// ds_read_b128 at addr + OFF, OFF an immediate (16-bit instruction offset)
template <int OFF>
__device__ __forceinline__ void lds_read_b128_at(v4i& d, uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF));
}

__device__ __forceinline__ float lane_add_swap32(float x, float y) {
  // lanes 0-31: x[l] + x[l+32]; lanes 32-63: y[l-32] + y[l]
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// FP4: the MXFP4 index plane -- query and key rows are packed E2M1 (Di/2
// bytes) and the FP32 scale slots hold four E8M0 bytes, one per 32 dims; the
// dots run on the scaled FP4 MFMA with those bytes as its block scales.
__device__ __forceinline__ v8i lo_v8i(v4i x) {
  return __builtin_shufflevector(x, v4i{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
}

// FP8: the FP8 index plane -- E4M3 codes in the INT8 plane's layout (Di
// bytes per row, FP32 per-row key and per-(row, head) query scales); the
// dots run on the block-scaled FP8 MFMA with unit block scales, each 64-dim
// operand being two of the INT8 path's 32-dim fragments (a dot does not
// depend on the order of its terms, and both operands pair the same dims).
template <int KK, bool FP4, bool FP8 = false>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kIdxWaves, kIdxWaves))) index_score_kernel(
    const int8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ head_w, const int8_t* __restrict__ idx_kv,
    const float* __restrict__ idx_scale, int num_blocks, const int32_t* __restrict__ bt,
    int max_blocks, const int32_t* __restrict__ qsl, const int32_t* __restrict__ positions,
    int B, int num_tokens, int Hi, int Di, int ratio, float* __restrict__ scores,
    long long stride, int pages_per_wg, int32_t* err) {
  // one array per ring stage: with a single array indexed by a run-time
  // stage, the compiler cannot tell which stage a direct-to-LDS load writes
  // and drains every load in flight before each LDS read of keys
  __shared__ __attribute__((aligned(16))) int8_t keys0[kPage * kRowBytes];
  __shared__ __attribute__((aligned(16))) int8_t keys1[kPage * kRowBytes];
  __shared__ __attribute__((aligned(16))) int8_t keys2[kPage * kRowBytes];
  __shared__ __attribute__((aligned(16))) float ks0[kPage];
  __shared__ __attribute__((aligned(16))) float ks1[kPage];
  __shared__ __attribute__((aligned(16))) float ks2[kPage];
  __shared__ int blk_s[kMaxPPW];
  __shared__ int nvis_s[kRowsPerWG];
  __shared__ int scratch[kThreads / 64 + 2];
  // folded head weights of the group's rows, [row][head] (w * qs * 2^21 for
  // INT8, w * qs for FP8, w for FP4): one coalesced load per thread with the
  // rows' metadata, read back by each wave in its MFMA result order
  __shared__ __attribute__((aligned(16))) float ww_s[kRowsPerWG * 64];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases in SGPRs
  const int lane = tid & 63;
  // direct-to-LDS loads per wave per page (FP4 rows take 64 LDS bytes, INT8
  // rows 128), and vector-memory operations per page with the scale load
  constexpr int LPWv = FP4 ? kLoadsPerWave / 2 : kLoadsPerWave;
  constexpr int VMPv = LPWv + 1;
  const long long stride_pages = (stride + kPage - 1) / kPage;
  const int page0 = blockIdx.x * pages_per_wg;
  const int npages = static_cast<int>(min(static_cast<long long>(pages_per_wg),
                                          stride_pages - page0));
  if (npages <= 0) return;
  const float neg_inf = -__builtin_huge_valf();

  // The request and rows of work-group y, with the positions of those rows and
  // the block ids of this run's pages.  First guess that the B requests own
  // equal runs of rows from row 0 (qsl[b] = b * num_tokens / B, the usual
  // decode batch): the guessed rows' positions and block ids are then fetched
  // in the same round trip as query_start_loc, and the guess is checked
  // against every entry of it.  Otherwise the groups are located by a scan
  // over query_start_loc and the rows' metadata fetched after it.
  // Groups are taken in reverse launch order: in a causal prefill a later
  // group sees more pages, so its work-groups are dispatched first and the
  // short ones fill in behind them instead of trailing them.
  const int gy = static_cast<int>(gridDim.y) - 1 - static_cast<int>(blockIdx.y);
  int row0 = 0, nrows = 0, b = -1;
  int pos_v = 0, blk_v = -1;
  // thread tid's element of ww_s: row tid / 64 of the group, head tid % 64
  const int w_row = tid >> 6, w_head = tid & 63;
  float hw_v = 0.0f, qs_v = 0.0f;
  auto load_w = [&](int r0w, int nrw) {
    if (w_row < nrw && w_head < Hi) {
      const long long hc = static_cast<long long>(r0w + w_row) * Hi + w_head;
      hw_v = head_w[hc];
      if constexpr (!FP4) qs_v = q_scale[hc];
    }
  };
  bool located = false;
  if (B > 0 && B < kThreads && num_tokens % B == 0) {
    const int R = num_tokens / B;
    const int gpr = (R + kRowsPerWG - 1) / kRowsPerWG;   // groups per request
    const int bg = gy / gpr;
    const int r0 = bg * R + (gy % gpr) * kRowsPerWG;
    const int nr = bg < B ? min(kRowsPerWG, (bg + 1) * R - r0) : 0;
    const int qv = tid <= B ? min(max(qsl[tid], 0), num_tokens) : 0;
    if (tid < nr) pos_v = positions[r0 + tid];
    load_w(r0, nr);
    if (bg < B && tid < npages) {
      const int page = page0 + tid;
      blk_v = (page < max_blocks) ? bt[static_cast<long long>(bg) * max_blocks + page] : -1;
    }
    const bool ok = __all(tid > B || qv == tid * R);
    if (lane == 0) scratch[wave] = ok ? 1 : 0;
    lds_barrier();
    bool all_ok = true;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) all_ok = all_ok && scratch[w] != 0;
    if (all_ok) {
      if (bg >= B) return;   // every row is owned, and these groups are past them
      located = true;
      b = bg;
      row0 = r0;
      nrows = nr;
    }
  }
  if (!located) {
    b = locate_group(qsl, B, num_tokens, gy, &row0, &nrows, scratch);
    if (b >= 0) {
      pos_v = tid < nrows ? positions[row0 + tid] : 0;
      hw_v = 0.0f;
      qs_v = 0.0f;
      load_w(row0, nrows);
      blk_v = -1;
      if (tid < npages) {
        const int page = page0 + tid;
        blk_v = (page < max_blocks) ? bt[static_cast<long long>(b) * max_blocks + page] : -1;
      }
    }
  }
  if (b < 0) {
    // rows that no request owns: the first groups past the owned ones cover them
    const int owned_end = (B > 0) ? min(max(qsl[B], 0), num_tokens) : 0;
    const int owned_begin = (B > 0) ? min(max(qsl[0], 0), num_tokens) : 0;
    int gfirst = 0;
    for (int bb = 0; bb < B; ++bb) {
      const int lo = min(max(qsl[bb], 0), num_tokens);
      const int hi = min(max(qsl[bb + 1], 0), num_tokens);
      gfirst += hi > lo ? (hi - lo + kRowsPerWG - 1) / kRowsPerWG : 0;
    }
    const int u = gy - gfirst;  // index among unowned 4-row blocks
    const int n_unowned = owned_begin + (num_tokens - owned_end);
    if (u < 0 || u * kRowsPerWG >= n_unowned) return;
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

  // (a block id is used only if its page turns out to be visible to some row)
  if (tid < kRowsPerWG) {
    int n = 0;
    if (tid < nrows) {
      n = visible_count(pos_v, ratio);
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
      blk = blk_v;
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
  const int col = lane & 31;    // MFMA column: key within a 32-key tile
  const int half = lane >> 5;   // which 16-byte half of each 32-dim k-step

  // A operand (this wave's query row: 32-head tiles x 32-dim k-steps, lane
  // (col, half) holding head mt*32 + col, dims ks*32 + half*16 .. +15) and
  // the folded head weights w*qs in the MFMA result order (result j of lane
  // (col, half) is head mt*32 + 8*(j/4) + 4*half + j%4), loaded once, after
  // the first pages' loads are issued
  constexpr int MT = 2;
  // k-steps of 32 bytes: 32 INT8 dims, or 64 FP4 dims (32x32x64 MFMA)
  constexpr int KS = FP4 ? KK : 2 * KK;
  const int RB = FP4 ? Di / 2 : Di;   // bytes per query / key row
  v4i qa[MT][KS];
  float ww[MT][16];
  int sa[MT][KS];   // FP4: the E8M0 byte of lane (col, half)'s 32 dims
  auto load_query = [&]() {
    if (!active) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = mt * 32 + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = ks * 32 + half * 16;
        qa[mt][ks] = (h < Hi && off < RB)
                         ? *reinterpret_cast<const v4i*>(
                               q_idx + (static_cast<long long>(my_t) * Hi + h) * RB + off)
                         : v4i{0, 0, 0, 0};
      }
      if constexpr (FP4) {
        const uint32_t qsw =
            h < Hi ? __float_as_uint(q_scale[static_cast<long long>(my_t) * Hi + h]) : 0u;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sa[mt][ks] = (qsw >> (8 * (ks * 2 + half))) & 0xff;
      }
    }
  };
  // INT8: times 2^21, as the epilogue's ReLU leaves dot * 2^-21 (see the page
  // loop); FP4: the scales are inside the MFMA
  constexpr float kWScale = FP8 ? 1.0f : 2097152.0f;
  ww_s[tid] = (w_row < nrows && w_head < Hi) ? (FP4 ? hw_v : hw_v * qs_v * kWScale) : 0.0f;
  __syncthreads();  // blk_s and ww_s ready (no direct-to-LDS load is in flight yet)
  // result 4q + i of lane (col, half) in M tile mt is head mt*32 + 8q + 4*half
  // + i: four consecutive heads, one 16-byte LDS read (heads past Hi are 0)
  if (active) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 wv =
            *reinterpret_cast<const float4*>(&ww_s[wave * 64 + mt * 32 + 8 * q4 + 4 * half]);
        ww[mt][4 * q4] = wv.x;
        ww[mt][4 * q4 + 1] = wv.y;
        ww[mt][4 * q4 + 2] = wv.z;
        ww[mt][4 * q4 + 3] = wv.w;
      }
  }

  // ---- page pi -> LDS stage pi % kStages with direct-to-LDS loads.  LDS
  //      slot q of a page holds 16-byte chunk (q & 7) ^ ((key >> 1) & 7) of key
  //      q >> 3 (the XOR swizzle that makes the operand reads conflict-free),
  //      so each lane picks its source chunk.  FP4 rows are 64 bytes: slot q
  //      holds chunk (q & 3) ^ ((key >> 2) & 3) of key q >> 2, so sixteen
  //      lanes reading one chunk of sixteen keys touch sixteen different
  //      16-byte bank groups.  Every wave issues exactly LPWv + 1 loads per
  //      page (pages with nothing to stage read a dummy 16 bytes), which keeps
  //      the vmcnt bookkeeping uniform.
  auto keys_of = [&](auto stg) -> int8_t* {
    constexpr int S = decltype(stg)::value;
    if constexpr (S == 0) return keys0;
    else if constexpr (S == 1) return keys1;
    else return keys2;
  };
  auto ks_of = [&](auto stg) -> float* {
    constexpr int S = decltype(stg)::value;
    if constexpr (S == 0) return ks0;
    else if constexpr (S == 1) return ks1;
    else return ks2;
  };
  // byte offset inside a page of this lane's source chunk for the wave's
  // load u: the same for every page (hoisted out of the page loop), so a
  // page's loads take one uniform base and no per-lane address arithmetic.
  // FP4: 64-byte rows, four chunks per key; INT8: 128-byte LDS rows, and a
  // padding slot past Di takes any bytes of the same key.
  auto lane_off = [&](int u) -> uint32_t {
    const int q = (wave * LPWv + u) * 64 + lane;
    const int key = FP4 ? (q >> 2) : (q >> 3);
    int c = FP4 ? ((q & 3) ^ ((key >> 2) & 3)) : ((q & 7) ^ ((key >> 1) & 7));
    c = (c * 16 >= RB) ? 0 : c;
    return static_cast<uint32_t>(key * RB + c * 16);
  };
  auto issue = [&](int pi, auto stg) {
    int8_t* keys = keys_of(stg);
    float* ksd = ks_of(stg);
    const int blk = __builtin_amdgcn_readfirstlane(blk_s[pi]);
    if (blk >= 0) {
      const int8_t* pbase = idx_kv + static_cast<long long>(blk) * kPage * RB;
      const float* sbase = idx_scale + static_cast<long long>(blk) * kPage;
#pragma unroll
      for (int u = 0; u < LPWv; ++u)
        __builtin_amdgcn_global_load_lds(
            pbase + static_cast<int>(lane_off(u)),
            (__attribute__((address_space(3))) void*)(keys + (wave * LPWv + u) * 1024), 16, 0,
            0);
      // key scales: wave w brings keys 32w .. 32w+31, 16 bytes per lane
      // (each active lane writes 16 LDS bytes, so only lanes 0-7 run it)
      if (lane < 8)
        __builtin_amdgcn_global_load_lds(
            sbase + (lane & 7) * 4 + wave * 32,
            (__attribute__((address_space(3))) void*)(ksd + wave * 32), 16, 0, 0);
    } else {
      // nothing to stage: the same number of loads, of 16 valid bytes
#pragma unroll
      for (int u = 0; u < LPWv; ++u)
        __builtin_amdgcn_global_load_lds(
            q_idx, (__attribute__((address_space(3))) void*)(keys + (wave * LPWv + u) * 1024),
            16, 0, 0);
      if (lane < 8)
        __builtin_amdgcn_global_load_lds(
            q_idx, (__attribute__((address_space(3))) void*)(ksd + wave * 32), 16, 0, 0);
    }
  };

  // one page: wait for it, barrier, refill the stage freed by the previous
  // page, score this one
  auto step = [&](int pi, auto stg) {
    constexpr int S = decltype(stg)::value;
    // page pi has landed once only the newer pages and the score stores
    // issued since may still be in flight (vector memory completes in issue
    // order): an active wave issues both of a page's two stores on every
    // page but the last of the score row (only there can the row end cut
    // the second to no lanes), which is the last page of its work-group's
    // run, so no wait comes after it.  Counting every store matters: a
    // count one short per page makes each page wait for the stores of the
    // page two back to reach memory.
    const int newer = min(kStages - 2, npages - 1 - pi);
    wait_vm_rt(__builtin_amdgcn_readfirstlane(VMPv * newer +
                                              (active ? 2 * min(kStages - 1, pi) : 0)));
    lds_barrier();
    const int blk_here = blk_s[pi];   // read before the refill's loads go out
    if (pi + kStages - 1 < npages)
      issue(pi + kStages - 1, std::integral_constant<int, (S + kStages - 1) % kStages>{});
    if (!active) return;
    const int8_t* keys = keys_of(stg);
    const float* ksd = ks_of(stg);
    const int c0 = (page0 + pi) * kPage;
    float* out_row = scores + static_cast<long long>(my_t) * stride + c0;
    float w0 = neg_inf, w1 = neg_inf;
    if (blk_here >= 0 && c0 < my_n) {
      // Key operands come from LDS through inline ds_read instructions with
      // explicit lgkmcnt waits.  The compiler cannot tell a read of this
      // page's stage from the direct-to-LDS loads of the later pages still in
      // flight, and guards a plain LDS read with vmcnt(0), which would make
      // every page wait for the page just requested; this page's own loads
      // are already waited for (the vmcnt wait and barrier above).
      // Each wait names the registers it covers, which orders their uses
      // after it.
      uint32_t kbase = lds_addr(keys);
      uint32_t sbase = lds_addr(ksd);
      // The stage's LDS bases pass through an empty asm, so the per-lane
      // addresses below are formed here, for each page, instead of being
      // hoisted out of the page loop as one live set per stage: those sets
      // spilled, and each reload's vmcnt(0) waited for the next pages' loads.
      asm volatile("" : "+s"(kbase), "+s"(sbase));
      uint32_t ksw0 = 0u, ksw1 = 0u;   // INT8: the FP32 scales of keys lane, 64 + lane
      if constexpr (!FP4) {
        lds_read_b32(ksw0, sbase + 4 * lane);
        lds_read_b32(ksw1, sbase + 4 * (64 + lane));
      }
      // eight (32-head, 32-key) tiles p = 2*nt + mt, each scored as soon as
      // its MFMAs are issued: the epilogue waits for them, and the SIMD's
      // other waves fill that wait.  Key operands are double-buffered by key
      // tile: the reads for tile nt + 1 go out before tile nt's MFMAs, into
      // the set whose MFMAs (tile nt - 1) the epilogue has already waited for.
      float x[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      v4i bk[kIdxDB ? 2 : 1][KS];
      uint32_t kw[kIdxDB ? 2 : 1] = {};   // FP4: the key's E8M0 bytes (its scale slot)
      // Key kj = nt * 32 + col: its swizzle does not depend on nt (32 keys
      // move the XOR pattern by whole periods), so one address per k-step
      // serves every key tile, with the tile's row offset as an immediate
      constexpr int RBL = FP4 ? 64 : kRowBytes;   // LDS bytes per key row
      uint32_t kaddr[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kaddr[ks] = kbase + static_cast<uint32_t>(
                                FP4 ? col * 64 + (((ks * 2 + half) ^ ((col >> 2) & 3)) * 16)
                                    : col * kRowBytes + swz_chunk(col, ks * 2 + half) * 16);
      auto read_b = [&](int nt, int buf) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          switch (nt) {
            case 0: lds_read_b128_at<0>(bk[buf][ks], kaddr[ks]); break;
            case 1: lds_read_b128_at<32 * RBL>(bk[buf][ks], kaddr[ks]); break;
            case 2: lds_read_b128_at<64 * RBL>(bk[buf][ks], kaddr[ks]); break;
            default: lds_read_b128_at<96 * RBL>(bk[buf][ks], kaddr[ks]); break;
          }
        }
        if constexpr (FP4) lds_read_b32(kw[buf], sbase + 4 * (nt * 32 + col));
      };
      // The accumulators start at 0x40800000, the bits of 4.0f.  A dot
      // product of Di <= 128 INT8 pairs lies in [-2^21, 2^21], so the INT32
      // result read as a float is 4 + dot * 2^-21 when dot >= 0 (the
      // mantissa step of [4, 8) is 2^-21) and below 4 otherwise.  One
      // clamped add of -4 (v_add_f32 ... clamp) then gives relu(dot) * 2^-21
      // exactly, in [0, 1], and the weight, pre-scaled by 2^21, multiplies it
      // back: the same product as w * relu(dot), with no separate max and
      // int-to-float conversion (two VALU ops per head and key, not three).
      constexpr int kBias = 0x40800000;
      constexpr v16i kBiasV = {kBias, kBias, kBias, kBias, kBias, kBias, kBias, kBias,
                               kBias, kBias, kBias, kBias, kBias, kBias, kBias, kBias};
      if constexpr (kIdxDB) read_b(0, 0);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int cur = kIdxDB ? (nt & 1) : 0;
        if constexpr (!kIdxDB) {
          // one set: tile nt's reads go out once tile nt - 1's MFMAs are
          // done (its epilogue has consumed their results)
          read_b(nt, 0);
          if constexpr (FP4)
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bk[0][0]), "+v"(bk[0][1]),
                         "+v"(bk[0][2]), "+v"(bk[0][3]), "+v"(kw[0]));
          else
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bk[0][0]), "+v"(bk[0][1]),
                         "+v"(bk[0][2]), "+v"(bk[0][3]), "+v"(ksw0), "+v"(ksw1));
        } else if (nt + 1 < 4) {
          read_b(nt + 1, cur ^ 1);
        }
        // LDS operations complete in order: once at most the next tile's
        // reads are outstanding, this tile's (and the scales') have landed
        if constexpr (!kIdxDB) {
        } else if constexpr (FP4) {
          if (nt + 1 < 4)
            asm volatile("s_waitcnt lgkmcnt(5)" : "+v"(bk[cur][0]), "+v"(bk[cur][1]),
                         "+v"(bk[cur][2]), "+v"(bk[cur][3]), "+v"(kw[cur]));
          else
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bk[cur][0]), "+v"(bk[cur][1]),
                         "+v"(bk[cur][2]), "+v"(bk[cur][3]), "+v"(kw[cur]));
        } else {
          if (nt == 0)
            asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(bk[0][0]), "+v"(bk[0][1]),
                         "+v"(bk[0][2]), "+v"(bk[0][3]), "+v"(ksw0), "+v"(ksw1));
          else if (nt + 1 < 4)
            asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(bk[cur][0]), "+v"(bk[cur][1]),
                         "+v"(bk[cur][2]), "+v"(bk[cur][3]));
          else
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(bk[cur][0]), "+v"(bk[cur][1]),
                         "+v"(bk[cur][2]), "+v"(bk[cur][3]));
        }
        int sb[KS];
        if constexpr (FP4) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) sb[ks] = (kw[cur] >> (8 * (ks * 2 + half))) & 0xff;
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          float xs = x[nt];
          if constexpr (FP4) {
            // FP32 dots of the dequantised rows (E2M1 values, E8M0 scales of
            // each 32 dims applied by the MFMA); ReLU and the head weight
            const v16f zero16 = {};
            v16f accf;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              accf = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  lo_v8i(qa[mt][ks]), lo_v8i(bk[cur][ks]), ks == 0 ? zero16 : accf, 4, 4, 0,
                  sa[mt][ks], 0, sb[ks]);
#pragma unroll
            for (int j = 0; j < 16; ++j) xs = fmaf(ww[mt][j], fmaxf(accf[j], 0.0f), xs);
          } else if constexpr (FP8) {
            // FP32 dots of the E4M3 rows (block scales 2^0), ReLU, head weight
            const v16f zero16 = {};
            v16f accf;
#pragma unroll
            for (int s2 = 0; s2 < KS / 2; ++s2) {
              const v8i a8 = __builtin_shufflevector(qa[mt][2 * s2], qa[mt][2 * s2 + 1], 0, 1, 2,
                                                     3, 4, 5, 6, 7);
              const v8i b8 = __builtin_shufflevector(bk[cur][2 * s2], bk[cur][2 * s2 + 1], 0, 1,
                                                     2, 3, 4, 5, 6, 7);
              accf = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  a8, b8, s2 == 0 ? zero16 : accf, 0, 0, 0, 127, 0, 127);
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) xs = fmaf(ww[mt][j], fmaxf(accf[j], 0.0f), xs);
          } else {
            v16i acc;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[mt][ks], bk[cur][ks],
                                                          ks == 0 ? kBiasV : acc, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 16; ++j)
              xs = fmaf(ww[mt][j],
                        __builtin_amdgcn_fmed3f(__int_as_float(acc[j]) - 4.0f, 0.0f, 1.0f), xs);
          }
          x[nt] = xs;
        }
      }
      // head sums: lanes l and l + 32 hold the two 32-head halves of the
      // same key, so one swap per key pair finishes them; lane l of w0 ends
      // with key l of this page, of w1 with key 64 + l
      w0 = lane_add_swap32(x[0], x[1]);
      w1 = lane_add_swap32(x[2], x[3]);
      // adding +0.0 turns a -0.0 score into +0.0 (one zero) and leaves every
      // other value unchanged; it folds into the scale multiply as an FMA
      const int vis = my_n - c0;   // visible keys of this page (> 0 here)
      w0 = (lane < vis) ? (FP4 ? w0 + 0.0f : fmaf(__uint_as_float(ksw0), w0, 0.0f)) : neg_inf;
      w1 = (64 + lane < vis) ? (FP4 ? w1 + 0.0f : fmaf(__uint_as_float(ksw1), w1, 0.0f))
                             : neg_inf;
    }
    // the score row ends at stride (a page may reach past it)
    const int lim = static_cast<int>(min(static_cast<long long>(kPage), stride - c0));
    if (lane < lim) out_row[lane] = w0;
    if (64 + lane < lim) out_row[64 + lane] = w1;
  };

  static_assert(kStages == 3, "the page loop is unrolled over three stages");
  if (npages > 0) issue(0, std::integral_constant<int, 0>{});
  if (npages > 1) issue(1, std::integral_constant<int, 1>{});
  // the query loads go after the first pages' loads, so their latencies
  // overlap (the first page's wait then also covers them: vector memory
  // completes in issue order)
  load_query();
  for (int pi = 0; pi < npages; pi += kStages) {
    step(pi, std::integral_constant<int, 0>{});
    if (pi + 1 < npages) step(pi + 1, std::integral_constant<int, 1>{});
    if (pi + 2 < npages) step(pi + 2, std::integral_constant<int, 2>{});
  }
}

// ---------------------------------------------------------------------------
// Reindex scoring: the same score, evaluated only at the slots of each row's
// candidate mask (pypto-lib "DeepSeek V4.1 Flash", section "Decode
// composition": reindex layers score with their own index query inside the
// full layer's candidate blocks).  Slot s of row t is position
// cand[t][s / block] * block + s % block.  A work-group scores 256 slots of
// one row, 64 per wave, as the 32x32x32 INT8 MFMA tiles and biased-
// accumulator epilogue of index_score_kernel in the same order, so a slot's
// score is bit-identical to the full scorer's at that position.  Keys are
// gathered straight into operand registers (each lane 16 bytes of one key).
constexpr int kCandSlots = 256;   // slots per work-group

template <int KS>
__global__ void __launch_bounds__(kThreads) index_cand_kernel(
    const int8_t* __restrict__ q_idx, const float* __restrict__ q_scale,
    const float* __restrict__ head_w, const int8_t* __restrict__ idx_kv,
    const float* __restrict__ idx_scale, int num_blocks, const int32_t* __restrict__ bt,
    int max_blocks, const int32_t* __restrict__ qsl, const int32_t* __restrict__ positions,
    int B, int num_tokens, int Hi, int Di, int ratio, const int32_t* __restrict__ cand, int kb,
    int block, float* __restrict__ out, long long ostride, int32_t* __restrict__ count,
    int32_t* err) {
  __shared__ long long base_s[kCandSlots];   // pool row of an entry's first slot, or -1
  __shared__ int elig_s[kCandSlots];         // eligible leading slots of the entry
  __shared__ int err_s;
  const int t = blockIdx.y;
  if (t >= num_tokens) return;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int nslot = kb * block;
  const int s0 = blockIdx.x * kCandSlots;
  const int e0 = s0 / block;                 // first mask entry of this work-group
  const int ne = kCandSlots / block;         // entries it covers
  if (tid == 0) err_s = 0;

  // metadata, this work-group's mask entries (and the entry before them),
  // then the query: nothing here depends on another load
  const int qsl_v = qsl_lane_load(qsl, B);
  const int p = positions[t];
  const int32_t* crow = cand + static_cast<long long>(t) * kb;
  const int my_e = e0 + tid;
  const int cb = (tid < ne && my_e < kb) ? crow[my_e] : -1;
  const int prev_cb = (s0 > 0) ? crow[e0 - 1] : -1;
  v4i qa[2][KS];
  float ww[2][16];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int h = mt * 32 + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = ks * 32 + half * 16;
      qa[mt][ks] = (h < Hi && off < Di)
                       ? *reinterpret_cast<const v4i*>(
                             q_idx + (static_cast<long long>(t) * Hi + h) * Di + off)
                       : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int hh = mt * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
      // unguarded loads of a valid head, then the select (one round trip)
      const long long hc = static_cast<long long>(t) * Hi + (hh < Hi ? hh : 0);
      const float wv = head_w[hc] * q_scale[hc] * 2097152.0f;
      ww[mt][j] = (hh < Hi) ? wv : 0.0f;
    }
  }
  const int b = owner_from_lanes(qsl_v, qsl, B, t);
  const int nv = (b >= 0) ? visible_count(p, ratio) : 0;

  // ---- each mask entry: visibility, then its page through the block table
  int ebits = 0;
  if (tid < ne) {
    long long base = -1;
    int elig = 0;
    if (cb >= 0 && my_e < kb) {
      const long long c = static_cast<long long>(cb) * block;
      if (c >= nv) {
        if (b >= 0) ebits |= CSA_EFLAG_TOPK_RANGE;   // a candidate the row may not see
      } else {
        const long long r = page_row(bt + static_cast<long long>(b) * max_blocks, max_blocks,
                                     num_blocks, static_cast<int>(c));
        if (r >= 0) {
          base = r;
          elig = static_cast<int>(min(static_cast<long long>(block), nv - c));
        } else {
          ebits |= CSA_EFLAG_BLOCK_RANGE;
        }
      }
    }
    base_s[tid] = base;
    elig_s[tid] = elig;
  }
  if (ebits) atomicOr(&err_s, ebits);
  __syncthreads();

  // ---- the row's eligible slots form a prefix when the mask ascends with
  //      trailing -1 (as csa_candidate_blocks writes it); the work-group that
  //      holds its end (with the slot before its range eligible) records it
  if (tid == 0) {
    const bool prev_full =
        s0 == 0 || (b >= 0 && prev_cb >= 0 &&
                    (static_cast<long long>(prev_cb) + 1) * block <= static_cast<long long>(nv));
    if (prev_full && b >= 0) {
      int c = -1;
      for (int e = 0; e < ne; ++e) {
        if (e0 + e >= kb || elig_s[e] < block) {
          c = min(nslot, s0 + e * block + (e0 + e < kb ? elig_s[e] : 0));
          break;
        }
      }
      if (c >= 0 || s0 + kCandSlots >= nslot) count[t] = c >= 0 ? c : nslot;
    } else if (b < 0 && s0 == 0) {
      count[t] = 0;
    }
    if (err_s) flag_error(err, err_s);
    if (b < 0 && s0 == 0) flag_error(err, CSA_EFLAG_META);
  }

  // ---- this wave's 64 slots: key of B-operand column kj, and (for the
  //      epilogue) the slot of lane l
  const int neg_bits = 0xff800000;
  const float neg_inf = __int_as_float(neg_bits);
  auto slot_row = [&](int sl, bool& ok) -> long long {
    const int e = sl / block - e0;
    const int o = sl - (e0 + e) * block;
    ok = sl < nslot && e < ne && o < elig_s[e];
    return ok ? base_s[e] + o : 0;
  };
  v4i bk[2][KS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    bool ok;
    const long long r = slot_row(s0 + wave * 64 + nt * 32 + col, ok);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = ks * 32 + half * 16;
      bk[nt][ks] = (ok && off < Di)
                       ? *reinterpret_cast<const v4i*>(idx_kv + r * Di + off)
                       : v4i{0, 0, 0, 0};
    }
  }
  bool my_ok;
  const int my_slot = s0 + wave * 64 + lane;
  const long long my_row = slot_row(my_slot, my_ok);
  const float my_ks = my_ok ? idx_scale[my_row] : 0.0f;

  constexpr int kBias = 0x40800000;
  constexpr v16i kBiasV = {kBias, kBias, kBias, kBias, kBias, kBias, kBias, kBias,
                           kBias, kBias, kBias, kBias, kBias, kBias, kBias, kBias};
  float x[2] = {0.0f, 0.0f};
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    const int nt = pt >> 1, mt = pt & 1;
    v16i acc;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[mt][ks], bk[nt][ks],
                                                  ks == 0 ? kBiasV : acc, 0, 0, 0);
    float xs = x[nt];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      xs = fmaf(ww[mt][j], __builtin_amdgcn_fmed3f(__int_as_float(acc[j]) - 4.0f, 0.0f, 1.0f),
                xs);
    x[nt] = xs;
  }
  // lanes l and l + 32 hold the two 32-head halves of a key: after the swap
  // lane l holds the head sum of slot l of this wave
  float w = lane_add_swap32(x[0], x[1]);
  w = my_ok ? my_ks * w : neg_inf;
  if (w == 0.0f) w = 0.0f;   // one zero: +0.0
  if (my_slot < nslot) out[static_cast<long long>(t) * ostride + my_slot] = w;
}

}  // namespace

}  // namespace csa

namespace {
template <bool FP8>
int index_entry(const int8_t* q_idx, const float* q_scale, const float* head_w,
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
  // one resident round of work-groups (three per CU on 256 CUs): short rows
  // put every page in flight at once, long rows stream through each
  // work-group's page ring; a grid just past one round would leave a
  // straggler round, so pages per work-group round up
  // (the group count is estimated from below: every request owns at least
  // one group, and four rows fill one; decode batches of 2-row requests
  // have B groups, not num_tokens / 4)
  constexpr long long kSlots = csa::kIdxWaves * 256;
  const long long groups_est = std::max<long long>((num_tokens + 3) / 4, std::min(B, num_tokens));
  long long ppw = (pages * groups_est + kSlots - 1) / kSlots;
  if (ppw < 1) ppw = 1;
  if (ppw > csa::kMaxPPW) ppw = csa::kMaxPPW;
  const long long gx = (pages + ppw - 1) / ppw;
  if (gx > 0x7fffffffll || groups > 65535) return CSA_ERR_UNSUPPORTED;
  dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(groups));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (Di <= 64) {
    hipLaunchKernelGGL((csa::index_score_kernel<1, false, FP8>), grid, dim3(csa::kThreads), 0, st, q_idx,
                       q_scale, head_w, idx_kv, idx_scale, num_blocks, block_table, max_blocks,
                       query_start_loc, positions, B, num_tokens, Hi, Di, ratio, scores,
                       static_cast<long long>(score_stride), static_cast<int>(ppw), err);
  } else {
    hipLaunchKernelGGL((csa::index_score_kernel<2, false, FP8>), grid, dim3(csa::kThreads), 0, st, q_idx,
                       q_scale, head_w, idx_kv, idx_scale, num_blocks, block_table, max_blocks,
                       query_start_loc, positions, B, num_tokens, Hi, Di, ratio, scores,
                       static_cast<long long>(score_stride), static_cast<int>(ppw), err);
  }
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}

}  // namespace

extern "C" int csa_index_score(const int8_t* q_idx, const float* q_scale, const float* head_w,
                               const int8_t* idx_kv, const float* idx_scale, int32_t num_blocks,
                               const int32_t* block_table, int32_t max_blocks,
                               const int32_t* query_start_loc, const int32_t* positions,
                               int32_t B, int32_t T, int32_t num_tokens, int32_t Hi, int32_t Di,
                               int32_t ratio, float* scores, int64_t score_stride, int32_t* err,
                               void* stream) {
  return index_entry<false>(q_idx, q_scale, head_w, idx_kv, idx_scale, num_blocks, block_table,
                            max_blocks, query_start_loc, positions, B, T, num_tokens, Hi, Di,
                            ratio, scores, score_stride, err, stream);
}

extern "C" int csa_index_score_fp8(const uint8_t* q_fp8, const float* q_scale,
                                   const float* head_w, const uint8_t* idx_fp8,
                                   const float* idx_scale, int32_t num_blocks,
                                   const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* query_start_loc, const int32_t* positions,
                                   int32_t B, int32_t T, int32_t num_tokens, int32_t Hi,
                                   int32_t Di, int32_t ratio, float* scores,
                                   int64_t score_stride, int32_t* err, void* stream) {
  return index_entry<true>(reinterpret_cast<const int8_t*>(q_fp8), q_scale, head_w,
                           reinterpret_cast<const int8_t*>(idx_fp8), idx_scale, num_blocks,
                           block_table, max_blocks, query_start_loc, positions, B, T, num_tokens,
                           Hi, Di, ratio, scores, score_stride, err, stream);
}

extern "C" int csa_index_score_candidates(
    const int8_t* q_idx, const float* q_scale, const float* head_w, const int8_t* idx_kv,
    const float* idx_scale, int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
    const int32_t* query_start_loc, const int32_t* positions, int32_t B, int32_t T,
    int32_t num_tokens, int32_t Hi, int32_t Di, int32_t ratio, const int32_t* cand_blocks,
    int32_t kb, int32_t block, float* cand_scores, int64_t cand_stride, int32_t* cand_count,
    int32_t* err, void* stream) {
  if (T < 0 || B < 0 || num_blocks < 0 || max_blocks < 0 || cand_stride < 0) return CSA_ERR_SHAPE;
  if (num_tokens < 0 || num_tokens > T || ratio < 1 || kb < 1 || block < 1 || block > 128 ||
      (csa::kPage % block) != 0 || cand_stride < static_cast<int64_t>(kb) * block ||
      static_cast<long long>(kb) * block > (1ll << 30))
    return CSA_ERR_RANGE;
  if (num_tokens == 0) return CSA_OK;
  if (!q_idx || !q_scale || !head_w || !query_start_loc || !positions || !cand_blocks ||
      !cand_scores || !cand_count)
    return CSA_ERR_NULL;
  if (num_blocks > 0 && max_blocks > 0 && B > 0 && (!idx_kv || !idx_scale || !block_table))
    return CSA_ERR_NULL;
  if (Hi < 1 || Hi > 64 || Di < 16 || Di > 128 || (Di % 16) != 0) return CSA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(q_idx) | reinterpret_cast<uintptr_t>(idx_kv)) & 15)
    return CSA_ERR_UNSUPPORTED;
  if (static_cast<long long>(num_blocks) * csa::kPage * Di >= (1ll << 40)) return CSA_ERR_SHAPE;
  const long long nslot = static_cast<long long>(kb) * block;
  const long long gx = (nslot + csa::kCandSlots - 1) / csa::kCandSlots;
  if (num_tokens > 65535) return CSA_ERR_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(num_tokens));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (Di <= 64) {
    hipLaunchKernelGGL(csa::index_cand_kernel<2>, grid, dim3(csa::kThreads), 0, st, q_idx,
                       q_scale, head_w, idx_kv, idx_scale, num_blocks, block_table, max_blocks,
                       query_start_loc, positions, B, num_tokens, Hi, Di, ratio, cand_blocks, kb,
                       block, cand_scores, static_cast<long long>(cand_stride), cand_count, err);
  } else {
    hipLaunchKernelGGL(csa::index_cand_kernel<4>, grid, dim3(csa::kThreads), 0, st, q_idx,
                       q_scale, head_w, idx_kv, idx_scale, num_blocks, block_table, max_blocks,
                       query_start_loc, positions, B, num_tokens, Hi, Di, ratio, cand_blocks, kb,
                       block, cand_scores, static_cast<long long>(cand_stride), cand_count, err);
  }
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}

extern "C" int csa_index_score_mxfp4(const uint8_t* q_fp4, const uint8_t* q_sc,
                                     const float* head_w, const uint8_t* idx_fp4,
                                     const uint8_t* idx_sc, int32_t num_blocks,
                                     const int32_t* block_table, int32_t max_blocks,
                                     const int32_t* query_start_loc, const int32_t* positions,
                                     int32_t B, int32_t T, int32_t num_tokens, int32_t Hi,
                                     int32_t Di, int32_t ratio, float* scores,
                                     int64_t score_stride, int32_t* err, void* stream) {
  if (T < 0 || B < 0 || num_blocks < 0 || max_blocks < 0 || score_stride < 0) return CSA_ERR_SHAPE;
  if (num_tokens < 0 || num_tokens > T || ratio < 1) return CSA_ERR_RANGE;
  if (num_tokens == 0 || score_stride == 0) return CSA_OK;
  if (!q_fp4 || !q_sc || !head_w || !query_start_loc || !positions || !scores)
    return CSA_ERR_NULL;
  if (num_blocks > 0 && max_blocks > 0 && B > 0 && (!idx_fp4 || !idx_sc || !block_table))
    return CSA_ERR_NULL;
  if (Hi < 1 || Hi > 64 || Di != 128) return CSA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(q_fp4) | reinterpret_cast<uintptr_t>(idx_fp4) |
       reinterpret_cast<uintptr_t>(q_sc) | reinterpret_cast<uintptr_t>(idx_sc)) & 15)
    return CSA_ERR_UNSUPPORTED;
  if (static_cast<long long>(num_blocks) * csa::kPage * Di >= (1ll << 40)) return CSA_ERR_SHAPE;
  const long long pages = (score_stride + csa::kPage - 1) / csa::kPage;
  const long long groups = (num_tokens + 3) / 4 + B;
  constexpr long long kSlots = csa::kIdxWaves * 256;
  const long long groups_est = std::max<long long>((num_tokens + 3) / 4, std::min(B, num_tokens));
  long long ppw = (pages * groups_est + kSlots - 1) / kSlots;
  if (ppw < 1) ppw = 1;
  if (ppw > csa::kMaxPPW) ppw = csa::kMaxPPW;
  const long long gx = (pages + ppw - 1) / ppw;
  if (gx > 0x7fffffffll || groups > 65535) return CSA_ERR_UNSUPPORTED;
  dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(groups));
  // the E8M0 bytes of a row (Di / 32 = 4) travel in the FP32 scale slots
  hipLaunchKernelGGL((csa::index_score_kernel<2, true>), grid, dim3(csa::kThreads), 0,
                     static_cast<hipStream_t>(stream), reinterpret_cast<const int8_t*>(q_fp4),
                     reinterpret_cast<const float*>(q_sc), head_w,
                     reinterpret_cast<const int8_t*>(idx_fp4),
                     reinterpret_cast<const float*>(idx_sc), num_blocks, block_table, max_blocks,
                     query_start_loc, positions, B, num_tokens, Hi, Di, ratio, scores,
                     static_cast<long long>(score_stride), static_cast<int>(ppw), err);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}
