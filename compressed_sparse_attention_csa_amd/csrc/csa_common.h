// Device helpers shared by the CSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

constexpr int kPage = CSA_PAGE;  // tokens per cache block

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef unsigned short v4us __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Two floats -> packed bf16 pair (lo in bits 0-15) with gfx950's conversion
// instruction, round to nearest even.
typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f_t{lo, hi}, v2bf_t));
}

// float -> bf16 bits with the same instruction, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Compressed slots visible to a query at absolute position p: c < (p+1)/ratio.
__device__ __forceinline__ int visible_count(int p, int ratio) {
  return p < 0 ? 0 : (p + 1) / ratio;
}

// Request owning packed row t (query_start_loc is nondecreasing, B+1 long);
// -1 when no request owns it.
__device__ __forceinline__ int owner_request(const int32_t* __restrict__ qsl, int B, int t) {
  if (B <= 0 || t < qsl[0] || t >= qsl[B]) return -1;
  int lo = 0, hi = B;  // invariant: qsl[lo] <= t < qsl[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (qsl[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// owner_request with one memory round trip when B < 64, in two halves so
// other loads can be issued between them: every lane of the wave loads one
// entry of query_start_loc, then a ballot counts the entries <= t.  Both
// halves must be called by all 64 lanes of a wave with the same t.
__device__ __forceinline__ int qsl_lane_load(const int32_t* __restrict__ qsl, int B) {
  const int lane = threadIdx.x & 63;
  return (B < 64 && lane <= B) ? qsl[lane] : 0x7fffffff;
}

__device__ __forceinline__ int owner_from_lanes(int v, const int32_t* __restrict__ qsl, int B,
                                                int t) {
  if (B >= 64) return owner_request(qsl, B, t);
  if (B <= 0) return -1;
  const int lane = threadIdx.x & 63;
  const uint64_t le = __ballot(v <= t);
  const int first = __builtin_amdgcn_readfirstlane(lane == 0 ? v : 0);
  const int last = __builtin_amdgcn_readlane(v, B);
  if (t < first || t >= last) return -1;
  return __popcll(le) - 1;   // qsl is nondecreasing: the entries <= t are a prefix
}

__device__ __forceinline__ int owner_request_wave(const int32_t* __restrict__ qsl, int B, int t) {
  return owner_from_lanes(qsl_lane_load(qsl, B), qsl, B, t);
}

__device__ __forceinline__ void flag_error(int32_t* err, int bits) {
  if (err != nullptr && bits) atomicOr(err, bits);
}

// Pool row of request-local position c through a 128-token block table;
// -1 when the page lies past the table or names an invalid block.
__device__ __forceinline__ long long page_row(const int32_t* __restrict__ bt_row,
                                              int max_blocks, int num_blocks, int c) {
  int page = c / kPage;
  if (page >= max_blocks) return -1;
  int blk = bt_row[page];
  if (blk < 0 || blk >= num_blocks) return -1;
  return static_cast<long long>(blk) * kPage + (c % kPage);
}

// Wave-wide xor shuffle (wave64).
__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Reductions with lane l ^ 16 and lane l ^ 32 on the VALU (gfx950 lane
// swaps; a shuffle through ds_bpermute costs an LDS round trip).  With both
// operands equal, the permlane32 swap returns lane l's and lane l ^ 32's
// values in its two results (in some order), and the permlane16 swap does
// the same for l ^ 16 within each 32-lane half.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Whole-wave max and sum on the VALU: DPP quad swaps and row mirrors combine
// the 16 lanes of a row, then the two lane swaps above.  Every lane ends with
// the same value (each step adds or compares symmetric pairs).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xb1>(v));    // quad_perm 1,0,3,2: lane ^ 1
  v = fmaxf(v, dpp_f<0x4e>(v));    // quad_perm 2,3,0,1: lane ^ 2
  v = fmaxf(v, dpp_f<0x141>(v));   // row_half_mirror: the other quad of 8
  v = fmaxf(v, dpp_f<0x140>(v));   // row_mirror: the other half of 16
  return max_xor32(max_xor16(v));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xb1>(v);
  v += dpp_f<0x4e>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return sum_xor32(sum_xor16(v));
}

// Work-group barrier that orders LDS only.  A __syncthreads() is a
// work-group release/acquire and waits for every vector-memory operation in
// flight (vmcnt(0)), direct-to-LDS loads and prefetches included; here each
// wave waits for its own LDS operations only (lgkmcnt(0)), and the caller
// waits explicitly (vmcnt) for exactly the loads the next phase reads.  The
// signal fences keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt immediate that waits until at most N vector-memory operations are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace csa
