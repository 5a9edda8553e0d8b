// RoPE-row materialisation: pypto-lib "DeepSeek V4.1 Flash", section
// "Serving-owned full RoPE tables" -- gather FP32 half-width rows of
// caller-owned tables for the active token rows; a negative position writes
// the identity rotation; padding rows stay untouched.
#include "csa_common.h"

namespace csa {

// One thread per (row, column) element; a pure copy, so it is HBM/latency
// bound and needs nothing beyond coalesced row reads and writes.
__global__ void __launch_bounds__(256) rope_rows_kernel(
    const float* __restrict__ fcos, const float* __restrict__ fsin, int cap, int half,
    const int32_t* __restrict__ pos, int num_tokens, float* __restrict__ rcos,
    float* __restrict__ rsin, int32_t* err) {
  long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  long long n = static_cast<long long>(num_tokens) * half;
  if (i >= n) return;
  int t = static_cast<int>(i / half);
  int j = static_cast<int>(i % half);
  int p = pos[t];
  if (p < 0) {
    rcos[i] = 1.0f;
    rsin[i] = 0.0f;
  } else if (p < cap) {
    long long src = static_cast<long long>(p) * half + j;
    rcos[i] = fcos[src];
    rsin[i] = fsin[src];
  } else if (j == 0) {
    flag_error(err, CSA_EFLAG_POS_RANGE);
  }
}

}  // namespace csa

extern "C" int csa_materialize_rope_rows(const float* freqs_cos, const float* freqs_sin,
                                         int32_t table_capacity, int32_t half_rope_dim,
                                         const int32_t* position_ids, int32_t T,
                                         int32_t num_tokens, float* rope_cos, float* rope_sin,
                                         int32_t* err, void* stream) {
  if (T < 0 || table_capacity < 0 || half_rope_dim < 0) return CSA_ERR_SHAPE;
  if (num_tokens < 0 || num_tokens > T) return CSA_ERR_RANGE;
  if (num_tokens == 0 || half_rope_dim == 0) return CSA_OK;
  if (!freqs_cos || !freqs_sin || !position_ids || !rope_cos || !rope_sin) return CSA_ERR_NULL;
  long long n = static_cast<long long>(num_tokens) * half_rope_dim;
  unsigned grid = static_cast<unsigned>((n + 255) / 256);
  hipLaunchKernelGGL(csa::rope_rows_kernel, dim3(grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), freqs_cos, freqs_sin, table_capacity,
                     half_rope_dim, position_ids, num_tokens, rope_cos, rope_sin, err);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}
