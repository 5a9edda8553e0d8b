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

// Inverse RoPE of the attention output (ROCm ATOM "DeepSeek-V4.1 native paged
// runtime": an inverse RoPE kernel follows the V4 attention): the rope span of
// every head of active row t is multiplied by the conjugate of row t's rope
// row, (x, y) -> (x c + y s, y c - x s).  One thread per group of four
// channels of a head (8 bytes of BF16): groups inside the span are rotated in
// FP32 and rounded to nearest even, the others are copied (nothing to do in
// place).
__global__ void __launch_bounds__(256) inverse_rope_kernel(
    const uint16_t* __restrict__ in, uint16_t* __restrict__ out, const float* __restrict__ rcos,
    const float* __restrict__ rsin, int half, int rope_offset, int num_tokens, int H, int D) {
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int G = D / 4;
  if (i >= static_cast<long long>(num_tokens) * H * G) return;
  const int t = static_cast<int>(i / (static_cast<long long>(H) * G));
  const int c0 = static_cast<int>(i % G) * 4;
  const uint2 v = *reinterpret_cast<const uint2*>(in + i * 4);
  const bool touches = c0 + 4 > rope_offset && c0 < rope_offset + 2 * half;
  if (!touches) {
    if (in != out) *reinterpret_cast<uint2*>(out + i * 4) = v;
    return;
  }
  uint32_t w[2] = {v.x, v.y};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = c0 + 2 * j - rope_offset;   // even: rope_offset is even
    if (r < 0 || r >= 2 * half) continue;
    const float c = rcos[static_cast<long long>(t) * half + (r >> 1)];
    const float sn = rsin[static_cast<long long>(t) * half + (r >> 1)];
    const float x = bf16_to_f32(static_cast<uint16_t>(w[j] & 0xffffu));
    const float y = bf16_to_f32(static_cast<uint16_t>(w[j] >> 16));
    w[j] = pack_bf16x2(fmaf(x, c, y * sn), fmaf(y, c, -x * sn));
  }
  *reinterpret_cast<uint2*>(out + i * 4) = make_uint2(w[0], w[1]);
}

}  // namespace csa

extern "C" int csa_inverse_rope(const uint16_t* in, uint16_t* out, const float* rope_cos,
                                const float* rope_sin, int32_t rope_dim, int32_t rope_offset,
                                int32_t T, int32_t num_tokens, int32_t H, int32_t D,
                                void* stream) {
  if (T < 0 || H < 0 || D < 0 || rope_dim < 0 || rope_offset < 0) return CSA_ERR_SHAPE;
  if (num_tokens < 0 || num_tokens > T) return CSA_ERR_RANGE;
  if ((rope_dim & 1) || (rope_offset & 1) || rope_offset + rope_dim > D || (D & 3))
    return CSA_ERR_UNSUPPORTED;
  if (num_tokens == 0 || H == 0 || D == 0) return CSA_OK;
  if (!in || !out || (rope_dim > 0 && (!rope_cos || !rope_sin))) return CSA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 7)
    return CSA_ERR_UNSUPPORTED;
  const long long n = static_cast<long long>(num_tokens) * H * (D / 4);
  if ((n + 255) / 256 > 0x7fffffffll) return CSA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(csa::inverse_rope_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                     dim3(256), 0, static_cast<hipStream_t>(stream), in, out, rope_cos, rope_sin,
                     rope_dim / 2, rope_offset, num_tokens, H, D);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}

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
