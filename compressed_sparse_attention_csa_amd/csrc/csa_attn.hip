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
// Two schedules share the same tile code.
//
// Ring kernel (prefill, large decode batches): a work-group (4 waves) owns
// one query row and walks its whole key list; wave w owns heads 16w..16w+15.
// The key list is virtual -- entry i < W_len is window position w_lo + i,
// later entries are topk_idx[t][i - W_len] -- and the work-group resolves it
// through the block tables in one parallel pass into LDS, compacting the
// valid rows to the front.  Rows then stream into a four-tile LDS ring (32
// rows per tile) with gfx950's direct global->LDS loads -- one wave-wide
// 16-byte-per-lane load moves a whole 1 KiB row, no registers involved --
// keeping three tiles in flight behind the one being multiplied.
//
// Decode kernel (small batches): a work-group owns one (row, 16-head group,
// 128-entry span); each wave gathers and multiplies its own 32-row tile, so a
// span costs one memory latency and every key byte is read from LDS once.
// FP16 partials of the spans, normalised by their own sums and scaled by a power
// of two per channel quarter, are merged with the
// sink by a third kernel.
//
// Tile code.  Rows sit at a 16-byte-padded stride so the K operand reads
// (A of S^T = K Q^T) and the transposed V reads (A of O^T = V^T P^T) spread
// over the LDS banks.  S^T puts one head per lane, so the softmax needs only
// two cross-lane steps per tile, and P^T leaves the MFMA already laid out as
// the B operand of the P*V product (the key order inside the MFMA is permuted
// identically on both operands).  The rotated query stays in registers as the
// B operand of S^T.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "csa_common.h"

// Allocation-free decode: the span partials live in a file-scope device array
// instead of a caller workspace, for callers that cannot allocate (code under
// HIP graph capture, tight serving loops).  Each GPU the library runs on holds
// its own copy of the array until the process ends; its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever handed to kernels -- the array's name in host
// code is a host-side stand-in, not a device address.  The partials are
// always written before they are read, so nothing needs clearing, and every
// call on one GPU shares the array: calls that overlap on one GPU race.
static constexpr size_t kScratchBytes = size_t{32} << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace csa {

namespace {

constexpr int kTile = 32;       // key rows per LDS tile
constexpr int kAttnWaves = 4;   // 16 heads per wave
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kRingWaves = 8;   // ring kernel: 4 softmax waves + 4 P*V waves
constexpr int kRingThreads = 64 * kRingWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const uint16_t* q;
  const float* rope_cos;
  const float* rope_sin;
  int half_rope;
  int rope_offset;
  // full RoPE tables [tab_cap][half_rope] instead of rope rows (rope_cos is
  // then NULL): row t takes table row rope_pos[t], the identity rotation
  // when that is negative; with rope_out_cos the work-group of head group 0
  // and span 0 also stores the row there (rows past the tables are flagged
  // and left untouched)
  const int32_t* rope_pos;
  const float* tab_cos;
  const float* tab_sin;
  int tab_cap;
  float* rope_out_cos;
  float* rope_out_sin;
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
  // low-bit planes (decode kernel with MX = true): window rows as MXFP8 E4M3
  // codes [.][D] with one E8M0 byte per 32 channels, compressed rows as packed
  // E2M1 codes [.][D/2] with one E4M3 byte per 16 channels
  const uint8_t* win_fp8;
  const uint8_t* win_sc;
  const uint8_t* cmp_fp4;
  const uint8_t* cmp_sc;
  const float* sink;
  float scale_log2;  // softmax_scale * log2(e)
  const int32_t* qsl;
  const int32_t* positions;
  int B;
  int num_tokens;
  int H;
  uint16_t* out;
  float* lse;
  uint16_t* part_o;  // FP16 [T][splits][H][D]: span partials normalised by their sum,
                     // times a power of two per channel quarter
  float2* part_ml;   // [T][splits][H]: (max, sum) of each span, base-2 logits
  float* part_mult;  // [T][splits][H][4]: the inverse of each quarter's power of two
  int splits;
  int ring_span;     // ring schedule with splits > 1: list entries per span
  int items_per_xcd;
  int32_t* err;
};

// Element j of the rope row at position p, gathered from the full tables
// (pypto-lib "DeepSeek V4.1 Flash", section "Serving-owned full RoPE
// tables"): a negative position takes the identity rotation, and so (for
// this kernel's own use) does a position past the tables, which
// publish_rope_row flags.
__device__ __forceinline__ void rope_from_tables(const float* __restrict__ tc,
                                                 const float* __restrict__ ts, int cap, int half,
                                                 int p, int j, float& c, float& s) {
  c = 1.0f;
  s = 0.0f;
  if (p >= 0 && p < cap) {
    c = tc[static_cast<long long>(p) * half + j];
    s = ts[static_cast<long long>(p) * half + j];
  }
}

// The rope row of token t as the materialisation step writes it: thread j <
// half stores element j; a row past the tables stays untouched and raises
// POS_RANGE (in the work-group's LDS error word).
__device__ __forceinline__ void publish_rope_row(float* __restrict__ oc, float* __restrict__ os,
                                                 int cap, int half, int t, int p, int j, float c,
                                                 float s, int* err_lds) {
  if (p >= cap) {
    if (j == 0 && half > 0) atomicOr(err_lds, CSA_EFLAG_POS_RANGE);
    return;
  }
  if (j < half) {
    oc[static_cast<long long>(t) * half + j] = c;
    os[static_cast<long long>(t) * half + j] = s;
  }
}

constexpr int kMaxSplit = 4224;  // longest key list of the ring schedule: window + k
constexpr int kMaxDenseK = 1 << 20;   // bound on k without a selection array
constexpr int kDecodeCUs = 256;       // MI355X compute units: the split-ring target
constexpr uint32_t kWinBit = 0x80000000u;
constexpr uint32_t kNoRow = 0xffffffffu;
constexpr int kRing = 4;          // key tiles resident in LDS (in flight or in use)

__device__ __forceinline__ v8bf as_v8bf(v4i x) { return __builtin_bit_cast(v8bf, x); }

// Span partials travel as FP16 with a power-of-two factor per (span, head,
// channel quarter): the factor puts the quarter's largest magnitude mx in
// [0.5, 1), so every stored value keeps 11 bits relative to that maximum and
// none overflows.  Returns (factor, its inverse); a zero, subnormal,
// infinite or NaN maximum keeps the values as they are.
__device__ __forceinline__ float2 fp16_block_scale(float mx) {
  const uint32_t e = (__float_as_uint(mx) >> 23) & 0xffu;
  if (e == 0u || e == 255u) return make_float2(1.0f, 1.0f);
  const uint32_t ec = e < 252u ? e : 252u;
  return make_float2(__uint_as_float((253u - ec) << 23), __uint_as_float((ec + 1u) << 23));
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const _Float16 a = static_cast<_Float16>(lo), b = static_cast<_Float16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Max over the 16 lanes of a DPP row.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false)));
  return v;
}

// Two E2M1 codes (byte BS of w, the lower-indexed one in bits 0-3) times an
// FP32 scale, as a BF16 pair.  The products are BF16 values (at most 6
// significant bits for an E4M3 scale), so their upper halves are exact.
template <int BS>
__device__ __forceinline__ uint32_t fp4_pair_bf16(uint32_t w, float sc) {
  const v2f_t e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, BS);
  const float lo = e[0] * sc, hi = e[1] * sc;
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo),
                               0x07060302u);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr uint32_t kMxWin = 0x100u;    // scale word flags: a window row,
constexpr uint32_t kMxMasked = 0x200u; // an entry past the valid rows

// The low-bit planes as values (read once from the kernel arguments: a
// choice between two argument fields made per lane would otherwise become a
// per-lane load from the argument block, and its wait would hold up every
// load issued before it).
struct MxPlanes {
  const uint8_t* win_fp8;
  const uint8_t* win_sc;
  const uint8_t* cmp_fp4;
  const uint8_t* cmp_sc;
  const uint8_t* dummy;   // the query's first bytes, read for masked entries
};

// One lane's share of a low-bit row r (a compacted entry: pool row, bit 31
// for the window pool, kNoRow when masked): the codes of channels 8 * chunk
// .. + 7 and their group's scale byte, with the flags above.  One 8-byte
// payload load and one scale-byte load, from addresses picked without
// branches: an E2M1 chunk is the half (chunk & 1) of an aligned 8-byte word
// shared with its neighbour; a masked entry reads the dummy bytes and is
// zeroed by the conversion.  UNIFORM: r is the same in every lane (one row
// per load instruction), so the row's bases are formed on the scalar unit and
// only the lane's chunk offset is per lane.
template <int D, bool UNIFORM>
__device__ __forceinline__ void mx_load(const MxPlanes& p, uint32_t r, int chunk, u32x2& pay,
                                        uint32_t& sc) {
  if constexpr (UNIFORM) r = __builtin_amdgcn_readfirstlane(r);
  const bool win = (r & kWinBit) != 0u;
  const bool masked = r == kNoRow;
  const long long row = static_cast<long long>(r & ~kWinBit);
  // (pointer selects, not integer arithmetic, so the loads stay global ones)
  const uint8_t* pbase = masked ? p.dummy : (win ? p.win_fp8 + row * D : p.cmp_fp4 + row * (D / 2));
  const uint8_t* sbase = masked ? p.dummy : (win ? p.win_sc + row * (D / 32) : p.cmp_sc + row * (D / 16));
  const uint32_t poff = masked ? 0u : (win ? chunk * 8u : (chunk >> 1) * 8u);
  const uint32_t soff = masked ? 0u : (win ? (chunk >> 2) : (chunk >> 1));
  pay = *reinterpret_cast<const u32x2*>(pbase + poff);
  sc = static_cast<uint32_t>(sbase[soff]) | (win ? kMxWin : 0u) | (masked ? kMxMasked : 0u);
}

// The eight channels as BF16, exactly (an E4M3 code times a power of two, or
// an E2M1 code times an E4M3 code, has at most 6 significant bits).
__device__ __forceinline__ uint4 mx_bf16x8(u32x2 pay, uint32_t sc, bool odd_chunk) {
  uint4 v;
  if (sc & kMxWin) {
    // the E8M0 byte as the exponent field of the FP32 scale operand: the
    // conversion multiplies by 2^(byte - 127) (byte 255: NaN)
    const float f = __builtin_bit_cast(float, (sc & 0xffu) << 23);
    v = uint4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pay[0], f, false)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pay[0], f, true)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pay[1], f, false)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pay[1], f, true))};
  } else {
    const float f = __builtin_amdgcn_cvt_f32_fp8(sc & 0xffu, 0);
    const uint32_t w = odd_chunk ? pay[1] : pay[0];
    v = uint4{fp4_pair_bf16<0>(w, f), fp4_pair_bf16<1>(w, f), fp4_pair_bf16<2>(w, f),
              fp4_pair_bf16<3>(w, f)};
  }
  if (sc & kMxMasked) v = uint4{0u, 0u, 0u, 0u};
  return v;
}



// Exclusive scan over a work-group of NW waves (scratch: one int per wave).
template <int NW>
__device__ int block_excl_scan_n(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int s = wsum[w];
    if (w < wave) before += s;
    tot += s;
  }
  *total = tot;
  return before + incl - v;
}

// block_excl_scan_n with LDS-only barriers (vector loads in flight are not
// waited for).
template <int NW>
__device__ int block_excl_scan_lds(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  lds_barrier();   // wsum of an earlier scan has been read
  if (lane == 63) wsum[wave] = incl;
  lds_barrier();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int s = wsum[w];
    if (w < wave) before += s;
    tot += s;
  }
  *total = tot;
  return before + incl - v;
}

// ds_read_b128 of K step `step` (64 bytes apart) as an inline instruction with
// an immediate offset; `step` is a compile-time constant after unrolling, so
// the switch folds away.
__device__ __forceinline__ void lds_read128_step(v4i& d, uint32_t addr, int step) {
  switch (step) {
    case 0: asm volatile("ds_read_b128 %0, %1 offset:0" : "=v"(d) : "v"(addr)); break;
    case 1: asm volatile("ds_read_b128 %0, %1 offset:64" : "=v"(d) : "v"(addr)); break;
    case 2: asm volatile("ds_read_b128 %0, %1 offset:128" : "=v"(d) : "v"(addr)); break;
    case 3: asm volatile("ds_read_b128 %0, %1 offset:192" : "=v"(d) : "v"(addr)); break;
    case 4: asm volatile("ds_read_b128 %0, %1 offset:256" : "=v"(d) : "v"(addr)); break;
    case 5: asm volatile("ds_read_b128 %0, %1 offset:320" : "=v"(d) : "v"(addr)); break;
    case 6: asm volatile("ds_read_b128 %0, %1 offset:384" : "=v"(d) : "v"(addr)); break;
    case 7: asm volatile("ds_read_b128 %0, %1 offset:448" : "=v"(d) : "v"(addr)); break;
    case 8: asm volatile("ds_read_b128 %0, %1 offset:512" : "=v"(d) : "v"(addr)); break;
    case 9: asm volatile("ds_read_b128 %0, %1 offset:576" : "=v"(d) : "v"(addr)); break;
    case 10: asm volatile("ds_read_b128 %0, %1 offset:640" : "=v"(d) : "v"(addr)); break;
    case 11: asm volatile("ds_read_b128 %0, %1 offset:704" : "=v"(d) : "v"(addr)); break;
    case 12: asm volatile("ds_read_b128 %0, %1 offset:768" : "=v"(d) : "v"(addr)); break;
    case 13: asm volatile("ds_read_b128 %0, %1 offset:832" : "=v"(d) : "v"(addr)); break;
    case 14: asm volatile("ds_read_b128 %0, %1 offset:896" : "=v"(d) : "v"(addr)); break;
    case 15: asm volatile("ds_read_b128 %0, %1 offset:960" : "=v"(d) : "v"(addr)); break;
    default: asm volatile("ds_read_b128 %0, %1" : "=v"(d) : "v"(addr + 64 * step)); break;
  }
}

template <int LPW>
__device__ __forceinline__ void wait_tiles_behind(int behind) {
  // at most `behind` later tiles (LPW loads each) may still be in flight
  switch (behind) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<LPW>(); break;
    case 2: wait_vmcnt<2 * LPW>(); break;
    default: wait_vmcnt<3 * LPW>(); break;
  }
}

template <int D, bool MX>
__global__ void __launch_bounds__(kRingThreads, 1) attn_kernel(AttnArgs a) {
  constexpr int KS = D / 32;                 // K steps of S^T
  constexpr int RB = 2 * D;                  // bytes per key row
  constexpr int NC = D / 8;                  // 16-byte chunks per row
  constexpr int RPI = 64 / NC;               // rows one wave-wide load moves
  constexpr int LPT = kTile / RPI;           // loads per tile
  constexpr int LPW = LPT >= kRingWaves ? LPT / kRingWaves : 1;   // loads per loading wave
  constexpr int NLW = LPT / LPW;             // waves that load
  constexpr int GS = RPI * RB + 16;          // LDS stride of one load's rows (+16 B pad)
  constexpr int TS = (kTile / RPI) * GS;     // LDS bytes per tile
  constexpr int HT = 4;                      // 16-head tiles (64 heads)
  constexpr int DW = D / 4;                  // channels per P*V wave
  constexpr int DTW = DW / 16;               // 16-channel O^T tiles per P*V wave
  static_assert(kRing == 4, "the step loop is unrolled over four ring slots");
  // one array per ring slot: with a single array indexed by a run-time slot
  // the compiler cannot tell which slot a direct-to-LDS load writes and
  // drains every load in flight before LDS reads
  __shared__ __attribute__((aligned(16))) uint8_t kv0[TS];
  __shared__ __attribute__((aligned(16))) uint8_t kv1[TS];
  __shared__ __attribute__((aligned(16))) uint8_t kv2[TS];
  __shared__ __attribute__((aligned(16))) uint8_t kv3[TS];
  __shared__ uint32_t row_s[kMaxSplit];   // pool row of each valid entry (bit 31: window pool)
  __shared__ int scan_s[kRingWaves];
  __shared__ int err_s;
  __shared__ float rope_s[2 * 256];            // rope row of t: cos, then sin
  __shared__ v4i p_s[2][HT][64];               // P^T fragments, double-buffered by tile
  __shared__ float f_s[64];                    // per-head output factor
  __shared__ int ovf_s[HT];

  // XCD-aware work mapping: consecutive rows land on one XCD.
  // An item is one row, or with splits > 1 one span of ring_span entries of
  // a row's key list (a long decode list): the span's FP32 partial goes to
  // the merge kernel.
  const int L = blockIdx.x;
  const int item = (L & 7) * a.items_per_xcd + (L >> 3);
  const int t = item / a.splits;
  const int split = item - t * a.splits;
  if (t >= a.num_tokens) return;
  const int i0 = split * a.ring_span;   // first list entry of this item

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;  // head within a 16-head tile (B/C column index)
  const int grp = lane >> 4;  // lane group
  // waves 0-3 compute S and the softmax of heads 16w .. 16w+15; waves 4-7
  // multiply P*V for channels (w-4)*D/4 .. of every head, one tile behind
  const bool s_wave = wave < HT;
  const int h0 = (wave & (HT - 1)) * 16;
  const int h = h0 + col;
  const bool hv = s_wave && h < a.H;

  if (tid == 0) err_s = 0;

  // metadata loads first, then the rope row and the sink.  The selected
  // indices of this thread's first two list entries are fetched with them on
  // the guess that the row's window is full (every row but a request's first
  // window - 1 tokens), which takes a dependent round trip off the
  // resolution.  The query (64 KiB per row, usually cold) is loaded only
  // after the resolution and the first two tile gathers: vector memory
  // counts complete in order, so loaded here it would hold up every wait of
  // the resolution.
  const int qsl_v = qsl_lane_load(a.qsl, a.B);
  const int p = a.positions[t];
  const int rp = a.tab_cos ? a.rope_pos[t] : -1;   // the rope row's position
  // (no selection array: the compressed set is every visible row, 0 .. n_vis-1)
  const int32_t* topk_row = a.topk ? a.topk + static_cast<long long>(t) * a.k : nullptr;
  const int i_spec0 = i0 + tid - a.window, i_spec1 = i0 + kRingThreads + tid - a.window;
  const int c_spec0 = (topk_row && i_spec0 >= 0 && i_spec0 < a.k) ? topk_row[i_spec0] : -1;
  const int c_spec1 = (topk_row && i_spec1 >= 0 && i_spec1 < a.k) ? topk_row[i_spec1] : -1;
  float rcv = 0.0f, rsv = 0.0f;
  if (tid < a.half_rope && !a.tab_cos) {
    rcv = a.rope_cos[static_cast<long long>(t) * a.half_rope + tid];
    rsv = a.rope_sin[static_cast<long long>(t) * a.half_rope + tid];
  }
  const float sink2 = hv ? a.sink[h] * kLog2e : 0.0f;
  const int b = owner_from_lanes(qsl_v, a.qsl, a.B, t);
  const int nv = visible_count(p, a.ratio);
  // from the full tables: row rp, fetched once rp is in, ahead of the
  // resolution's lookups (whose waits then cover it)
  if (tid < a.half_rope && a.tab_cos)
    rope_from_tables(a.tab_cos, a.tab_sin, a.tab_cap, a.half_rope, rp, tid, rcv, rsv);
  int w_len = 0, w_lo = 0;
  if (b >= 0 && p >= 0 && a.window > 0) {
    w_lo = max(0, p - a.window + 1);
    w_len = p - w_lo + 1;
  }
  const int list_len = (b >= 0) ? (w_len + a.k) : 0;
  const int n_my = a.splits == 1 ? list_len : max(0, min(list_len, i0 + a.ring_span) - i0);
  // LDS-only barriers in the prologue: a __syncthreads() would also wait for
  // the query loads still streaming in from HBM
  lds_barrier();   // err_s is cleared

  // ---- resolve every entry of the key list through the block tables at once;
  //      valid rows are compacted to the front (softmax does not depend on
  //      their order), so a tile's mask is just j < n_valid
  int n_valid = 0;
  {
    int ebits = 0;
    const bool spec_ok = w_len == a.window;
    if (!topk_row && a.k > 0 && b >= 0 && nv > a.k && split == 0 && tid == 0)
      ebits |= CSA_EFLAG_TOPK_RANGE;
    for (int j0 = 0, r = 0; j0 < n_my; j0 += kRingThreads, ++r) {
      const int i = i0 + j0 + tid;   // list entry
      uint32_t rr = kNoRow;
      // each entry names a table and a position; one page lookup serves
      // both kinds (lookups in two divergent branches cost two round trips)
      const int32_t* bt_row = nullptr;
      int lk_pos = 0, lk_max = 0, lk_num = 0;
      uint32_t lk_bit = 0u;
      if (j0 + tid >= n_my) {
        // past the list: nothing to resolve
      } else if (i < w_len) {
        bt_row = a.win_bt + static_cast<long long>(b) * a.max_win_blocks;
        lk_pos = w_lo + i;
        lk_max = a.max_win_blocks;
        lk_num = a.num_win_blocks;
        lk_bit = kWinBit;
      } else {
        const int c = !topk_row ? i - w_len
                      : (spec_ok && r < 2) ? (r == 0 ? c_spec0 : c_spec1) : topk_row[i - w_len];
        if (c >= 0) {
          if (c >= nv) {
            if (topk_row) ebits |= CSA_EFLAG_TOPK_RANGE;   // past n_vis: not selected
          } else {
            bt_row = a.cmp_bt + static_cast<long long>(b) * a.max_cmp_blocks;
            lk_pos = c;
            lk_max = a.max_cmp_blocks;
            lk_num = a.num_cmp_blocks;
          }
        }
      }
      const int lk_page = lk_pos / kPage;
      const int blk = (bt_row && lk_page < lk_max) ? bt_row[lk_page] : -1;
      if (bt_row) {
        if (blk >= 0 && blk < lk_num)
          rr = static_cast<uint32_t>(static_cast<long long>(blk) * kPage + (lk_pos % kPage)) | lk_bit;
        else
          ebits |= CSA_EFLAG_BLOCK_RANGE;
      }
      int total = 0;
      const int slot = n_valid + block_excl_scan_lds<kRingWaves>(rr != kNoRow ? 1 : 0, scan_s, &total);
      if (rr != kNoRow) row_s[slot] = rr;
      n_valid += total;
    }
    if (ebits) atomicOr(&err_s, ebits);
  }

  if (tid < a.half_rope) {
    rope_s[tid] = rcv;
    rope_s[256 + tid] = rsv;
  }
  if (a.rope_out_cos && split == 0)
    publish_rope_row(a.rope_out_cos, a.rope_out_sin, a.tab_cap, a.half_rope, t, rp, tid, rcv,
                     rsv, &err_s);
  lds_barrier();  // row_s and rope_s ready

  // ---- direct-to-LDS gather of one 32-row tile into ring slot tt % kRing
  //      (a compile-time constant).  Lane l of a wave-wide load moves chunk
  //      l % NC of row l / NC; each load's rows start 16 bytes past the
  //      previous load's, which spreads the K and V^T operand reads over the
  //      LDS banks.  Masked rows read finite dummy bytes (the query) so every
  //      loading wave issues exactly LPW loads per tile; P = 0 keeps them out
  //      of the result.
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.q);
  const bool loader = wave < NLW;
  auto slot_of = [&](auto sl) -> uint8_t* {
    constexpr int S = decltype(sl)::value;
    if constexpr (S == 0) return kv0;
    else if constexpr (S == 1) return kv1;
    else if constexpr (S == 2) return kv2;
    else return kv3;
  };
  auto issue = [&](int tt, auto sl) {
    if (!loader) return;
    uint8_t* slot = slot_of(sl);
    uint32_t rr[LPW];
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int j = tt * kTile + (wave * LPW + u) * RPI + lane / NC;   // compacted entry
      rr[u] = (j < n_valid) ? row_s[j] : kNoRow;
    }
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int ins = wave * LPW + u;
      // with one row per load the row is the same for the whole wave: its
      // address is computed once, on the scalar unit
      const uint32_t r = (RPI == 1) ? __builtin_amdgcn_readfirstlane(rr[u]) : rr[u];
      const uint16_t* pool = (r & kWinBit) ? a.win_kv : a.cmp_kv;
      const uint8_t* row = reinterpret_cast<const uint8_t*>(
          pool + static_cast<long long>(r & ~kWinBit) * D);
      const uint8_t* src = (r == kNoRow) ? dummy : row;
      __builtin_amdgcn_global_load_lds(
          src + (lane % NC) * 16, (__attribute__((address_space(3))) void*)(slot + ins * GS), 16,
          0, 0);
    }
  };
  // Low-bit rows (MX): a loading wave's share of tile tt goes to register
  // set tt & 1 (codes and scale words) and is dequantised into the tile's
  // ring slot one step before the tile is used, the same lanes writing the
  // same 16 bytes a direct-to-LDS load would.
  [[maybe_unused]] const MxPlanes mp{a.win_fp8, a.win_sc, a.cmp_fp4, a.cmp_sc, dummy};
  [[maybe_unused]] u32x2 mxp[2][MX ? LPW : 1];
  [[maybe_unused]] uint32_t mxs[2][MX ? LPW : 1];
  auto mx_issue = [&](int tt, auto set) {
    constexpr int Q = decltype(set)::value;
    if (!loader) return;
    uint32_t rr[LPW];
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int j = tt * kTile + (wave * LPW + u) * RPI + lane / NC;
      rr[u] = (j < n_valid) ? row_s[j] : kNoRow;
    }
#pragma unroll
    for (int u = 0; u < LPW; ++u) mx_load<D, RPI == 1>(mp, rr[u], lane % NC, mxp[Q][u], mxs[Q][u]);
  };
  auto mx_land = [&](auto set, auto sl) {
    constexpr int Q = decltype(set)::value;
    if (!loader) return;
    uint8_t* slot = slot_of(sl);
#pragma unroll
    for (int u = 0; u < LPW; ++u)
      *reinterpret_cast<uint4*>(slot + (wave * LPW + u) * GS + lane * 16) =
          mx_bf16x8(mxp[Q][u], mxs[Q][u], ((lane % NC) & 1) != 0);
  };
  auto row_off = [](int r) { return (r / RPI) * GS + (r % RPI) * RB; };

  const float neg_inf = -__builtin_huge_valf();
  const int ntiles = (n_valid + kTile - 1) / kTile;

  // Step k (k = 0 .. ntiles) begins with the step's one barrier: by then
  // every wave's loads of tile k have landed, the S waves have published
  // P(k-1), and tile k-2 is finished, so its slot takes tile k+2.  The S
  // waves then compute S(k) and P(k) while the P*V waves multiply tile k-1:
  // each SIMD runs one wave of each kind.
  auto step_sync = [&](int k, auto sl) {
    constexpr int S = decltype(sl)::value;
    if constexpr (MX) {
      lds_barrier();   // every wave has written its rows of tile k (mx_end)
    } else {
      // only tile k + 1 was issued after tile k
      wait_tiles_behind<LPW>((k + 1 < ntiles) ? 1 : 0);
      lds_barrier();
      if (k + 2 < ntiles) issue(k + 2, std::integral_constant<int, (S + 2) % kRing>{});
    }
  };

  // Softmax against a fixed reference: m_ref is the first tile's max, and
  // P = exp2(logit - m_ref) needs no rescaling of O as later tiles arrive
  // while no logit passes m_ref by more than kOvf (P then stays below
  // 2^kOvf, far inside BF16 and FP32 range).  A row where one does is run
  // again with m_ref set to its exact max, which the first pass recorded.
  constexpr float kOvf = 64.0f;
  float m_ref = neg_inf;    // this lane's head (base-2 logits)
  float m_seen = neg_inf;   // exact max over the whole list
  float l_run = 0.0f;

  // both kinds of wave run the same barrier sequence: per pass, one barrier
  // per step, then the overflow vote and the normalisation hand-off
  auto prime = [&]() {
    if constexpr (MX) {
      if (ntiles > 0) mx_issue(0, std::integral_constant<int, 0>{});
      if (ntiles > 1) mx_issue(1, std::integral_constant<int, 1>{});
    } else {
      if (ntiles > 0) issue(0, std::integral_constant<int, 0>{});
      if (ntiles > 1) issue(1, std::integral_constant<int, 1>{});
    }
  };
  // MX, after step k's work: tile k + 1 lands in its slot (free since tile
  // k - 3 finished), and tile k + 3 goes out to the register set that frees.
  // Landing after the step's work gives every load two steps' work to arrive.
  auto mx_end = [&](int k, auto sl) {
    if constexpr (MX) {
      constexpr int S = decltype(sl)::value;
      constexpr int Q = (S + 1) & 1;
      if (k + 1 < ntiles)
        mx_land(std::integral_constant<int, Q>{}, std::integral_constant<int, (S + 1) % kRing>{});
      if (k + 3 < ntiles) mx_issue(k + 3, std::integral_constant<int, Q>{});
    }
  };
  // MX: tile 0 lands and tile 2 goes out before the first step
  auto prime_land = [&]() {
    if constexpr (MX) {
      if (ntiles > 0)
        mx_land(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
      if (ntiles > 2) mx_issue(2, std::integral_constant<int, 0>{});
    }
  };

  // first two tiles of the first pass, then the query behind them
  prime();
  v4i qraw[KS];
  {
    const uint16_t* qrow = a.q + (static_cast<long long>(t) * a.H + (hv ? h : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qraw[ks] = hv ? *reinterpret_cast<const v4i*>(qrow + ks * 32 + grp * 8) : v4i{0, 0, 0, 0};
  }
  prime_land();

  // ---- query fragments (B operand of S^T) of the S waves: lane (head col,
  //      group grp) holds channels ks*32 + grp*8 .. +8, rotated where they
  //      fall in the rope span
  v8bf qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    v4i raw = qraw[ks];
    const int r0 = ks * 32 + grp * 8 - a.rope_offset;
    if (hv && r0 + 8 > 0 && r0 < 2 * a.half_rope) {
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const int rr = r0 + 2 * pr;
        if (rr >= 0 && rr < 2 * a.half_rope) {
          const float c = rope_s[rr >> 1], sn = rope_s[256 + (rr >> 1)];
          const uint32_t e = static_cast<uint32_t>(raw[pr]);
          const float x = bf16_to_f32(e & 0xffffu), y = bf16_to_f32(e >> 16);
          raw[pr] = static_cast<int>(pack_bf16x2(x * c - y * sn, x * sn + y * c));
        }
      }
    }
    qf[ks] = as_v8bf(raw);
  }


  if (s_wave) {
    // the softmax waves are the critical path of every step: their
    // instructions go first when both waves of a SIMD are ready
    __builtin_amdgcn_s_setprio(2);
    for (int pass = 0; pass < 2; ++pass) {
      if (pass > 0) {
        prime();
        prime_land();
      }
      bool ovf = false;
      l_run = 0.0f;
      // S^T tile: rows = 32 keys (two 16-row M tiles), columns = this wave's
      // 16 heads.  M-tile mt row i holds key mt*16 + i/4 + 4*(i%4), so the
      // four keys a lane group later needs for one transposed V read are 4
      // rows apart.  A wave past the last head multiplies its zero query.
      auto s_step = [&](int k, auto sl) {
        step_sync(k, sl);
        if (k >= ntiles) return;
        const uint8_t* tile = slot_of(sl);
        // K reads PF steps ahead of their MFMAs.  They are issued as inline
        // ds_read_b128 with explicit partial lgkmcnt waits: the compiler
        // counts the direct-to-LDS gathers in flight as pending LDS work and
        // would wait for every outstanding read (lgkmcnt(0)) before each use.
        // The wait takes the read registers as operands, which orders every
        // MFMA after the wait for its operands; PF + 1 register slots keep a
        // new read off the registers the previous MFMA pair read.
        constexpr int PF = KS < 4 ? KS : 4;
        constexpr int NB = PF + 1;
        const int krow = (col >> 2) + 4 * (col & 3);
        const uint32_t a0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
            (__attribute__((address_space(3))) const uint8_t*)(tile + row_off(krow) + grp * 16)));
        const uint32_t a1 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
            (__attribute__((address_space(3))) const uint8_t*)(tile + row_off(16 + krow) +
                                                                grp * 16)));
        v4i kb0[NB], kb1[NB];
#pragma unroll
        for (int i = 0; i < PF; ++i) {
          lds_read128_step(kb0[i], a0, i);
          lds_read128_step(kb1[i], a1, i);
        }
        // two accumulators per M tile (even and odd K steps) keep the
        // dependent MFMA chains short
        v4f sacc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i) sacc[i][0] = sacc[i][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int s = ks % NB;
          // reads issued after this step's two: those of the next PF - 1 steps
          const int later = 2 * ((KS - 1 - ks) < (PF - 1) ? (KS - 1 - ks) : (PF - 1));
          switch (later) {
            case 6: asm volatile("s_waitcnt lgkmcnt(6)" : "+v"(kb0[s]), "+v"(kb1[s])); break;
            case 4: asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(kb0[s]), "+v"(kb1[s])); break;
            case 2: asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(kb0[s]), "+v"(kb1[s])); break;
            default: asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kb0[s]), "+v"(kb1[s])); break;
          }
          sacc[0][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(kb0[s]), qf[ks],
                                                                    sacc[0][ks & 1], 0, 0, 0);
          sacc[1][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(kb1[s]), qf[ks],
                                                                    sacc[1][ks & 1], 0, 0, 0);
          if (ks + PF < KS) {
            lds_read128_step(kb0[(ks + PF) % NB], a0, ks + PF);
            lds_read128_step(kb1[(ks + PF) % NB], a1, ks + PF);
          }
        }
        const v4f s0 = sacc[0][0] + sacc[0][1];
        const v4f s1 = sacc[1][0] + sacc[1][1];
        // lane (head col, group grp) holds keys grp + 4r (s0[r]) and
        // 16 + grp + 4r (s1[r]) of the tile
        float lg[8];
        float tmax = neg_inf;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ja = k * kTile + grp + 4 * r, jb = ja + 16;
          lg[r] = ja < n_valid ? s0[r] * a.scale_log2 : neg_inf;
          lg[4 + r] = jb < n_valid ? s1[r] * a.scale_log2 : neg_inf;
          tmax = fmaxf(tmax, fmaxf(lg[r], lg[4 + r]));
        }
        tmax = max_xor32(max_xor16(tmax));
        m_seen = fmaxf(m_seen, tmax);
        // the first tile always holds a valid key (valid entries are
        // compacted to the front), so its max is finite
        if (k == 0 && pass == 0) m_ref = tmax;
        ovf = ovf || tmax > m_ref + kOvf;
        // lg - m_ref <= kOvf on every tile that matters (a row where it is
        // not runs again), so the bare exponential instruction suffices
        float psum = 0.0f;
        v4i pw;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const float p0 = __builtin_amdgcn_exp2f(lg[j] - m_ref);
          const float p1 = __builtin_amdgcn_exp2f(lg[j + 1] - m_ref);
          psum += p0 + p1;
          pw[j >> 1] = static_cast<int>(pack_bf16x2(p0, p1));
        }
        l_run += sum_xor32(sum_xor16(psum));
        p_s[k & 1][wave][lane] = pw;
      };
      for (int k = 0; k <= ntiles; k += kRing) {
        s_step(k, std::integral_constant<int, 0>{});
        mx_end(k, std::integral_constant<int, 0>{});
        if (k + 1 <= ntiles) {
          s_step(k + 1, std::integral_constant<int, 1>{});
          mx_end(k + 1, std::integral_constant<int, 1>{});
        }
        if (k + 2 <= ntiles) {
          s_step(k + 2, std::integral_constant<int, 2>{});
          mx_end(k + 2, std::integral_constant<int, 2>{});
        }
        if (k + 3 <= ntiles) {
          s_step(k + 3, std::integral_constant<int, 3>{});
          mx_end(k + 3, std::integral_constant<int, 3>{});
        }
      }
      // a second pass only when a logit outran the first tile's max (no load
      // is in flight here: the last step waited for all of them)
      if (lane == 0) ovf_s[wave] = (__ballot(ovf) != 0ull) ? 1 : 0;
      __syncthreads();
      const bool again = (ovf_s[0] | ovf_s[1] | ovf_s[2] | ovf_s[3]) != 0;
      __syncthreads();
      if (again) {
        m_ref = m_seen;
        continue;
      }
      // per-head normalisation, handed to the P*V waves; a span of a split
      // list publishes its (max, sum) for the merge instead
      if (hv && grp == 0) {
        if (a.splits > 1) {
          // the span's (max, sum); its partial is O / sum
          a.part_ml[static_cast<long long>(item) * a.H + h] = make_float2(m_ref, l_run);
          f_s[h] = l_run > 0.0f ? 1.0f / l_run : 0.0f;
        } else {
          const float M = fmaxf(m_ref, sink2);
          const float corr = (m_ref == neg_inf) ? 0.0f : exp2f(m_ref - M);
          const float Z = l_run * corr + exp2f(sink2 - M);
          f_s[h] = corr / Z;
          if (a.lse) a.lse[static_cast<long long>(t) * a.H + h] = (M + log2f(Z)) * kLn2;
        }
      }
      __syncthreads();   // f_s is complete
      break;
    }
  } else {
    // O^T += V^T P^T for this wave's channels and all four head tiles: each
    // transposed V fragment (in lane group g, source lane 4e + q points at 8
    // bytes of key row g + 4e [then 16 + g + 4e], channels n0 + 4q .. +3;
    // lane i of the group receives those rows' channel n0 + i -- the keys
    // P^T holds in elements e and 4 + e) feeds four MFMAs
    const int d0 = (wave - HT) * DW;
    v4f o_acc[DTW][HT];
    for (int pass = 0; pass < 2; ++pass) {
      if (pass > 0) {
        prime();
        prime_land();
      }
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) o_acc[dt][ht] = v4f{0.f, 0.f, 0.f, 0.f};
      auto pv_step = [&](int k, auto sl) {
        constexpr int S = decltype(sl)::value;
        step_sync(k, sl);
        if (k == 0) return;
        const uint8_t* tile = slot_of(std::integral_constant<int, (S + kRing - 1) % kRing>{});
        constexpr int VPF = DTW < 4 ? DTW : 4;
        const int e_src = (lane & 15) >> 2, q_src = lane & 3;
        const uint8_t* v0p = tile + row_off(grp + 4 * e_src) + q_src * 8 + d0 * 2;
        const uint8_t* v1p = tile + row_off(16 + grp + 4 * e_src) + q_src * 8 + d0 * 2;
        v4s vlo[VPF], vhi[VPF];
#pragma unroll
        for (int i = 0; i < VPF; ++i) {
          vlo[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s*)(v0p + i * 32));
          vhi[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s*)(v1p + i * 32));
        }
        v8bf pf[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) pf[ht] = as_v8bf(p_s[(k - 1) & 1][ht][lane]);
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) {
          const v4s lo = vlo[dt % VPF], hi = vhi[dt % VPF];
          if (dt + VPF < DTW) {
            vlo[dt % VPF] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s*)(v0p + (dt + VPF) * 32));
            vhi[dt % VPF] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s*)(v1p + (dt + VPF) * 32));
          }
          const v8bf va =
              __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
            o_acc[dt][ht] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[ht], o_acc[dt][ht], 0, 0, 0);
        }
      };
      for (int k = 0; k <= ntiles; k += kRing) {
        pv_step(k, std::integral_constant<int, 0>{});
        mx_end(k, std::integral_constant<int, 0>{});
        if (k + 1 <= ntiles) {
          pv_step(k + 1, std::integral_constant<int, 1>{});
          mx_end(k + 1, std::integral_constant<int, 1>{});
        }
        if (k + 2 <= ntiles) {
          pv_step(k + 2, std::integral_constant<int, 2>{});
          mx_end(k + 2, std::integral_constant<int, 2>{});
        }
        if (k + 3 <= ntiles) {
          pv_step(k + 3, std::integral_constant<int, 3>{});
          mx_end(k + 3, std::integral_constant<int, 3>{});
        }
      }
      __syncthreads();   // the S waves' overflow vote
      const bool again = (ovf_s[0] | ovf_s[1] | ovf_s[2] | ovf_s[3]) != 0;
      __syncthreads();
      if (again) continue;
      __syncthreads();   // f_s is complete
      // the BF16 output rows, or with splits > 1 the span's FP16 partial (f
      // is then 1 / its sum) scaled for this wave's channel quarter
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const int hh = ht * 16 + col;
        const float f = f_s[hh < a.H ? hh : 0];
        const long long roff = static_cast<long long>(hh) * D + d0;
        if (a.splits > 1) {
          float mx = 0.0f;
#pragma unroll
          for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(o_acc[dt][ht][r] * f));
          mx = max_xor32(max_xor16(mx));   // the four lane groups of head hh
          if (hh >= a.H) continue;
          const float2 sc = fp16_block_scale(mx);
          const float fs = f * sc.x;
          uint16_t* prow = a.part_o + static_cast<long long>(item) * a.H * D + roff;
#pragma unroll
          for (int dt = 0; dt < DTW; ++dt) {
            uint2 w;
            w.x = pack_f16x2(o_acc[dt][ht][0] * fs, o_acc[dt][ht][1] * fs);
            w.y = pack_f16x2(o_acc[dt][ht][2] * fs, o_acc[dt][ht][3] * fs);
            *reinterpret_cast<uint2*>(prow + dt * 16 + grp * 4) = w;
          }
          if (grp == 0)
            a.part_mult[(static_cast<long long>(item) * a.H + hh) * 4 + (wave - HT)] = sc.y;
        } else if (hh < a.H) {
          uint16_t* orow = a.out + static_cast<long long>(t) * a.H * D + roff;
#pragma unroll
          for (int dt = 0; dt < DTW; ++dt) {
            // o_acc[dt][ht][r] is channel d0 + dt*16 + grp*4 + r of head hh
            uint2 w;
            w.x = pack_bf16x2(o_acc[dt][ht][0] * f, o_acc[dt][ht][1] * f);
            w.y = pack_bf16x2(o_acc[dt][ht][2] * f, o_acc[dt][ht][3] * f);
            *reinterpret_cast<uint2*>(orow + dt * 16 + grp * 4) = w;
          }
        }
      }
      break;
    }
  }

  if (tid == 0 && err_s) flag_error(a.err, err_s);
  if (b < 0 && split == 0 && tid == 0) flag_error(a.err, CSA_EFLAG_META);
}

// ---------------------------------------------------------------------------
// Decode schedule: a work-group owns one (row, 16-head group, 128-entry span of
// the key list).  Each of its four waves gathers its own 32 rows into a private
// LDS slot with direct-to-LDS loads -- all at once, so a work-group pays one
// memory latency -- and runs one 32-key tile (S^T, softmax, P*V) for the
// group's 16 heads; no key byte is read from LDS by more than one wave.  The
// four per-wave softmax states are then combined in LDS.  With one span the
// work-group writes the output rows directly; with several it writes an FP16
// partial (16 heads x D, normalised by its own sum and scaled by a power of
// two per channel quarter) with the FP32 (max, sum)
// for the merge kernel.
constexpr int kSpan = kAttnWaves * kTile;   // list entries per decode work-group

template <int D, bool MX>
__global__ void __launch_bounds__(kAttnThreads, 1) attn_decode_kernel(AttnArgs a) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int RB = 2 * D;
  constexpr int NC = D / 8;
  constexpr int RPI = 64 / NC;
  constexpr int GS = RPI * RB + 16;
  constexpr int TS = (kTile / RPI) * GS;     // one wave's slot: 32 rows
  constexpr int OSTR = D + 4;                // padded FP32 row of the per-wave output
  constexpr int SS = (TS > 16 * OSTR * 4) ? TS : 16 * OSTR * 4;   // slot bytes
  __shared__ __attribute__((aligned(16))) uint8_t slot_s[kAttnWaves * SS];
  __shared__ uint32_t row_s[kSpan];
  __shared__ float ml_s[kAttnWaves][2][16];
  __shared__ float rope_s[2 * kAttnThreads];   // rope row of t: cos, then sin
  __shared__ int scan_s[kAttnWaves];
  __shared__ int err_s;

  const int HG = (a.H + 15) / 16;
  const int L = blockIdx.x;
  const int item = (L & 7) * a.items_per_xcd + (L >> 3);
  const int hg = item % HG;
  const int ts = item / HG;                 // t * splits + split
  const int t = ts / a.splits;
  const int split = ts % a.splits;
  if (t >= a.num_tokens) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int h = hg * 16 + col;
  const bool hv = h < a.H;
  if (tid == 0) err_s = 0;
  // metadata loads first, then the first use of the metadata.  The selected
  // index of this thread's entry is fetched with them on the guess that the
  // row's window is full (position >= window - 1, every row but a request's
  // first few tokens), which takes a dependent round trip off the
  // resolution.
  const int qsl_v = qsl_lane_load(a.qsl, a.B);
  const int p = a.positions[t];
  const int rp = a.tab_cos ? a.rope_pos[t] : -1;   // the rope row's position
  // (no selection array: the compressed set is every visible row, 0 .. n_vis-1)
  const int32_t* topk_row = a.topk ? a.topk + static_cast<long long>(t) * a.k : nullptr;
  const int i_spec = split * kSpan + tid - a.window;
  const int c_spec = (topk_row && i_spec >= 0 && i_spec < a.k) ? topk_row[i_spec] : -1;

  const int b = owner_from_lanes(qsl_v, a.qsl, a.B, t);
  const int nv = visible_count(p, a.ratio);
  int w_len = 0, w_lo = 0;
  if (b >= 0 && p >= 0 && a.window > 0) {
    w_lo = max(0, p - a.window + 1);
    w_len = p - w_lo + 1;
  }
  const int list_len = (b >= 0) ? (w_len + a.k) : 0;
  const int i_begin = split * kSpan;
  const int n_my = max(0, min(list_len, i_begin + kSpan) - i_begin);
  // LDS-only barriers in the prologue: a __syncthreads() would also wait for
  // the query loads still streaming in from HBM
  lds_barrier();   // err_s is cleared

  v4i qraw[KS];
  float rcv = 0.0f, rsv = 0.0f;
  // ---- resolve this span through the block tables; compact valid rows
  int n_valid = 0;
  {
    int ebits = 0;
    if (!topk_row && a.k > 0 && b >= 0 && nv > a.k && split == 0 && tid == 0)
      ebits |= CSA_EFLAG_TOPK_RANGE;   // bound below n_vis (k = 0: the window alone)
    // each entry names a table and a position; one page lookup serves both
    // kinds (two lookups in divergent branches would cost two round trips)
    uint32_t rr = kNoRow;
    const int j = tid;
    const int32_t* bt_row = nullptr;
    int lk_pos = 0, lk_max = 0, lk_num = 0;
    uint32_t lk_bit = 0u;
    if (j < n_my) {
      const int i = i_begin + j;
      if (i < w_len) {
        bt_row = a.win_bt + static_cast<long long>(b) * a.max_win_blocks;
        lk_pos = w_lo + i;
        lk_max = a.max_win_blocks;
        lk_num = a.num_win_blocks;
        lk_bit = kWinBit;
      } else {
        const int c = !topk_row ? i - w_len : (w_len == a.window) ? c_spec : topk_row[i - w_len];
        if (c >= 0) {
          if (c >= nv) {
            if (topk_row) ebits |= CSA_EFLAG_TOPK_RANGE;   // past n_vis: not selected
          } else {
            bt_row = a.cmp_bt + static_cast<long long>(b) * a.max_cmp_blocks;
            lk_pos = c;
            lk_max = a.max_cmp_blocks;
            lk_num = a.num_cmp_blocks;
          }
        }
      }
    }
    const int lk_page = lk_pos / kPage;
    const int blk = (bt_row && lk_page < lk_max) ? bt_row[lk_page] : -1;
    // the query and the rope row, behind the page lookup: unguarded loads of
    // a valid head (a head past H gets zeros below), so the lookup's wait
    // does not include them; complete before the gather is issued
    {
      const uint16_t* qrow = a.q + (static_cast<long long>(t) * a.H + (hv ? h : 0)) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qraw[ks] = *reinterpret_cast<const v4i*>(qrow + ks * 32 + grp * 8);
    }
    if (a.half_rope > 0) {   // uniform: no table without a rope span
      const int rt = tid < a.half_rope ? tid : 0;
      if (a.tab_cos) {
        rope_from_tables(a.tab_cos, a.tab_sin, a.tab_cap, a.half_rope, rp, rt, rcv, rsv);
      } else {
        rcv = a.rope_cos[static_cast<long long>(t) * a.half_rope + rt];
        rsv = a.rope_sin[static_cast<long long>(t) * a.half_rope + rt];
      }
    }
    if (bt_row) {
      if (blk >= 0 && blk < lk_num)
        rr = static_cast<uint32_t>(static_cast<long long>(blk) * kPage + (lk_pos % kPage)) | lk_bit;
      else
        ebits |= CSA_EFLAG_BLOCK_RANGE;
    }
    if (ebits && hg == 0) atomicOr(&err_s, ebits);
    int total = 0;
    const int slot = block_excl_scan_lds<kAttnWaves>(rr != kNoRow ? 1 : 0, scan_s, &total);
    if (rr != kNoRow) row_s[slot] = rr;
    n_valid = total;
  }
  if (tid < a.half_rope) {
    rope_s[tid] = rcv;
    rope_s[kAttnThreads + tid] = rsv;
  }
  if (a.rope_out_cos && split == 0 && hg == 0)
    publish_rope_row(a.rope_out_cos, a.rope_out_sin, a.tab_cap, a.half_rope, t, rp, tid, rcv,
                     rsv, &err_s);
  __syncthreads();

  // ---- this wave's 32 rows straight into its LDS slot (masked rows read the
  //      query: finite bytes that P = 0 keeps out).  All row indices are read
  //      from LDS first, so the direct-to-LDS loads issue back to back.
  uint8_t* myslot = slot_s + wave * SS;
  const int j0 = wave * kTile;
  constexpr int NI = kTile / RPI;
  // low-bit rows go through registers: lane (row ins * RPI + lane / NC,
  // chunk lane % NC) holds its codes and scale word until the conversion below
  [[maybe_unused]] u32x2 mx_pay[MX ? NI : 1];
  [[maybe_unused]] uint32_t mx_sc[MX ? NI : 1];
  if constexpr (MX) {
    if (j0 < n_valid) {
      uint32_t rr[NI];
#pragma unroll
      for (int ins = 0; ins < NI; ++ins) {
        const int j = j0 + ins * RPI + lane / NC;
        rr[ins] = (j < n_valid) ? row_s[j] : kNoRow;
      }
      const MxPlanes mp{a.win_fp8, a.win_sc, a.cmp_fp4, a.cmp_sc,
                        reinterpret_cast<const uint8_t*>(a.q)};
#pragma unroll
      for (int ins = 0; ins < NI; ++ins)
        mx_load<D, RPI == 1>(mp, rr[ins], lane % NC, mx_pay[ins], mx_sc[ins]);
    }
  } else if (j0 < n_valid) {
    uint32_t rr[NI];
#pragma unroll
    for (int ins = 0; ins < NI; ++ins) {
      const int j = j0 + ins * RPI + lane / NC;
      rr[ins] = (j < n_valid) ? row_s[j] : kNoRow;
    }
    const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.q);
#pragma unroll
    for (int ins = 0; ins < NI; ++ins) {
      const uint32_t r = rr[ins];
      const uint16_t* pool = (r & kWinBit) ? a.win_kv : a.cmp_kv;
      const uint8_t* row = reinterpret_cast<const uint8_t*>(
          pool + static_cast<long long>(r & ~kWinBit) * D);
      const uint8_t* src = (r == kNoRow) ? dummy : row;
      __builtin_amdgcn_global_load_lds(
          src + (lane % NC) * 16, (__attribute__((address_space(3))) void*)(myslot + ins * GS),
          16, 0, 0);
    }
  }
  auto row_off = [](int r) { return (r / RPI) * GS + (r % RPI) * RB; };

  // ---- query fragments of head h (B operand of S^T), rotated on the rope
  //      span while the gather is in flight
  v8bf qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    v4i raw = hv ? qraw[ks] : v4i{0, 0, 0, 0};
    const int r0 = ks * 32 + grp * 8 - a.rope_offset;
    if (hv && r0 + 8 > 0 && r0 < 2 * a.half_rope) {
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const int rr = r0 + 2 * pr;
        if (rr >= 0 && rr < 2 * a.half_rope) {
          const float c = rope_s[rr >> 1], sn = rope_s[kAttnThreads + (rr >> 1)];
          const uint32_t e = static_cast<uint32_t>(raw[pr]);
          const float x = bf16_to_f32(e & 0xffffu), y = bf16_to_f32(e >> 16);
          raw[pr] = static_cast<int>(pack_bf16x2(x * c - y * sn, x * sn + y * c));
        }
      }
    }
    qf[ks] = as_v8bf(raw);
  }

  const float neg_inf = -__builtin_huge_valf();
  float m_w = neg_inf, l_w = 0.0f;
  v4f o_acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o_acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  if constexpr (MX) {
    if (j0 < n_valid) {
#pragma unroll
      for (int ins = 0; ins < NI; ++ins)
        *reinterpret_cast<uint4*>(myslot + ins * GS + lane * 16) =
            mx_bf16x8(mx_pay[ins], mx_sc[ins], ((lane % NC) & 1) != 0);
    }
  } else {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's rows have landed in its slot
  }

  if (j0 < n_valid) {
    const uint8_t* tile = myslot;
    v4f s0 = v4f{0.f, 0.f, 0.f, 0.f}, s1 = v4f{0.f, 0.f, 0.f, 0.f};
    v4f s2 = v4f{0.f, 0.f, 0.f, 0.f}, s3 = v4f{0.f, 0.f, 0.f, 0.f};
    const int krow = (col >> 2) + 4 * (col & 3);
    const uint8_t* k0p = tile + row_off(krow) + grp * 16;
    const uint8_t* k1p = tile + row_off(16 + krow) + grp * 16;
#pragma unroll
    for (int kg = 0; kg < KS; kg += 4) {
#pragma unroll
      for (int ks = kg; ks < kg + 4 && ks < KS; ks += 2) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_v8bf(*reinterpret_cast<const v4i*>(k0p + ks * 64)), qf[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_v8bf(*reinterpret_cast<const v4i*>(k1p + ks * 64)), qf[ks], s1, 0, 0, 0);
        if (ks + 1 < KS) {
          s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_v8bf(*reinterpret_cast<const v4i*>(k0p + (ks + 1) * 64)), qf[ks + 1], s2, 0, 0, 0);
          s3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_v8bf(*reinterpret_cast<const v4i*>(k1p + (ks + 1) * 64)), qf[ks + 1], s3, 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    s0 += s2;
    s1 += s3;
    float lg[8];
    float tmax = neg_inf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ja = j0 + grp + 4 * r, jb = ja + 16;
      lg[r] = ja < n_valid ? s0[r] * a.scale_log2 : neg_inf;
      lg[4 + r] = jb < n_valid ? s1[r] * a.scale_log2 : neg_inf;
      tmax = fmaxf(tmax, fmaxf(lg[r], lg[4 + r]));
    }
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
    m_w = tmax;   // finite: the wave has at least one valid row
    float psum = 0.0f;
    v4i pw;
#pragma unroll
    for (int jj = 0; jj < 8; jj += 2) {
      const float p0 = exp2f(lg[jj] - m_w), p1 = exp2f(lg[jj + 1] - m_w);
      psum += p0 + p1;
      pw[jj >> 1] = static_cast<int>(pack_bf16x2(p0, p1));
    }
    psum += shfl_xor_f(psum, 16);
    psum += shfl_xor_f(psum, 32);
    l_w = psum;
    const v8bf pf = as_v8bf(pw);
    const int e_src = (lane & 15) >> 2, q_src = lane & 3;
    const uint8_t* v0p = tile + row_off(grp + 4 * e_src) + q_src * 8;
    const uint8_t* v1p = tile + row_off(16 + grp + 4 * e_src) + q_src * 8;
#pragma unroll
    for (int dg = 0; dg < DT; dg += 8) {
#pragma unroll
      for (int dt = dg; dt < dg + 8 && dt < DT; ++dt) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(v0p + dt * 32));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(v1p + dt * 32));
        const v8s va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o_acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, va), pf,
                                                             o_acc[dt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // ---- combine the four waves: each parks (m, l, O) in LDS (its own slot)
  {
    float* ow = reinterpret_cast<float*>(myslot);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<v4f*>(ow + col * OSTR + dt * 16 + grp * 4) = o_acc[dt];
    if (grp == 0) {
      ml_s[wave][0][col] = m_w;
      ml_s[wave][1][col] = l_w;
    }
  }
  __syncthreads();
  if (tid == 0 && err_s) flag_error(a.err, err_s);
  if (b < 0 && split == 0 && hg == 0 && tid == 0) flag_error(a.err, CSA_EFLAG_META);
  {
    // thread (head hh, lane c4) combines channels c4*4 + 64m: consecutive
    // lanes touch consecutive 16-byte LDS words and output bytes
    const int hh = tid >> 4;
    const int c4 = (tid & 15) * 4;
    const int head = hg * 16 + hh;
    if (head < a.H) {
      float mw[kAttnWaves], e[kAttnWaves];
      float M = neg_inf;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        mw[w] = ml_s[w][0][hh];
        M = fmaxf(M, mw[w]);
      }
      float Lsum = 0.0f;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        e[w] = (mw[w] == neg_inf) ? 0.0f : exp2f(mw[w] - M);
        Lsum += ml_s[w][1][hh] * e[w];
      }
      float scale;
      if (a.splits == 1) {
        const float sink2 = a.sink[head] * kLog2e;
        const float Mt = fmaxf(M, sink2);
        const float corr = (M == neg_inf) ? 0.0f : exp2f(M - Mt);
        const float Z = Lsum * corr + exp2f(sink2 - Mt);
        scale = corr / Z;
        if (a.lse && c4 == 0) a.lse[static_cast<long long>(t) * a.H + head] = (Mt + log2f(Z)) * kLn2;
      } else {
        // the span's partial, normalised by its own sum (an empty span: 0)
        scale = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
        if (c4 == 0) a.part_ml[static_cast<long long>(ts) * a.H + head] = make_float2(M, Lsum);
      }
      // channels c4 + 64 m, m < D / 64, of head `head`, combined over the waves
      v4f accs[D / 64];
      float mx = 0.0f;
#pragma unroll
      for (int m = 0; m < D / 64; ++m) {
        v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w)
          acc += *reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(slot_s + w * SS) +
                                               hh * OSTR + c4 + 64 * m) * e[w];
        accs[m] = acc * scale;
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(accs[m][r]));
      }
      if (a.splits == 1) {
        uint16_t* dst = a.out + (static_cast<long long>(t) * a.H + head) * D;
#pragma unroll
        for (int m = 0; m < D / 64; ++m) {
          uint2 pk;
          pk.x = pack_bf16x2(accs[m][0], accs[m][1]);
          pk.y = pack_bf16x2(accs[m][2], accs[m][3]);
          *reinterpret_cast<uint2*>(dst + c4 + 64 * m) = pk;
        }
      } else {
        // one factor for the head's four quarters: the max over its 16 lanes
        const float2 sc = fp16_block_scale(row16_max(mx));
        uint16_t* pdst = a.part_o + (static_cast<long long>(ts) * a.H + head) * D;
#pragma unroll
        for (int m = 0; m < D / 64; ++m) {
          uint2 pk;
          pk.x = pack_f16x2(accs[m][0] * sc.x, accs[m][1] * sc.x);
          pk.y = pack_f16x2(accs[m][2] * sc.x, accs[m][3] * sc.x);
          *reinterpret_cast<uint2*>(pdst + c4 + 64 * m) = pk;
        }
        if (c4 == 0)
          *reinterpret_cast<float4*>(a.part_mult + (static_cast<long long>(ts) * a.H + head) * 4) =
              make_float4(sc.y, sc.y, sc.y, sc.y);
      }
    }
  }
}

// Combine the span partials of each (row, head) with the sink: one wave per
// (row, head).  Span s contributes its normalised partial O_s with weight
// l_s * 2^(m_s - M) (M the max over the spans' maxima and the sink), so
//   out = sum_s w_s O_s / (sum_s w_s + 2^(sink - M)),  lse = (M + log2 Z) ln 2.
// O_s arrives as FP16 times a power of two per channel quarter, whose inverse
// joins the weight of the lane's quarter.
// Lane l owns channels [8l, 8l + 8) of every partial (D = 512; D / 64
// channels in general).  With at most 64 spans (MANY false) lane s holds span
// s's (max, sum) and the weights travel by lane reads; with more, lanes
// stride over the spans for the max and the denominator and each chunk of
// eight partials loads its spans' pairs too.  The first chunk goes out with
// the pairs of the max pass, so a row of at most 64 spans costs one memory
// latency before its sums.
constexpr int kMergeChunk = 8;

template <int D, bool MANY>
__global__ void __launch_bounds__(64) attn_merge_kernel(
    const uint16_t* __restrict__ part_o, const float2* __restrict__ part_ml,
    const float* __restrict__ part_mult, const float* __restrict__ sink, int splits, int H,
    int num_tokens, int items_per_xcd,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int CPL = D / 64;            // channels per lane
  static_assert(CPL == 1 || CPL == 2 || CPL == 4 || CPL == 8, "channels per lane");
  // (row, head) items in row-major order, consecutive items on one XCD: the
  // same split of rows over XCDs as the span work-groups, whose partials
  // are then still in that XCD's L2
  const int L = blockIdx.x;
  const int item = (L & 7) * items_per_xcd + (L >> 3);
  const int t = item / H;
  const int h = item % H;
  if (t >= num_tokens) return;
  const int lane = threadIdx.x;
  const float neg_inf = -__builtin_huge_valf();
  const long long tbase = static_cast<long long>(t) * splits;
  // loads read a valid span in every lane (a clamped index) and the select
  // follows, so they issue together rather than one guarded round trip each
  float2 ml = part_ml[(tbase + (lane < splits ? lane : 0)) * H + h];
  if (lane >= splits) ml = make_float2(neg_inf, 0.0f);
  const float sinkv = sink[h];
  float acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.0f;
  float chunk[kMergeChunk][CPL];
  float cmult[kMergeChunk];
  float2 cml[kMergeChunk];
  const int quarter = lane >> 4;   // channels lane * CPL .. lie in quarter lane / 16
  auto load_chunk = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      const int sp = s0 + u;
      const long long sl = tbase + (sp < splits ? sp : 0);
      if constexpr (MANY) {
        cml[u] = part_ml[sl * H + h];
        if (sp >= splits) cml[u] = make_float2(neg_inf, 0.0f);
      }
      // a span past the list reads span 0; its weight is never applied
      cmult[u] = part_mult[(sl * H + h) * 4 + quarter];
      const uint16_t* po = part_o + (sl * H + h) * D + lane * CPL;
      uint32_t w[(CPL + 1) / 2];
      if constexpr (CPL == 8) {
        const uint4 x = *reinterpret_cast<const uint4*>(po);
        w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
      } else if constexpr (CPL == 4) {
        const uint2 x = *reinterpret_cast<const uint2*>(po);
        w[0] = x.x; w[1] = x.y;
      } else if constexpr (CPL == 2) {
        w[0] = *reinterpret_cast<const uint32_t*>(po);
      } else {
        w[0] = *po;
      }
#pragma unroll
      for (int i = 0; i < CPL; ++i)
        chunk[u][i] = static_cast<float>(
            __builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i >> 1] >> (16 * (i & 1)))));
    }
  };
  load_chunk(0);
  // the first chunk's loads are issued before the span statistics are
  // reduced: these empty instructions consume one value of each span, so
  // all of them share one memory latency with the statistics' loads
#pragma unroll
  for (int u = 0; u < kMergeChunk; ++u) asm volatile("" ::"v"(chunk[u][0]));
  // running max and denominator over the spans, with the sink
  const float sink2 = sinkv * kLog2e;
  float M = ml.x;
  if constexpr (MANY)
    for (int s = lane + 64; s < splits; s += 64) M = fmaxf(M, part_ml[(tbase + s) * H + h].x);
  M = fmaxf(wave_max(M), sink2);
  const float w_l = ml.x == neg_inf ? 0.0f : ml.y * exp2f(ml.x - M);   // lane's span weight
  float z = w_l;
  if constexpr (MANY) {
    for (int s = lane + 64; s < splits; s += 64) {
      const float2 m2 = part_ml[(tbase + s) * H + h];
      z += m2.x == neg_inf ? 0.0f : m2.y * exp2f(m2.x - M);
    }
  }
  z = wave_sum(z) + exp2f(sink2 - M);
  for (int s0 = 0; s0 < splits; s0 += kMergeChunk) {
    if (s0 > 0) load_chunk(s0);
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      float w;
      if constexpr (MANY) w = cml[u].x == neg_inf ? 0.0f : cml[u].y * exp2f(cml[u].x - M);
      else w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), (s0 + u) & 63));
      if (s0 + u < splits) {
        w *= cmult[u];
#pragma unroll
        for (int i = 0; i < CPL; ++i) acc[i] += chunk[u][i] * w;
      }
    }
  }
  const float f = 1.0f / z;
  uint16_t* orow = out + (static_cast<long long>(t) * H + h) * D + lane * CPL;
  if constexpr (CPL % 2 == 0) {
    uint32_t* o32 = reinterpret_cast<uint32_t*>(orow);
#pragma unroll
    for (int i = 0; i < CPL; i += 2) o32[i >> 1] = pack_bf16x2(acc[i] * f, acc[i + 1] * f);
  } else {
#pragma unroll
    for (int i = 0; i < CPL; ++i) orow[i] = f32_to_bf16(acc[i] * f);
  }
  if (lse && lane == 0) lse[static_cast<long long>(t) * H + h] = (M + log2f(z)) * kLn2;
}

// Schedule shared by the launcher and the workspace helper.  Prefill and
// large decode batches walk each row's whole key list in one work-group (the
// ring kernel, no partials); small decode batches split the list into
// kSpan-entry spans per 16-head group (the decode kernel) and merge.
struct SplitPlan {
  bool ring;
  int splits;
  int ring_span;
};

// Decode lists at least this long walk spans through the ring kernel (all
// 64 heads per work-group, tiles pipelined through the LDS ring) instead of
// one 16-head work-group per 128 entries, whose setup latency repeats for
// every span and every head group.
constexpr int kRingSplitMin = 1024;

// Decode batches of at least this many active rows fill the CUs with one
// work-group per row.
constexpr int kRingRowsMin = 256;

SplitPlan plan_splits(int T, int k, int window, bool prefill) {
  const int lmax = max(1, window + k);
  if (prefill || T >= kRingRowsMin) return SplitPlan{true, 1, lmax};
  if (lmax < kRingSplitMin) return SplitPlan{false, (lmax + kSpan - 1) / kSpan, 0};
  // spans sized so that the row x span items fill the CUs about once
  long long span = (static_cast<long long>(lmax) * T + kDecodeCUs - 1) / kDecodeCUs;
  span = std::max<long long>(span, 4 * kTile);
  span = std::min<long long>((span + kTile - 1) / kTile * kTile, kMaxSplit - kMaxSplit % kTile);
  const int sp = static_cast<int>(span);
  return SplitPlan{true, (lmax + sp - 1) / sp, sp};
}

// Decode workspace: the FP16 scaled partials [T][splits][H][D], their FP32
// (max, sum) pairs [T][splits][H], then (16-byte aligned) the quarter factors
// [T][splits][H][4].
inline size_t attn_ws_mult_offset(int T, int splits, int H, int D) {
  const size_t n = static_cast<size_t>(T) * splits * H;
  return (n * (static_cast<size_t>(D) * 2 + 8) + 15) / 16 * 16;
}
inline size_t attn_ws_bytes(int T, int splits, int H, int D) {
  return attn_ws_mult_offset(T, splits, H, D) + static_cast<size_t>(T) * splits * H * 16;
}

// Largest decode workspace over the active counts 1 .. T: counts from
// kRingRowsMin on run whole lists without partials, so at most
// kRingRowsMin - 1 plans are compared.
size_t attn_ws_bytes_max(int T, int H, int D, int k, int window) {
  size_t need = 0;
  const int n_hi = std::min(T, kRingRowsMin - 1);
  for (int n = 1; n <= n_hi; ++n) {
    const SplitPlan plan = plan_splits(n, k, window, false);
    if (plan.splits > 1) need = std::max(need, attn_ws_bytes(n, plan.splits, H, D));
  }
  return need;
}

template <int D>
int launch_attn(const AttnArgs& in, bool ring, bool mx, hipStream_t st) {
  AttnArgs a = in;
  const long long items = static_cast<long long>(a.num_tokens) * a.splits *
                          (ring ? 1 : (a.H + 15) / 16);
  a.items_per_xcd = static_cast<int>((items + 7) / 8);
  const long long grid = static_cast<long long>(a.items_per_xcd) * 8;
  if (grid > 0x7fffffffll) return CSA_ERR_UNSUPPORTED;
  if (ring && mx)
    hipLaunchKernelGGL((attn_kernel<D, true>), dim3(static_cast<unsigned>(grid)),
                       dim3(kRingThreads), 0, st, a);
  else if (ring)
    hipLaunchKernelGGL((attn_kernel<D, false>), dim3(static_cast<unsigned>(grid)),
                       dim3(kRingThreads), 0, st, a);
  else if (mx)
    hipLaunchKernelGGL((attn_decode_kernel<D, true>), dim3(static_cast<unsigned>(grid)),
                       dim3(kAttnThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_decode_kernel<D, false>), dim3(static_cast<unsigned>(grid)),
                       dim3(kAttnThreads), 0, st, a);
  if (hipGetLastError() != hipSuccess) return CSA_ERR_LAUNCH;
  if (a.splits > 1) {
    const long long items = static_cast<long long>(a.num_tokens) * a.H;
    const long long mpx = (items + 7) / 8;
    const long long mgrid = 8 * mpx;
    if (a.splits <= 64)
      hipLaunchKernelGGL((attn_merge_kernel<D, false>), dim3(static_cast<unsigned>(mgrid)),
                         dim3(64), 0, st, a.part_o, a.part_ml, a.part_mult, a.sink, a.splits, a.H,
                         a.num_tokens, static_cast<int>(mpx), a.out, a.lse);
    else
      hipLaunchKernelGGL((attn_merge_kernel<D, true>), dim3(static_cast<unsigned>(mgrid)),
                         dim3(64), 0, st, a.part_o, a.part_ml, a.part_mult, a.sink, a.splits, a.H,
                         a.num_tokens, static_cast<int>(mpx), a.out, a.lse);
    if (hipGetLastError() != hipSuccess) return CSA_ERR_LAUNCH;
  }
  return CSA_OK;
}

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch array (looked up on first use).
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA_ERR_LAUNCH;
  std::lock_guard<std::mutex> guard(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSA_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA_OK;
}

// cmp_kv / win_kv: BF16 pools, or with mx the low-bit payload planes (packed
// E2M1 compressed rows, E4M3 window rows) whose scale planes are cmp_sc / win_sc.
int attn_entry(bool prefill, const uint16_t* q, const float* rope_cos, const float* rope_sin,
               int32_t rope_dim, int32_t rope_offset, const void* cmp_kv,
               int32_t num_cmp_blocks, const int32_t* cmp_block_table, int32_t max_cmp_blocks,
               const int32_t* topk_idx, int32_t k, int32_t ratio, const void* win_kv,
               int32_t num_win_blocks, const int32_t* win_block_table, int32_t max_win_blocks,
               int32_t window, const float* attn_sink, float softmax_scale,
               const int32_t* query_start_loc, const int32_t* positions, int32_t B, int32_t T,
               int32_t num_tokens, int32_t H, int32_t D, uint16_t* out, float* lse,
               void* workspace, size_t workspace_bytes, int32_t* err, void* stream,
               bool static_scratch = false, bool mx = false, const uint8_t* cmp_sc = nullptr,
               const uint8_t* win_sc = nullptr, const int32_t* rope_pos = nullptr,
               const float* tab_cos = nullptr,
               const float* tab_sin = nullptr, int32_t tab_cap = 0,
               float* rope_out_cos = nullptr, float* rope_out_sin = nullptr) {
  if (T < 0 || B < 0 || num_cmp_blocks < 0 || num_win_blocks < 0 || max_cmp_blocks < 0 ||
      max_win_blocks < 0 || window < 0 || k < 0)
    return CSA_ERR_SHAPE;
  // a selection array holds at most 4096 entries per row (csa_topk's bound);
  // without one, k bounds the visible compressed rows of a row
  if (num_tokens < 0 || num_tokens > T || ratio < 1 || (topk_idx && k > 4096) ||
      k > kMaxDenseK)
    return CSA_ERR_RANGE;
  if (num_tokens == 0) return CSA_OK;
  if (!q || !attn_sink || !query_start_loc || !positions || !out) return CSA_ERR_NULL;
  if (tab_cos || tab_sin) {   // rope rows gathered from the full tables
    if (tab_cap < 0) return CSA_ERR_SHAPE;
    if (rope_dim > 0 && (!tab_cos || !tab_sin || !rope_pos)) return CSA_ERR_NULL;
    if (!rope_out_cos != !rope_out_sin) return CSA_ERR_NULL;
  } else if (rope_dim > 0 && (!rope_cos || !rope_sin)) {
    return CSA_ERR_NULL;
  }
  if (H < 1 || H > 64) return CSA_ERR_UNSUPPORTED;
  if (D != 64 && D != 128 && D != 256 && D != 512) return CSA_ERR_UNSUPPORTED;
  if (rope_dim < 0 || (rope_dim & 1) || rope_offset < 0 || (rope_offset & 1) ||
      rope_offset + rope_dim > D)
    return CSA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) |
       reinterpret_cast<uintptr_t>(cmp_kv) | reinterpret_cast<uintptr_t>(win_kv)) & 15)
    return CSA_ERR_UNSUPPORTED;
  // a low-bit payload plane comes with its scale plane
  if (mx && ((cmp_kv && !cmp_sc) || (win_kv && !win_sc))) return CSA_ERR_NULL;
  // pool rows are packed in 31 bits
  if (static_cast<long long>(num_cmp_blocks) * kPage >= (1ll << 31) ||
      static_cast<long long>(num_win_blocks) * kPage >= (1ll << 31))
    return CSA_ERR_UNSUPPORTED;
  const SplitPlan plan = plan_splits(num_tokens, k, window, prefill);
  // the ring schedule holds a row's whole key list in LDS
  if (plan.ring && plan.splits == 1 && window + k > kMaxSplit) return CSA_ERR_UNSUPPORTED;
  AttnArgs a{};
  a.q = q;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.half_rope = rope_dim / 2;
  a.rope_offset = rope_offset;
  if (tab_cos && rope_dim > 0) {
    a.rope_cos = nullptr;
    a.rope_sin = nullptr;
    a.rope_pos = rope_pos;
    a.tab_cos = tab_cos;
    a.tab_sin = tab_sin;
    a.tab_cap = tab_cap;
    a.rope_out_cos = rope_out_cos;
    a.rope_out_sin = rope_out_sin;
  }
  if (mx) {
    a.cmp_fp4 = static_cast<const uint8_t*>(cmp_kv);
    a.cmp_sc = cmp_sc;
    a.win_fp8 = static_cast<const uint8_t*>(win_kv);
    a.win_sc = win_sc;
  } else {
    a.cmp_kv = static_cast<const uint16_t*>(cmp_kv);
    a.win_kv = static_cast<const uint16_t*>(win_kv);
  }
  a.num_cmp_blocks = cmp_kv ? num_cmp_blocks : 0;
  a.cmp_bt = cmp_block_table;
  a.max_cmp_blocks = cmp_block_table ? max_cmp_blocks : 0;
  a.topk = topk_idx;
  a.k = k;
  a.ratio = ratio;
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
  a.ring_span = plan.ring_span;
  a.err = err;
  if (plan.splits > 1) {
    const size_t need = attn_ws_bytes(num_tokens, plan.splits, H, D);
    if (static_scratch) {   // the library's own array instead of a workspace
      if (need > kScratchBytes) return CSA_ERR_SCRATCH;
      const int st = scratch_for_current_device(&workspace);
      if (st != CSA_OK) return st;
      workspace_bytes = kScratchBytes;
    }
    if (!workspace || workspace_bytes < need) return CSA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 15) return CSA_ERR_UNSUPPORTED;
    char* w = static_cast<char*>(workspace);
    const size_t n_part = static_cast<size_t>(num_tokens) * plan.splits * H;
    a.part_o = reinterpret_cast<uint16_t*>(w);
    a.part_ml = reinterpret_cast<float2*>(w + n_part * D * sizeof(uint16_t));
    a.part_mult = reinterpret_cast<float*>(w + attn_ws_mult_offset(num_tokens, plan.splits, H, D));
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (D) {
    case 64: return launch_attn<64>(a, plan.ring, mx, st);
    case 128: return launch_attn<128>(a, plan.ring, mx, st);
    case 256: return launch_attn<256>(a, plan.ring, mx, st);
    default: return launch_attn<512>(a, plan.ring, mx, st);
  }
}

}  // namespace

}  // namespace csa

// The launcher plans on the active count, which a padded batch ([V41]
// "Compressor state ownership": T may include trailing storage padding)
// keeps below T; the size returned covers the plan of every count 1 .. T.
extern "C" size_t csa_sparse_attn_workspace_bytes(int32_t T, int32_t H, int32_t D, int32_t k,
                                                  int32_t window) {
  if (T <= 0 || H <= 0 || D <= 0 || k < 0 || window < 0) return 0;
  return csa::attn_ws_bytes_max(T, H, D, k, window);
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

extern "C" int csa_sparse_attn_decode_rope(
    const uint16_t* q, const float* freqs_cos, const float* freqs_sin, int32_t table_capacity,
    const int32_t* position_ids, int32_t rope_dim, int32_t rope_offset, const uint16_t* cmp_kv,
    int32_t num_cmp_blocks,
    const int32_t* cmp_block_table, int32_t max_cmp_blocks, const int32_t* topk_idx, int32_t k,
    int32_t ratio, const uint16_t* win_kv, int32_t num_win_blocks,
    const int32_t* win_block_table, int32_t max_win_blocks, int32_t window,
    const float* attn_sink, float softmax_scale, const int32_t* query_start_loc,
    const int32_t* positions, int32_t B, int32_t T, int32_t num_tokens, int32_t H, int32_t D,
    uint16_t* out, float* lse, float* rope_cos, float* rope_sin, void* workspace,
    size_t workspace_bytes, int32_t* err, void* stream) {
  if (table_capacity < 0) return CSA_ERR_SHAPE;
  if (rope_dim > 0 && (!freqs_cos || !freqs_sin || !position_ids)) return CSA_ERR_NULL;
  if (rope_dim == 0) freqs_cos = freqs_sin = nullptr;   // no rope span: nothing to gather
  return csa::attn_entry(false, q, nullptr, nullptr, rope_dim, rope_offset, cmp_kv,
                         num_cmp_blocks, cmp_block_table, max_cmp_blocks, topk_idx, k, ratio,
                         win_kv, num_win_blocks, win_block_table, max_win_blocks, window,
                         attn_sink, softmax_scale, query_start_loc, positions, B, T, num_tokens,
                         H, D, out, lse, workspace, workspace_bytes, err, stream,
                         /*static_scratch=*/false, /*mx=*/false, nullptr, nullptr,
                         position_ids, freqs_cos, freqs_sin, table_capacity, rope_cos, rope_sin);
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

// The low-bit planes run the schedules of csa_sparse_attn_decode.
extern "C" size_t csa_sparse_attn_mx_workspace_bytes(int32_t T, int32_t H, int32_t D, int32_t k,
                                                     int32_t window) {
  return csa_sparse_attn_workspace_bytes(T, H, D, k, window);
}

extern "C" int csa_sparse_attn_decode_mx(
    const uint16_t* q, const float* rope_cos, const float* rope_sin, int32_t rope_dim,
    int32_t rope_offset, const uint8_t* cmp_fp4, const uint8_t* cmp_scale,
    int32_t num_cmp_blocks, const int32_t* cmp_block_table, int32_t max_cmp_blocks,
    const int32_t* topk_idx, int32_t k, int32_t ratio, const uint8_t* win_fp8,
    const uint8_t* win_scale, int32_t num_win_blocks, const int32_t* win_block_table,
    int32_t max_win_blocks, int32_t window, const float* attn_sink, float softmax_scale,
    const int32_t* query_start_loc, const int32_t* positions, int32_t B, int32_t T,
    int32_t num_tokens, int32_t H, int32_t D, uint16_t* out, float* lse, void* workspace,
    size_t workspace_bytes, int32_t* err, void* stream) {
  return csa::attn_entry(false, q, rope_cos, rope_sin, rope_dim, rope_offset, cmp_fp4,
                         num_cmp_blocks, cmp_block_table, max_cmp_blocks, topk_idx, k, ratio,
                         win_fp8, num_win_blocks, win_block_table, max_win_blocks, window,
                         attn_sink, softmax_scale, query_start_loc, positions, B, T, num_tokens,
                         H, D, out, lse, workspace, workspace_bytes, err, stream,
                         /*static_scratch=*/false, /*mx=*/true, cmp_scale, win_scale);
}

extern "C" int csa_sparse_attn_decode_mx_rope(
    const uint16_t* q, const float* freqs_cos, const float* freqs_sin, int32_t table_capacity,
    const int32_t* position_ids, int32_t rope_dim, int32_t rope_offset, const uint8_t* cmp_fp4,
    const uint8_t* cmp_scale, int32_t num_cmp_blocks, const int32_t* cmp_block_table,
    int32_t max_cmp_blocks, const int32_t* topk_idx, int32_t k, int32_t ratio,
    const uint8_t* win_fp8, const uint8_t* win_scale, int32_t num_win_blocks,
    const int32_t* win_block_table, int32_t max_win_blocks, int32_t window,
    const float* attn_sink, float softmax_scale, const int32_t* query_start_loc,
    const int32_t* positions, int32_t B, int32_t T, int32_t num_tokens, int32_t H, int32_t D,
    uint16_t* out, float* lse, float* rope_cos, float* rope_sin, void* workspace,
    size_t workspace_bytes, int32_t* err, void* stream) {
  if (table_capacity < 0) return CSA_ERR_SHAPE;
  if (rope_dim > 0 && (!freqs_cos || !freqs_sin || !position_ids)) return CSA_ERR_NULL;
  if (rope_dim == 0) freqs_cos = freqs_sin = nullptr;   // no rope span: nothing to gather
  return csa::attn_entry(false, q, nullptr, nullptr, rope_dim, rope_offset, cmp_fp4,
                         num_cmp_blocks, cmp_block_table, max_cmp_blocks, topk_idx, k, ratio,
                         win_fp8, num_win_blocks, win_block_table, max_win_blocks, window,
                         attn_sink, softmax_scale, query_start_loc, positions, B, T, num_tokens,
                         H, D, out, lse, workspace, workspace_bytes, err, stream,
                         /*static_scratch=*/false, /*mx=*/true, cmp_scale, win_scale,
                         position_ids, freqs_cos, freqs_sin, table_capacity, rope_cos, rope_sin);
}

extern "C" size_t csa_sparse_attn_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int csa_sparse_attn_decode_noalloc(
    const uint16_t* q, const float* rope_cos, const float* rope_sin, int32_t rope_dim,
    int32_t rope_offset, const uint16_t* cmp_kv, int32_t num_cmp_blocks,
    const int32_t* cmp_block_table, int32_t max_cmp_blocks, const int32_t* topk_idx, int32_t k,
    int32_t ratio, const uint16_t* win_kv, int32_t num_win_blocks,
    const int32_t* win_block_table, int32_t max_win_blocks, int32_t window,
    const float* attn_sink, float softmax_scale, const int32_t* query_start_loc,
    const int32_t* positions, int32_t B, int32_t T, int32_t num_tokens, int32_t H, int32_t D,
    uint16_t* out, float* lse, int32_t* err, void* stream) {
  return csa::attn_entry(false, q, rope_cos, rope_sin, rope_dim, rope_offset, cmp_kv,
                         num_cmp_blocks, cmp_block_table, max_cmp_blocks, topk_idx, k, ratio,
                         win_kv, num_win_blocks, win_block_table, max_win_blocks, window,
                         attn_sink, softmax_scale, query_start_loc, positions, B, T, num_tokens,
                         H, D, out, lse, nullptr, 0, err, stream, /*static_scratch=*/true);
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
    case CSA_ERR_SCRATCH:
      return "CSA_ERR_SCRATCH: the call needs more than the library's static scratch holds";
    default: return "unknown csa_status";
  }
}
