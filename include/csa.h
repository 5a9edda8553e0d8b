/*
 * csa.h -- C ABI of libcsa.so: one compressed-sparse-attention (CSA) layer
 * step on AMD Instinct MI355X (gfx950).
 *
 * The step, per query row:
 *   1. csa_materialize_rope_rows  -- gather FP32 half-width RoPE rows
 *   2. csa_index_score            -- INT8 lightning-indexer scores over the
 *                                    causally visible compressed positions
 *      (csa_index_score_mxfp4 / csa_index_score_fp8: the same scores from
 *      the MXFP4 or FP8 index plane)
 *   3. csa_topk                   -- the k best positions, ascending, -1 padded
 *      (hierarchical layers: csa_candidate_blocks publishes a block mask;
 *      csa_index_score_candidates + csa_topk_candidates select inside it)
 *   4. csa_sparse_attn_decode /   -- shared-KV attention over the 128-token
 *      csa_sparse_attn_prefill       window and the selected compressed rows,
 *                                    with one sink logit per head
 *      (csa_sparse_attn_decode_mx: the same over the MXFP8 window and MXFP4
 *      compressed KV planes; csa_sparse_attn_decode_rope / _mx_rope: step 1
 *      folded into the decode attention, which reads the full tables and
 *      writes the rope rows out)
 *   5. csa_inverse_rope           -- the output's rope span rotated back by the
 *                                    query row's angles
 * and the step before the path: csa_compress_pairs publishes ratio-2
 * compressed rows from the projections and its FP32 state ring
 * (csa_compress_pairs_rope: with its rope rows read from the full tables).
 *
 * Pages the contracts follow (cited by title and section):
 *   [V41]  pypto-lib "DeepSeek V4.1 Flash": "Serving-owned full RoPE tables",
 *          "Compressor state ownership" (query_start_loc / positions /
 *          num_tokens contract; indices checked before table indexing),
 *          "Decode composition" (top-k checks, -1 padding, 128-token block
 *          tables, padding rows).
 *   [HP]   gitcode hyper-parallel issue #2 (DeepSeek V4 CP notes): Stage-2
 *          operator calls (sinks, softmax_scale, ori_win_left = 127,
 *          ori_win_right = 0), sections 8.2 / 10.3 (causal compressed
 *          visibility c < (p+1)//ratio), 9.1 (window KV and compressed KV
 *          joined, indices are the union), 10.2 (indexer indices are
 *          compressed slot ids).
 *   [MTP]  pypto-lib "DeepSeek V4-Flash, MTP point": "What is quantized"
 *          (INT8 index keys with FP32 per-row scale, BF16 KV, FP32 sinks),
 *          "Deployment configuration" (4 requests x S=2 decode rows, 128-token
 *          pages, work scales with the visible context).
 *   [ATOM] ROCm ATOM "DeepSeek-V4.1 native paged runtime": "Current execution
 *          scope" (per-row bounds read on the device; padding sentinels).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees or retains them; scratch space is a caller
 *     workspace whose size a *_workspace_bytes helper returns.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream). Sizes are host scalars. Per-row bounds (visible span, window,
 *     owning request) are derived on the device, so the same launch serves any
 *     batch contents (graph-capturable; [ATOM]).
 *   - Tensors are dense, row-major (C order) with the shapes given below. BF16
 *     values are passed as their uint16 bit patterns.
 *   - PAGE = 128: row c of a request lives at pool row
 *       block_table[b * max_blocks + c / 128] * 128 + c % 128.
 *   - Active rows are t < num_tokens; rows t >= num_tokens of every output are
 *     never read or written ([V41]). num_tokens == 0 returns CSA_OK with no
 *     launch. Row t belongs to the request b with
 *     query_start_loc[b] <= t < query_start_loc[b+1] (equal neighbours are an
 *     empty request).
 *   - Return value: a csa_status. A negative status means nothing was
 *     launched (host-checkable argument errors). Device-detected contract
 *     violations OR a CSA_EFLAG_* bit into *err (if err != NULL; the caller
 *     zeroes it) and are handled as each function states -- never by an
 *     out-of-range access.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_PAGE 128

typedef enum {
  CSA_OK = 0,
  CSA_ERR_NULL = -1,        /* a required pointer is NULL                        */
  CSA_ERR_SHAPE = -2,       /* a size is negative or inconsistent                */
  CSA_ERR_RANGE = -3,       /* num_tokens outside [0, T], k > width, ratio < 1   */
  CSA_ERR_UNSUPPORTED = -4, /* a shape this build has no kernel for              */
  CSA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than the helper's size  */
  CSA_ERR_LAUNCH = -6,      /* the HIP runtime refused a launch                  */
  CSA_ERR_SCRATCH = -7      /* needs more than the static scratch of a *_noalloc */
} csa_status;

/* device error word bits, OR-ed into *err */
#define CSA_EFLAG_POS_RANGE 1   /* position >= table capacity, or a visible span past its storage */
#define CSA_EFLAG_BLOCK_RANGE 2 /* a needed page lies past the block table or names an invalid block */
#define CSA_EFLAG_TOPK_RANGE 4  /* a selected index is not visible to its row                  */
#define CSA_EFLAG_META 8        /* an active row that no request owns                          */

/* Human-readable name of a csa_status. */
const char* csa_status_string(int status);

/*
 * csa_materialize_rope_rows -- [V41] "Serving-owned full RoPE tables".
 *
 *   freqs_cos, freqs_sin  FP32 [table_capacity, half_rope_dim], read only
 *   position_ids          INT32 [T]
 *   rope_cos, rope_sin    FP32 [T, half_rope_dim], written for t < num_tokens
 *
 * Row t < num_tokens: position p = position_ids[t]; p < 0 writes the identity
 * (cos = 1.0, sin = +0.0); 0 <= p < table_capacity copies table row p bit for
 * bit; p >= table_capacity flags CSA_EFLAG_POS_RANGE and leaves the row
 * untouched.
 */
int csa_materialize_rope_rows(const float* freqs_cos, const float* freqs_sin,
                              int32_t table_capacity, int32_t half_rope_dim,
                              const int32_t* position_ids, int32_t T, int32_t num_tokens,
                              float* rope_cos, float* rope_sin, int32_t* err, void* stream);

/*
 * csa_inverse_rope -- inverse RoPE of the attention output ([ATOM]
 * "DeepSeek-V4.1 native paged runtime", introduction and "Current execution
 * scope": the V4 attention is followed by an inverse RoPE kernel, which the
 * pages name but do not define).  Reading: K = V rows carry their rope span
 * rotated by their own positions, so the output's rope span mixes rotated
 * values; this call rotates that span back by the query row's angles.  For
 * every head of active row t and pair i of channels
 * (rope_offset + 2i, rope_offset + 2i + 1):
 *     (x, y) -> (x c + y s, y c - x s),  c = rope_cos[t][i], s = rope_sin[t][i]
 * (multiplication by the conjugate of the rope row), in FP32, rounded to
 * nearest even BF16; the other channels are copied.
 *
 *   in, out            BF16 [T, H, D]; out may equal in (in place)
 *   rope_cos/sin       FP32 [T, rope_dim / 2]: the rows the query was rotated
 *                      with (csa_materialize_rope_rows)
 *
 * Rows t >= num_tokens of out are not written.  Supported: D a multiple of 4,
 * rope_dim and rope_offset even, rope_offset + rope_dim <= D, in and out
 * 8-byte aligned.
 */
int csa_inverse_rope(const uint16_t* in, uint16_t* out, const float* rope_cos,
                     const float* rope_sin, int32_t rope_dim, int32_t rope_offset, int32_t T,
                     int32_t num_tokens, int32_t H, int32_t D, void* stream);
/*
 * csa_index_score -- lightning-indexer scores ([HP] 10.2 / 10.3; [MTP] INT8
 * index keys with an FP32 per-row scale; per-row bounds as in [ATOM]).
 *
 *   q_idx        INT8 [T, Hi, Di]   quantised indexer query
 *   q_scale      FP32 [T, Hi]       its per-(row, head) scale, > 0
 *   head_w       FP32 [T, Hi]       per-head weights
 *   idx_kv       INT8 [num_blocks, 128, Di]  index keys (one per position)
 *   idx_scale    FP32 [num_blocks, 128]      key scales, > 0
 *   block_table  INT32 [B, max_blocks]
 *   query_start_loc INT32 [B + 1], positions INT32 [T] (causal positions)
 *   scores       FP32 [T, score_stride], written for t < num_tokens
 *
 * For active row t of request b at position p and c < n = (p + 1) / ratio:
 *   scores[t][c] = sum_h head_w[t][h] * relu(q_scale[t][h] * idx_scale[c]
 *                                            * <q_idx[t][h], idx_kv[c]>)
 * with exact INT32 dots and an FP32 epilogue (evaluated as
 * idx_scale[c] * sum_h (head_w * q_scale)[t][h] * relu(dot), which equals the
 * formula for positive scales); -0.0 results are written as +0.0. Entries
 * c in [n, score_stride) are set to -inf.
 * Violations: a row no request owns -> CSA_EFLAG_META, whole row -inf; n past
 * score_stride or past 128 * max_blocks -> CSA_EFLAG_POS_RANGE, n is cut;
 * a visible position on a page with an invalid block id ->
 * CSA_EFLAG_BLOCK_RANGE, that position scores -inf.
 * Supported: 1 <= Hi <= 64, 16 <= Di <= 128 with Di a multiple of 16,
 * ratio >= 1; q_idx and idx_kv 16-byte aligned (else CSA_ERR_UNSUPPORTED).
 */
int csa_index_score(const int8_t* q_idx, const float* q_scale, const float* head_w,
                    const int8_t* idx_kv, const float* idx_scale, int32_t num_blocks,
                    const int32_t* block_table, int32_t max_blocks,
                    const int32_t* query_start_loc, const int32_t* positions,
                    int32_t B, int32_t T, int32_t num_tokens, int32_t Hi, int32_t Di,
                    int32_t ratio, float* scores, int64_t score_stride, int32_t* err,
                    void* stream);

/*
 * csa_topk -- per active row, the k best of its visible positions
 * ([V41] "Decode composition": eligibility, uniqueness, logical-position
 * order, trailing -1; [HP] 7.4: width capped by the key length).
 *
 *   scores     FP32 [T, score_stride]
 *   positions  INT32 [T]; the visible span of row t is n = (p + 1) / ratio,
 *              cut to score_stride (CSA_EFLAG_POS_RANGE if cut)
 *   topk_idx   INT32 [T, k]: the m = min(k, n) chosen positions ascending,
 *              then -1
 *   topk_val   FP32 [T, k] or NULL: the chosen scores, -inf for padding
 *   workspace  device scratch of csa_topk_workspace_bytes(T, score_stride, k)
 *              bytes, 16-byte aligned (may be NULL when that size is 0): per
 *              row a threshold word, one count per 2,048 positions and one
 *              8-byte slot per score. No state survives a call, so it needs no
 *              initialisation (calls that overlap on different streams need
 *              separate workspaces).
 *
 * Ranking: score descending, ties to the lower position; -0.0 equals +0.0;
 * NaN ranks below every number. Supported: 1 <= k <= 4096, score_stride a
 * multiple of 4 and at most 2^24, scores 16-byte aligned. Rows whose span
 * exceeds 8,192 in a launch with score_stride > 32,768 take a three-kernel
 * path (sampled threshold, candidate filter, exact select among the
 * candidates); when the sample leaves fewer than min(k, n) or more than 8,192
 * candidates, that row falls back to an exact whole-row select.
 */
size_t csa_topk_workspace_bytes(int32_t T, int64_t score_stride, int32_t k);
int csa_topk(const float* scores, int64_t score_stride, const int32_t* positions,
             int32_t ratio, int32_t T, int32_t num_tokens, int32_t k, int32_t* topk_idx,
             float* topk_val, void* workspace, size_t workspace_bytes, int32_t* err,
             void* stream);

/*
 * csa_sparse_attn_decode -- shared-KV sparse attention with sink
 * ([HP] Stage-2 calls and 9.1; [MTP] BF16 KV, FP32 attn_sink).
 *
 *   q            BF16 [T, H, D]
 *   rope_cos/sin FP32 [T, rope_dim / 2]: rope rows of each query row
 *                (csa_materialize_rope_rows); channels
 *                [rope_offset, rope_offset + rope_dim) of q are rotated in
 *                adjacent pairs (2i, 2i+1) by angle i before use
 *   cmp_kv       BF16 [num_cmp_blocks, 128, D]  compressed KV (K = V)
 *   cmp_block_table INT32 [B, max_cmp_blocks]
 *   topk_idx     INT32 [T, k]: request-local compressed positions; negative
 *                entries are padding.  NULL selects, for each row, every
 *                causally visible compressed row, positions 0 .. n_vis - 1
 *                (the indexer-less ratio-128 HCA layers: [MTP] "Layer
 *                schedule" and "Attention paths"; the [HP] Stage-2 call for
 *                ratio=128 passes no sparse indices); k then bounds n_vis,
 *                and a row with n_vis > k keeps positions 0 .. k - 1 and sets
 *                CSA_EFLAG_TOPK_RANGE.  k = 0 leaves the window alone (the
 *                SWA-only layers; no flag); topk_idx and the compressed pool
 *                may then be NULL
 *   win_kv       BF16 [num_win_blocks, 128, D]  raw-token (window) KV
 *   win_block_table INT32 [B, max_win_blocks], indexed by raw position
 *   attn_sink    FP32 [H]
 *   out          BF16 [T, H, D]  (round to nearest even of the FP32 result)
 *   lse          FP32 [T, H] or NULL
 *   workspace    csa_sparse_attn_workspace_bytes(T, H, D, k, window) bytes,
 *                16-byte aligned (NULL when that size is 0); scratch for the
 *                split partials, always written before it is read (calls
 *                that overlap on different streams need separate workspaces).
 *                The schedule is chosen from num_tokens; the helper's size,
 *                taken with the storage extent T, covers every num_tokens in
 *                [0, T], so a padded batch sized by T never gets
 *                CSA_ERR_WORKSPACE.
 *
 * Row t of request b at position p attends, with every head, over the window
 * rows at raw positions [max(0, p - window + 1), p] followed by the selected
 * compressed rows (no deduplication between the two caches):
 *   l_j = softmax_scale * <rot(q[t][h]), K_j>,  M = max(sink_h, max_j l_j),
 *   Z = exp(sink_h - M) + sum_j exp(l_j - M),
 *   out = sum_j exp(l_j - M) / Z * K_j,  lse = M + log Z.
 * An empty set gives out = 0, lse = sink. Violations: a row no request owns
 * -> CSA_EFLAG_META, treated as empty; a selected entry >= (p + 1) / ratio ->
 * CSA_EFLAG_TOPK_RANGE, left out; a window or selected row whose page is past
 * the table or names an invalid block -> CSA_EFLAG_BLOCK_RANGE, left out.
 * Supported: 1 <= H <= 64, D in {64, 128, 256, 512}, rope_dim and rope_offset
 * even, rope_offset + rope_dim <= D, window >= 0, 0 <= k <= 4096 with a
 * selection array and k <= 2^20 without one, pools of fewer than 2^31 rows;
 * the prefill schedule (and decode batches of 256 rows or more) needs
 * window + k <= 4224, the decode schedule takes any key-list length.
 * Arithmetic: the rotated query and the probabilities are rounded to BF16 as
 * MFMA operands; logits, softmax and accumulation are FP32.
 */
size_t csa_sparse_attn_workspace_bytes(int32_t T, int32_t H, int32_t D, int32_t k,
                                       int32_t window);
int csa_sparse_attn_decode(const uint16_t* q, const float* rope_cos, const float* rope_sin,
                           int32_t rope_dim, int32_t rope_offset, const uint16_t* cmp_kv,
                           int32_t num_cmp_blocks, const int32_t* cmp_block_table,
                           int32_t max_cmp_blocks, const int32_t* topk_idx, int32_t k,
                           int32_t ratio, const uint16_t* win_kv, int32_t num_win_blocks,
                           const int32_t* win_block_table, int32_t max_win_blocks,
                           int32_t window, const float* attn_sink, float softmax_scale,
                           const int32_t* query_start_loc, const int32_t* positions,
                           int32_t B, int32_t T, int32_t num_tokens, int32_t H, int32_t D,
                           uint16_t* out, float* lse, void* workspace,
                           size_t workspace_bytes, int32_t* err, void* stream);

/*
 * csa_sparse_attn_decode_rope -- csa_sparse_attn_decode with the RoPE-row
 * materialisation ([V41] "Serving-owned full RoPE tables") folded into the
 * same launch: the query of row t is rotated by row position_ids[t] of the
 * full tables, and that row is also written out, so a decode step needs no
 * separate csa_materialize_rope_rows launch.
 *
 *   freqs_cos, freqs_sin  FP32 [table_capacity, rope_dim / 2], read only
 *   position_ids          INT32 [T]: each row's RoPE position (as for
 *                         csa_materialize_rope_rows; positions still gives
 *                         the cache position); the three may be NULL when
 *                         rope_dim = 0
 *   rope_cos, rope_sin    FP32 [T, rope_dim / 2], written for t < num_tokens
 *                         exactly as csa_materialize_rope_rows writes them
 *                         (identity for a negative position, table row p bit
 *                         for bit, untouched and CSA_EFLAG_POS_RANGE when
 *                         p >= table_capacity); both NULL: not written
 *
 * Every other argument, the result and its arithmetic are those of
 * csa_sparse_attn_decode (same workspace size): out and lse are bit for bit
 * what csa_materialize_rope_rows followed by csa_sparse_attn_decode give for
 * rows whose position lies inside the tables.  A row past the tables attends
 * with the identity rotation.  CSA_ERR_SHAPE for table_capacity < 0;
 * CSA_ERR_NULL for a missing table or position_ids with rope_dim > 0, or
 * only one of rope_cos and rope_sin.
 */
int csa_sparse_attn_decode_rope(const uint16_t* q, const float* freqs_cos, const float* freqs_sin,
                                int32_t table_capacity, const int32_t* position_ids,
                                int32_t rope_dim, int32_t rope_offset,
                                const uint16_t* cmp_kv, int32_t num_cmp_blocks,
                                const int32_t* cmp_block_table, int32_t max_cmp_blocks,
                                const int32_t* topk_idx, int32_t k, int32_t ratio,
                                const uint16_t* win_kv, int32_t num_win_blocks,
                                const int32_t* win_block_table, int32_t max_win_blocks,
                                int32_t window, const float* attn_sink, float softmax_scale,
                                const int32_t* query_start_loc, const int32_t* positions,
                                int32_t B, int32_t T, int32_t num_tokens, int32_t H, int32_t D,
                                uint16_t* out, float* lse, float* rope_cos, float* rope_sin,
                                void* workspace, size_t workspace_bytes, int32_t* err,
                                void* stream);

/*
 * csa_sparse_attn_prefill -- the same operation and arguments as
 * csa_sparse_attn_decode, scheduled for many query rows (a prefill walk in
 * 128-token tiles, [MTP] "Deployment configuration"): one 512-thread
 * work-group per query row, consecutive rows kept on one XCD so their shared
 * window rows and popular compressed rows stay in that XCD's L2. Needs no
 * workspace (csa_sparse_attn_workspace_bytes is still accepted).
 */
int csa_sparse_attn_prefill(const uint16_t* q, const float* rope_cos, const float* rope_sin,
                            int32_t rope_dim, int32_t rope_offset, const uint16_t* cmp_kv,
                            int32_t num_cmp_blocks, const int32_t* cmp_block_table,
                            int32_t max_cmp_blocks, const int32_t* topk_idx, int32_t k,
                            int32_t ratio, const uint16_t* win_kv, int32_t num_win_blocks,
                            const int32_t* win_block_table, int32_t max_win_blocks,
                            int32_t window, const float* attn_sink, float softmax_scale,
                            const int32_t* query_start_loc, const int32_t* positions,
                            int32_t B, int32_t T, int32_t num_tokens, int32_t H, int32_t D,
                            uint16_t* out, float* lse, void* workspace,
                            size_t workspace_bytes, int32_t* err, void* stream);

/*
 * csa_sparse_attn_decode_mx -- csa_sparse_attn_decode reading the low-bit KV
 * planes of the production cache ABI ([V41], the paragraph on the production
 * cache ABI before "Compressor state ownership": window KV as MXFP8 E4M3 with
 * E8M0 group-of-32 scales, compressed KV as packed MXFP4 E2M1 with E4M3
 * group-of-16 scales; the references quantise on cache publication and
 * dequantise on cache reads).  Every argument but the four planes is that of
 * csa_sparse_attn_decode, with the same meaning, checks and flags.
 *
 *   cmp_fp4   UINT8 [num_cmp_blocks, 128, D / 2]: packed E2M1 codes, channel
 *             2i in bits 0-3 of byte i, channel 2i + 1 in bits 4-7
 *   cmp_scale UINT8 [num_cmp_blocks, 128, D / 16]: E4M3 (OCP E4M3FN) codes;
 *             channel c of a row is e2m1(c) * e4m3(cmp_scale[c / 16])
 *   win_fp8   UINT8 [num_win_blocks, 128, D]: E4M3 codes
 *   win_scale UINT8 [num_win_blocks, 128, D / 32]: E8M0 bytes; channel c of a
 *             row is e4m3(c) * 2^(win_scale[c / 32] - 127) (byte 255 is NaN)
 *   workspace csa_sparse_attn_mx_workspace_bytes(T, H, D, k, window) bytes
 *             (the same size as csa_sparse_attn_workspace_bytes), 16-byte
 *             aligned, NULL when that size is 0; it covers every num_tokens
 *             up to T.
 *
 * Each row is dequantised exactly (an E4M3 code times a power of two, or an
 * E2M1 code times an E4M3 code, is a BF16 value; only products outside BF16's
 * normal range, from extreme E8M0 bytes, are rounded) into the BF16 tile the
 * attention multiplies, so the result is csa_sparse_attn_decode's on the
 * dequantised rows.  NaN codes propagate as NaN.  A payload plane given without its scale plane returns
 * CSA_ERR_NULL; a NULL pair is an empty pool (its rows flag BLOCK_RANGE).
 * Plane pointers are 16-byte aligned.  The schedules are those of
 * csa_sparse_attn_decode (its kernels with the rows dequantised on their way
 * into LDS), so the result has the same bits as csa_sparse_attn_decode on
 * BF16 pools holding the dequantised rows.  There is no prefill form.
 */
size_t csa_sparse_attn_mx_workspace_bytes(int32_t T, int32_t H, int32_t D, int32_t k,
                                          int32_t window);
int csa_sparse_attn_decode_mx(const uint16_t* q, const float* rope_cos, const float* rope_sin,
                              int32_t rope_dim, int32_t rope_offset, const uint8_t* cmp_fp4,
                              const uint8_t* cmp_scale, int32_t num_cmp_blocks,
                              const int32_t* cmp_block_table, int32_t max_cmp_blocks,
                              const int32_t* topk_idx, int32_t k, int32_t ratio,
                              const uint8_t* win_fp8, const uint8_t* win_scale,
                              int32_t num_win_blocks, const int32_t* win_block_table,
                              int32_t max_win_blocks, int32_t window, const float* attn_sink,
                              float softmax_scale, const int32_t* query_start_loc,
                              const int32_t* positions, int32_t B, int32_t T,
                              int32_t num_tokens, int32_t H, int32_t D, uint16_t* out,
                              float* lse, void* workspace, size_t workspace_bytes,
                              int32_t* err, void* stream);

/*
 * csa_sparse_attn_decode_mx_rope -- csa_sparse_attn_decode_mx with the RoPE
 * rows gathered from the full tables in the same launch, exactly as
 * csa_sparse_attn_decode_rope does for the BF16 pools: freqs_cos / freqs_sin
 * / table_capacity / position_ids replace the rope rows, and rope_cos /
 * rope_sin (both or neither) receive them.  Every other argument, check and
 * flag is csa_sparse_attn_decode_mx's.
 */
int csa_sparse_attn_decode_mx_rope(const uint16_t* q, const float* freqs_cos,
                                   const float* freqs_sin, int32_t table_capacity,
                                   const int32_t* position_ids, int32_t rope_dim,
                                   int32_t rope_offset, const uint8_t* cmp_fp4,
                                   const uint8_t* cmp_scale, int32_t num_cmp_blocks,
                                   const int32_t* cmp_block_table, int32_t max_cmp_blocks,
                                   const int32_t* topk_idx, int32_t k, int32_t ratio,
                                   const uint8_t* win_fp8, const uint8_t* win_scale,
                                   int32_t num_win_blocks, const int32_t* win_block_table,
                                   int32_t max_win_blocks, int32_t window,
                                   const float* attn_sink, float softmax_scale,
                                   const int32_t* query_start_loc, const int32_t* positions,
                                   int32_t B, int32_t T, int32_t num_tokens, int32_t H,
                                   int32_t D, uint16_t* out, float* lse, float* rope_cos,
                                   float* rope_sin, void* workspace, size_t workspace_bytes,
                                   int32_t* err, void* stream);

/*
 * csa_sparse_attn_decode_noalloc -- csa_sparse_attn_decode for callers that
 * cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * operation, arguments (without the workspace), kernels and results; the
 * split partials go to a static device array of the library,
 * csa_sparse_attn_noalloc_max_bytes() bytes (32 MiB) per GPU, held by each
 * GPU the library runs on until the process ends.  Its device address is
 * looked up on the first call on a device (the stream must belong to the
 * current device).  The call allocates nothing and frees nothing.
 *
 * Limit: a call whose schedule needs more partial bytes than the array holds
 * (csa_sparse_attn_workspace_bytes(num_tokens, H, D, k, window) for a batch
 * of num_tokens rows) returns CSA_ERR_SCRATCH and launches nothing.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (partials are written before they are read, so nothing needs
 * clearing): calls that overlap on one GPU (different streams, or a graph
 * replayed concurrently) race and must be serialized by the caller.
 */
size_t csa_sparse_attn_noalloc_max_bytes(void);
int csa_sparse_attn_decode_noalloc(const uint16_t* q, const float* rope_cos,
                                   const float* rope_sin, int32_t rope_dim, int32_t rope_offset,
                                   const uint16_t* cmp_kv, int32_t num_cmp_blocks,
                                   const int32_t* cmp_block_table, int32_t max_cmp_blocks,
                                   const int32_t* topk_idx, int32_t k, int32_t ratio,
                                   const uint16_t* win_kv, int32_t num_win_blocks,
                                   const int32_t* win_block_table, int32_t max_win_blocks,
                                   int32_t window, const float* attn_sink, float softmax_scale,
                                   const int32_t* query_start_loc, const int32_t* positions,
                                   int32_t B, int32_t T, int32_t num_tokens, int32_t H,
                                   int32_t D, uint16_t* out, float* lse, int32_t* err,
                                   void* stream);

/*
 * csa_index_score_mxfp4 -- csa_index_score with the FP4 index plane
 * ([V41] cache ABI: index keys packed MXFP4 E2M1 with group-of-32 E8M0
 * scales; [ATOM] "Current execution scope": the FP4 index arithmetic is E2M1
 * with one E8M0 scale per 32 dims).  The query side uses the same format, and
 * the score is
 *     score[t,c] = sum_h w[t,h] * relu( <mx(q[t,h]), mx(k[c])> )
 * where mx() multiplies each E2M1 value by 2^(s - 127), s the E8M0 byte of its
 * group of 32 dims.  Visibility, metadata, flags and the output layout are
 * csa_index_score's.
 *
 *   q_fp4    UINT8 [T, Hi, Di/2]: packed E2M1, the lower-indexed element of a
 *            pair in bits 0-3
 *   q_sc     UINT8 [T, Hi, Di/32]: E8M0 scales of the query rows
 *   head_w   FP32 [T, Hi]
 *   idx_fp4  UINT8 [num_blocks, 128, Di/2]; idx_sc UINT8 [num_blocks, 128,
 *            Di/32]: the key pool, paged like csa_index_score's
 *
 * Supported: Di = 128, Hi <= 64; q_fp4, q_sc, idx_fp4, idx_sc 16-byte
 * aligned.  The dots run on gfx950's block-scaled FP4 MFMA in FP32.
 */
int csa_index_score_mxfp4(const uint8_t* q_fp4, const uint8_t* q_sc, const float* head_w,
                          const uint8_t* idx_fp4, const uint8_t* idx_sc, int32_t num_blocks,
                          const int32_t* block_table, int32_t max_blocks,
                          const int32_t* query_start_loc, const int32_t* positions, int32_t B,
                          int32_t T, int32_t num_tokens, int32_t Hi, int32_t Di, int32_t ratio,
                          float* scores, int64_t score_stride, int32_t* err, void* stream);

/*
 * csa_index_score_fp8 -- csa_index_score with the FP8 index plane ([ATOM]
 * "Current execution scope": FP8 is the default index cache dtype; the pages
 * give no layout, so it is read as the INT8 plane's with OCP E4M3FN codes in
 * place of INT8 ones).  The score is
 *     score[t,c] = sum_h w[t,h] * relu( qs[t,h] * ks[c] * <e4m3(q[t,h]), e4m3(k[c])> )
 * with every argument, layout, check and flag as in csa_index_score, except:
 *
 *   q_fp8    UINT8 [T, Hi, Di]: E4M3 codes of the query rows
 *   idx_fp8  UINT8 [num_blocks, 128, Di]: E4M3 codes of the key rows
 *
 * The codes must not be NaN (0x7F, 0xFF).  The dots run on gfx950's
 * block-scaled FP8 MFMA with unit block scales; products of two E4M3 values
 * are exact in FP32, so only the accumulation order differs from an exact
 * dot.  Supported: as csa_index_score (16 <= Di <= 128, Di a multiple of 16,
 * Hi <= 64).
 */
int csa_index_score_fp8(const uint8_t* q_fp8, const float* q_scale, const float* head_w,
                        const uint8_t* idx_fp8, const float* idx_scale, int32_t num_blocks,
                        const int32_t* block_table, int32_t max_blocks,
                        const int32_t* query_start_loc, const int32_t* positions, int32_t B,
                        int32_t T, int32_t num_tokens, int32_t Hi, int32_t Di, int32_t ratio,
                        float* scores, int64_t score_stride, int32_t* err, void* stream);

/*
 * csa_compress_pairs -- the ratio-2 compressor's publication and its FP32
 * state ring, the step before the path ([V41] "Compressor state ownership";
 * the cache ABI paragraph: a ring row is the token's KV projection followed by
 * its gate score).  For request b (rows query_start_loc[b] .. [b+1] of the
 * active prefix, consecutive positions) with state block
 * blk = state_block_table[b]:
 *   - a token at odd position p closes the pair (p - 1, p) and publishes
 *     compressed position p / 2 of request b; its predecessor is the
 *     preceding input row, or for the chunk's first row the ring row
 *     blk * state_capacity + (p - 1) % state_capacity;
 *   - publication: per channel, the softmax of the pair's gate scores weights
 *     its KV projections; the result is rounded to BF16, normalised
 *     (x * rsqrt(mean(x^2) + rms_eps) * rms_gamma), its rope span
 *     [rope_offset, rope_offset + rope_dim) rotated in adjacent pairs by the
 *     rope row given for the token (the pair's start position: the pages'
 *     group-start RoPE rows), and stored rounded to nearest even BF16 in the
 *     compressed pool through cmp_block_table (128-row pages);
 *   - after every ring read of the call, the last min(chunk, state_capacity)
 *     rows of each chunk are stored at slot blk * state_capacity + p %
 *     state_capacity ([kv_proj row | gate row], FP32).
 * The pooling, rounding, normalisation and rope steps are named but not
 * defined on the pages; the above is the plain reading.
 *
 *   kv_proj, gate      FP32 [T, D]
 *   state_block_table  INT32 [B]: -1 disables the request (no access at all)
 *   state_cache        FP32 [num_state_blocks, state_capacity, 2 * D], in/out
 *   rms_gamma          FP32 [D]; rms_eps >= 0
 *   rope_cos/sin       FP32 [T, rope_dim / 2]
 *   cmp_kv             BF16 [num_cmp_blocks, 128, D], written at published rows
 *   cmp_block_table    INT32 [B, max_cmp_blocks]
 *
 * Negative positions neither publish nor write.  A state block >= the pool
 * size or a publication page past the table or naming an invalid block sets
 * CSA_EFLAG_BLOCK_RANGE and that access is skipped; an active row no request
 * owns sets CSA_EFLAG_META.  Supported: D even and <= 2048, rope_dim and
 * rope_offset even, rope_offset + rope_dim <= D, state_capacity >= 1, the FP32
 * arrays and cmp_kv 8-byte aligned.  Requests must not share a state block
 * (their ring accesses would race).  One kernel launch on `stream`: the work-
 * group of a request's first row does its only ring read and then writes the
 * request's ring rows, in row order (a later row with the same slot wins).
 */
int csa_compress_pairs(const float* kv_proj, const float* gate, int32_t D,
                       const int32_t* query_start_loc, const int32_t* positions, int32_t B,
                       int32_t T, int32_t num_tokens, const int32_t* state_block_table,
                       float* state_cache, int32_t num_state_blocks, int32_t state_capacity,
                       const float* rms_gamma, float rms_eps, const float* rope_cos,
                       const float* rope_sin, int32_t rope_dim, int32_t rope_offset,
                       uint16_t* cmp_kv, int32_t num_cmp_blocks,
                       const int32_t* cmp_block_table, int32_t max_cmp_blocks, int32_t* err,
                       void* stream);

/*
 * csa_compress_pairs_rope -- csa_compress_pairs with each token's rope row
 * gathered from the full tables ([V41] "Serving-owned full RoPE tables") in
 * the same launch instead of read from materialised rows: the row of token t
 * is table row rope_position_ids[t] (the pair's start position; identity for
 * a negative one).  A position >= table_capacity sets CSA_EFLAG_POS_RANGE, as
 * csa_materialize_rope_rows would, and a publication of that token rotates
 * by the identity.  Every other argument, check and flag is
 * csa_compress_pairs's; the published rows and the ring are bit for bit
 * those of csa_materialize_rope_rows followed by csa_compress_pairs for
 * positions inside the tables.
 *
 *   freqs_cos, freqs_sin  FP32 [table_capacity, rope_dim / 2]
 *   rope_position_ids     INT32 [T]
 * (the three may be NULL when rope_dim = 0; CSA_ERR_SHAPE for
 * table_capacity < 0)
 */
int csa_compress_pairs_rope(const float* kv_proj, const float* gate, int32_t D,
                            const int32_t* query_start_loc, const int32_t* positions, int32_t B,
                            int32_t T, int32_t num_tokens, const int32_t* state_block_table,
                            float* state_cache, int32_t num_state_blocks,
                            int32_t state_capacity, const float* rms_gamma, float rms_eps,
                            const float* freqs_cos, const float* freqs_sin,
                            int32_t table_capacity, const int32_t* rope_position_ids,
                            int32_t rope_dim, int32_t rope_offset, uint16_t* cmp_kv,
                            int32_t num_cmp_blocks, const int32_t* cmp_block_table,
                            int32_t max_cmp_blocks, int32_t* err, void* stream);

/*
 * Hierarchical selection ([V41] "Decode composition"): a full layer publishes
 * a candidate mask of blocks of `block` consecutive compressed positions
 * (2,048 blocks of eight in V4.1); a later reindex layer scores only the
 * mask's positions with its own index query and selects its final k
 * positions there.  A reuse layer takes another layer's selection as it is:
 * it calls the attention entry points with that topk_idx and needs nothing
 * below.  Masks stay in request-local compressed-position space.
 *
 * csa_candidate_blocks -- the full layer's mask.  Block j of row t covers
 * positions j*block .. j*block + block - 1; its score is the largest score
 * among its visible positions (c < (p + 1) / ratio, cut to score_stride with
 * CSA_EFLAG_POS_RANGE), NaN when all of them are NaN.  Blocks with no visible
 * position are not eligible.
 *
 *   scores       FP32 [T, score_stride] (csa_index_score's output)
 *   cand_blocks  INT32 [T, kb]: the min(kb, eligible) best blocks (block score
 *                descending, the lower block first, NaN below every number)
 *                ascending, then -1
 *   workspace    csa_candidate_blocks_workspace_bytes(T, score_stride, block,
 *                kb) bytes, 16-byte aligned: the block scores, one count per
 *                row, then the selection's scratch; nothing survives a call
 *
 * Supported: block divides 128, 1 <= kb <= 4096, score_stride a multiple of
 * 4, scores 16-byte aligned.
 */
size_t csa_candidate_blocks_workspace_bytes(int32_t T, int64_t score_stride, int32_t block,
                                            int32_t kb);
int csa_candidate_blocks(const float* scores, int64_t score_stride, const int32_t* positions,
                         int32_t ratio, int32_t T, int32_t num_tokens, int32_t block, int32_t kb,
                         int32_t* cand_blocks, void* workspace, size_t workspace_bytes,
                         int32_t* err, void* stream);

/*
 * csa_index_score_candidates -- a reindex layer's scores.  Slot s of row t is
 * position cand_blocks[t][s / block] * block + s % block; it scores exactly as
 * csa_index_score does at that position (the same arithmetic, bit for bit).
 * Query, key, block-table and metadata arguments are csa_index_score's.
 *
 *   cand_blocks  INT32 [T, kb]: ascending block ids, then -1 (as
 *                csa_candidate_blocks writes them)
 *   cand_scores  FP32 [T, cand_stride], cand_stride >= kb * block: slots
 *                0 .. kb*block - 1 written; a slot that is not eligible (block
 *                -1, position not visible, or its page invalid) is -inf
 *   cand_count   INT32 [T]: the number of leading eligible slots (with an
 *                ascending mask the eligible slots are exactly that prefix)
 *
 * Errors: a block past the row's visible span sets CSA_EFLAG_TOPK_RANGE, an
 * invalid page CSA_EFLAG_BLOCK_RANGE, a row no request owns CSA_EFLAG_META
 * (count 0); those slots are left out.  With a mask that does not ascend,
 * cand_count covers only its eligible prefix.
 */
int csa_index_score_candidates(const int8_t* q_idx, const float* q_scale, const float* head_w,
                               const int8_t* idx_kv, const float* idx_scale, int32_t num_blocks,
                               const int32_t* block_table, int32_t max_blocks,
                               const int32_t* query_start_loc, const int32_t* positions,
                               int32_t B, int32_t T, int32_t num_tokens, int32_t Hi, int32_t Di,
                               int32_t ratio, const int32_t* cand_blocks, int32_t kb,
                               int32_t block, float* cand_scores, int64_t cand_stride,
                               int32_t* cand_count, int32_t* err, void* stream);

/*
 * csa_topk_candidates -- a reindex layer's final selection: per active row,
 * the k best of its first cand_count[t] slots, reported as compressed
 * positions (slot s -> cand_blocks[t][s / block] * block + s % block), in
 * csa_topk's output contract (ascending, -1 / -inf padding, the same
 * ranking; with an ascending mask slot order is position order, so ties go to
 * the lower position).  workspace: csa_topk_candidates_workspace_bytes(T,
 * cand_stride, k) bytes (0 for cand_stride <= 32,768).  Supported as csa_topk,
 * with cand_stride >= kb * block.
 */
size_t csa_topk_candidates_workspace_bytes(int32_t T, int64_t cand_stride, int32_t k);
int csa_topk_candidates(const float* cand_scores, int64_t cand_stride, const int32_t* cand_count,
                        const int32_t* cand_blocks, int32_t kb, int32_t block, int32_t T,
                        int32_t num_tokens, int32_t k, int32_t* topk_idx, float* topk_val,
                        void* workspace, size_t workspace_bytes, int32_t* err, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
