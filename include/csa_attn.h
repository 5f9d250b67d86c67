/*
 * csa_attn.h -- C ABI of the CSA / HCA hybrid-attention hot path for MI355X
 * (gfx950).  Every call enqueues hand-written HIP kernels on the caller's
 * stream and returns; nothing here synchronises, allocates or frees device
 * memory.
 *
 * The method (DeepSeek-V4 hybrid attention) as the pages describe it:
 *   - "DeepSeek-V4 ... open-source declaration" (peacm.com), section 3.2
 *     "hybrid attention": CSA compresses every m tokens into one KV entry,
 *     scores the compressed blocks with a lightweight "lightning indexer" and
 *     keeps the top-k per query, runs multi-query attention over those blocks,
 *     and ends with a grouped output projection of the head-dim-512 outputs;
 *     HCA compresses 128:1 and attends every compressed entry densely.  The
 *     "four tricks" list adds RMSNorm on queries and KV before the core
 *     attention, RoPE on the last 64 dims only with a RoPE at position -i on
 *     the output, a raw sliding window of the latest 128 tokens visible to
 *     every query, and a learnable sink logit in the softmax denominator.
 *   - "DeepSeek-V4 technical report digest" (gitcode.csdn.net), section 2.1.4
 *     (KV cache: RoPE dims in BF16, the others in FP8) and section 3.2 (the
 *     indexer's QK path in FP4 E2M1 with 1x32 sub-block scales, converted
 *     losslessly to FP8).
 *   - "DeepSeek V4 (Flash & Pro)" (github wiki article), hybrid-attention
 *     section: HCA is a dense MQA stream over 128:1-compressed KV plus a
 *     128-token sliding window.
 *
 * Conventions shared by every call
 *   - Pointers inside the structs and every array argument are DEVICE
 *     pointers, owned by the caller; the structs themselves are host memory
 *     and are read during the call only.  `stream` is a hipStream_t (NULL =
 *     the null stream).
 *   - Arguments are validated on the host before any HIP call; a non-OK
 *     status means nothing was enqueued.  csa_last_error() returns a
 *     thread-local message for the last non-OK status of the calling thread.
 *   - Positions (token indices) are int32 device arrays.  A position p's
 *     compressed block is j = floor(p / m); block j is complete, and visible
 *     to a query at position t, when (j+1)*m - 1 <= t.
 *   - Kernels never read or write outside the buffers described below:
 *     block indices beyond a linear cache's capacity are not stored and not
 *     visible; top-k entries that are negative or not visible are skipped.
 *     Positions are device data, so the host cannot compare them with a
 *     linear cache's capacity: a compressed or indexer-key cache smaller
 *     than the positions need is clipped silently (the blocks at or beyond
 *     cap do not exist for the call), never reported as CSA_ERR_CAPACITY.
 *     CSA_ERR_CAPACITY is returned only for the window ring, whose needed
 *     size (window + Tq - 1) the host does know.
 *   - Results are bitwise deterministic and do not depend on the batch size B
 *     (no floating-point atomics; fixed split sizes; fixed-order merges).
 *   - Calls on one stream run in order; calls on different streams that
 *     write the same buffers race.
 */
#ifndef CSA_ATTN_H
#define CSA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CSA_OK = 0,
    CSA_ERR_INVALID_ARG = -1,  /* null pointer, bad size or inconsistent shape */
    CSA_ERR_UNSUPPORTED = -2,  /* dtype / shape combination without a kernel */
    CSA_ERR_CAPACITY = -3,     /* the window ring too small for the request */
    CSA_ERR_WORKSPACE = -4,    /* workspace missing or smaller than required */
    CSA_ERR_HIP = -5           /* a HIP launch failed (message has the HIP error) */
} csa_status;

typedef enum {
    CSA_F32 = 0,
    CSA_BF16 = 1,
    CSA_FP8_E4M3 = 2,          /* OCP E4M3FN: bias 7, max 448, no infinities */
    CSA_FP4_E2M1 = 3           /* OCP E2M1 codes with E8M0 scales per 32 values */
} csa_dtype;

/* KV cache: one record per entry, [B][cap] records, one KV head (MQA), the
 * same vector serving as key and value.  Record layout by fmt (d = head dim,
 * dr = RoPE dims, the last dr of the d):
 *   CSA_F32      : d x f32                                  (4d bytes)
 *   CSA_BF16     : d x bf16                                 (2d bytes)
 *   CSA_FP8_E4M3 : (d-dr) x E4M3 code | dr x bf16 | f32 row scale | zero pad
 *                  to a multiple of 16 bytes (592 bytes at d=512, dr=64).
 *                  Non-RoPE dim i has the value e4m3(code_i) * scale, with
 *                  scale = max|non-RoPE dims| / 448 (1 for an all-zero row);
 *                  RoPE dims stay in bf16 (technical-report digest 2.1.4).
 * ring = 0: entry index e lives in slot e (entries >= cap are dropped).
 * ring = 1: slot e mod cap (the raw sliding-window cache, indexed by token
 *           position; it must hold the last window + Tq - 1 positions). */
typedef struct {
    void* rec;
    int32_t fmt;
    int32_t d;
    int32_t d_rope;
    int32_t ring;
    int64_t cap;
} csa_kv_cache;

/* Indexer key cache, [B][cap] rows of di values (linear, no ring):
 *   CSA_F32 : codes = di x f32;  CSA_BF16 : codes = di x bf16;
 *   CSA_FP4_E2M1 : codes = di/2 bytes (element 2i in the low nibble of byte
 *                  i), scales = [B][cap][di/32] E8M0 bytes (value 2^(s-127)). */
typedef struct {
    void* codes;
    uint8_t* scales;
    int32_t fmt;
    int32_t di;
    int64_t cap;
} csa_idx_cache;

/* Attention parameters.  head_dim = d, rope_dim = dr (even, <= d), window =
 * W raw tokens (0 disables the window), m = compression ratio of `comp`,
 * rope_base = RoPE base (frequency of pair i is base^(-2i/dr)),
 * softmax_scale = logit scale (1/sqrt(d) in the method), rms_eps = RMSNorm
 * epsilon of the query prologue.
 * split_policy (the technical-report digest, section 5.3: batch-invariant,
 * deterministic kernels, a high-throughput and a low-latency one with the
 * same accumulation order):
 *   CSA_SPLIT_BY_CHUNK (0): chunks of fewer than 64 queries (decode) cut a
 *     row's entry list into fixed-size splits merged in split order; longer
 *     chunks (prefill) take the row in one pass.  A row's result then depends
 *     on whether its chunk is shorter than 64 queries (within rounding);
 *   CSA_SPLIT_FIXED (1): every chunk takes the decode splits and merge, so a
 *     row's bits depend only on the row and the caches, whatever the chunk
 *     length and the batch; a long chunk then needs the split partials'
 *     workspace (csa_attn_workspace_size) and their memory traffic. */
enum { CSA_SPLIT_BY_CHUNK = 0, CSA_SPLIT_FIXED = 1 };
typedef struct {
    int32_t head_dim;
    int32_t rope_dim;
    int32_t window;
    int32_t m;
    float rope_base;
    float softmax_scale;
    float rms_eps;
    int32_t split_policy;
} csa_attn_params;

/* Bytes of one KV record of format fmt (see csa_kv_cache); 0 if invalid. */
size_t csa_kv_record_bytes(int32_t fmt, int32_t d, int32_t d_rope);

/* ---------------------------------------------------------------------------
 * csa_compress_kv -- CSA step 1 / HCA compression (peacm 3.2: every m tokens
 * become one compressed KV entry through an attention-like mechanism; 128:1
 * for HCA), plus the KV normalisation and partial RoPE of the four tricks.
 *
 * x         : [B][T][d] raw tokens, x_dtype CSA_F32 or CSA_BF16; row (b, i)
 *             is the token at position tok_start[b] + i.
 * tok_start : device int32 [B], each a multiple of m.
 * Each complete run of m tokens (i = 0 .. T/m - 1; a ragged tail of T mod m
 * tokens is ignored) is block j = tok_start[b]/m + i and is written as
 *     z_r = score_bias[r] + <score_proj, x_r>   (score_proj NULL: no term)
 *     c   = sum_r softmax(z)_r x_r               (r < m)
 *     e   = RoPE_{j*m}( RMSNorm_gamma(c) )       (gamma NULL: no norm;
 *                                                 rope_dim 0: no RoPE)
 * into exactly one of kv_out (a KV record, m = 1 gives raw window entries)
 * or idx_out (an indexer key row, d == di).  The quantisers round to nearest
 * even: bf16; E4M3 with saturation to +-448; FP4 per 32 values with
 * e = floor(log2 amax) - 2 raised to at least (row max e) - 14, codes E2M1
 * saturating at +-6.
 * score_bias: device f32 [m]; score_proj, gamma: device f32 [d] or NULL.
 * Errors: INVALID_ARG (nulls, B or T < 0, d odd or outside [2, 1024], m
 * outside [1, 1024], rope_dim odd or > d, both or neither output, an output
 * whose d / d_rope differ from the call's, cap < 1), UNSUPPORTED (dtypes,
 * rope_dim > 128, B beyond the grid limit; FP4 needs di % 32 == 0), HIP.
 * ------------------------------------------------------------------------- */
csa_status csa_compress_kv(const void* x, int32_t x_dtype, int32_t B, int64_t T, int32_t d,
                           const int32_t* tok_start, int32_t m, const float* score_bias,
                           const float* score_proj, const float* gamma, float eps,
                           int32_t rope_dim, float rope_base, const csa_kv_cache* kv_out,
                           const csa_idx_cache* idx_out, void* stream);

/* ---------------------------------------------------------------------------
 * csa_compress_kv_batch -- several csa_compress_kv calls enqueued as one
 * launch (a decode step's window entry, compressed block and indexer key of
 * the same layer: peacm 3.2 CSA step 1 for each).  Job k has exactly the
 * arguments and the result of csa_compress_kv(jobs[k].x, x_dtype, ...), so
 * the semantics, error statuses and rounding are those above.
 * jobs     : host array of njobs descriptors (read during the call only).
 * x_dtype  : CSA_F32 or CSA_BF16, shared by every job.
 * The jobs run concurrently: their outputs must not overlap and no job may
 * read what another writes.  All jobs are validated before anything is
 * enqueued.  Up to 4 jobs that take the latency kernel (no content score,
 * d a multiple of 32, at most 16 token rows per thread) share one launch;
 * otherwise the jobs are launched one after another on the stream.
 * Errors: INVALID_ARG (njobs < 0, or jobs NULL with njobs > 0), and those of
 * csa_compress_kv for any job.
 * ------------------------------------------------------------------------- */
typedef struct {
    const void* x;
    int32_t B;
    int64_t T;
    int32_t d;
    const int32_t* tok_start;
    int32_t m;
    const float* score_bias;
    const float* score_proj;
    const float* gamma;
    float eps;
    int32_t rope_dim;
    float rope_base;
    const csa_kv_cache* kv_out;
    const csa_idx_cache* idx_out;
} csa_compress_job;
csa_status csa_compress_kv_batch(const csa_compress_job* jobs, int32_t njobs, int32_t x_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * csa_compress_kv_step -- the compression of csa_compress_kv fed one token
 * per sequence per call (decode; peacm 3.2 CSA step 1: every m tokens become
 * one compressed entry, 128:1 for HCA).  For job k and sequence b the token
 * x[b] (row of d values, x_dtype) sits at position t = tok_pos[b] (device
 * int32 [B]; a negative t writes nothing), token r = t mod m of block
 * j = t / m, with score z = score_bias[r] + <score_proj, x[b]>.
 * The pooling softmax over the block's m scores runs as an online softmax
 * over its tokens, in the caller's state: device f32 [B][d + 2] per job
 * (m > 1; NULL for m == 1) holding the running sum of weighted tokens, the
 * running maximum score and the running sum of exp(score - maximum):
 *   r == 0       the state starts from the token (its contents are not read);
 *   0 < r        max' = max(max, z); both sums are scaled by exp(max - max')
 *                and the token added with weight exp(z - max');
 *   r == m - 1   the block is finished from (weighted sum / sum) exactly as
 *                csa_compress_kv finishes a block (RMSNorm, RoPE at j*m,
 *                quantiser into slot j of the one output), and the state is
 *                left as it was before this token (the call can be repeated).
 * The tokens of a block must come in order, one call per token, starting at
 * r == 0.  The entry equals csa_compress_kv's over the same m tokens up to
 * the rounding of the pooling sums (the same terms, added in another form);
 * m == 1 entries (window entries) are the same bits.  Jobs run concurrently
 * (outputs and states must not overlap); up to 4 share a launch.
 * Errors: those of csa_compress_kv for a call over one block of m tokens, and
 * INVALID_ARG (njobs < 0, jobs NULL with njobs > 0, m > 1 without a state).
 * ------------------------------------------------------------------------- */
typedef struct {
    const void* x;
    int32_t B;
    int32_t d;
    const int32_t* tok_pos;
    int32_t m;
    const float* score_bias;
    const float* score_proj;
    const float* gamma;
    float eps;
    int32_t rope_dim;
    float rope_base;
    float* state;
    const csa_kv_cache* kv_out;
    const csa_idx_cache* idx_out;
} csa_compress_step_job;
csa_status csa_compress_kv_step(const csa_compress_step_job* jobs, int32_t njobs, int32_t x_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * csa_indexer_topk -- CSA step 2 (peacm 3.2: the lightning indexer scores
 * each query against the compressed blocks and keeps the most relevant
 * top-k; digest 3.2: the QK path in FP4).
 *
 * For query row (b, i) at position t = q_pos[b][i], over the visible blocks
 * j < n_t = min(floor((t+1)/m), keys->cap):
 *     S_j = sum_h w_idx[b][i][h] * max(0, <q_idx[b][i][h], key_j>)
 * (fp32 accumulation) and out_idx[b][i][:] = the min(topk, n_t) blocks with
 * the largest S, ties to the smaller j, in ascending j order, padded with -1.
 * NaN scores rank lowest; -0 equals +0.
 * q_idx   : [B][Tq][Hi] rows of di = keys->di values in q_dtype (F32, BF16,
 *           or FP4 codes with q_idx_scales [B][Tq][Hi][di/32]).
 * w_idx   : device f32 [B][Tq][Hi].   q_pos: device int32 [B][Tq].
 * out_idx : device int32 [B][Tq][topk].
 * workspace: csa_indexer_topk_workspace_size(B, Tq, keys->cap, topk) bytes
 *           (contents are scratch; need not be zeroed).
 * Errors: INVALID_ARG, UNSUPPORTED (di not a multiple of 32 or > 256;
 * Hi > 16; topk > 2048), WORKSPACE, HIP.
 * ------------------------------------------------------------------------- */
size_t csa_indexer_topk_workspace_size(int32_t B, int32_t Tq, int64_t key_cap, int32_t topk);
csa_status csa_indexer_topk(const void* q_idx, const uint8_t* q_idx_scales, int32_t q_dtype,
                            const float* w_idx, const csa_idx_cache* keys, const int32_t* q_pos,
                            int32_t B, int32_t Tq, int32_t Hi, int32_t m, int32_t topk,
                            int32_t* out_idx, void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * csa_indexer_topk_noalloc -- csa_indexer_topk for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments without the
 * workspace, the same result, bit for bit.  The scratch is a static device
 * array of 64 MiB in the library, one per GPU the library runs on, held until
 * the process ends; its address is looked up (hipGetSymbolAddress) on the
 * first call with each device current.  Nothing is allocated or freed.
 * The array is shared by every call on that GPU and keeps the last call's
 * contents (the kernels need no cleared scratch): calls that overlap on one
 * GPU (different streams, different threads) race and must be serialised by
 * the caller.
 * Errors: those of csa_indexer_topk, and WORKSPACE when the call needs more
 * than 64 MiB of scratch (csa_indexer_topk_workspace_size of the same
 * arguments), HIP when the array's address cannot be taken.
 * ------------------------------------------------------------------------- */
csa_status csa_indexer_topk_noalloc(const void* q_idx, const uint8_t* q_idx_scales, int32_t q_dtype,
                                    const float* w_idx, const csa_idx_cache* keys, const int32_t* q_pos,
                                    int32_t B, int32_t Tq, int32_t Hi, int32_t m, int32_t topk,
                                    int32_t* out_idx, void* stream);

/* ---------------------------------------------------------------------------
 * csa_sparse_mqa_attn -- CSA step 3 (peacm 3.2: multi-query attention over
 * the top-k blocks) with the four tricks (query RMSNorm, partial RoPE with
 * the -i output RoPE, the raw window, the sink logit).
 *
 * For query row (b, i) at position t = q_pos[b][i] and head h < H:
 *   q^  = RoPE_t( RMSNorm_{gamma_q}(q[b][i][h]) )   (eps = p->rms_eps)
 *   E   = { comp entry j : j = topk_idx[b][i][r], 0 <= j < visible }
 *         + { win entry s : max(0, t-W+1) <= s <= t }   (a multiset: a token
 *           both in a block and in the window counts twice)
 *   z_e = softmax_scale * <q^, e>
 *   p_e = exp(z_e) / (exp(sink[h]) + sum_e' exp(z_e'))
 *   o   = sum_e p_e e,  then the last dr dims of o rotated by RoPE_{-t}
 * with o = 0 when E is empty.  Arithmetic in fp32 (bf16 MFMA inputs where q
 * and the cache are bf16/fp8).
 * q       : [B][Tq][H][d], q_dtype F32 or BF16.  gamma_q: f32 [d] or NULL.
 * sink    : f32 [H].   topk_idx: int32 [B][Tq][topk].
 * comp    : linear compressed cache with p->m; win: ring window cache.
 * out     : [B][Tq][H][d], out_dtype F32 or BF16.
 * workspace: csa_attn_workspace_size(...) bytes with max_entries = topk and
 *           the call's split_policy.
 * Errors: INVALID_ARG (incl. cache d / dr differing from p, split_policy not
 * 0 or 1), UNSUPPORTED, CAPACITY (win->cap < window + Tq - 1), WORKSPACE, HIP.
 * ------------------------------------------------------------------------- */
size_t csa_attn_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t head_dim,
                               int64_t max_comp_entries, int32_t window, int32_t q_dtype,
                               int32_t comp_fmt, int32_t split_policy);
csa_status csa_sparse_mqa_attn(const void* q, int32_t q_dtype, const int32_t* q_pos,
                               const int32_t* topk_idx, int32_t topk, const csa_kv_cache* comp,
                               const csa_kv_cache* win, const float* gamma_q, const float* sink,
                               const csa_attn_params* p, int32_t B, int32_t Tq, int32_t H,
                               void* out, int32_t out_dtype, void* workspace, size_t ws_bytes,
                               void* stream);

/* ---------------------------------------------------------------------------
 * hca_dense_mqa_attn -- HCA (peacm 3.2: no sparse selection, dense attention
 * over every compressed entry; wiki article: a dense MQA stream plus the
 * 128-token window).  As csa_sparse_mqa_attn with E = { comp entry j :
 * j < min(floor((t+1)/m), comp->cap) } + the window.
 * workspace: csa_attn_workspace_size(...) bytes with max_entries = comp->cap.
 * ------------------------------------------------------------------------- */
csa_status hca_dense_mqa_attn(const void* q, int32_t q_dtype, const int32_t* q_pos,
                              const csa_kv_cache* comp, const csa_kv_cache* win,
                              const float* gamma_q, const float* sink, const csa_attn_params* p,
                              int32_t B, int32_t Tq, int32_t H, void* out, int32_t out_dtype,
                              void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * attn_out_proj_grouped -- CSA step 4 (peacm 3.2: the head-dim-512 outputs
 * are projected in groups to cut the cost).  Block-diagonal, heads grouped
 * consecutively, no bias:
 *   y[r][g*(D/G) + i] = sum_c o[r][g*(Hd/G) + c] * W[g][i][c]
 * o: [M][Hd] (o_dtype F32 / BF16), W: [G][D/G][Hd/G] (w_dtype, same as
 * o_dtype), y: [M][D] (y_dtype F32 / BF16).  fp32 accumulation in a fixed
 * order, no split of the reduction across workgroups; any Hd/G (widths that
 * are not a whole number of 16-byte vectors, or of 32-wide slabs for bf16
 * with M > 4, take a scalar kernel).  Rows are computed independently, so a
 * row's result does not depend on the other rows; the order of its fp32 sum
 * (hence its last bits) depends on M's size class only: M <= 4, M <= 128
 * (bf16), larger.
 * Errors: INVALID_ARG (sizes < 1, M < 0, Hd % G, D % G, null pointers with
 * M > 0), UNSUPPORTED (dtypes, M beyond the grid limit), HIP.
 * ------------------------------------------------------------------------- */
csa_status attn_out_proj_grouped(const void* o, int32_t o_dtype, const void* W, int32_t w_dtype,
                                 int64_t M, int32_t Hd, int32_t D, int32_t G, void* y,
                                 int32_t y_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * csa_linear_fp8 -- a projection with FP8 weights.  The pages store every
 * parameter outside the MoE experts in FP8 ("DeepSeek-V4 preview review"
 * (deepseek.csdn.net), section 6.2; "DeepSeek V4 (Flash & Pro)" (github wiki
 * article), specification table: FP4 + FP8 mixed precision).  Reading: E4M3
 * codes with one fp32 scale per output row, activations not quantised, no
 * bias, G groups of consecutive rows (G = 1 a dense map; G > 1 the
 * block-diagonal grouped output projection of CSA step 4):
 *   y[r][g*(N/G) + i] = w_scale[g*(N/G) + i]
 *                       * sum_c x[r][g*(K/G) + c] * e4m3(W[g*(N/G) + i][c])
 * x: [M][K] bf16 (x_dtype CSA_BF16), W: [N][K/G] E4M3 codes (0x7F / 0xFF are
 * NaN), w_scale: f32 [N], y: [M][N] in y_dtype (F32 / BF16, nearest even).
 * The products are exact (every E4M3 value is a bf16 number) and summed in
 * fp32 in a fixed order with no split across workgroups; the row scale
 * multiplies the sum.  Rows are independent; the order of a row's sum, hence
 * its last bits, depends only on the weight shape and on M's size class
 * (M <= 32, M <= 64, larger).  Activations are finite numbers.
 * Errors: INVALID_ARG (sizes < 1, M < 0, K % G, N % G, null pointers with
 * M > 0), UNSUPPORTED (x not bf16, y not F32 / BF16, K/G not a multiple of
 * 64, x or W not 16-byte aligned, shapes beyond one launch's grid), HIP.
 * ------------------------------------------------------------------------- */
csa_status csa_linear_fp8(const void* x, int32_t x_dtype, int64_t M, int32_t K, const uint8_t* W,
                          const float* w_scale, int32_t N, int32_t G, void* y, int32_t y_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * csa_layer_in_proj -- the input projections of one CSA layer from its hidden
 * states, one FP8-weight product for all of them (weights as in
 * csa_linear_fp8, one dense map each; the pages name the outputs, not their
 * maps: the queries of the core attention, the KV token that CSA step 1
 * compresses and the window keeps, the lightning indexer's queries, head
 * weights and key token).
 * h: [M][D] bf16 (h_dtype CSA_BF16).  W: [N][D] E4M3 codes, w_scale: f32
 * [N], with N = H*d + d + di + Hi*di + Hi and the rows in this order:
 *   q     : H*d rows  -> q     [M][H][d]   bf16  (input of the attention)
 *   kv    : d rows    -> kv    [M][d]      bf16  (raw token of csa_compress_kv)
 *   k_idx : di rows   -> k_idx [M][di]     bf16  (raw indexer-key token)
 *   q_idx : Hi*di rows-> q_idx [M][Hi][di/2] FP4 codes, q_idx_scales
 *                        [M][Hi][di/32] E8M0 (csa_indexer_topk's FP4 queries)
 *   w_idx : Hi rows   -> w_idx [M][Hi]     f32   (indexer head weights)
 * Each output is the projected value as an fp32 sum times the row scale,
 * then rounded: bf16 nearest even; q_idx quantised per head row of di values
 * by the indexer-key FP4 rule of csa_compress_kv (blocks of 32 with
 * e = floor(log2 amax) - 2 raised to at least (row max e) - 14, E2M1 codes
 * nearest even, saturating at +-6).
 * workspace: csa_layer_in_proj_workspace_size(M, Hi, di) bytes, 4-byte
 * aligned (the fp32 indexer queries before quantisation); need not be zeroed.
 * Errors: those of csa_linear_fp8 (K = D, G = 1), INVALID_ARG (H, d, di or
 * Hi < 1, null outputs), UNSUPPORTED (di not a multiple of 32 or > 256),
 * WORKSPACE, HIP.
 * ------------------------------------------------------------------------- */
size_t csa_layer_in_proj_workspace_size(int64_t M, int32_t Hi, int32_t di);
csa_status csa_layer_in_proj(const void* h, int32_t h_dtype, int64_t M, int32_t D, const uint8_t* W,
                             const float* w_scale, int32_t H, int32_t d, int32_t di, int32_t Hi, void* q,
                             void* kv, void* k_idx, uint8_t* q_idx, uint8_t* q_idx_scales, float* w_idx,
                             void* workspace, size_t ws_bytes, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* csa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA_ATTN_H */
