/*
 * oscar.h -- C ABI of the OSCAR INT2 KV-cache decode library for AMD MI355X
 * (gfx950).
 *
 * The method (MarkTechPost article on OSCAR, "The Serving System"; ModelScope/
 * CSDN page, design section): every sequence keeps a three-segment token pool,
 *   BF16 sink (first S0 tokens) | INT2 history | BF16 recent (last W tokens),
 * new tokens enter the recent window and the oldest recent token is rotated by
 * R_K (keys), clipped to a per-head threshold, quantized per token to 2-bit
 * codes with a bf16 scale and zero per group of G channels, packed 4 codes per
 * byte and demoted into the history.  Decode attends the INT2 and BF16
 * segments separately and merges the partial results by online softmax.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Device pointers are HIP device memory owned by the caller; the library
 *    never allocates or frees device memory.  Host pointers are marked "host".
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null
 *    stream).  Kernel faults surface at the caller's next synchronization.
 *  - bf16 tensors are uint16 bit patterns (IEEE binary32 upper halves).
 *  - Row-vector convention: a rotated vector is x' = x R with R stored
 *    row-major [D_in][D_out] as fp32, one matrix per KV head: R[Hkv][D][D].
 *  - Query head h reads KV head h / (Hq / Hkv).
 *  - Positions of a sequence of length L (L counts every stored token):
 *      sink [0, min(L, S0)), history [S0, max(S0, L-W)),
 *      recent [max(S0, L-W), L).
 *    Keys in the BF16 segments are unrotated.  Values: with v_absorbed = 1
 *    (R_V absorbed into the projection weights, MarkTechPost article, "The
 *    Serving System") every segment stores V in the pool's V basis and the
 *    decode output is in that basis; with v_absorbed = 0 the BF16 segments
 *    store V itself, the INT2 history stores V R_V (rotated at demotion like
 *    K), and decode rotates the history's contribution back by R_V^T, so the
 *    output is in the model basis.
 *  - Errors: functions return an oscar_status; arguments are validated on the
 *    host before anything is launched, and nothing is launched on error.
 *    oscar_last_error() gives a human-readable reason (thread-local).
 *
 * Pool layout (16-token pages, all KV heads of a page together)
 * -------------------------------------------------------------
 * BF16 pool: page p occupies bf16_page_bytes = Hkv * 64*D bytes; head k's
 *   block starts at (p*Hkv + k) * 64*D and holds
 *     K: [16 tokens][D] bf16 (32*D bytes), then
 *     V: [4 token quads][D channels][4 tokens] bf16 (32*D bytes)
 *   (token s of the page is quad s/4, slot s%4).  A sequence's BF16 page table
 *   maps logical page pos/16 to a physical page; only logical pages that
 *   overlap the sink or recent segment are read or written.
 *
 * INT2 pool: page p occupies int2_page_bytes = Hkv * (8*D + 128*n_g) bytes
 *   (n_g = D/G); head k's block starts at (p*Hkv + k) * (8*D + 128*n_g):
 *     codes: 64 records of D/8 bytes.  Record lam = 16*j + r (j = 0..3,
 *       r = 0..15) holds
 *       - K part, D/64 little-endian 32-bit words: word w holds the K codes of
 *         token r for channels w*64 + j*16 + m, m = 0..15, in bits 2m..2m+1;
 *       - V part, D/64 words: word w holds the V codes of tokens 4j..4j+3 for
 *         channels c = (4w + b)*16 + r, b = 0..3; token 4j+i of channel block
 *         b sits in bits 16*(i&1) + 2*(2b + (i>>1)).
 *     scales: [4 token quads][K: 4 tokens][n_g][scale, zero] bf16, then
 *       [V: 4 tokens][n_g][scale, zero] bf16, i.e. 32*n_g bytes per quad.
 *   A dequantized value is scale * (code - zero).  The history token at
 *   position pos lives in logical INT2 page (pos - S0)/16, slot (pos - S0)%16.
 *   Bytes per history token and head: 2*D/4 + 8*n_g (72 at D = G = 128,
 *   2.25 bits per element).
 *
 * Page tables are int32 [batch][stride] (host value -1 or any id outside
 * [0, num_pages) marks an absent page: its tokens are skipped, never read).
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  OSCAR_OK = 0,
  OSCAR_ERR_INVALID = 1,     /* null pointer, bad shape, misaligned buffer */
  OSCAR_ERR_UNSUPPORTED = 2, /* valid request outside what this build implements */
  OSCAR_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  OSCAR_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} oscar_status;

/* Configuration of one attention layer's pool.
 * Supported: head_dim 64 or 128; group_size 64 or 128 dividing head_dim;
 * num_q_heads / num_kv_heads in {2, 4, 8}; page_size 16; sink_tokens a
 * multiple of 16 (64 by default, MarkTechPost article, "The Serving System");
 * recent_tokens >= 1 (256 by default, same section); v_absorbed 1 or 0
 * (see the value basis above).
 *
 * Codebook (ModelScope/CSDN page, closing section: the rotation combined with
 * a Lloyd-Max codebook).  codebook = 0: the history levels are 0, 1, 2, 3 in
 * code units (dequantized value scale * (code - zero)), codes by
 * round-to-nearest-even and clamp.  codebook = 1: the levels are
 * levels_k[code] (keys) and levels_v[code] (values), each with
 * 0 = L[0] < L[1] < L[2] < L[3] = 3 and L[1], L[2] multiples of 1/32 (else
 * OSCAR_ERR_INVALID); the dequantized value is scale * (L[code] - zero), and
 * the code of t = c/scale + zero is the number of midpoints
 * (L[k] + L[k+1]) / 2 strictly below t.  Scale and zero are the same as with
 * codebook = 0, so the pool layout is unchanged.  oscar_calib_codebook fits
 * the levels. */
typedef struct {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t group_size;
  int32_t page_size;
  int32_t sink_tokens;
  int32_t recent_tokens;
  int32_t v_absorbed;
  float sm_scale; /* softmax scale; 0 selects 1/sqrt(head_dim) */
  int32_t codebook;
  float levels_k[4];
  float levels_v[4];
} oscar_config;

/* Byte sizes of the pool layout described above, filled by oscar_pool_create. */
typedef struct {
  size_t int2_page_bytes;       /* one INT2 page, all KV heads */
  size_t bf16_page_bytes;       /* one BF16 page, all KV heads */
  size_t int2_head_block_bytes; /* one KV head's block inside an INT2 page */
  size_t bf16_head_block_bytes; /* one KV head's block inside a BF16 page */
} oscar_layout;

/* Opaque host-side handle holding a validated, immutable configuration. */
typedef struct oscar_pool oscar_pool;

/* Validate `cfg` and create a handle (host memory only).  `layout` may be
 * NULL.  Errors: OSCAR_ERR_INVALID for null/negative fields,
 * OSCAR_ERR_UNSUPPORTED for shapes outside the supported set. */
oscar_status oscar_pool_create(const oscar_config* cfg, oscar_pool** out, oscar_layout* layout);
void oscar_pool_destroy(oscar_pool* pool);

/* Bytes of device workspace oscar_decode_attention (bf16_only = 0) or
 * oscar_bf16_decode_attention (bf16_only = 1) needs for `batch` sequences of
 * at most `max_seq_len` tokens.  The workspace must be zero-filled before its
 * first use; each successful call leaves its counters zero again, so one
 * zero-fill serves every later call.  Calls that share a workspace must not
 * overlap in time. */
oscar_status oscar_decode_workspace_bytes(const oscar_pool* pool, int32_t batch, int32_t max_seq_len,
                                          int32_t bf16_only, size_t* bytes);

/* Decode-time write path (ModelScope/CSDN page, design section: new tokens
 * are written to the recent window; the oldest recent token is rotated,
 * clipped, quantized, packed and demoted into the INT2 history).
 * For every sequence b with length L_b = seq_lens[b] BEFORE the call:
 *   - writes k_new[b], v_new[b] (bf16 [batch][Hkv][D]; v_new in the pool's V
 *     basis) at position L_b of the BF16 pool;
 *   - if d = L_b - W >= S0, reads token d's K and V from the BF16 pool and
 *     writes  k_d R_K[k]  (fp32 accumulation) and  v_d  (absorbed V) or
 *     v_d R_V[k]  (fp32 accumulation, v_absorbed = 0), each
 *     clipped to +-tau[k] and quantized with bf16 scale = bf16((max-min)/3)
 *     (1 if max = min) and zero = bf16(-min/scale), code =
 *     clamp(rne(c/scale + zero), 0, 3), into INT2 history slot d - S0.
 * seq_lens is not advanced; the caller owns lengths.  r_k: fp32 [Hkv][D][D];
 * r_v: fp32 [Hkv][D][D] when v_absorbed = 0, NULL otherwise (either
 * mismatch is OSCAR_ERR_INVALID); tau_k, tau_v: fp32 [Hkv] (+inf disables).
 * Page tables must hold a valid entry for every page written.  Sequences that
 * share a page must not demote into it in the same call. */
oscar_status oscar_append_demote(const oscar_pool* pool, int32_t batch, const void* k_new, const void* v_new,
                                 const int32_t* seq_lens, const int32_t* bf16_page_table,
                                 int32_t bf16_pt_stride, int32_t bf16_num_pages,
                                 const int32_t* int2_page_table, int32_t int2_pt_stride,
                                 int32_t int2_num_pages, void* bf16_pool, void* int2_pool, const float* r_k,
                                 const float* r_v, const float* tau_k, const float* tau_v, void* stream);

/* Decode attention over the three-segment pool (ModelScope/CSDN page, design
 * section: INT2 kernel unpacks and dequantizes, BF16 kernel handles sink and
 * recent, online-softmax merge; MarkTechPost article, "Outcome": the online
 * rotation is absorbed into the decode kernels).  For each sequence b and
 * query head h:
 *   out[b][h] = softmax_t(sm * q.k_t) . v_t  over all L_b tokens,
 * with history keys k^ = s(code - z) R_K^T (computed as q' = q R_K against
 * the codes) and history values s(code - z), times R_V^T when v_absorbed = 0
 * (applied once per head to the merged history partial; r_v as for
 * oscar_append_demote).
 * q: bf16 [batch][Hq][D] (model basis); seq_lens: int32 [batch] device, L_b
 * counting the current token, at most max_seq_len (longer lengths are
 * clamped to max_seq_len and to what the page tables can address; lengths
 * of 0 or less select no token and give zero output rows); out:
 * bf16 [batch][Hq][D].
 * seq_lens_host: NULL, or the same lengths in host memory (int32 [batch]).
 * With them (and batch <= 128) the split-K plan follows each sequence's own
 * history: every sequence gets as many chunks as its pages need, and the
 * chunk size is the smallest that fills whole rounds of workgroups over the
 * compute units (ModelScope/CSDN page, design section: split INT2 and BF16
 * kernels merged by online softmax; the chunk count per sequence length).
 * Without them every sequence is planned for max_seq_len.  The device
 * lengths must not exceed the host ones (tokens past a sequence's planned
 * history would not be attended).
 * workspace: oscar_decode_workspace_bytes(pool, batch, max_seq_len, 0) bytes,
 * 256-byte aligned, zero-filled before first use.
 * Value range: the history's P.V runs on fp16 matrix cores with weights
 * p * s_V * 2^-E, where E follows the largest value group scale s_V seen by
 * the softmax state (clamped to [-96, 96]); every s_V in [2^-96, 2^96] keeps
 * the weights inside fp16's normal range, whatever tau_V was (+inf included).
 * Larger scales are outside the supported range (the weights overflow).
 * Query precision: q' = q R_K enters the int8 matrix cores as
 * sq (a + b/256) (~16 significant bits relative to max|q'|), and as
 * sq (a + b/256 + c/65536) for a workgroup whose heads include a q' with one
 * channel above 8x its rms (group_size = head_dim; with two scale groups per
 * head the two-term split is kept). */
oscar_status oscar_decode_attention(const oscar_pool* pool, int32_t batch, int32_t max_seq_len, const void* q,
                                    const int32_t* seq_lens, const int32_t* seq_lens_host, const int32_t* bf16_page_table,
                                    int32_t bf16_pt_stride, int32_t bf16_num_pages,
                                    const int32_t* int2_page_table, int32_t int2_pt_stride,
                                    int32_t int2_num_pages, const void* bf16_pool, const void* int2_pool,
                                    const float* r_k, const float* r_v, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* oscar_decode_attention for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, kernels and result as oscar_decode_attention,
 * without the workspace: the decode's partials and tickets live in a
 * library-owned device array of OSCAR_NOALLOC_SCRATCH_BYTES per GPU, kept
 * until the process ends.  The call allocates nothing.  A request whose
 * decode workspace (oscar_decode_workspace_bytes) exceeds that size returns
 * OSCAR_ERR_UNSUPPORTED and launches nothing.  The first call on a device
 * also enqueues a clear of the array on `stream`; every call leaves the
 * array's tickets at zero.  All calls on one GPU share the array, so calls
 * that overlap in time on one GPU (concurrent streams, threads) race and
 * give undefined results. */
#define OSCAR_NOALLOC_SCRATCH_BYTES (8u << 20)
oscar_status oscar_decode_attention_noalloc(const oscar_pool* pool, int32_t batch, int32_t max_seq_len, const void* q,
                                            const int32_t* seq_lens, const int32_t* seq_lens_host, const int32_t* bf16_page_table,
                                            int32_t bf16_pt_stride, int32_t bf16_num_pages,
                                            const int32_t* int2_page_table, int32_t int2_pt_stride,
                                            int32_t int2_num_pages, const void* bf16_pool, const void* int2_pool,
                                            const float* r_k, const float* r_v, void* out, void* stream);

/* Prefix-shared ("cascade") decode.  The pages keep the paged pool's prefix
 * sharing intact (MarkTechPost article, "Visual Explainer / How-To", the
 * inference step: the radix cache and prefix reuse work unchanged) and report
 * the largest gains where long prefixes are shared (ModelScope/CSDN page,
 * evaluation section, Figure 6).  Shared pages are stored once; this call
 * also reads them once per group of sequences.  A prefix group names sequences
 * first_seq .. first_seq + num_seqs - 1 whose INT2 page tables hold the same
 * physical pages for logical history pages 0 .. shared_pages - 1, as far as
 * each member's history reaches (the caller guarantees this; the pages are
 * read through the table of the member with the longest history).
 * Groups must be ordered by first_seq and disjoint; a group with
 * shared_pages = 0 is ignored.  The shared pages are attended once for up to
 * 16 / (Hq/Hkv) member sequences together (2 at GQA 8, 4 at GQA 4), in a
 * launch of prefix workgroups that precedes the decode launch; each member's
 * own history pages and its BF16 segments are attended by the decode launch,
 * which merges the prefix partials in.  A member whose history is shorter
 * than the shared range sees only its own tokens.  The result equals
 * oscar_decode_attention's up to fp32 summation order.  At most 32 units
 * (groups split into 16 / (Hq/Hkv) sequences) per call (else
 * OSCAR_ERR_UNSUPPORTED).  groups: host array.  workspace:
 * oscar_decode_cascade_workspace_bytes(...) bytes, 256-byte aligned, zeroed
 * before first use (as for oscar_decode_attention). */
typedef struct {
  int32_t first_seq;
  int32_t num_seqs;
  int32_t shared_pages;
} oscar_prefix_group;

oscar_status oscar_decode_cascade_workspace_bytes(const oscar_pool* pool, int32_t batch, int32_t max_seq_len,
                                                  int32_t int2_pt_stride, const oscar_prefix_group* groups,
                                                  int32_t num_groups, size_t* bytes);
oscar_status oscar_decode_attention_cascade(const oscar_pool* pool, int32_t batch, int32_t max_seq_len,
                                            const void* q, const int32_t* seq_lens, const int32_t* seq_lens_host,
                                            const int32_t* bf16_page_table, int32_t bf16_pt_stride,
                                            int32_t bf16_num_pages, const int32_t* int2_page_table,
                                            int32_t int2_pt_stride, int32_t int2_num_pages, const void* bf16_pool,
                                            const void* int2_pool, const float* r_k, const float* r_v, void* out,
                                            const oscar_prefix_group* groups, int32_t num_groups, void* workspace,
                                            size_t workspace_bytes, void* stream);

/* Log-sum-exp merge of partial attentions (ModelScope/CSDN page, design
 * section, online-softmax merge).  Row i (0 <= i < rows) merges partials
 * row_offsets[i] .. row_offsets[i+1]-1:
 *   out[i] = sum_j exp(lse_j - LSE) o_j,  LSE = ln sum_j exp(lse_j);
 * a partial with lse = -inf contributes nothing; a row with no finite lse is
 * written as zeros.  row_offsets: int32 [rows+1] device (non-decreasing,
 * row_offsets[0] = 0); o_partials: fp32 [nnz][head_dim] normalized outputs;
 * lse_partials: fp32 [nnz] natural log; out: bf16 [rows][head_dim].
 * head_dim must be 64 or 128. */
oscar_status oscar_merge(int32_t rows, int32_t head_dim, const int32_t* row_offsets, const float* o_partials,
                         const float* lse_partials, void* out, void* stream);

/* Bulk write path (prefill of history): quantizes tokens 0..num_tokens-1 of
 * dense K and V (bf16 [num_tokens][Hkv][D]; V already in the pool's V basis
 * when absorbed, else V itself) exactly as oscar_append_demote quantizes one
 * token, with K rotated by R_K (and, v_absorbed = 0, V by R_V; r_v as for
 * oscar_append_demote) on the matrix cores, and writes token t to slot t%16
 * of INT2 page
 * page_ids[t/16] (int32 device [ceil(num_tokens/16)]).  Pages are written
 * whole; token slots past num_tokens in the last page are zero-filled. */
oscar_status oscar_quantize_pack(const oscar_pool* pool, int32_t num_tokens, const void* k, const void* v,
                                 const int32_t* page_ids, int32_t int2_num_pages, void* int2_pool,
                                 const float* r_k, const float* r_v, const float* tau_k, const float* tau_v,
                                 void* stream);

/* Prefill of BF16 pages: writes tokens t = 0..num_tokens-1 of dense k and v
 * (bf16 [num_tokens][Hkv][D], v in the pool's V basis) to positions
 * first_position + t of one sequence, i.e. to slot (first_position + t) % 16
 * of BF16 page bf16_page_table[(first_position + t) / 16] (int32 device
 * [bf16_pt_stride]).  Tokens whose page entry is outside [0, bf16_num_pages)
 * or past the table are skipped.  Used to stage the sink and recent windows
 * (and, for the BF16-only comparator, whole sequences). */
oscar_status oscar_write_bf16(const oscar_pool* pool, int32_t num_tokens, int32_t first_position, const void* k,
                              const void* v, const int32_t* bf16_page_table, int32_t bf16_pt_stride,
                              int32_t bf16_num_pages, void* bf16_pool, void* stream);

/* All-BF16 paged decode (the comparator for the INT2 path): plain softmax
 * attention over every position 0..L_b-1 stored in the BF16 pool (layout
 * above), through bf16_page_table.  Arguments as oscar_decode_attention;
 * workspace from oscar_decode_workspace_bytes(..., bf16_only = 1). */
oscar_status oscar_bf16_decode_attention(const oscar_pool* pool, int32_t batch, int32_t max_seq_len,
                                         const void* q, const int32_t* seq_lens,
                                         const int32_t* bf16_page_table, int32_t bf16_pt_stride,
                                         int32_t bf16_num_pages, const void* bf16_pool, void* out,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Offline calibration (MarkTechPost article on OSCAR, "What OSCAR Does
 * Differently"; ModelScope/CSDN page, design section: per layer and head, a
 * fixed rotation and clip threshold are estimated from a small calibration
 * set).  All fp32.  Calibration activations of one layer:
 *   q: [Hkv][g][N][D] contiguous, the queries of the g query heads that read
 *      each KV head (model basis, before any rotation);
 *   k, v: element (h, n, c) at h * kv_head_stride + n * kv_token_stride + c
 *      (strides in elements, multiples of 4, kv_token_stride >= D), e.g.
 *      [Hkv][N][D] or [N][Hkv][D]; values in the model basis.
 * head_dim is 64 or 128.  Pointers are device memory, 16-byte aligned; every
 * head's addressed span must stay below 2 GiB.
 * ------------------------------------------------------------------------ */

/* C = scale * X^T X for each of `heads` matrices X [rows][head_dim], row r of
 * head h at x + h * head_stride + r * row_stride.  out: fp32
 * [heads][head_dim][head_dim].  The sum over rows is split over workgroups
 * and reduced in a fixed order (deterministic). */
oscar_status oscar_calib_gram_workspace_bytes(int32_t heads, int32_t rows, int32_t head_dim, size_t* bytes);
oscar_status oscar_calib_gram(int32_t heads, int32_t rows, int32_t head_dim, const float* x, int64_t head_stride,
                              int64_t row_stride, float scale, float* out, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Causal softmax attention of the calibration draw: for KV head h, query head
 * j and row n, out[h][j][n] = sum_{t <= n} p_t v_t with p = softmax over
 * t <= n of sm * q[h][j][n] . k_t (sm_scale 0 selects 1/sqrt(head_dim)).
 * out: fp32 [Hkv][g][N][D]; lse: fp32 [Hkv][g][N] natural-log normalizer, or
 * NULL.  The score-weighted value covariance C_S of a KV head is the gram of
 * its g*N output rows scaled by 1/(g*N). */
oscar_status oscar_calib_attention(int32_t kv_heads, int32_t gqa, int32_t tokens, int32_t head_dim, float sm_scale,
                                   const float* q, const float* k, const float* v, int64_t kv_head_stride,
                                   int64_t kv_token_stride, float* out, float* lse, void* stream);

/* Eigenbasis and rotation of symmetric matrices cov [heads][D][D]: U holds
 * the eigenvectors as columns ordered by descending eigenvalue, each column
 * signed so that its largest-magnitude entry (the first of equal ones) is
 * positive; with mix = 1, r = U H P_br (H the Sylvester Walsh-Hadamard
 * matrix / sqrt(D); column j of H P_br is column bitreverse(j) of H), with
 * mix = 0, r = U.  r: fp32 [heads][D][D] row-major [D_in][D_out];
 * eigvals: fp32 [heads][D] descending, or NULL.  One-sided Jacobi in fp32. */
oscar_status oscar_calib_rotation(int32_t heads, int32_t head_dim, const float* cov, int32_t mix, float* r,
                                  float* eigvals, void* stream);

/* Clip thresholds: tau[h] = the `quantile` quantile (linear interpolation
 * between the order statistics at rank (M-1)*quantile, M = rows*D) of
 * |x R[h]| over all rows of head h (x laid out as for oscar_calib_gram;
 * r NULL: no rotation), rounded to fp32.  The order statistics are exact
 * (radix selection); y = x R is fp32 on the matrix cores. */
oscar_status oscar_calib_clip_workspace_bytes(int32_t heads, int32_t rows, int32_t head_dim, size_t* bytes);
oscar_status oscar_calib_clip(int32_t heads, int32_t rows, int32_t head_dim, const float* x, int64_t head_stride,
                              int64_t row_stride, const float* r, double quantile, float* tau, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Codebook fit (the levels of oscar_config.codebook = 1; ModelScope/CSDN
 * page, closing section): for x laid out as for oscar_calib_gram, rotated by
 * r (NULL: none) and clipped to +-tau[h] (device fp32 [heads]), every value's
 * normalized position t = c/scale + zero (scale and zero per group of
 * group_size channels of a row, exactly as the write path forms them); then
 * Lloyd-Max with the end levels fixed at 0 and 3: 100 steps from the uniform
 * levels, each moving L[1], L[2] to the mean of the values in their cells
 * [midpoint below, midpoint above), sums in fp64; finally L[1], L[2] rounded
 * to the nearest multiple of 1/32 (half to even).  levels: device fp32 [4].
 * One codebook for all heads (a layer's keys, or its values). */
oscar_status oscar_calib_codebook_workspace_bytes(int32_t heads, int32_t rows, int32_t head_dim, size_t* bytes);
oscar_status oscar_calib_codebook(int32_t heads, int32_t rows, int32_t head_dim, int32_t group_size, const float* x,
                                  int64_t head_stride, int64_t row_stride, const float* r, const float* tau,
                                  float* levels, void* workspace, size_t workspace_bytes, void* stream);

/* The whole calibration of one layer: C_Q = gram(q)/(g N), R_K = U_Q H P_br,
 * C_S from the causal attention outputs, R_V = U_S H P_br, tau_K and tau_V
 * the clip_quantile quantiles of |k R_K| and |v R_V| (the pages give the
 * clip as a ratio without fixing its estimator; the synthetic workloads use
 * the 0.995 quantile).  r_k, r_v: fp32 [Hkv][D][D]; tau_k, tau_v: fp32
 * [Hkv]; c_q, c_s: fp32 [Hkv][D][D] or NULL. */
oscar_status oscar_calib_workspace_bytes(int32_t kv_heads, int32_t gqa, int32_t tokens, int32_t head_dim,
                                         size_t* bytes);
oscar_status oscar_calibrate(int32_t kv_heads, int32_t gqa, int32_t tokens, int32_t head_dim, float sm_scale,
                             const float* q, const float* k, const float* v, int64_t kv_head_stride,
                             int64_t kv_token_stride, double clip_quantile, float* r_k, float* r_v, float* tau_k,
                             float* tau_v, float* c_q, float* c_s, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Rotation error chain (ModelScope/CSDN page, motivation section and its
 * Figure 1: rotations are judged by attention-score KL and attention output
 * error, not by K/V reconstruction error).
 *
 * oscar_dequantize: reads INT2 history records of tokens 0..num_tokens-1
 * (token t in slot t%16 of page page_ids[t/16], the layout written by
 * oscar_quantize_pack) and writes k_out, v_out fp32 [num_tokens][Hkv][D]:
 * s (code - z) R_K^T for keys and s (code - z) R_V^T for values; a NULL
 * r_k / r_v returns that tensor in its stored basis.
 *
 * oscar_attention_error: causal attention of q (layout as above) over the
 * reference (k, v) and over the quantized (k_hat, v_hat), same strides; per
 * KV head h, query head j and row n, stats[h][j][n] = {KL(p || p^),
 * sum_{t <= n} (l^_t - l_t)^2, ||o - o^||^2, ||o||^2} with l = sm q.k,
 * p = softmax(l), o = p v (fp32 [Hkv][g][N][4]).  Both softmaxes are taken
 * against one running maximum, so a row whose every quantized logit sits
 * more than ~87 below every reference logit underflows (not met in practice). */
oscar_status oscar_dequantize(const oscar_pool* pool, int32_t num_tokens, const int32_t* page_ids,
                              int32_t int2_num_pages, const void* int2_pool, const float* r_k, const float* r_v,
                              float* k_out, float* v_out, void* stream);
oscar_status oscar_attention_error(int32_t kv_heads, int32_t gqa, int32_t tokens, int32_t head_dim, float sm_scale,
                                   const float* q, const float* k, const float* v, const float* k_hat,
                                   const float* v_hat, int64_t kv_head_stride, int64_t kv_token_stride,
                                   float* stats, void* stream);

const char* oscar_status_string(oscar_status status);
/* Reason for the last error returned on this thread ("" if none). */
const char* oscar_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_H */
