/*
 * bsattn.h -- block-sparse self-attention (forward, backward, attention layer)
 * for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbsattn.so.  Plain pointers and sizes only; no C++ or framework
 * types cross this boundary, and no C++ exception escapes it.
 *
 * The operation (Adaptive Sparse Transformer page, "Adapt or Perish: 新手入门指南 –
 * Adaptive Sparse Transformer 核心原理与实战", the SparseAttention formula):
 *   O = softmax(scale * Q K^T under a 0/1 mask M) V,
 * with masked scores treated as -inf (the primer page's and the multi-head
 * page's code fill masked scores with a large negative value) and one softmax
 * over the union of all patterns.  M comes from a layout object:
 *   - a BigBird-style block layout (BigBird page, "BigBird 稀疏注意力机制解析：如何突破
 *     Transformer 的序列长度限制", section 核心实现: global, sliding-window and random
 *     patterns) on 32-, 64- or 128-token blocks, stored in block-CSR form over
 *     64x64 tiles (SQA page, "Transformer计算效率优化：SQA稀疏注意力机制详解",
 *     section 3.1: block-sparse mask, attention only on non-zero blocks;
 *     section 5: 64x64 blocks), optionally refined per token by a key padding
 *     length (bsattn_make_layout);
 *   - a token band |t - s| <= w, alone or in the routed-query variant (SQA page,
 *     section 2.1) (bsattn_make_band_layout, bsattn_forward_routed);
 *   - the token-granular BigBird pattern: linspace global tokens, a token
 *     window and random tokens per row (bsattn_make_token_layout);
 *   - a content-adaptive block layout whose key blocks are chosen from Q and K
 *     at every call (bsattn_make_adaptive_layout).
 * The gradients (bsattn_backward) take the BigBird-style block layouts and the
 * token band; the attention layer around the kernel (bsattn_layer_forward)
 * takes these and the token-granular pattern.
 *
 * Tensor layout everywhere: [B, H, L, D] row-major, D innermost, contiguous.
 * LSE is [B, H, L] fp32: the natural-log log-sum-exp of the scaled, masked
 * scores of each query row (the normaliser of the softmax, kept for a
 * backward pass).
 *
 * Errors: every function returns a bsattn_status.  Arguments are validated
 * before anything is enqueued; on failure nothing is launched and
 * bsattn_last_error() returns a thread-local description.  Launch failures
 * are reported as BSATTN_ERR_HIP.  NaN inputs propagate to the outputs.  A
 * query row with no allowed key gets O = 0 and LSE = -inf.
 *
 * Asynchrony: the compute calls (forward, backward, layer, router) enqueue
 * work on their hipStream_t and return without synchronising; they are
 * reentrant.  Set-up calls (bsattn_layout_upload, bsattn_prepare) allocate and
 * synchronise their stream; a compute call of a shape that was never prepared
 * does the same once, on first use.  Calls that share a workspace must be
 * ordered (same stream, or synchronised).
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BSATTN_OK = 0,
    BSATTN_ERR_INVALID_ARG = 1,   /* bad pointer, size, shape or layout mismatch */
    BSATTN_ERR_UNSUPPORTED = 2,   /* valid request the library does not implement (e.g. D=96) */
    BSATTN_ERR_HIP = 3,           /* a HIP runtime call or kernel launch failed */
    BSATTN_ERR_NO_MEMORY = 4,     /* host or device allocation failed */
    BSATTN_ERR_STATE = 5          /* layout not uploaded to the current device */
} bsattn_status;

typedef enum {
    BSATTN_F32 = 0,               /* fp32 Q/K/V/O, fp32 arithmetic */
    BSATTN_BF16 = 1               /* bf16 Q/K/V/O, bf16 MFMA with fp32 accumulation */
} bsattn_dtype;

/* Opaque, immutable once built.  Owns its host CSR arrays and, after
 * bsattn_layout_upload, a device copy plus the scheduled work list. */
typedef struct bsattn_layout bsattn_layout;

/* Build a BigBird-style block layout on the host (no HIP call).
 * BigBird page, section 核心实现 (global / sliding window / random patterns);
 * SQA page, section 3.1 (block-sparse storage).
 *   num_heads      H >= 1; the layout is per head and shared by the batch.
 *   seq_len        L, a positive multiple of 64 and of block.
 *   block          32, 64 or 128 tokens (the SQA page recommends 64x64
 *                  blocks, section 5, and treats the size as a tuning knob;
 *                  128 halves the layout's granularity, 32 doubles it).  The
 *                  rule below runs on blocks of this size; the stored CSR is
 *                  always over 64-token tiles.  A 128-token block (I, J) is
 *                  the tiles 2I..2I+1 x 2J..2J+1.  A 32-token block (I, J)
 *                  is the quarter (I mod 2, J mod 2) of tile (I/2, J/2): a
 *                  tile is stored when any of its quarters is in the layout,
 *                  and bsattn_layout_tile_masks says which quarters are.
 *   window_blocks  odd >= 1: query block i sees key blocks j with
 *                  |i-j| <= (window_blocks-1)/2, clipped to [0, L/block).
 *   global_blocks  host array of num_global distinct block indices in range
 *                  (may be NULL when num_global == 0).  A global block's row
 *                  is every block, and every row contains every global block.
 *   random_blocks  r >= 0 extra blocks per non-global row, drawn without
 *                  replacement from the blocks not already in the row by a
 *                  splitmix64-driven partial Fisher-Yates shuffle: row stream
 *                  state s = sm(sm(sm(seed)^h)^i), sm(x) = first splitmix64
 *                  output from state x; draw j swaps candidate j with
 *                  candidate j + (u_j mod (n-j)), u_j the (j+1)-th output from
 *                  state s, candidates in ascending order.  If r exceeds the
 *                  candidates, all are taken.
 *   seed           hash seed.
 *   out            receives the new layout (caller frees with bsattn_layout_destroy).
 * Rows are ascending and duplicate-free.  Limits: window_blocks <= 63,
 * num_global <= 64, random_blocks <= 64, H * (L/64) <= 2^20, L/64 <= 2^18.
 * Layouts of 32-token blocks run in bf16 without key padding (the forward
 * and backward calls return UNSUPPORTED otherwise). */
bsattn_status bsattn_make_layout(int32_t num_heads, int32_t seq_len, int32_t block,
                                 int32_t window_blocks, const int32_t* global_blocks,
                                 int32_t num_global, int32_t random_blocks, uint64_t seed,
                                 bsattn_layout** out);

/* Build the block layout of a token band (routed-query variant, SQA page,
 * section 2.1: non-routed queries see only a local window of keys), read as
 * |t - s| <= band_tokens.  Row i lists every key block the band of query
 * block i touches (i-1, i, i+1 for band_tokens <= 64), and the kernels mask
 * the band per token.  band_tokens in [0, seq_len).  Host only. */
bsattn_status bsattn_make_band_layout(int32_t num_heads, int32_t seq_len, int32_t block,
                                      int32_t band_tokens, bsattn_layout** out);

/* Build the token-granular BigBird pattern on the host (no HIP call).
 * BigBird page, section 核心实现: global tokens chosen uniformly by the code
 * example's linspace, a sliding window of w neighbours on each side (typical
 * w = 64), r random remote tokens per token (typical r = 8); section 避坑指南:
 * global tokens at 5-10% of L.  Query t attends key s iff t is global, s is
 * global, |t - s| <= band_tokens, or s is one of t's random tokens.
 *   num_heads      H >= 1; the pattern is per head and shared by the batch.
 *   seq_len        L, a positive multiple of 64.
 *   band_tokens    w in [0, L).
 *   num_global     n in [0, min(L, 2048)]: global tokens floor(i (L-1)/(n-1)),
 *                  i = 0..n-1 (exact integers; n = 1 gives token 0).
 *   random_tokens  r in [0, 64]: per non-global row, r distinct tokens drawn
 *                  from those outside the window and the global tokens, by the
 *                  same splitmix64 partial Fisher-Yates as bsattn_make_layout
 *                  with the token index in place of the block index (the rule
 *                  of bsattn_make_layout on 1-token blocks); all of them if
 *                  fewer than r.  Global rows draw none.
 *   seed           hash seed.
 *   out            receives the new layout (caller frees with bsattn_layout_destroy).
 * The stored CSR lists, per row of 64-token tiles, the tiles the band touches
 * and then the gathered tiles L/64 .. L/64 + ceil(n/64) - 1 that hold the
 * global tokens' keys.  Forward only (bf16, no key padding); the backward,
 * the layer and the routed call return UNSUPPORTED or INVALID_ARG for it.
 * Limits: H * L * r <= 2^28. */
bsattn_status bsattn_make_token_layout(int32_t num_heads, int32_t seq_len, int32_t band_tokens,
                                       int32_t num_global, int32_t random_tokens, uint64_t seed,
                                       bsattn_layout** out);

/* A content-adaptive block layout: its key blocks are chosen on the device
 * from q and k at every bsattn_forward call (Adaptive Sparse Transformer
 * page, importance evaluation: score candidate positions and keep the highest
 * r% per query; here the candidates are 64-token key blocks, SQA page
 * sections 3.1 and 5).  For each (b, h):
 *   qs[i, d] = sum over u = 0..63 of q[64 i + u, d], added in that order in fp64
 *   (ks likewise from k); S[i, j] = sum over d = 0..D-1 of qs[i, d] * ks[j, d],
 *   each product rounded and added in order of d in fp64, no fused
 *   multiply-add; query block i attends the keep_blocks key blocks of highest
 *   S[i, j], ties to the lower j.  NaN scores give an unspecified (but valid,
 *   distinct) choice.
 *   num_heads     H >= 1.
 *   seq_len       L, a positive multiple of 64, L/64 <= 1024.
 *   keep_blocks   in [1, L/64]; floor(r L/64) keeps the fraction r.
 *   out           receives the new layout (caller frees with bsattn_layout_destroy).
 * Host only.  The stored CSR holds, per row, the positions 0 .. keep_blocks-1
 * (the blocks themselves are per call).  bsattn_forward on it is bf16 only
 * and takes no key padding; its workspace (bsattn_workspace_size) also holds
 * the block sums and the chosen blocks.  No backward. */
bsattn_status bsattn_make_adaptive_layout(int32_t num_heads, int32_t seq_len, int32_t keep_blocks,
                                          bsattn_layout** out);

/* The selection step of a forward over an adaptive layout alone: writes the
 * kept key blocks of every query block, ascending, to selected_blocks (device
 * int32 [B, H, L/64, keep_blocks]).  q, k device bf16 [B, H, L, D], D in
 * {64, 128}; workspace as for bsattn_forward.  Enqueued on `stream`. */
bsattn_status bsattn_adaptive_select(const bsattn_layout* layout, int32_t batch, int32_t num_heads,
                                     int32_t seq_len, int32_t head_dim, const void* q, const void* k,
                                     int32_t* selected_blocks, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* A per-query top-keep layout (Adaptive Sparse Transformer page, the
 * importance-evaluation step: each query keeps its floor(L r) best-scoring
 * keys and attends to those alone).  For each (b, h) and query t:
 *   rank[t, s] = sum over d = 0..D-1 of q[t, d] * k[s, d] in fp32, products
 *   added in order of d from +0 (each bf16 product is exact in fp32, so the
 *   value is reproducible bit for bit); query t keeps the keep_tokens keys of
 *   highest rank, ties to the lower s, and attends to them with the usual
 *   softmax of scale * q.k.  NaN ranks give an unspecified (but valid) choice
 *   of exactly keep_tokens keys.
 *   num_heads     H >= 1.
 *   seq_len       L, a positive multiple of 64, L <= 8192.
 *   keep_tokens   in [1, L]; floor(r L) keeps the fraction r.
 *   out           receives the new layout (caller frees with bsattn_layout_destroy).
 * Host only.  The stored CSR is the dense block grid (every key block in
 * every row); the kept keys are chosen per call.  bsattn_forward on it is
 * bf16 only and takes no key padding; its workspace (bsattn_workspace_size)
 * also holds the kept-key words.  No backward. */
bsattn_status bsattn_make_topr_layout(int32_t num_heads, int32_t seq_len, int32_t keep_tokens,
                                      bsattn_layout** out);

/* The selection step of a forward over a top-keep layout alone: writes the
 * kept keys of every query to keep_bits (device uint64 [B, H, L, L/64],
 * 16-byte aligned): bit b of word (b, h, t, j) is set iff query t keeps key
 * 64 j + b, and every query has exactly keep_tokens bits set.  q, k device
 * bf16 [B, H, L, D], D in {64, 128}; workspace as for bsattn_forward.
 * Enqueued on `stream`. */
bsattn_status bsattn_topr_select(const bsattn_layout* layout, int32_t batch, int32_t num_heads,
                                 int32_t seq_len, int32_t head_dim, const void* q, const void* k,
                                 uint64_t* keep_bits, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Candidate positions of every query from the hidden states (Adaptive
 * Sparse Transformer page, "Adapt or Perish: 新手入门指南 – Adaptive Sparse
 * Transformer 核心原理与实战", its candidate generator: a Conv1d from the
 * model width to k channels, kernel 3, padding 1, predicts k relevant
 * positions per query).  y[b, t, j] = bias[j] + sum over taps u = 0, 1, 2
 * and channels c of w[u][c][j] * x[b, t + u - 1, c] (zeros outside the
 * sequence; w is PyTorch's Conv1d weight W[j, c, u] stored tap-major).  The
 * sum is taken in fp64 in one fixed order -- from bias[j], taps u = 0, 1, 2
 * in turn, channels c = 0 .. C - 1 within a tap -- so the position is
 * reproducible: positions[b, t, j] = y rounded to the nearest integer (ties
 * to even), clamped to [0, L - 1] (NaN: 0).
 *   x          device bf16 [batch, seq_len, channels], the hidden states.
 *   w          device fp32 [3, channels, num_candidates].
 *   bias       device fp32 [num_candidates].
 *   positions  device int32 [batch, seq_len, num_candidates], written.
 * 1 <= num_candidates <= 64; channels >= 1; seq_len >= 1.  Enqueued on
 * `stream`; allocates nothing. */
bsattn_status bsattn_candidate_positions(const void* x, const float* w, const float* bias, int32_t batch,
                                         int32_t seq_len, int32_t channels, int32_t num_candidates,
                                         int32_t* positions, hipStream_t stream);

/* Attention over each query's best candidates (the same page: its importance
 * evaluation scores the candidate positions and keeps the best r%; then the
 * SparseAttention formula with M = 1 on the kept keys).  For every (batch,
 * head, query): the distinct positions among positions[b, t, 0 .. k) (values
 * outside [0, seq_len) are ignored) are ranked by the fp32 score q.k taken in
 * order of d from +0 (each bf16 product is exact in fp32, so the rank is
 * reproducible), ties to the lower position; the first `keep` are kept (all
 * of them when fewer are distinct).  out = softmax(scale * q.k) over the kept
 * keys times their V rows, lse = the log-sum-exp of those scaled scores.
 *   dtype        BSATTN_BF16 (others: UNSUPPORTED).
 *   q, k, v      device bf16 [B, H, L, D], D in {64, 128}, 16-byte aligned.
 *   positions    device int32 [B, L, num_candidates] (shared by the heads),
 *                e.g. from bsattn_candidate_positions.
 *   keep         1 <= keep <= num_candidates <= 64 (the page: floor(k r)).
 *   out, lse     device bf16 [B, H, L, D] and fp32 [B, H, L], written; a
 *                query with no candidate in range gets O = 0, lse = -inf.
 *   kept         optional device int32 [B, H, L, keep]: the kept positions,
 *                ascending, -1 past their count; NULL to skip.
 * Enqueued on `stream`; allocates nothing. */
bsattn_status bsattn_candidate_forward(bsattn_dtype dtype, int32_t batch, int32_t num_heads, int32_t seq_len,
                                       int32_t head_dim, const void* q, const void* k, const void* v,
                                       const int32_t* positions, int32_t num_candidates, int32_t keep,
                                       float scale, void* out, float* lse, int32_t* kept, hipStream_t stream);

/* Borrowed host view of a token layout (valid until destroy): the global
 * tokens [num_global], ascending, and the random tokens [H][L][links_per_row],
 * each row ascending and padded with -1.  INVALID_ARG for other layouts.  Any
 * output pointer may be NULL. */
bsattn_status bsattn_layout_token_links(const bsattn_layout* layout, const int32_t** global_tokens,
                                        int32_t* num_global, const int32_t** links, int32_t* links_per_row);

/* Borrowed host view of the block-CSR arrays (valid until destroy).
 *   row_ptr [num_rows + 1], col_idx [nnz], num_rows = H * L / 64 (rows of
 *   64-token tiles whatever the layout's block), rows ordered head-major
 *   (row h*nb + i).  Any output pointer may be NULL. */
bsattn_status bsattn_layout_csr(const bsattn_layout* layout, const int32_t** row_ptr,
                                const int32_t** col_idx, int32_t* num_rows, int64_t* nnz);

/* Borrowed host view of the quarter masks of a layout of 32-token blocks
 * (valid until destroy): masks[nnz], parallel to col_idx; bit 2a + b set
 * when query half a of the tile's row block (tokens 32a .. 32a + 31 of it)
 * attends key half b of its column block.  For 64- and 128-token layouts
 * *masks is NULL and *n is 0 (every quarter of a stored tile is in).  Either
 * output pointer may be NULL. */
bsattn_status bsattn_layout_tile_masks(const bsattn_layout* layout, const uint8_t** masks, int64_t* n);

/* Copy the CSR and the layout's work items to the current HIP device
 * (hipMalloc + copies enqueued on `stream`, then synchronised).  Must precede
 * the forward calls that use the layout; calling it again re-uploads to the
 * then-current device and drops the schedules built so far.  The device copy
 * is freed by bsattn_layout_destroy.  The per-shape schedules are built by
 * bsattn_prepare, or on a shape's first call. */
bsattn_status bsattn_layout_upload(bsattn_layout* layout, hipStream_t stream);

/* Rebuild the same layout on the device from its parameters (one thread per
 * row runs the identical integer rule) into caller-owned device arrays
 * row_ptr_dev [num_rows + 1] and col_idx_dev [nnz] (the 64-token tile CSR, as
 * bsattn_layout_csr), and for layouts of 32-token blocks tile_masks_dev [nnz]
 * (the quarter masks, as bsattn_layout_tile_masks; may be NULL otherwise).
 * Exists to prove that the host and device evaluations of the rule agree bit
 * for bit.  Window/global/random layouts of 32-, 64- and 128-token blocks
 * and band layouts; UNSUPPORTED for token, adaptive and top-keep layouts. */
bsattn_status bsattn_layout_build_device(const bsattn_layout* layout, int32_t* row_ptr_dev,
                                         int32_t* col_idx_dev, uint8_t* tile_masks_dev, hipStream_t stream);

/* Build and upload, ahead of time, the work schedule of one call shape of an
 * uploaded layout, so that every later bsattn_forward (and, with
 * num_routed = k on a band layout, bsattn_forward_routed) of that shape
 * allocates nothing and never synchronises -- it can then be captured in a
 * HIP graph.  A call of a shape that was not prepared builds its schedule on
 * first use (hipMalloc and a synchronous copy on its stream).
 *   batch, head_dim  the calls' B and D (D in {64, 128}); one schedule per pair.
 *   num_routed       0, or the calls' k for bsattn_forward_routed (band layouts).
 *   backward         non-zero: also upload the backward work lists
 *                    (window/global/random and band layouts), which
 *                    bsattn_backward otherwise uploads on its first call.
 * hipMalloc and copies enqueued on `stream`, then synchronised.  The device
 * arrays belong to the layout (freed by bsattn_layout_destroy or a re-upload).
 * Calling it again for a prepared shape does nothing.  fp32 forwards use no
 * schedule. */
bsattn_status bsattn_prepare(const bsattn_layout* layout, int32_t batch, int32_t head_dim,
                             int32_t num_routed, int32_t backward, hipStream_t stream);

/* Free a layout and its device copy.  NULL is a no-op. */
void bsattn_layout_destroy(bsattn_layout* layout);

/* Device workspace bytes needed by bsattn_forward (num_routed == 0) or
 * bsattn_forward_routed (num_routed = k) for this layout, batch and head
 * width: the fp32 partial outputs and partial LSEs of rows that are split
 * across workgroups (global rows, routed tiles), which a second kernel of the
 * same call merges by log-sum-exp.  Written to *bytes (0 when nothing is
 * split).  For a token layout (num_routed ignored): the partials of every
 * row and of the global rows, and the gathered K/V tiles of the global
 * tokens.  The workspace needs no initialisation and holds nothing between
 * calls; calls that share one must not overlap in time. */
bsattn_status bsattn_workspace_size(const bsattn_layout* layout, int32_t batch,
                                    int32_t head_dim, int32_t num_routed, size_t* bytes);

/* Block-sparse attention forward.
 *   layout         uploaded layout with num_heads == H and seq_len == L.  A
 *                  band layout (bsattn_make_band_layout) gives the
 *                  token-granular sliding window |t - s| <= band_tokens (the
 *                  primer page's window_size loop, the BigBird page's 64-256
 *                  token windows); it is bf16 only and takes no key padding
 *                  (BSATTN_ERR_UNSUPPORTED otherwise).  A token layout
 *                  (bsattn_make_token_layout) gives the token-granular
 *                  BigBird pattern, also bf16 only without key padding: the
 *                  call then runs a gather of the global tokens' K/V rows,
 *                  the attention kernel and a merge that adds every row's
 *                  random tokens.  An adaptive layout
 *                  (bsattn_make_adaptive_layout) chooses its key blocks from
 *                  q and k first, in the same call.
 *   dtype          element type of q, k, v and out.
 *   batch..head_dim  B >= 1, H, L as in the layout, D in {64, 128}.
 *   q, k, v        device [B, H, L, D], contiguous, 16-byte aligned.
 *   out            device [B, H, L, D] of dtype; must not alias q, k or v.
 *   lse            device [B, H, L] fp32 (natural log).
 *   key_valid_len  device int32 [B] or NULL: keys s >= key_valid_len[b] are
 *                  masked (the primer page's key mask); each value in [0, L].
 *                  Query rows past the valid length are computed normally.
 *   scale          score scale (1/sqrt(D) for the usual attention).
 *   workspace      device buffer of at least bsattn_workspace_size() bytes,
 *                  256-byte aligned, any contents (may be NULL if that size
 *                  is 0).
 * Enqueued on `stream`.  When bsattn_prepare has built this (batch, head_dim)
 * shape, the call allocates nothing and does not synchronise; otherwise its
 * first call builds the schedule (hipMalloc and a synchronous copy). */
bsattn_status bsattn_forward(const bsattn_layout* layout, bsattn_dtype dtype,
                             int32_t batch, int32_t num_heads, int32_t seq_len, int32_t head_dim,
                             const void* q, const void* k, const void* v,
                             void* out, float* lse, const int32_t* key_valid_len, float scale,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* bsattn_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same computation and kernels as bsattn_forward, without the workspace
 * arguments: the workspace is a device array of 64 MiB that the library
 * holds on each device it runs on until the process ends (resolved on the
 * first call on a device).  The call allocates nothing, so the shape must
 * have been built by bsattn_prepare(layout, batch, head_dim, 0, ...) first
 * (BSATTN_ERR_STATE otherwise); a call whose bsattn_workspace_size exceeds
 * 64 MiB returns BSATTN_ERR_UNSUPPORTED.  All calls on one device share the
 * array: calls that overlap in time on one device race (order them on one
 * stream).  Other arguments, layouts and errors as bsattn_forward. */
bsattn_status bsattn_forward_noalloc(const bsattn_layout* layout, bsattn_dtype dtype,
                                     int32_t batch, int32_t num_heads, int32_t seq_len, int32_t head_dim,
                                     const void* q, const void* k, const void* v,
                                     void* out, float* lse, const int32_t* key_valid_len, float scale,
                                     hipStream_t stream);

/* Routed-query selection (SQA page, section 2.1: a learned linear router
 * scores each query and keeps the top-k; section 3.2: the router runs in
 * higher precision than the model).  For each (b, h):
 *   score[t] = sum_{d=0}^{D-1} (double)q[b,h,t,d] * (double)w[d], summed left
 *   to right in fp64 (every product is exact, so the score is reproducible
 *   bit for bit), then the k rows with the largest score, ties to the lower
 *   row index, written ascending to routed_rows.
 *   q                device bf16 [B, H, L, D], D in {64, 128}, 16-byte aligned.
 *   w                device fp32 [D].
 *   k                1 <= k <= L; L <= 8192.
 *   routed_rows      device int32 [B, H, k].
 *   workspace        device buffer of at least bsattn_route_workspace_size()
 *                    bytes (B * H * L * 8: the fp64 scores), 16-byte
 *                    aligned; it needs no initialisation and holds nothing
 *                    between calls, and calls sharing it must not overlap.
 * Errors: INVALID_ARG for NULL pointers, bad k or a short workspace;
 * UNSUPPORTED for L > 8192 or another head_dim.  Nothing is allocated.
 * NaN scores give an unspecified (but valid, distinct) selection. */
bsattn_status bsattn_route_workspace_size(int32_t batch, int32_t num_heads, int32_t seq_len, int32_t k,
                                          size_t* bytes);
bsattn_status bsattn_route_topk(const void* q, const float* w, int32_t batch, int32_t num_heads,
                                int32_t seq_len, int32_t head_dim, int32_t k,
                                int32_t* routed_rows, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Routed-query attention forward (SQA page, section 2.1): rows listed in
 * routed_rows [B, H, num_routed] (device int32, distinct, in [0, L)) attend to
 * every key; all other rows attend to keys with |t - s| <= band, where
 * `band_layout` comes from bsattn_make_band_layout (and is uploaded).
 * dtype must be BSATTN_BF16.  Other arguments as bsattn_forward; the
 * workspace is sized with num_routed, and bsattn_prepare with num_routed = k
 * builds the schedule ahead of time. */
bsattn_status bsattn_forward_routed(const bsattn_layout* band_layout, bsattn_dtype dtype,
                                    int32_t batch, int32_t num_heads, int32_t seq_len,
                                    int32_t head_dim, const void* q, const void* k,
                                    const void* v, const int32_t* routed_rows,
                                    int32_t num_routed, void* out, float* lse, float scale,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Device workspace bytes needed by bsattn_backward for this layout, batch and
 * head width: delta = rowsum(dO * O) per query row (fp32 [B, H, L]), then the
 * fp32 partial gradients of rows and columns of the layout that are split
 * across workgroups (global rows and the key blocks every row attends; for a
 * token layout also its global rows' tiles and its global keys' partials).
 * Written to *bytes.  The workspace needs no initialisation and holds nothing
 * between calls; calls that share one must not overlap in time. */
bsattn_status bsattn_backward_workspace_size(const bsattn_layout* layout, int32_t batch,
                                             int32_t head_dim, size_t* bytes);

/* Block-sparse attention backward: the gradients of bsattn_forward (same
 * layout, key padding and scale) with respect to q, k and v for an upstream
 * gradient dout of the output.  The models on the pages are trained (SQA
 * page, sections 2.2 and 3.2; BigBird page, the pitfall guide on mixed
 * precision training); the backward is the derivative of the forward:
 *   P = exp(scale * q.k - lse) on allowed keys, delta = rowsum(dout * out),
 *   dv = P^T dout,  ds = P * (dout v^T - delta),
 *   dq = scale * ds k,  dk = scale * ds^T q.
 *   layout          uploaded window/global/random, band or token layout
 *                   (adaptive and top-keep layouts, and the routed variant:
 *                   UNSUPPORTED; band and token layouts take no key padding).
 *                   A token layout (BigBird page, its token-granular code
 *                   example) runs the band and its global rows through the
 *                   block passes and adds each non-global row's global keys
 *                   outside its band and its random tokens with gather
 *                   kernels, in place on dq, dk and dv (one more bf16
 *                   rounding there).  out and lse must come from
 *                   bsattn_forward on this layout: outputs of
 *                   bsattn_forward_routed are not detected and would give the
 *                   band's gradients for the routed rows.
 *   dtype           BSATTN_BF16 (others: UNSUPPORTED).
 *   batch..head_dim as bsattn_forward.
 *   q, k, v         the forward's inputs, device bf16 [B, H, L, D].
 *   out, lse        the forward's outputs for these inputs: bf16 [B, H, L, D]
 *                   and fp32 [B, H, L] (a row with lse = -inf has no allowed
 *                   key and gets zero gradient).
 *   dout            device bf16 [B, H, L, D].
 *   dq, dk, dv      device bf16 [B, H, L, D], written completely; must not
 *                   alias any input or each other.
 *   key_valid_len   as bsattn_forward.
 *   workspace       device buffer of at least bsattn_backward_workspace_size()
 *                   bytes, 256-byte aligned, any contents.
 * All pointers 16-byte aligned.  Enqueued on `stream`.  Unless
 * bsattn_prepare (backward != 0) uploaded them, the first call on a device
 * uploads the layout's backward work lists (hipMalloc and a synchronous
 * copy); later calls allocate nothing and do not synchronise. */
bsattn_status bsattn_backward(const bsattn_layout* layout, bsattn_dtype dtype,
                              int32_t batch, int32_t num_heads, int32_t seq_len, int32_t head_dim,
                              const void* q, const void* k, const void* v,
                              const void* out, const float* lse, const void* dout,
                              void* dq, void* dk, void* dv, const int32_t* key_valid_len,
                              float scale, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Backward of the routed-query forward (bsattn_forward_routed; SQA page,
 * sections 2.1 and 2.2: the routed model is trained end to end): dQ, dK and dV
 * of that forward for an upstream dout, with the mask "row t sees every key
 * if t is routed, else the keys with |t - s| <= band_tokens".
 *   band_layout   the band layout the forward used (uploaded).
 *   routed_rows   device int32 [B, H, num_routed], distinct rows in [0, L), as
 *                 given to the forward; out and lse are the forward's outputs.
 *   workspace     device buffer of at least
 *                 bsattn_backward_routed_workspace_size() bytes, 256-byte
 *                 aligned; needs no initialisation, holds nothing between calls.
 * dtype must be BSATTN_BF16.  Other arguments, layouts and errors as
 * bsattn_backward.  The first call for a routed tile count (ceil(num_routed /
 * 64)) builds and uploads its work lists with hipMalloc and a stream
 * synchronisation, unless bsattn_prepare(backward = 1, num_routed) did. */
bsattn_status bsattn_backward_routed_workspace_size(const bsattn_layout* band_layout, int32_t batch,
                                                    int32_t head_dim, int32_t num_routed, size_t* bytes);
bsattn_status bsattn_backward_routed(const bsattn_layout* band_layout, bsattn_dtype dtype, int32_t batch,
                                     int32_t num_heads, int32_t seq_len, int32_t head_dim, const void* q,
                                     const void* k, const void* v, const void* out, const float* lse,
                                     const void* dout, const int32_t* routed_rows, int32_t num_routed,
                                     void* dq, void* dk, void* dv, float scale, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* Device workspace bytes needed by bsattn_layer_forward: the fp32 qkv
 * projection, the per-head Q, K, V, O (bf16), LSE and the attention's own
 * workspace.  Written to *bytes. */
bsattn_status bsattn_layer_workspace_size(const bsattn_layout* layout, int32_t batch,
                                          int32_t head_dim, size_t* bytes);

/* The attention layer around the block-sparse attention (primer page, section
 * PyTorch 实现基础稀疏注意力, the SparseAttention module):
 *   qkv = x w_qkv^T + b_qkv            (width 3C, C = H * D; rows read as (3, H, D))
 *   O   = block-sparse attention of each head's q, k, v (bsattn_forward)
 *   out = concat_heads(O) w_proj^T + b_proj
 *   x        device bf16 [B, L, C], row-major.
 *   w_qkv    device bf16 [3C, C] (an nn.Linear weight: out x in); b_qkv bf16 [3C].
 *   w_proj   device bf16 [C, C]; b_proj bf16 [C].
 *   out      device bf16 [B, L, C]; must not alias an input.
 *   layout, key_valid_len, scale as bsattn_forward (the page divides by sqrt(C);
 *   pass the scale wanted).
 * The two projections are hipBLASLt GEMMs (bf16 inputs, fp32 accumulation)
 * whose epilogue adds the bias and writes bf16: the qkv projection token-major
 * [B L, 3C], from which the attention reads each head in place, and the output
 * projection from the attention's concatenated heads [B L, C].  Where
 * hipBLASLt has no algorithm for a shape, rocBLAS GEMMs with fp32 output and
 * this library's bias, head split and concatenation kernels are used instead.
 * q, k, v and the projections are rounded to bf16 once each.  Pointers 16-byte
 * aligned, workspace 256-byte aligned.
 * Enqueued on `stream`; the first call of a shape on a thread creates the
 * library handles and hipBLASLt's plan for the two projections (the first
 * algorithm of its heuristic). */
bsattn_status bsattn_layer_forward(const bsattn_layout* layout, int32_t batch, int32_t num_heads,
                                   int32_t seq_len, int32_t head_dim, const void* x,
                                   const void* w_qkv, const void* b_qkv, const void* w_proj,
                                   const void* b_proj, void* out, const int32_t* key_valid_len,
                                   float scale, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* Measurement hook: while set (non-NULL), every forward call made from this
 * thread records `before` on its stream immediately before the main attention
 * kernel and `after` immediately after it (over a top-keep layout: around the
 * key selection, its dominant kernel; in bsattn_candidate_forward: around its
 * attention kernel), and every backward call does the same around its dK/dV
 * kernel, so a caller can time that kernel alone with
 * hipEventElapsedTime.  Pass NULLs to clear.  Events are caller owned. */
bsattn_status bsattn_set_profile_events(hipEvent_t before, hipEvent_t after);

/* Static description of a status code; never NULL. */
const char* bsattn_status_string(bsattn_status status);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char* bsattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
