/*
 * nosa.h — C ABI of the NOSA per-decode-step block-sparse attention path on
 * AMD Instinct MI355X (gfx950).
 *
 * The method is NOSA ("NOSA: Native and Offloadable Sparse Attention",
 * technical summary pages, section Methodology). One decode step of one layer
 * runs, per row = one (batch, KV head) pair:
 *
 *   nosa_pool_blocks    sub-block mean / block max pooling of a newly complete
 *                       block (Methodology, "1. Algorithm", bullet
 *                       "Block-Wise Implementation")
 *   nosa_score_blocks   query-aware pooled block scores (bullets "Dual-Selection
 *                       Mechanism", "Block-Wise Implementation")
 *   nosa_select         Gamma_e: k_e blocks by pre-exponential eviction score
 *                       with strict eviction (bullets "Dual-Selection
 *                       Mechanism", "ED-DMA", "Locality Guarantee");
 *                       Gamma_q: top k_q of the rest by query-aware score
 *   nosa_swap_diff      set difference between the new selection and the
 *                       blocks cached in HBM (Methodology, "2. System: NOSI",
 *                       bullet "Optimized Memory Layout")
 *   nosa_fetch_blocks   copy of the missing blocks from pinned host memory
 *                       into HBM by a GPU kernel (bullet "High-Bandwidth
 *                       Communication")
 *   nosa_sparse_decode  attention over the selected blocks plus the newest
 *                       block, the eviction score added to each logit so its
 *                       exponential happens only in the softmax (bullet
 *                       "ED-DMA")
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership: the caller owns every buffer. Device buffers are plain device
 *   pointers; "pinned host" buffers come from nosa_host_alloc. The library
 *   keeps no allocation and no mutable state between calls, except the
 *   scratch array of nosa_sparse_decode_noalloc (one per GPU, for the life
 *   of the process) and the device addresses of that array it caches.
 * Streams: every call only enqueues work on `stream` (a hipStream_t, may be
 *   NULL for the null stream) and never synchronises. Host-side arguments
 *   (shape, step) are read during the call and may be reused afterwards.
 * Errors: arguments are validated on the host before anything is launched;
 *   a bad argument returns NOSA_ERR_INVALID_ARGUMENT (or NOSA_ERR_UNSUPPORTED
 *   for a valid but unimplemented shape) and launches nothing. A failed
 *   launch returns NOSA_ERR_HIP. Device *data* (block ids in lists) is trusted:
 *   out-of-range ids are undefined behaviour. No C++ exception crosses the ABI.
 * Rows: row r = b * n_kv_heads + g. Query heads g*G .. g*G+G-1 (G =
 *   n_q_heads / n_kv_heads) share KV head g.
 * Blocks: block j holds tokens [j*S, j*S + S), S = block_size. After a step
 *   has appended its token there are n_tokens tokens; the candidate blocks
 *   are 0 .. n_cand-1 with n_cand = (n_tokens - 1) / S; block n_cand (the
 *   newest, 1..S tokens) is always attended and is never a candidate.
 *
 * Layouts (element type = shape.dtype unless stated)
 * --------------------------------------------------
 * q, out     [batch][n_q_heads][D]
 * KV block   one block-unit of 2*S*D elements (S = 64): the K tile, S*D
 *            elements, then the V tile transposed (V^T, D rows of S
 *            positions), D*S elements. Position p of a V^T row holds token
 *            vt(p) of the block: inside each half of 32, positions 8j..8j+7
 *            hold tokens 4j..4j+3 and 16+4j..16+4j+3 of that half. Both tiles
 *            are stored as 1 KiB fragments of 64 16-byte vectors (E = 16 /
 *            element size elements each; vector l has col = l % 16, grp =
 *            l / 16), each fragment one matrix-core operand of a wave:
 *              K   fragment t*(D/4E) + s, vector l: token 16t + col,
 *                  dimensions (4s + grp)*E .. + E-1;
 *              V^T fragment dt*(S/4E) + s, vector l: dimension 16dt + col,
 *                  positions (4s + grp)*E .. + E-1.
 *            So K[tok][d] is at element
 *              ((tok/16 * D/4E + d/4E) * 64 + tok%16 + 16 * (d/E % 4)) * E + d%E
 *            and V[tok][d], with p the position of tok, at S*D +
 *              ((d/16 * S/4E + p/4E) * 64 + d%16 + 16 * (p/E % 4)) * E + p%E.
 *            A "KV buffer" is [rows][row_blocks][2*S*D]; the full KV, an HBM
 *            block cache (k slots per row) and the newest-block buffer (one
 *            block per row) all use it with their own row_blocks.
 * e_tok      float32 [rows][e_row_stride]: per-token eviction scores,
 *            pre-exponential. nosa_sparse_decode reads them a block at a
 *            time: e_tok is 16-byte aligned, e_row_stride a multiple of 4 and
 *            at least S * (n_cand + 1) (values past n_tokens are ignored).
 * kbar       pooled keys in the pooled dtype (shape.pooled_dtype), V = 16 /
 *            element size dimensions per 16-byte vector (4 for float32, 8 for
 *            bfloat16), in quads of 4 blocks: [rows][Q][D/V][16][V], Q =
 *            ceil(max_blocks / 4); the mean key of sub-block i of block j
 *            (sb = 4*j + i) is at [.][sb/16][d/V][sb%16][d%V]. Each mean is
 *            the sub-block's keys summed in double and rounded once to the
 *            pooled dtype (nearest, ties to even): for bfloat16 keys the
 *            exact mean rounded once. With bfloat16 keys and float32 pooled
 *            keys, the buffer continues (nosa_kbar_bytes bytes in all) with
 *            a bfloat16 rounding of every mean, in the bfloat16 layout, then
 *            a float32 radius per block [rows][max_blocks]: scores from the
 *            bfloat16 copy are within scale * sum_h ||q_h||_2 * radius of
 *            the float32 ones, which lets nosa_score_select rank on the
 *            copy and settle the near ties on float32 scores.
 * e_blk      float32 [rows][max_blocks]: pooled eviction score per block.
 * s_q        float32 [rows][max_blocks]: query-aware score per block.
 * bitmaps    uint32 [rows][W], W = (max_blocks + 31) / 32; bit j%32 of word
 *            j/32 stands for block j.
 * sel        int32 [rows][k]: selected block ids ascending, -1 padded;
 *            n_sel int32 [rows].
 * slot_block int32 [rows][k]: block held by each cache slot, -1 = empty.
 * block_slot int32 [rows][max_blocks]: slot of each cached block, -1 = none.
 */
#ifndef NOSA_H
#define NOSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t nosa_status;
enum {
    NOSA_OK = 0,
    NOSA_ERR_INVALID_ARGUMENT = 1,
    NOSA_ERR_UNSUPPORTED = 2,
    NOSA_ERR_HIP = 3,
    NOSA_ERR_WORKSPACE = 4
};

/* element types of q, K, V and out */
enum { NOSA_F32 = 0, NOSA_BF16 = 1 };

/* which source the decode reads selected blocks from */
enum { NOSA_KV_FULL = 0, NOSA_KV_CACHE = 1 };

/* decode kernel choice (nosa_shape.decode_kernel) */
enum { NOSA_DECODE_AUTO = 0, NOSA_DECODE_VALU = 1, NOSA_DECODE_MFMA = 2 };

/* Problem shape, in the pages' terms: block size, sub-block size, budgets
 * k = k_e + k_q, and GQA groups (n_q_heads / n_kv_heads).
 * Supported: block_size 64, sub_block 16, head_dim 64 or 128, G <= 8,
 * k <= 128, max_blocks <= 4096.
 * pooled_dtype: element type of the pooled keys (kbar) and of a prefill's
 * pooled queries (qbar). The pages fix the pooling (mean inside sub-blocks,
 * then max over the block; Methodology, "Block-Wise Implementation"), not
 * its precision. NOSA_F32 (0, the default of a zeroed shape): the means
 * rounded once to float32, which selects what the exact means select up to
 * float32 rounding of the scores. NOSA_BF16 (bfloat16 KV only): the means
 * rounded once to bfloat16, the variant for a stack that keeps pooled keys
 * in the model's dtype; it halves the scoring reads, and it changes which
 * blocks Gamma_q selects on a few percent of the steps of a long decode. */
typedef struct nosa_shape {
    int32_t batch;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t sub_block;
    int32_t k_e;           /* query-agnostic (eviction) budget, blocks */
    int32_t k_q;           /* query-aware budget, blocks */
    int32_t max_blocks;    /* capacity of per-row block arrays */
    int32_t dtype;         /* NOSA_F32 or NOSA_BF16 */
    int32_t decode_kernel; /* NOSA_DECODE_* */
    float scale;           /* logit scale; 0 means 1/sqrt(head_dim) */
    int32_t pooled_dtype;  /* NOSA_F32 (default) or NOSA_BF16: kbar and qbar */
} nosa_shape;

/* Where the decode is. The entry points below that take `const nosa_step
 * *step` read it on the host during the call; the *_step entry points
 * (graph-replayable steps, at the end of this header) take it in device
 * memory instead and read it in their kernels. */
typedef struct nosa_step {
    int32_t n_tokens;    /* tokens present, including the one appended this step */
    int32_t n_cand_prev; /* candidate blocks at the previous step; -1: no previous
                            step, so nosa_select (re)initialises Gamma_e */
} nosa_step;

/* Pool blocks [blk_begin, blk_end) of every row: kbar gets each sub-block's
 * mean key in the pooled dtype (layout and rounding above), e_blk the max over the
 * block's sub-blocks of the mean per-token eviction score (Methodology,
 * "Block-Wise Implementation": mean inside sub-blocks, then max over the
 * block). Block j of row r is read from the KV buffer `kv` at block index
 * kv_first_block + (j - blk_begin) of that row (kv_row_blocks blocks per row),
 * so the same call pools from the full KV or from the newest-block buffer.
 * With bf16 keys and float32 pooled keys it also writes the blocks' bfloat16
 * copies and radii (kbar must then hold nosa_kbar_bytes bytes).
 * kv may be a device pointer or the device alias of pinned host memory. */
nosa_status nosa_pool_blocks(const nosa_shape *shape, const void *kv, int64_t kv_row_blocks,
                             int32_t kv_first_block, const float *e_tok, int64_t e_row_stride,
                             int32_t blk_begin, int32_t blk_end, void *kbar, float *e_blk,
                             void *stream);

/* The step before the path, fused in one launch (Methodology, "2. System:
 * NOSI", Kernel Fusion: eviction head, QKV split and pooling together), for
 * token n_tokens - 1 of every row:
 *  - qkv [batch][(Hq + 2*Hkv) * D] (KV dtype) is one token's fused projection
 *    output, query heads first, then key heads, then value heads: the query
 *    heads go to q_out [batch][Hq][D]; the row's key and value go into token
 *    slot (n_tokens - 1) % S of block `block` of the KV buffer `kv`, as
 *    nosa_append_tokens writes them;
 *  - the eviction head (Dual-Selection Mechanism, query-agnostic part; kept
 *    pre-exponential, ED-DMA): e = x[b] . w_evict[g] + b_evict[g] with x
 *    [batch][hidden] and w_evict [n_kv_heads][hidden] in the KV dtype,
 *    b_evict float32 [n_kv_heads] or NULL (zero), summed in float32, goes to
 *    e_tok[row][n_tokens - 1];
 *  - when that token completes its block j = (n_tokens - 1) / S, the block is
 *    pooled exactly as nosa_pool_blocks pools it (kbar, e_blk), the other
 *    tokens of the block being read from `kv` and e_tok.
 * qkv and q_out are 16-byte aligned (x and w_evict may be, for vector loads);
 * e_row_stride >= n_tokens; block in [0, kv_row_blocks); j < max_blocks.
 * Invalid arguments return NOSA_ERR_INVALID_ARGUMENT before any launch. */
nosa_status nosa_ingest_tokens(const nosa_shape *shape, const void *qkv, const void *x,
                               const void *w_evict, const float *b_evict, int32_t hidden,
                               int32_t n_tokens, void *q_out, void *kv, int64_t kv_row_blocks,
                               int32_t block, float *e_tok, int64_t e_row_stride, void *kbar,
                               float *e_blk, void *stream);

/* ---- prefill (training-time forward) with the selection per query block ----
 * The method is trainable and native (Methodology, "1. Algorithm: NOSA"): the
 * same dual selection shapes attention over a whole sequence. Query blocks
 * are the S-token blocks of the sequence; query block i selects among the
 * complete blocks before it (0..i-1) as a decode step with those candidates
 * does, scoring with the block's pooled query; its tokens attend the selected
 * blocks and their own block causally. Call order: nosa_pool_blocks over the
 * complete blocks, nosa_prefill_pool_queries, nosa_prefill_select,
 * nosa_prefill_attention. */

/* Pooled query of every query block: qbar [n_qb][batch][Hq][D] (pooled
 * dtype, n_qb = ceil(n_tokens / S)) is the mean over the block's tokens of q
 * [batch][n_tokens][Hq][D] (KV dtype), summed in double and rounded once to
 * the pooled dtype. q and qbar must be
 * 16-byte aligned (NOSA_ERR_INVALID_ARGUMENT otherwise). */
nosa_status nosa_prefill_pool_queries(const nosa_shape *shape, const void *q, int32_t n_tokens,
                                      void *qbar, void *stream);

/* Selection of every query block i (candidates 0..i-1): sel [n_qb][rows][k]
 * ascending, -1 padded, and n_sel [n_qb][rows], as nosa_score_select with no
 * previous step would select for query qbar[i]. One launch for all query
 * blocks; n_qb <= max_blocks + 1 and n_qb <= 65535. */
nosa_status nosa_prefill_select(const nosa_shape *shape, const void *qbar, const void *kbar,
                                const float *e_blk, int32_t n_tokens, int32_t *sel,
                                int32_t *n_sel, void *stream);

/* Causal block-sparse attention of the whole sequence (bf16, matrix cores):
 * out[b][p][h] = softmax over the tokens of query block i = p / S's selected
 * blocks and of tokens S*i .. p of z = scale * q.k + e (e_tok as an additive
 * logit, ED-DMA), times V. kv is the block-unit KV [rows][kv_row_blocks][2*S*D]
 * (kv_row_blocks >= n_qb; the last block may be partial: its slots past
 * n_tokens are read as zeros, whatever they hold), e_tok [rows][stride]
 * (stride >= n_qb * S, a multiple of 4), q and out [batch][n_tokens][Hq][D].
 * float32: NOSA_ERR_UNSUPPORTED. */
nosa_status nosa_prefill_attention(const nosa_shape *shape, const void *q, int32_t n_tokens,
                                   const void *kv, int64_t kv_row_blocks, const float *e_tok,
                                   int64_t e_row_stride, const int32_t *sel, const int32_t *n_sel,
                                   void *out, void *stream);

/* Write the newest token of every row into the block-unit KV buffer `kv`
 * (device memory or the device alias of pinned host memory; kv_row_blocks
 * blocks per row): token slot pos (0..S-1) of block `block` receives
 * k_new[row][D] as token pos of the K tile and v_new[row][D] as token pos of
 * the V^T tile (the block layout above). k_new and v_new are [rows][D] in the
 * KV dtype, rows = batch * n_kv_heads. This is the KV-cache write the
 * decode step assumes (the pages keep the cache in block-sized units;
 * "2. System: NOSI", Optimized Memory Layout): with the newest-block buffer
 * as `kv`, an offloaded cache takes new tokens on the GPU and a completed
 * block goes to host memory with nosa_fetch_blocks (source: the newest-block
 * buffer, destination: the host KV). Invalid arguments (pos or block out of
 * range, NULL pointers) return NOSA_ERR_INVALID_ARGUMENT before any launch. */
nosa_status nosa_append_tokens(const nosa_shape *shape, const void *k_new, const void *v_new,
                               int32_t pos, void *kv, int64_t kv_row_blocks, int32_t block,
                               void *stream);

/* Query-aware block scores for candidates 0 .. n_cand-1 of every row:
 * s_q[r][j] = sum over the G heads of the row of max over sub-blocks i of
 * scale * q_h . kbar[j,i] (Methodology, "Dual-Selection Mechanism" and
 * "Block-Wise Implementation"). Entries j >= n_cand are left untouched. */
nosa_status nosa_score_blocks(const nosa_shape *shape, const void *q, const void *kbar,
                              const nosa_step *step, float *s_q, void *stream);

/* Dual selection for every row (Methodology, "Dual-Selection Mechanism",
 * "Locality Guarantee", "ED-DMA").
 * Gamma_e (bitmap ge_bits, in/out) keeps k_e blocks ranked by e_blk, the
 * pre-exponential eviction score. With step->n_cand_prev < 0 it is rebuilt
 * as the k_e best of all candidates and every other candidate is marked in
 * ev_bits (evicted). Otherwise each new candidate n_cand_prev .. n_cand-1 in
 * turn either enters, replacing the lowest-ranked member if it ranks above
 * it (the member moves to ev_bits), or is evicted at once; an evicted block
 * never re-enters. Ranking: higher score first, equal scores lower id first.
 * Gamma_q: the k_q best of the candidates outside Gamma_e by s_q (evicted
 * blocks are eligible). Outputs sel/n_sel (ascending union) and sel_bits. */
nosa_status nosa_select(const nosa_shape *shape, const float *s_q, const float *e_blk,
                        const nosa_step *step, uint32_t *ge_bits, uint32_t *ev_bits,
                        int32_t *sel, int32_t *n_sel, uint32_t *sel_bits, void *stream);

/* Set difference against the HBM block cache of k = k_e + k_q slots per row
 * (Methodology, "2. System: NOSI", "Optimized Memory Layout").
 * fetch = selected blocks not cached (ascending); free = slots that are
 * empty or hold a block no longer selected (ascending); fetch[i] goes to
 * free[i]; leftover free slots become empty. Updates slot_block and
 * block_slot (in/out; start with every entry -1), writes fetch_block /
 * fetch_slot [rows][k] and n_fetch [rows], and adds to counters
 * uint64 [rows][2]: {blocks fetched, selected blocks already cached}. */
nosa_status nosa_swap_diff(const nosa_shape *shape, const int32_t *sel, const int32_t *n_sel,
                           const uint32_t *sel_bits, int32_t *slot_block, int32_t *block_slot,
                           int32_t *fetch_block, int32_t *fetch_slot, int32_t *n_fetch,
                           uint64_t *counters, void *stream);

/* nosa_select followed by nosa_swap_diff, in one launch: the same outputs
 * and state updates as the two calls in sequence. */
nosa_status nosa_select_swap(const nosa_shape *shape, const float *s_q, const float *e_blk,
                             const nosa_step *step, uint32_t *ge_bits, uint32_t *ev_bits,
                             int32_t *sel, int32_t *n_sel, uint32_t *sel_bits,
                             int32_t *slot_block, int32_t *block_slot, int32_t *fetch_block,
                             int32_t *fetch_slot, int32_t *n_fetch, uint64_t *counters,
                             void *stream);

/* nosa_score_blocks and nosa_select (and, when the six cache pointers are
 * given, the set difference as in nosa_select_swap) in one call. With more
 * than 128 rows (bf16; more than 256 with bf16 keys and float32 pooled
 * keys), or float32 inputs, it is one launch: one workgroup per row computes
 * the row's query-aware scores into on-chip memory and selects from them.
 * With fewer bf16 rows, too few workgroups to fill the GPU that way, the
 * scores are computed on a grid split over each row's candidates and the
 * selection follows as a second launch on the same stream. With bf16 keys
 * and float32 pooled keys the scores come from the
 * pooled keys' bfloat16 copy (half the bytes); every candidate whose score
 * interval (copy score +- scale * sum_h ||q_h|| * radius) reaches the lowest
 * lower bound of that first top k_q is then scored again from the float32
 * means (float32 dot products, partial sums in a fixed order), and Gamma_q
 * is the top k_q of those: the selection is the one float32 scores give,
 * and s_q receives the copy's scores (within the radius bound of the
 * float32 ones). Otherwise s_q receives the scores. Selections and state updates are
 * those of the separate calls. The cache pointers are all NULL or all
 * non-NULL. */
nosa_status nosa_score_select(const nosa_shape *shape, const void *q, const void *kbar,
                              const float *e_blk, const nosa_step *step, float *s_q,
                              uint32_t *ge_bits, uint32_t *ev_bits, int32_t *sel, int32_t *n_sel,
                              uint32_t *sel_bits, int32_t *slot_block, int32_t *block_slot,
                              int32_t *fetch_block, int32_t *fetch_slot, int32_t *n_fetch,
                              uint64_t *counters, void *stream);

/* nosa_select (and, when the six cache pointers are given, the set
 * difference as in nosa_select_swap) that also writes the two parts of the
 * selection as ascending lists: ge_list int32 [rows][k_e] (Gamma_e) with
 * n_ge [rows], and gq_list int32 [rows][k_q] (Gamma_q) with n_gq [rows],
 * -1 padded. The cache pointers are all NULL or all non-NULL. A step that
 * completes no block leaves Gamma_e unchanged (strict eviction only acts on
 * new candidates), so the previous step's ge_list already names this step's
 * eviction set: attention over it can start before this step's scores. */
nosa_status nosa_select_parts(const nosa_shape *shape, const float *s_q, const float *e_blk,
                              const nosa_step *step, uint32_t *ge_bits, uint32_t *ev_bits,
                              int32_t *sel, int32_t *n_sel, uint32_t *sel_bits, int32_t *ge_list,
                              int32_t *n_ge, int32_t *gq_list, int32_t *n_gq,
                              int32_t *slot_block, int32_t *block_slot, int32_t *fetch_block,
                              int32_t *fetch_slot, int32_t *n_fetch, uint64_t *counters,
                              void *stream);

/* Copy fetch_block[r][i] of the source KV buffer to slot fetch_slot[r][i] of
 * the destination KV buffer, for i < n_fetch[r] (at most max_fetch), every
 * row (Methodology, "High-Bandwidth Communication"). The copy is a GPU kernel
 * with 16-byte loads; src_kv is normally the device alias of pinned host
 * memory (nosa_host_alloc), so the loads travel over PCIe. Whole blocks of
 * 2*S*D elements are moved; layout inside a block is preserved. */
nosa_status nosa_fetch_blocks(const nosa_shape *shape, const void *src_kv, int64_t src_row_blocks,
                              const int32_t *fetch_block, const int32_t *fetch_slot,
                              const int32_t *n_fetch, int32_t max_fetch, void *dst_kv,
                              int64_t dst_row_blocks, void *stream);

/* Bytes of the kbar buffer for this shape (layout above); 0 for an invalid
 * shape. */
size_t nosa_kbar_bytes(const nosa_shape *shape);

/* Element offsets inside one KV block-unit of K[tok][d] (k_off) and of
 * V[tok][d] (v_off) for the shape's head_dim and dtype, the layout under
 * "KV block" above: each a host array of S*D int64 written as [tok][d].
 * Host only (no device work). Errors: the shape's (NOSA_ERR_INVALID_ARGUMENT,
 * NOSA_ERR_UNSUPPORTED), NOSA_ERR_INVALID_ARGUMENT for a NULL array. */
nosa_status nosa_block_offsets(const nosa_shape *shape, int64_t *k_off, int64_t *v_off);

/* Workspace bytes the attention calls need for this shape: split-K partials
 * of up to k + 2 chunks per row (one call over the whole selection, or two
 * partial calls over its parts). Calls that overlap in time need separate
 * workspaces, or disjoint chunk ranges of one (nosa_decode_partial). */
size_t nosa_decode_workspace_size(const nosa_shape *shape);

/* Chunks a partial-attention call over list_len list entries (plus the
 * newest block when with_newest = 1) occupies; -1 for invalid arguments. */
int32_t nosa_decode_chunks(const nosa_shape *shape, int32_t list_len, int32_t with_newest);

/* Sparse decode attention for every query head (Methodology, "ED-DMA"):
 * over the tokens T of the listed blocks plus the newest block (block n_cand,
 * tokens [S*n_cand, n_tokens)),
 *   z_i = scale * q_h . k_i + e_tok[r][i],  out_h = sum_i softmax(z)_i v_i.
 * kv_mode NOSA_KV_FULL: entry i < n_list[r] of row r is block list[r*k + i]
 *   of the KV buffer kv (kv_row_blocks per row); entries are block ids.
 * kv_mode NOSA_KV_CACHE: entry i < k is slot i of the cache kv; list is the
 *   slot_block table (block id per slot, -1 = empty, skipped); n_list unused.
 * The newest block of row r is block 0 of row r of cur_kv (cur_row_blocks
 *   blocks per row); for the full KV pass kv advanced by n_cand blocks.
 * Split-K partials go to ws (at least nosa_decode_workspace_size bytes); a
 * second kernel merges each row's partials in a fixed order and writes out
 * (float32 accumulation, bf16 stores round to nearest even). When the MFMA
 * kernel serves each row with a single chunk (nosa_decode_chunks(shape, k, 1)
 * == 1), that kernel normalizes and writes out itself, in one launch. shape.decode_kernel picks the partial kernel: MFMA (bf16
 * only; the default for bf16) or VALU (the default for float32). */
nosa_status nosa_sparse_decode(const nosa_shape *shape, const void *q, const void *kv,
                               int64_t kv_row_blocks, int32_t kv_mode, const int32_t *list,
                               const int32_t *n_list, const void *cur_kv, int64_t cur_row_blocks,
                               const nosa_step *step, const float *e_tok, int64_t e_row_stride,
                               void *out, void *ws, size_t ws_bytes, void *stream);

/* nosa_sparse_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same attention with the same arguments minus the
 * workspace. The split-K partials go to a scratch array the library holds in
 * device memory, NOSA_NOALLOC_SCRATCH_BYTES per GPU (its address is taken
 * once per device, on the first call there), with a row's partials packed
 * at the chunk count this call uses. Needs rows * chunks * G * (D + 2) * 4
 * bytes (chunks = nosa_decode_chunks(shape, k, 1); none when the MFMA kernel
 * serves each row with a single chunk); a shape that needs more returns
 * NOSA_ERR_WORKSPACE before any launch. The call allocates nothing and
 * synchronises nothing. Every call on one GPU shares that GPU's scratch: two
 * calls whose kernels overlap in time (other streams, other threads) race on
 * it and give undefined results. Results are bit for bit those of
 * nosa_sparse_decode. */
#define NOSA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
nosa_status nosa_sparse_decode_noalloc(const nosa_shape *shape, const void *q, const void *kv,
                                       int64_t kv_row_blocks, int32_t kv_mode,
                                       const int32_t *list, const int32_t *n_list,
                                       const void *cur_kv, int64_t cur_row_blocks,
                                       const nosa_step *step, const float *e_tok,
                                       int64_t e_row_stride, void *out, void *stream);

/* The first half of nosa_sparse_decode over an arbitrary block list: for
 * every row, attention partials (running max, sum and weighted values per
 * head) over list entries 0 .. list_len-1 of row r (list[r*list_stride + i];
 * NOSA_KV_FULL: block ids, the first n_list[r] valid; NOSA_KV_CACHE: slot i
 * holds block list[...], -1 skipped) and, when with_newest = 1, the newest
 * block. They fill workspace chunks chunk0 .. chunk0 + nosa_decode_chunks()-1.
 * Two calls over disjoint lists and disjoint chunk ranges may run
 * concurrently on different streams; nosa_decode_combine then merges.
 * kv may be NULL when list_len is 0. */
nosa_status nosa_decode_partial(const nosa_shape *shape, const void *q, const void *kv,
                                int64_t kv_row_blocks, int32_t kv_mode, const int32_t *list,
                                const int32_t *n_list, int32_t list_stride, int32_t list_len,
                                int32_t with_newest, const void *cur_kv, int64_t cur_row_blocks,
                                const nosa_step *step, const float *e_tok, int64_t e_row_stride,
                                void *ws, size_t ws_bytes, int32_t chunk0, void *stream);

/* nosa_decode_partial with its partial kernel bracketed by two HIP events
 * (hipEvent_t, created by the caller with hipEventCreate or
 * hipEventCreateWithFlags): the kernel is launched through
 * hipExtLaunchKernelGGL, which records start_event when the kernel starts
 * and stop_event when it ends, so hipEventElapsedTime of the pair is the
 * kernel's own duration, without the launch in front of it. For measuring
 * the attention kernel inside a running decode loop. Both events must be
 * non-NULL (NOSA_ERR_INVALID_ARGUMENT otherwise); everything else is as in
 * nosa_decode_partial. */
nosa_status nosa_decode_partial_timed(const nosa_shape *shape, const void *q, const void *kv,
                                      int64_t kv_row_blocks, int32_t kv_mode,
                                      const int32_t *list, const int32_t *n_list,
                                      int32_t list_stride, int32_t list_len, int32_t with_newest,
                                      const void *cur_kv, int64_t cur_row_blocks,
                                      const nosa_step *step, const float *e_tok,
                                      int64_t e_row_stride, void *ws, size_t ws_bytes,
                                      int32_t chunk0, void *start_event, void *stop_event,
                                      void *stream);

/* The second half: merges workspace chunks 0 .. n_chunks-1 of every row in
 * chunk order and writes out [batch][n_q_heads][D]. */
nosa_status nosa_decode_combine(const nosa_shape *shape, int32_t n_chunks, void *out, void *ws,
                                size_t ws_bytes, void *stream);

/* nosa_decode_combine that then moves the device step record step_dev on, as
 * nosa_step_advance does: the last call of a step replayed from a captured
 * graph, one kernel fewer per replay. Its merge reads no step record, and
 * every kernel of the step that does is enqueued before it on the stream.
 * step_dev must be non-NULL (NOSA_ERR_INVALID_ARGUMENT otherwise). */
nosa_status nosa_decode_combine_step(const nosa_shape *shape, int32_t n_chunks, void *out,
                                     void *ws, size_t ws_bytes, nosa_step *step_dev,
                                     void *stream);

/* nosa_decode_partial over every chunk (chunk0 = 0) and the merge, as one
 * call: NOSA's sparse attention for the given list (Methodology, "ED-DMA"),
 * output out [batch][n_q_heads][D] in the input dtype, workspace ws as for
 * nosa_decode_partial. When the matrix-core kernel (bf16) serves each row
 * with a single chunk (nosa_decode_chunks() == 1: many rows), it is one
 * launch: each workgroup normalizes its row's output and writes it, and ws
 * (still required and validated) is not written. Otherwise the partial kernel is followed by the merge kernel,
 * as nosa_decode_partial + nosa_decode_combine. start_event / stop_event:
 * both NULL, or both hipEvent_t recorded at the attention kernel's own start
 * and end, as in nosa_decode_partial_timed. list_len + with_newest must be
 * at least 1. Errors: NOSA_ERR_INVALID_ARGUMENT for a NULL out, one event
 * without the other or nothing to attend, else as nosa_decode_partial. */
nosa_status nosa_decode_attend(const nosa_shape *shape, const void *q, const void *kv,
                               int64_t kv_row_blocks, int32_t kv_mode, const int32_t *list,
                               const int32_t *n_list, int32_t list_stride, int32_t list_len,
                               int32_t with_newest, const void *cur_kv, int64_t cur_row_blocks,
                               const nosa_step *step, const float *e_tok, int64_t e_row_stride,
                               void *ws, size_t ws_bytes, void *out, void *start_event,
                               void *stop_event, void *stream);

/* ---- steps replayed from a captured graph ----
 * The step record lives in device memory (step_dev: a nosa_step, 8 bytes,
 * 4-byte aligned) and every call of a step reads it in its kernels, so one
 * decode step, captured once into a hipGraph, can be replayed step after
 * step: nosa_step_advance, the step's last call, moves the record on. The
 * calls take the same arguments as their host-step forms and compute the same
 * results for the same record. No call allocates, synchronises or memsets.
 * Values the record holds are clamped to the shape's capacity (n_tokens to
 * 1 .. max_blocks * S), so buffers sized for max_blocks are never left; the
 * caller keeps n_tokens within that capacity for meaningful results. One
 * token per step: at most one block completes per step. */

/* step_dev->n_cand_prev = (n_tokens - 1) / S; step_dev->n_tokens += 1. */
nosa_status nosa_step_advance(const nosa_shape *shape, nosa_step *step_dev, void *stream);

/* nosa_pool_blocks for the block completed since the previous step: when
 * n_cand_prev >= 0 and n_cand = (n_tokens - 1) / S exceeds it, pools block
 * n_cand_prev of kv (the full block-unit KV, kv_row_blocks >= max_blocks);
 * otherwise does nothing. e_row_stride >= max_blocks * S. */
nosa_status nosa_pool_step(const nosa_shape *shape, const void *kv, int64_t kv_row_blocks,
                           const float *e_tok, int64_t e_row_stride, const nosa_step *step_dev,
                           void *kbar, float *e_blk, void *stream);

/* nosa_append_tokens with pos = (n_tokens - 1) % S and block = (n_tokens - 1) / S
 * of the full KV (kv_row_blocks >= max_blocks). */
nosa_status nosa_append_step(const nosa_shape *shape, const void *k_new, const void *v_new,
                             void *kv, int64_t kv_row_blocks, const nosa_step *step_dev,
                             void *stream);

/* nosa_score_select with the step record in device memory. */
nosa_status nosa_score_select_step(const nosa_shape *shape, const void *q, const void *kbar,
                                   const float *e_blk, const nosa_step *step_dev, float *s_q,
                                   uint32_t *ge_bits, uint32_t *ev_bits, int32_t *sel,
                                   int32_t *n_sel, uint32_t *sel_bits, int32_t *slot_block,
                                   int32_t *block_slot, int32_t *fetch_block,
                                   int32_t *fetch_slot, int32_t *n_fetch, uint64_t *counters,
                                   void *stream);

/* nosa_decode_partial with the step record in device memory. With
 * NOSA_KV_FULL, cur_kv is the full KV (cur_row_blocks >= max_blocks) and the
 * newest block is its block n_cand; with NOSA_KV_CACHE, block 0 of cur_kv (the
 * newest-block buffer). Validated against the capacity: e_row_stride >=
 * max_blocks * S, and with NOSA_KV_FULL kv_row_blocks >= max_blocks. */
nosa_status nosa_decode_partial_step(const nosa_shape *shape, const void *q, const void *kv,
                                     int64_t kv_row_blocks, int32_t kv_mode, const int32_t *list,
                                     const int32_t *n_list, int32_t list_stride,
                                     int32_t list_len, int32_t with_newest, const void *cur_kv,
                                     int64_t cur_row_blocks, const nosa_step *step_dev,
                                     const float *e_tok, int64_t e_row_stride, void *ws,
                                     size_t ws_bytes, int32_t chunk0, void *stream);

/* Pinned host memory readable by GPU kernels: *host is the host address,
 * *dev the device alias to pass as a kernel source. coherent != 0 asks for
 * fine-grained (host-coherent) memory, the form the Python layer uses for
 * the host KV; coherent == 0 for coarse-grained memory. Free with
 * nosa_host_free. */
nosa_status nosa_host_alloc(size_t bytes, int32_t coherent, void **host, void **dev);
nosa_status nosa_host_free(void *host);

/* Measurement utility, not a step of the method: reads `bytes` (> 0, a
 * multiple of 16) of device memory at src (16-byte aligned) once with
 * `workgroups` workgroups of 256 threads, 16-byte loads, eight in flight per
 * thread; sink (one uint32, device memory) is written only on a magic value.
 * Timing it gives the achievable streaming-read bandwidth, the second
 * denominator for the HBM-bound kernels. */
nosa_status nosa_read_probe(const void *src, int64_t bytes, uint32_t *sink, int32_t workgroups,
                            void *stream);

const char *nosa_status_string(nosa_status s);
/* Text of the last HIP error seen by a call on this thread ("" if none). */
const char *nosa_last_error(void);
int32_t nosa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* NOSA_H */
