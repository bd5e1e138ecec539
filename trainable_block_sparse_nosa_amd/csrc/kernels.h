// Launchers of the NOSA gfx950 kernels (internal to the library).
#pragma once

#include "common.h"

namespace nosa {

// Template parameters: T is the KV dtype (q, K, V, out), TK the pooled dtype
// (kbar, and the pooled queries of a prefill): float32, or bfloat16 with
// bfloat16 KV.
template <typename T, typename TK, int D>
hipError_t launch_pool(const Dims &dm, const void *kv, int64_t kv_row_blocks, int kv_first,
                       const float *e_tok, int64_t e_stride, int blk_begin, int blk_end,
                       void *kbar, float *e_blk, hipStream_t st);
// Pool the block completed at the device step, if any (candidates went from
// n_cand_prev >= 0 to n_cand_prev + 1): block j of kv's rows (the full KV).
template <typename T, typename TK, int D>
hipError_t launch_pool_step(const Dims &dm, const void *kv, int64_t kv_row_blocks,
                            const float *e_tok, int64_t e_stride, const int32_t *dstep,
                            void *kbar, float *e_blk, hipStream_t st);
hipError_t launch_step_advance(const Dims &dm, int32_t *dstep, hipStream_t st);

// Block scores of candidates 0..n_cand-1 into s_q over a grid split along
// each row's candidates (dstep: n_cand from the device step record, the grid
// sized for the capacity): bfloat16 pooled keys on the matrix cores, float32
// pooled keys on the VALU.
template <typename T, typename TK, int D, int G>
hipError_t launch_score(const Dims &dm, const void *q, const void *kbar, int n_cand, float *s_q,
                        hipStream_t st, const int32_t *dstep = nullptr);

struct SwapPtrs {
    int32_t *slot_block, *block_slot, *fetch_block, *fetch_slot, *n_fetch;
    uint64_t *counters;
};

struct SelectLists {
    int32_t *ge_list, *n_ge, *gq_list, *n_gq;
};

// swap == nullptr: selection only; else the set difference runs in the same
// launch. parts != nullptr: also write Gamma_e and Gamma_q as ascending lists.
hipError_t launch_select(const Dims &dm, const float *s_q, const float *e_blk, int n_cand,
                         int n_prev, uint32_t *ge, uint32_t *ev, int32_t *sel, int32_t *n_sel,
                         uint32_t *sel_bits, const SwapPtrs *swap, const SelectLists *parts,
                         hipStream_t st);

// Scores and selection (and the set difference when swap != nullptr): with
// bf16 KV and at most SPLIT_SCORE_MAX_ROWS rows (CERT_SPLIT_MAX_ROWS with
// float32 pooled keys, certified scoring), the scores come from a grid
// split over each row's candidates into s_q and a second launch selects from
// them; otherwise the selecting workgroup (one per row) computes its row's
// scores itself, writing them to s_q as well. dstep != nullptr: n_cand and
// n_prev come from the device step record.
template <typename T, typename TK, int D, int G>
hipError_t launch_score_select(const Dims &dm, const void *q, const void *kbar, float *s_q,
                               const float *e_blk, int n_cand, int n_prev, uint32_t *ge,
                               uint32_t *ev, int32_t *sel, int32_t *n_sel, uint32_t *sel_bits,
                               const SwapPtrs *swap, hipStream_t st,
                               const int32_t *dstep = nullptr);

// Selection of every query block i < n_qb of a sequence (candidates 0..i-1,
// no previous step) in one launch: sel [n_qb][rows][k], n_sel [n_qb][rows].
template <typename T, typename TK, int D, int G>
hipError_t launch_prefill_select(const Dims &dm, const void *qbar, const void *kbar,
                                 const float *e_blk, int n_qb, int32_t *sel, int32_t *n_sel,
                                 hipStream_t st);

hipError_t launch_swap(const Dims &dm, const int32_t *sel, const int32_t *n_sel,
                       const uint32_t *sel_bits, const SwapPtrs &swap, hipStream_t st);

template <typename T, typename TK, int D, int G>
hipError_t launch_ingest(const Dims &dm, const void *qkv, const void *x, const void *w_e,
                         const float *b_e, int hidden, int tok, void *q_out, void *kv,
                         int64_t kv_row_blocks, int block, float *e_tok, int64_t e_stride,
                         void *kbar, float *e_blk, hipStream_t st);

// dstep != nullptr: pos and block come from the device step record (the
// newest token n_tokens - 1: slot (n_tokens - 1) % S of block (n_tokens - 1) / S).
template <typename T, int D>
hipError_t launch_append(const Dims &dm, const void *k_new, const void *v_new, int pos, void *kv,
                         int64_t kv_row_blocks, int block, hipStream_t st,
                         const int32_t *dstep = nullptr);

hipError_t launch_fetch(const Dims &dm, const void *src, int64_t src_row_blocks,
                        const int32_t *fblk, const int32_t *fslot, const int32_t *nfetch,
                        int max_fetch, void *dst, int64_t dst_row_blocks, hipStream_t st);

// Split-K plan of one partial-attention call: its entries are list entries
// 0..list_len-1 plus (optionally) the newest block as entry list_len; a
// chunk of `cb` consecutive entries is one workgroup (the MFMA kernel's last
// chunk runs to the end, newest block included).
struct DecodePlan {
    int cb;        // entries per chunk
    int n_chunks;  // chunks of this call
};
int decode_kind(const Dims &dm, int requested);  // NOSA_DECODE_VALU or _MFMA
DecodePlan decode_plan(const Dims &dm, int kind, int list_len, int with_newest);
// Workspace rows hold this many chunk partials: enough for the whole
// selection plus the newest block in one call, or split over two calls.
inline int decode_chunk_cap(const Dims &dm) { return dm.k + 2; }

struct DecodeArgs {
    const void *q;
    const void *kv;
    int64_t kv_row_blocks;
    int kv_mode;
    const int32_t *list;
    const int32_t *n_list;  // per-row entry counts (NOSA_KV_FULL), else null
    int list_stride;        // list row stride
    int list_len;           // list entries per row
    int with_newest;        // 1: entry list_len is the newest block
    const void *cur;
    int64_t cur_row_blocks;
    int n_tokens, n_cand;
    const float *e_tok;
    int64_t e_stride;
    float *ws_o;   // [rows][chunk_cap][G][D]
    float *ws_ml;  // [rows][chunk_cap][G][2]
    int chunk0;    // first workspace chunk of this call
    int chunk_cap;
    int cb;        // entries per chunk (from the plan)
    const int32_t *dstep = nullptr;  // device step record: overrides n_tokens / n_cand
    int cur_at_step = 0;             // 1: the newest block is block n_cand of cur's rows
    // MFMA kernel with one chunk per row: with out set, each workgroup
    // normalizes its row's output and writes it, leaving no partials
    void *out = nullptr;
};

template <typename T, int D, int G>
hipError_t launch_decode_valu(const Dims &dm, const DecodePlan &pl, const DecodeArgs &a,
                              hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
template <int D, int G>
hipError_t launch_decode_mfma(const Dims &dm, const DecodePlan &pl, const DecodeArgs &a,
                              hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
// qbar in the pooled dtype TK.
template <typename T, typename TK, int D>
hipError_t launch_pool_queries(const Dims &dm, const void *q, int n_tokens, void *qbar,
                               hipStream_t st);
template <int D, int G>
hipError_t launch_prefill(const Dims &dm, const void *q, int n_tokens, const void *kv,
                          int64_t kv_row_blocks, const float *e_tok, int64_t e_stride,
                          const int32_t *sel, const int32_t *n_sel, void *out, hipStream_t st);
template <typename T, int D, int G>
// dstep_adv != nullptr: the device step record is advanced at the end.
hipError_t launch_combine(const Dims &dm, int n_chunks, int chunk_cap, const float *ws_o,
                          const float *ws_ml, void *out, hipStream_t st,
                          int32_t *dstep_adv = nullptr);

// Streaming read of `bytes` (a multiple of 16) from src by `wgs` workgroups.
hipError_t launch_read_probe(const void *src, int64_t bytes, uint32_t *sink, int wgs,
                             hipStream_t st);

}  // namespace nosa
