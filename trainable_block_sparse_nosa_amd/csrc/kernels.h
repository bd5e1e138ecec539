// Launchers of the NOSA gfx950 kernels (internal to the library).
#pragma once

#include "common.h"

namespace nosa {

template <typename T, int D>
hipError_t launch_pool(const Dims &dm, const void *kv, int64_t kv_row_blocks, int kv_first,
                       const float *e_tok, int64_t e_stride, int blk_begin, int blk_end,
                       float *kbar, float *e_blk, hipStream_t st);

template <typename T, int D, int G>
hipError_t launch_score(const Dims &dm, const void *q, const float *kbar, int n_cand, float *s_q,
                        hipStream_t st);

struct SwapPtrs {
    int32_t *slot_block, *block_slot, *fetch_block, *fetch_slot, *n_fetch;
    uint64_t *counters;
};

// swap == nullptr: selection only; else the set difference runs in the same launch
hipError_t launch_select(const Dims &dm, const float *s_q, const float *e_blk, int n_cand,
                         int n_prev, uint32_t *ge, uint32_t *ev, int32_t *sel, int32_t *n_sel,
                         uint32_t *sel_bits, const SwapPtrs *swap, hipStream_t st);

hipError_t launch_swap(const Dims &dm, const int32_t *sel, const int32_t *n_sel,
                       const uint32_t *sel_bits, const SwapPtrs &swap, hipStream_t st);

hipError_t launch_fetch(const Dims &dm, const void *src, int64_t src_row_blocks,
                        const int32_t *fblk, const int32_t *fslot, const int32_t *nfetch,
                        int max_fetch, void *dst, int64_t dst_row_blocks, hipStream_t st);

// Split-K plan of the decode: list entries 0..k-1 are the selected blocks and
// entry k is the newest block; a chunk of `cb` consecutive entries is one
// workgroup.
struct DecodePlan {
    int cb;        // entries per chunk
    int n_chunks;  // chunks per row
    int npw;       // MFMA kernel: blocks per wave (1, 2, 4 or 8)
};
int decode_kind(const Dims &dm, int requested);  // NOSA_DECODE_VALU or _MFMA
DecodePlan decode_plan(const Dims &dm, int kind);

struct DecodeArgs {
    const void *q;
    const void *kv;
    int64_t kv_row_blocks;
    int kv_mode;
    const int32_t *list;
    const int32_t *n_list;
    const void *cur;
    int64_t cur_row_blocks;
    int n_tokens, n_cand;
    const float *e_tok;
    int64_t e_stride;
    void *out;
    float *ws_o;   // [rows][n_chunks][G][D]
    float *ws_ml;  // [rows][n_chunks][G][2]
};

template <typename T, int D, int G>
hipError_t launch_decode_valu(const Dims &dm, const DecodePlan &pl, const DecodeArgs &a,
                              hipStream_t st);
template <int D, int G>
hipError_t launch_decode_mfma(const Dims &dm, const DecodePlan &pl, const DecodeArgs &a,
                              hipStream_t st);

}  // namespace nosa
