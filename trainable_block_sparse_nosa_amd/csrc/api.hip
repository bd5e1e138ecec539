// C ABI of the NOSA decode path: argument validation, dispatch, launches.
#include <math.h>

#include <string>
#include <type_traits>

#include <mutex>

#include "kernels.h"

using namespace nosa;

// Scratch of nosa_sparse_decode_noalloc: split-K partials for callers that
// cannot allocate. Each GPU the library runs on holds its own copy, for the
// life of the process. In host code `noalloc_scratch` is a host-side stand-in
// for the symbol, not a device address: kernels get the per-device address
// that hipGetSymbolAddress returns, never the name.
static __device__ __align__(256) unsigned char noalloc_scratch[NOSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];  // device address of noalloc_scratch, per device

// The current device's scratch address, taken on the first call there.
hipError_t noalloc_scratch_ptr(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

thread_local std::string g_last_error;

nosa_status hip_status(hipError_t e) {
    if (e == hipSuccess) return NOSA_OK;
    g_last_error = hipGetErrorString(e);
    return NOSA_ERR_HIP;
}

nosa_status make_dims(const nosa_shape *s, Dims *dm) {
    if (!s) return NOSA_ERR_INVALID_ARGUMENT;
    if (s->batch <= 0 || s->n_q_heads <= 0 || s->n_kv_heads <= 0 || s->head_dim <= 0 ||
        s->block_size <= 0 || s->sub_block <= 0 || s->k_e < 0 || s->k_q < 0 ||
        s->max_blocks <= 0)
        return NOSA_ERR_INVALID_ARGUMENT;
    if (s->n_q_heads % s->n_kv_heads) return NOSA_ERR_INVALID_ARGUMENT;
    if (s->block_size % s->sub_block) return NOSA_ERR_INVALID_ARGUMENT;
    if (s->k_e + s->k_q <= 0) return NOSA_ERR_INVALID_ARGUMENT;
    if (s->dtype != NOSA_F32 && s->dtype != NOSA_BF16) return NOSA_ERR_INVALID_ARGUMENT;
    if (s->decode_kernel < NOSA_DECODE_AUTO || s->decode_kernel > NOSA_DECODE_MFMA)
        return NOSA_ERR_INVALID_ARGUMENT;
    if (!(s->scale >= 0.f) || isinf(s->scale)) return NOSA_ERR_INVALID_ARGUMENT;
    if (s->pooled_dtype != NOSA_F32 && s->pooled_dtype != NOSA_BF16)
        return NOSA_ERR_INVALID_ARGUMENT;
    if (s->pooled_dtype == NOSA_BF16 && s->dtype != NOSA_BF16) return NOSA_ERR_UNSUPPORTED;
    const int G = s->n_q_heads / s->n_kv_heads;
    if (s->block_size != 64 || s->sub_block != 16) return NOSA_ERR_UNSUPPORTED;
    if (s->head_dim != 64 && s->head_dim != 128) return NOSA_ERR_UNSUPPORTED;
    if (s->dtype == NOSA_F32 && s->head_dim != 64) return NOSA_ERR_UNSUPPORTED;
    if (G > 8 || s->k_e + s->k_q > 128 || s->max_blocks > 4096) return NOSA_ERR_UNSUPPORTED;
    if ((int64_t)s->batch * s->n_kv_heads > 65535) return NOSA_ERR_UNSUPPORTED;
    dm->B = s->batch;
    dm->Hq = s->n_q_heads;
    dm->Hkv = s->n_kv_heads;
    dm->G = G;
    dm->D = s->head_dim;
    dm->S = s->block_size;
    dm->sub = s->sub_block;
    dm->m = s->block_size / s->sub_block;
    dm->k_e = s->k_e;
    dm->k_q = s->k_q;
    dm->k = s->k_e + s->k_q;
    dm->max_blocks = s->max_blocks;
    dm->W = (s->max_blocks + 31) / 32;
    dm->rows = s->batch * s->n_kv_heads;
    dm->dtype = s->dtype;
    dm->pdtype = s->pooled_dtype;
    dm->scale = s->scale > 0.f ? s->scale : 1.0f / sqrtf((float)s->head_dim);
    return NOSA_OK;
}

// Step fields checked against the shape: returns n_cand or -1.
int step_cand(const Dims &dm, const nosa_step *st) {
    if (!st || st->n_tokens <= 0) return -1;
    const int n_cand = (st->n_tokens - 1) / dm.S;
    if (n_cand >= dm.max_blocks) return -1;
    if (st->n_cand_prev > n_cand) return -1;
    return n_cand;
}

template <typename F> nosa_status by_type_dim(const Dims &dm, F &&f) {
    if (dm.dtype == NOSA_F32)
        return f((float *)nullptr, std::integral_constant<int, 64>{});
    if (dm.D == 64) return f((bf16_t *)nullptr, std::integral_constant<int, 64>{});
    return f((bf16_t *)nullptr, std::integral_constant<int, 128>{});
}

// f(T *, TK *, D): KV dtype, pooled dtype (kbar, qbar) and head dim.
template <typename F> nosa_status by_types(const Dims &dm, F &&f) {
    return by_type_dim(dm, [&](auto tp, auto dc) -> nosa_status {
        using T = std::remove_pointer_t<decltype(tp)>;
        if constexpr (std::is_same_v<T, bf16_t>) {
            if (dm.pdtype == NOSA_BF16) return f(tp, (bf16_t *)nullptr, dc);
        }
        return f(tp, (float *)nullptr, dc);
    });
}

template <typename F> nosa_status by_group(const Dims &dm, F &&f) {
    switch (dm.G) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 3: return f(std::integral_constant<int, 3>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 5: return f(std::integral_constant<int, 5>{});
    case 6: return f(std::integral_constant<int, 6>{});
    case 7: return f(std::integral_constant<int, 7>{});
    case 8: return f(std::integral_constant<int, 8>{});
    default: return NOSA_ERR_UNSUPPORTED;
    }
}

// Workspace: partial outputs [rows][chunk_cap][G][D], then partial (max, sum)
// [rows][chunk_cap][G][2], float32.
size_t decode_ws_bytes(const Dims &dm) {
    const size_t parts = (size_t)dm.rows * decode_chunk_cap(dm) * dm.G;
    return parts * dm.D * sizeof(float) + parts * 2 * sizeof(float);
}

// Validation shared by the attention entry points; fills everything in `a`
// except the list description and the chunk placement.
nosa_status decode_common(const Dims &dm, int kind, const void *q, const void *kv,
                          int64_t kv_row_blocks, int32_t kv_mode, const void *cur_kv,
                          int64_t cur_row_blocks, const nosa_step *step, const float *e_tok,
                          int64_t e_row_stride, void *ws, size_t ws_bytes, DecodeArgs &a) {
    if (!q || !cur_kv || !e_tok || !ws) return NOSA_ERR_INVALID_ARGUMENT;
    if (kv_mode != NOSA_KV_FULL && kv_mode != NOSA_KV_CACHE) return NOSA_ERR_INVALID_ARGUMENT;
    if (kind == NOSA_DECODE_MFMA && dm.dtype != NOSA_BF16) return NOSA_ERR_UNSUPPORTED;
    if (kv_row_blocks <= 0 || cur_row_blocks <= 0) return NOSA_ERR_INVALID_ARGUMENT;
    const int n_cand = step_cand(dm, step);
    if (n_cand < 0) return NOSA_ERR_INVALID_ARGUMENT;
    // eviction-score rows cover whole blocks and are 16-byte aligned
    if (e_row_stride < (int64_t)(n_cand + 1) * dm.S || (e_row_stride & 3) ||
        ((uintptr_t)e_tok & 15u))
        return NOSA_ERR_INVALID_ARGUMENT;
    if (kv_mode == NOSA_KV_FULL && kv && kv_row_blocks < n_cand + 1) return NOSA_ERR_INVALID_ARGUMENT;
    if (ws_bytes < decode_ws_bytes(dm)) return NOSA_ERR_WORKSPACE;
    if (((uintptr_t)q | (uintptr_t)kv | (uintptr_t)cur_kv | (uintptr_t)ws) & 15u)
        return NOSA_ERR_INVALID_ARGUMENT;
    a = DecodeArgs{};
    a.q = q;
    a.kv = kv;
    a.kv_row_blocks = kv_row_blocks;
    a.kv_mode = kv_mode;
    a.cur = cur_kv;
    a.cur_row_blocks = cur_row_blocks;
    a.n_tokens = step->n_tokens;
    a.n_cand = n_cand;
    a.e_tok = e_tok;
    a.e_stride = e_row_stride;
    a.chunk_cap = decode_chunk_cap(dm);
    a.ws_o = static_cast<float *>(ws);
    a.ws_ml = a.ws_o + (size_t)dm.rows * a.chunk_cap * dm.G * dm.D;
    return NOSA_OK;
}

nosa_status launch_partial(const Dims &dm, int kind, const DecodePlan &pl, const DecodeArgs &a,
                           hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr) {
    return by_type_dim(dm, [&](auto tp, auto dc) -> nosa_status {
        using T = std::remove_pointer_t<decltype(tp)>;
        constexpr int D = decltype(dc)::value;
        return by_group(dm, [&](auto gc) -> nosa_status {
            constexpr int G = decltype(gc)::value;
            if constexpr (std::is_same<T, bf16_t>::value) {
                if (kind == NOSA_DECODE_MFMA)
                    return hip_status(launch_decode_mfma<D, G>(dm, pl, a, st, ev0, ev1));
            }
            return hip_status(launch_decode_valu<T, D, G>(dm, pl, a, st, ev0, ev1));
        });
    });
}

nosa_status launch_merge(const Dims &dm, int n_chunks, const DecodeArgs &a, void *out,
                         hipStream_t st, int32_t *dstep_adv = nullptr) {
    return by_type_dim(dm, [&](auto tp, auto dc) -> nosa_status {
        using T = std::remove_pointer_t<decltype(tp)>;
        constexpr int D = decltype(dc)::value;
        return by_group(dm, [&](auto gc) -> nosa_status {
            constexpr int G = decltype(gc)::value;
            return hip_status(
                launch_combine<T, D, G>(dm, n_chunks, a.chunk_cap, a.ws_o, a.ws_ml, out, st,
                                        dstep_adv));
        });
    });
}

}  // namespace

extern "C" {

nosa_status nosa_pool_blocks(const nosa_shape *shape, const void *kv, int64_t kv_row_blocks,
                             int32_t kv_first_block, const float *e_tok, int64_t e_row_stride,
                             int32_t blk_begin, int32_t blk_end, void *kbar, float *e_blk,
                             void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!kv || !e_tok || !kbar || !e_blk) return NOSA_ERR_INVALID_ARGUMENT;
    if (blk_begin < 0 || blk_end < blk_begin || blk_end > dm.max_blocks || kv_first_block < 0 ||
        kv_row_blocks < kv_first_block + (blk_end - blk_begin) ||
        e_row_stride < (int64_t)blk_end * dm.S)
        return NOSA_ERR_INVALID_ARGUMENT;
    if (blk_end == blk_begin) return NOSA_OK;
    return by_types(dm, [&](auto tp, auto tk, auto dc) -> nosa_status {
        using T = std::remove_pointer_t<decltype(tp)>;
        using TK = std::remove_pointer_t<decltype(tk)>;
        return hip_status(launch_pool<T, TK, decltype(dc)::value>(
            dm, kv, kv_row_blocks, kv_first_block, e_tok, e_row_stride, blk_begin, blk_end, kbar,
            e_blk, (hipStream_t)stream));
    });
}

nosa_status nosa_score_blocks(const nosa_shape *shape, const void *q, const void *kbar,
                              const nosa_step *step, float *s_q, void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!q || !kbar || !s_q) return NOSA_ERR_INVALID_ARGUMENT;
    const int n_cand = step_cand(dm, step);
    if (n_cand < 0) return NOSA_ERR_INVALID_ARGUMENT;
    if (n_cand == 0) return NOSA_OK;
    return by_types(dm, [&](auto tp, auto tk, auto dc) -> nosa_status {
        using T = std::remove_pointer_t<decltype(tp)>;
        using TK = std::remove_pointer_t<decltype(tk)>;
        constexpr int D = decltype(dc)::value;
        return by_group(dm, [&](auto gc) -> nosa_status {
            return hip_status(launch_score<T, TK, D, decltype(gc)::value>(
                dm, q, kbar, n_cand, s_q, (hipStream_t)stream));
        });
    });
}

nosa_status nosa_select(const nosa_shape *shape, const float *s_q, const float *e_blk,
                        const nosa_step *step, uint32_t *ge_bits, uint32_t *ev_bits, int32_t *sel,
                        int32_t *n_sel, uint32_t *sel_bits, void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!s_q || !e_blk || !ge_bits || !ev_bits || !sel || !n_sel || !sel_bits)
        return NOSA_ERR_INVALID_ARGUMENT;
    const int n_cand = step_cand(dm, step);
    if (n_cand < 0) return NOSA_ERR_INVALID_ARGUMENT;
    return hip_status(launch_select(dm, s_q, e_blk, n_cand, step->n_cand_prev, ge_bits, ev_bits,
                                    sel, n_sel, sel_bits, nullptr, nullptr, (hipStream_t)stream));
}

nosa_status nosa_select_swap(const nosa_shape *shape, const float *s_q, const float *e_blk,
                             const nosa_step *step, uint32_t *ge_bits, uint32_t *ev_bits,
                             int32_t *sel, int32_t *n_sel, uint32_t *sel_bits,
                             int32_t *slot_block, int32_t *block_slot, int32_t *fetch_block,
                             int32_t *fetch_slot, int32_t *n_fetch, uint64_t *counters,
                             void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!s_q || !e_blk || !ge_bits || !ev_bits || !sel || !n_sel || !sel_bits || !slot_block ||
        !block_slot || !fetch_block || !fetch_slot || !n_fetch || !counters)
        return NOSA_ERR_INVALID_ARGUMENT;
    const int n_cand = step_cand(dm, step);
    if (n_cand < 0) return NOSA_ERR_INVALID_ARGUMENT;
    const SwapPtrs sw{slot_block, block_slot, fetch_block, fetch_slot, n_fetch, counters};
    return hip_status(launch_select(dm, s_q, e_blk, n_cand, step->n_cand_prev, ge_bits, ev_bits,
                                    sel, n_sel, sel_bits, &sw, nullptr, (hipStream_t)stream));
}

nosa_status nosa_select_parts(const nosa_shape *shape, const float *s_q, const float *e_blk,
                              const nosa_step *step, uint32_t *ge_bits, uint32_t *ev_bits,
                              int32_t *sel, int32_t *n_sel, uint32_t *sel_bits, int32_t *ge_list,
                              int32_t *n_ge, int32_t *gq_list, int32_t *n_gq,
                              int32_t *slot_block, int32_t *block_slot, int32_t *fetch_block,
                              int32_t *fetch_slot, int32_t *n_fetch, uint64_t *counters,
                              void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!s_q || !e_blk || !ge_bits || !ev_bits || !sel || !n_sel || !sel_bits || !n_ge ||
        !n_gq || (dm.k_e > 0 && !ge_list) || (dm.k_q > 0 && !gq_list))
        return NOSA_ERR_INVALID_ARGUMENT;
    const bool any_swap = slot_block || block_slot || fetch_block || fetch_slot || n_fetch || counters;
    const bool all_swap = slot_block && block_slot && fetch_block && fetch_slot && n_fetch && counters;
    if (any_swap && !all_swap) return NOSA_ERR_INVALID_ARGUMENT;
    const int n_cand = step_cand(dm, step);
    if (n_cand < 0) return NOSA_ERR_INVALID_ARGUMENT;
    const SelectLists parts{ge_list, n_ge, gq_list, n_gq};
    const SwapPtrs sw{slot_block, block_slot, fetch_block, fetch_slot, n_fetch, counters};
    return hip_status(launch_select(dm, s_q, e_blk, n_cand, step->n_cand_prev, ge_bits, ev_bits,
                                    sel, n_sel, sel_bits, all_swap ? &sw : nullptr, &parts,
                                    (hipStream_t)stream));
}

nosa_status nosa_score_select(const nosa_shape *shape, const void *q, const void *kbar,
                              const float *e_blk, const nosa_step *step, float *s_q,
                              uint32_t *ge_bits, uint32_t *ev_bits, int32_t *sel, int32_t *n_sel,
                              uint32_t *sel_bits, int32_t *slot_block, int32_t *block_slot,
                              int32_t *fetch_block, int32_t *fetch_slot, int32_t *n_fetch,
                              uint64_t *counters, void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!q || !kbar || !s_q || !e_blk || !ge_bits || !ev_bits || !sel || !n_sel || !sel_bits)
        return NOSA_ERR_INVALID_ARGUMENT;
    const bool any_swap = slot_block || block_slot || fetch_block || fetch_slot || n_fetch || counters;
    const bool all_swap = slot_block && block_slot && fetch_block && fetch_slot && n_fetch && counters;
    if (any_swap && !all_swap) return NOSA_ERR_INVALID_ARGUMENT;
    const int n_cand = step_cand(dm, step);
    if (n_cand < 0) return NOSA_ERR_INVALID_ARGUMENT;
    const SwapPtrs sw{slot_block, block_slot, fetch_block, fetch_slot, n_fetch, counters};
    return by_types(dm, [&](auto tp, auto tk, auto dc) -> nosa_status {
        using T = std::remove_pointer_t<decltype(tp)>;
        using TK = std::remove_pointer_t<decltype(tk)>;
        constexpr int D = decltype(dc)::value;
        return by_group(dm, [&](auto gc) -> nosa_status {
            return hip_status(launch_score_select<T, TK, D, decltype(gc)::value>(
                dm, q, kbar, s_q, e_blk, n_cand, step->n_cand_prev, ge_bits, ev_bits, sel, n_sel,
                sel_bits, all_swap ? &sw : nullptr, (hipStream_t)stream));
        });
    });
}

nosa_status nosa_swap_diff(const nosa_shape *shape, const int32_t *sel, const int32_t *n_sel,
                           const uint32_t *sel_bits, int32_t *slot_block, int32_t *block_slot,
                           int32_t *fetch_block, int32_t *fetch_slot, int32_t *n_fetch,
                           uint64_t *counters, void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!sel || !n_sel || !sel_bits || !slot_block || !block_slot || !fetch_block ||
        !fetch_slot || !n_fetch || !counters)
        return NOSA_ERR_INVALID_ARGUMENT;
    const SwapPtrs sw{slot_block, block_slot, fetch_block, fetch_slot, n_fetch, counters};
    return hip_status(launch_swap(dm, sel, n_sel, sel_bits, sw, (hipStream_t)stream));
}

nosa_status nosa_fetch_blocks(const nosa_shape *shape, const void *src_kv, int64_t src_row_blocks,
                              const int32_t *fetch_block, const int32_t *fetch_slot,
                              const int32_t *n_fetch, int32_t max_fetch, void *dst_kv,
                              int64_t dst_row_blocks, void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!src_kv || !fetch_block || !fetch_slot || !n_fetch || !dst_kv)
        return NOSA_ERR_INVALID_ARGUMENT;
    if (max_fetch < 0 || max_fetch > dm.k || src_row_blocks <= 0 || dst_row_blocks <= 0)
        return NOSA_ERR_INVALID_ARGUMENT;
    if (max_fetch == 0) return NOSA_OK;
    return hip_status(launch_fetch(dm, src_kv, src_row_blocks, fetch_block, fetch_slot, n_fetch,
                                   max_fetch, dst_kv, dst_row_blocks, (hipStream_t)stream));
}

nosa_status nosa_ingest_tokens(const nosa_shape *shape, const void *qkv, const void *x,
                               const void *w_evict, const float *b_evict, int32_t hidden,
                               int32_t n_tokens, void *q_out, void *kv, int64_t kv_row_blocks,
                               int32_t block, float *e_tok, int64_t e_row_stride, void *kbar,
                               float *e_blk, void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!qkv || !x || !w_evict || !q_out || !kv || !e_tok || !kbar || !e_blk)
        return NOSA_ERR_INVALID_ARGUMENT;
    const int tok = n_tokens - 1;
    if (((reinterpret_cast<uintptr_t>(qkv) | reinterpret_cast<uintptr_t>(q_out)) & 15) != 0)
        return NOSA_ERR_INVALID_ARGUMENT;
    if (hidden <= 0 || n_tokens <= 0 || kv_row_blocks <= 0 || block < 0 ||
        block >= kv_row_blocks || e_row_stride < n_tokens || tok / dm.S >= dm.max_blocks)
        return NOSA_ERR_INVALID_ARGUMENT;
    return by_types(dm, [&](auto tp, auto tk, auto dc) -> nosa_status {
        using T = std::remove_pointer_t<decltype(tp)>;
        using TK = std::remove_pointer_t<decltype(tk)>;
        constexpr int D = decltype(dc)::value;
        return by_group(dm, [&](auto gc) -> nosa_status {
            return hip_status(launch_ingest<T, TK, D, decltype(gc)::value>(
                dm, qkv, x, w_evict, b_evict, hidden, tok, q_out, kv, kv_row_blocks, block, e_tok,
                e_row_stride, kbar, e_blk, (hipStream_t)stream));
        });
    });
}

nosa_status nosa_prefill_pool_queries(const nosa_shape *shape, const void *q, int32_t n_tokens,
                                      void *qbar, void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!q || !qbar || n_tokens <= 0) return NOSA_ERR_INVALID_ARGUMENT;
    // the kernel reads and writes 16-byte vectors
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(qbar)) & 15)
        return NOSA_ERR_INVALID_ARGUMENT;
    return by_types(dm, [&](auto tp, auto tk, auto dc) -> nosa_status {
        using T = std::remove_pointer_t<decltype(tp)>;
        using TK = std::remove_pointer_t<decltype(tk)>;
        constexpr int D = decltype(dc)::value;
        return hip_status(
            launch_pool_queries<T, TK, D>(dm, q, n_tokens, qbar, (hipStream_t)stream));
    });
}

nosa_status nosa_prefill_select(const nosa_shape *shape, const void *qbar, const void *kbar,
                                const float *e_blk, int32_t n_tokens, int32_t *sel,
                                int32_t *n_sel, void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!qbar || !kbar || !e_blk || !sel || !n_sel || n_tokens <= 0)
        return NOSA_ERR_INVALID_ARGUMENT;
    const int nqb = (n_tokens + dm.S - 1) / dm.S;
    if (nqb - 1 >= dm.max_blocks || nqb > 65535) return NOSA_ERR_INVALID_ARGUMENT;
    return by_types(dm, [&](auto tp, auto tk, auto dc) -> nosa_status {
        using T = std::remove_pointer_t<decltype(tp)>;
        using TK = std::remove_pointer_t<decltype(tk)>;
        constexpr int D = decltype(dc)::value;
        return by_group(dm, [&](auto gc) -> nosa_status {
            return hip_status(launch_prefill_select<T, TK, D, decltype(gc)::value>(
                dm, qbar, kbar, e_blk, nqb, sel, n_sel, (hipStream_t)stream));
        });
    });
}

nosa_status nosa_prefill_attention(const nosa_shape *shape, const void *q, int32_t n_tokens,
                                   const void *kv, int64_t kv_row_blocks, const float *e_tok,
                                   int64_t e_row_stride, const int32_t *sel, const int32_t *n_sel,
                                   void *out, void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!q || !kv || !e_tok || !sel || !n_sel || !out || n_tokens <= 0)
        return NOSA_ERR_INVALID_ARGUMENT;
    if (dm.dtype != NOSA_BF16) return NOSA_ERR_UNSUPPORTED;
    const int nqb = (n_tokens + dm.S - 1) / dm.S;
    if (kv_row_blocks < nqb || e_row_stride < (int64_t)nqb * dm.S) return NOSA_ERR_INVALID_ARGUMENT;
    if (((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kv) |
          reinterpret_cast<uintptr_t>(e_tok)) & 15) != 0 || (e_row_stride & 3) != 0)
        return NOSA_ERR_INVALID_ARGUMENT;
    return by_type_dim(dm, [&](auto, auto dc) -> nosa_status {
        constexpr int D = decltype(dc)::value;
        return by_group(dm, [&](auto gc) -> nosa_status {
            return hip_status(launch_prefill<D, decltype(gc)::value>(
                dm, q, n_tokens, kv, kv_row_blocks, e_tok, e_row_stride, sel, n_sel, out,
                (hipStream_t)stream));
        });
    });
}

nosa_status nosa_append_tokens(const nosa_shape *shape, const void *k_new, const void *v_new,
                               int32_t pos, void *kv, int64_t kv_row_blocks, int32_t block,
                               void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!k_new || !v_new || !kv) return NOSA_ERR_INVALID_ARGUMENT;
    if (pos < 0 || pos >= dm.S || kv_row_blocks <= 0 || block < 0 || block >= kv_row_blocks)
        return NOSA_ERR_INVALID_ARGUMENT;
    return by_type_dim(dm, [&](auto tp, auto dc) -> nosa_status {
        using T = std::remove_pointer_t<decltype(tp)>;
        constexpr int D = decltype(dc)::value;
        return hip_status(launch_append<T, D>(dm, k_new, v_new, pos, kv, kv_row_blocks, block,
                                              (hipStream_t)stream));
    });
}

size_t nosa_kbar_bytes(const nosa_shape *shape) {
    Dims dm;
    if (make_dims(shape, &dm) != NOSA_OK) return 0;
    return (size_t)kbar_bytes(dm);
}

nosa_status nosa_block_offsets(const nosa_shape *shape, int64_t *k_off, int64_t *v_off) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!k_off || !v_off) return NOSA_ERR_INVALID_ARGUMENT;
    return by_type_dim(dm, [&](auto tp, auto dc) -> nosa_status {
        using T = std::remove_pointer_t<decltype(tp)>;
        constexpr int D = decltype(dc)::value;
        for (int t = 0; t < 64; ++t)
            for (int d = 0; d < D; ++d) {
                k_off[t * D + d] = kv_k_off<T, D>(t, d);
                v_off[t * D + d] = kv_v_off<T, D>(t, d);
            }
        return NOSA_OK;
    });
}

size_t nosa_decode_workspace_size(const nosa_shape *shape) {
    Dims dm;
    if (make_dims(shape, &dm) != NOSA_OK) return 0;
    return decode_ws_bytes(dm);
}

int32_t nosa_decode_chunks(const nosa_shape *shape, int32_t list_len, int32_t with_newest) {
    Dims dm;
    if (make_dims(shape, &dm) != NOSA_OK || list_len < 0 || list_len > dm.k ||
        (with_newest != 0 && with_newest != 1))
        return -1;
    return decode_plan(dm, decode_kind(dm, shape->decode_kernel), list_len, with_newest).n_chunks;
}

nosa_status nosa_sparse_decode(const nosa_shape *shape, const void *q, const void *kv,
                               int64_t kv_row_blocks, int32_t kv_mode, const int32_t *list,
                               const int32_t *n_list, const void *cur_kv, int64_t cur_row_blocks,
                               const nosa_step *step, const float *e_tok, int64_t e_row_stride,
                               void *out, void *ws, size_t ws_bytes, void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!out || !kv || !list || (kv_mode == NOSA_KV_FULL && !n_list))
        return NOSA_ERR_INVALID_ARGUMENT;
    if (kv_mode == NOSA_KV_CACHE && kv_row_blocks < dm.k) return NOSA_ERR_INVALID_ARGUMENT;
    const int kind = decode_kind(dm, shape->decode_kernel);
    DecodeArgs a;
    s = decode_common(dm, kind, q, kv, kv_row_blocks, kv_mode, cur_kv, cur_row_blocks, step, e_tok,
                      e_row_stride, ws, ws_bytes, a);
    if (s != NOSA_OK) return s;
    a.list = list;
    a.n_list = kv_mode == NOSA_KV_FULL ? n_list : nullptr;
    a.list_stride = dm.k;
    a.list_len = dm.k;
    a.with_newest = 1;
    a.chunk0 = 0;
    const DecodePlan pl = decode_plan(dm, kind, dm.k, 1);
    a.cb = pl.cb;
    const hipStream_t st = (hipStream_t)stream;
    if (kind == NOSA_DECODE_MFMA && pl.n_chunks == 1) {
        a.out = out;  // one chunk per row: the attention launch writes the output
        return launch_partial(dm, kind, pl, a, st);
    }
    s = launch_partial(dm, kind, pl, a, st);
    if (s != NOSA_OK) return s;
    return launch_merge(dm, pl.n_chunks, a, out, st);
}

nosa_status nosa_sparse_decode_noalloc(const nosa_shape *shape, const void *q, const void *kv,
                                       int64_t kv_row_blocks, int32_t kv_mode,
                                       const int32_t *list, const int32_t *n_list,
                                       const void *cur_kv, int64_t cur_row_blocks,
                                       const nosa_step *step, const float *e_tok,
                                       int64_t e_row_stride, void *out, void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!out || !kv || !list || (kv_mode == NOSA_KV_FULL && !n_list))
        return NOSA_ERR_INVALID_ARGUMENT;
    if (kv_mode == NOSA_KV_CACHE && kv_row_blocks < dm.k) return NOSA_ERR_INVALID_ARGUMENT;
    const int kind = decode_kind(dm, shape->decode_kernel);
    const DecodePlan pl = decode_plan(dm, kind, dm.k, 1);
    const bool direct = kind == NOSA_DECODE_MFMA && pl.n_chunks == 1;
    // partials packed at this call's chunk count: [rows][chunks][G][D], then
    // [rows][chunks][G][2]
    const size_t parts = direct ? 0 : (size_t)dm.rows * pl.n_chunks * dm.G;
    const size_t need = parts * dm.D * sizeof(float) + parts * 2 * sizeof(float);
    if (need > NOSA_NOALLOC_SCRATCH_BYTES) return NOSA_ERR_WORKSPACE;
    void *scratch = nullptr;
    s = hip_status(noalloc_scratch_ptr(&scratch));
    if (s != NOSA_OK) return s;
    DecodeArgs a;
    // validation as nosa_sparse_decode's (the scratch stands for ws)
    s = decode_common(dm, kind, q, kv, kv_row_blocks, kv_mode, cur_kv, cur_row_blocks, step, e_tok,
                      e_row_stride, scratch, decode_ws_bytes(dm), a);
    if (s != NOSA_OK) return s;
    a.chunk_cap = direct ? 1 : pl.n_chunks;
    a.ws_o = static_cast<float *>(scratch);
    a.ws_ml = a.ws_o + parts * dm.D;
    a.list = list;
    a.n_list = kv_mode == NOSA_KV_FULL ? n_list : nullptr;
    a.list_stride = dm.k;
    a.list_len = dm.k;
    a.with_newest = 1;
    a.chunk0 = 0;
    a.cb = pl.cb;
    const hipStream_t st = (hipStream_t)stream;
    if (direct) {
        a.out = out;  // one chunk per row: the attention launch writes the output
        return launch_partial(dm, kind, pl, a, st);
    }
    s = launch_partial(dm, kind, pl, a, st);
    if (s != NOSA_OK) return s;
    return launch_merge(dm, pl.n_chunks, a, out, st);
}

static nosa_status decode_partial_impl(const nosa_shape *shape, const void *q, const void *kv,
                                       int64_t kv_row_blocks, int32_t kv_mode,
                                       const int32_t *list, const int32_t *n_list,
                                       int32_t list_stride, int32_t list_len, int32_t with_newest,
                                       const void *cur_kv, int64_t cur_row_blocks,
                                       const nosa_step *step, const float *e_tok,
                                       int64_t e_row_stride, void *ws, size_t ws_bytes,
                                       int32_t chunk0, hipEvent_t ev0, hipEvent_t ev1,
                                       void *stream, void *out = nullptr) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (list_len < 0 || list_len > dm.k || (with_newest != 0 && with_newest != 1))
        return NOSA_ERR_INVALID_ARGUMENT;
    if (list_len > 0 && (!kv || !list || list_stride < list_len ||
                         (kv_mode == NOSA_KV_FULL && !n_list)))
        return NOSA_ERR_INVALID_ARGUMENT;
    if (kv_mode == NOSA_KV_CACHE && list_len > 0 && kv_row_blocks < list_len)
        return NOSA_ERR_INVALID_ARGUMENT;
    const int kind = decode_kind(dm, shape->decode_kernel);
    DecodeArgs a;
    s = decode_common(dm, kind, q, kv ? kv : cur_kv, kv ? kv_row_blocks : cur_row_blocks,
                      kv_mode, cur_kv, cur_row_blocks, step, e_tok, e_row_stride, ws, ws_bytes, a);
    if (s != NOSA_OK) return s;
    const DecodePlan pl = decode_plan(dm, kind, list_len, with_newest);
    if (chunk0 < 0 || chunk0 + pl.n_chunks > a.chunk_cap) return NOSA_ERR_INVALID_ARGUMENT;
    a.list = list;
    a.n_list = kv_mode == NOSA_KV_FULL ? n_list : nullptr;
    a.list_stride = list_stride;
    a.list_len = list_len;
    a.with_newest = with_newest;
    a.chunk0 = chunk0;
    a.cb = pl.cb;
    if (!out) return launch_partial(dm, kind, pl, a, (hipStream_t)stream, ev0, ev1);
    // with the output: one launch when the MFMA kernel serves each row with a
    // single chunk, else the partials and then the merge kernel
    if (kind == NOSA_DECODE_MFMA && pl.n_chunks == 1) {
        a.out = out;
        return launch_partial(dm, kind, pl, a, (hipStream_t)stream, ev0, ev1);
    }
    s = launch_partial(dm, kind, pl, a, (hipStream_t)stream, ev0, ev1);
    if (s != NOSA_OK || pl.n_chunks == 0) return s;
    return launch_merge(dm, pl.n_chunks, a, out, (hipStream_t)stream);
}

nosa_status nosa_decode_partial(const nosa_shape *shape, const void *q, const void *kv,
                                int64_t kv_row_blocks, int32_t kv_mode, const int32_t *list,
                                const int32_t *n_list, int32_t list_stride, int32_t list_len,
                                int32_t with_newest, const void *cur_kv, int64_t cur_row_blocks,
                                const nosa_step *step, const float *e_tok, int64_t e_row_stride,
                                void *ws, size_t ws_bytes, int32_t chunk0, void *stream) {
    return decode_partial_impl(shape, q, kv, kv_row_blocks, kv_mode, list, n_list, list_stride,
                               list_len, with_newest, cur_kv, cur_row_blocks, step, e_tok,
                               e_row_stride, ws, ws_bytes, chunk0, nullptr, nullptr, stream);
}

nosa_status nosa_decode_partial_timed(const nosa_shape *shape, const void *q, const void *kv,
                                      int64_t kv_row_blocks, int32_t kv_mode,
                                      const int32_t *list, const int32_t *n_list,
                                      int32_t list_stride, int32_t list_len, int32_t with_newest,
                                      const void *cur_kv, int64_t cur_row_blocks,
                                      const nosa_step *step, const float *e_tok,
                                      int64_t e_row_stride, void *ws, size_t ws_bytes,
                                      int32_t chunk0, void *start_event, void *stop_event,
                                      void *stream) {
    if (!start_event || !stop_event) return NOSA_ERR_INVALID_ARGUMENT;
    return decode_partial_impl(shape, q, kv, kv_row_blocks, kv_mode, list, n_list, list_stride,
                               list_len, with_newest, cur_kv, cur_row_blocks, step, e_tok,
                               e_row_stride, ws, ws_bytes, chunk0, (hipEvent_t)start_event,
                               (hipEvent_t)stop_event, stream);
}

nosa_status nosa_decode_attend(const nosa_shape *shape, const void *q, const void *kv,
                               int64_t kv_row_blocks, int32_t kv_mode, const int32_t *list,
                               const int32_t *n_list, int32_t list_stride, int32_t list_len,
                               int32_t with_newest, const void *cur_kv, int64_t cur_row_blocks,
                               const nosa_step *step, const float *e_tok, int64_t e_row_stride,
                               void *ws, size_t ws_bytes, void *out, void *start_event,
                               void *stop_event, void *stream) {
    if (!out || (!start_event != !stop_event)) return NOSA_ERR_INVALID_ARGUMENT;
    if (list_len + with_newest == 0) return NOSA_ERR_INVALID_ARGUMENT;  // nothing to normalize
    return decode_partial_impl(shape, q, kv, kv_row_blocks, kv_mode, list, n_list, list_stride,
                               list_len, with_newest, cur_kv, cur_row_blocks, step, e_tok,
                               e_row_stride, ws, ws_bytes, 0, (hipEvent_t)start_event,
                               (hipEvent_t)stop_event, stream, out);
}

// ---- steps replayed from a captured graph: the step record in device memory ----

nosa_status nosa_step_advance(const nosa_shape *shape, nosa_step *step_dev, void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!step_dev) return NOSA_ERR_INVALID_ARGUMENT;
    return hip_status(launch_step_advance(dm, reinterpret_cast<int32_t *>(step_dev),
                                          (hipStream_t)stream));
}

nosa_status nosa_pool_step(const nosa_shape *shape, const void *kv, int64_t kv_row_blocks,
                           const float *e_tok, int64_t e_row_stride, const nosa_step *step_dev,
                           void *kbar, float *e_blk, void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!kv || !e_tok || !kbar || !e_blk || !step_dev) return NOSA_ERR_INVALID_ARGUMENT;
    if (kv_row_blocks < dm.max_blocks || e_row_stride < (int64_t)dm.max_blocks * dm.S)
        return NOSA_ERR_INVALID_ARGUMENT;
    return by_types(dm, [&](auto tp, auto tk, auto dc) -> nosa_status {
        using T = std::remove_pointer_t<decltype(tp)>;
        using TK = std::remove_pointer_t<decltype(tk)>;
        return hip_status(launch_pool_step<T, TK, decltype(dc)::value>(
            dm, kv, kv_row_blocks, e_tok, e_row_stride,
            reinterpret_cast<const int32_t *>(step_dev), kbar, e_blk, (hipStream_t)stream));
    });
}

nosa_status nosa_append_step(const nosa_shape *shape, const void *k_new, const void *v_new,
                             void *kv, int64_t kv_row_blocks, const nosa_step *step_dev,
                             void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!k_new || !v_new || !kv || !step_dev || kv_row_blocks < dm.max_blocks)
        return NOSA_ERR_INVALID_ARGUMENT;
    return by_type_dim(dm, [&](auto tp, auto dc) -> nosa_status {
        using T = std::remove_pointer_t<decltype(tp)>;
        constexpr int D = decltype(dc)::value;
        return hip_status(launch_append<T, D>(dm, k_new, v_new, 0, kv, kv_row_blocks, 0,
                                              (hipStream_t)stream,
                                              reinterpret_cast<const int32_t *>(step_dev)));
    });
}

nosa_status nosa_score_select_step(const nosa_shape *shape, const void *q, const void *kbar,
                                   const float *e_blk, const nosa_step *step_dev, float *s_q,
                                   uint32_t *ge_bits, uint32_t *ev_bits, int32_t *sel,
                                   int32_t *n_sel, uint32_t *sel_bits, int32_t *slot_block,
                                   int32_t *block_slot, int32_t *fetch_block,
                                   int32_t *fetch_slot, int32_t *n_fetch, uint64_t *counters,
                                   void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!q || !kbar || !s_q || !e_blk || !ge_bits || !ev_bits || !sel || !n_sel || !sel_bits ||
        !step_dev)
        return NOSA_ERR_INVALID_ARGUMENT;
    const bool any_swap = slot_block || block_slot || fetch_block || fetch_slot || n_fetch || counters;
    const bool all_swap = slot_block && block_slot && fetch_block && fetch_slot && n_fetch && counters;
    if (any_swap && !all_swap) return NOSA_ERR_INVALID_ARGUMENT;
    const SwapPtrs sw{slot_block, block_slot, fetch_block, fetch_slot, n_fetch, counters};
    return by_types(dm, [&](auto tp, auto tk, auto dc) -> nosa_status {
        using T = std::remove_pointer_t<decltype(tp)>;
        using TK = std::remove_pointer_t<decltype(tk)>;
        constexpr int D = decltype(dc)::value;
        return by_group(dm, [&](auto gc) -> nosa_status {
            return hip_status(launch_score_select<T, TK, D, decltype(gc)::value>(
                dm, q, kbar, s_q, e_blk, 0, -1, ge_bits, ev_bits, sel, n_sel, sel_bits,
                all_swap ? &sw : nullptr, (hipStream_t)stream,
                reinterpret_cast<const int32_t *>(step_dev)));
        });
    });
}

nosa_status nosa_decode_partial_step(const nosa_shape *shape, const void *q, const void *kv,
                                     int64_t kv_row_blocks, int32_t kv_mode, const int32_t *list,
                                     const int32_t *n_list, int32_t list_stride,
                                     int32_t list_len, int32_t with_newest, const void *cur_kv,
                                     int64_t cur_row_blocks, const nosa_step *step_dev,
                                     const float *e_tok, int64_t e_row_stride, void *ws,
                                     size_t ws_bytes, int32_t chunk0, void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!step_dev || list_len < 0 || list_len > dm.k || (with_newest != 0 && with_newest != 1))
        return NOSA_ERR_INVALID_ARGUMENT;
    if (list_len > 0 && (!kv || !list || list_stride < list_len ||
                         (kv_mode == NOSA_KV_FULL && !n_list)))
        return NOSA_ERR_INVALID_ARGUMENT;
    if (kv_mode == NOSA_KV_CACHE && list_len > 0 && kv_row_blocks < list_len)
        return NOSA_ERR_INVALID_ARGUMENT;
    // with the full KV the newest block is block n_cand of cur_kv's rows
    if (kv_mode == NOSA_KV_FULL && cur_row_blocks < dm.max_blocks) return NOSA_ERR_INVALID_ARGUMENT;
    const int kind = decode_kind(dm, shape->decode_kernel);
    // every step value the device record can hold: validate against the capacity
    const nosa_step cap{dm.max_blocks * dm.S, -1};
    DecodeArgs a;
    s = decode_common(dm, kind, q, kv ? kv : cur_kv, kv ? kv_row_blocks : cur_row_blocks,
                      kv_mode, cur_kv, cur_row_blocks, &cap, e_tok, e_row_stride, ws, ws_bytes, a);
    if (s != NOSA_OK) return s;
    const DecodePlan pl = decode_plan(dm, kind, list_len, with_newest);
    if (chunk0 < 0 || chunk0 + pl.n_chunks > a.chunk_cap) return NOSA_ERR_INVALID_ARGUMENT;
    a.list = list;
    a.n_list = kv_mode == NOSA_KV_FULL ? n_list : nullptr;
    a.list_stride = list_stride;
    a.list_len = list_len;
    a.with_newest = with_newest;
    a.chunk0 = chunk0;
    a.cb = pl.cb;
    a.dstep = reinterpret_cast<const int32_t *>(step_dev);
    a.cur_at_step = kv_mode == NOSA_KV_FULL ? 1 : 0;
    return launch_partial(dm, kind, pl, a, (hipStream_t)stream);
}

static nosa_status decode_combine_impl(const nosa_shape *shape, int32_t n_chunks, void *out,
                                       void *ws, size_t ws_bytes, int32_t *dstep_adv,
                                       void *stream) {
    Dims dm;
    nosa_status s = make_dims(shape, &dm);
    if (s != NOSA_OK) return s;
    if (!out || !ws || (((uintptr_t)ws) & 15u)) return NOSA_ERR_INVALID_ARGUMENT;
    if (ws_bytes < decode_ws_bytes(dm)) return NOSA_ERR_WORKSPACE;
    if (n_chunks < 1 || n_chunks > decode_chunk_cap(dm)) return NOSA_ERR_INVALID_ARGUMENT;
    DecodeArgs a{};
    a.chunk_cap = decode_chunk_cap(dm);
    a.ws_o = static_cast<float *>(ws);
    a.ws_ml = a.ws_o + (size_t)dm.rows * a.chunk_cap * dm.G * dm.D;
    return launch_merge(dm, n_chunks, a, out, (hipStream_t)stream, dstep_adv);
}

nosa_status nosa_decode_combine(const nosa_shape *shape, int32_t n_chunks, void *out, void *ws,
                                size_t ws_bytes, void *stream) {
    return decode_combine_impl(shape, n_chunks, out, ws, ws_bytes, nullptr, stream);
}

nosa_status nosa_decode_combine_step(const nosa_shape *shape, int32_t n_chunks, void *out,
                                     void *ws, size_t ws_bytes, nosa_step *step_dev,
                                     void *stream) {
    if (!step_dev) return NOSA_ERR_INVALID_ARGUMENT;
    return decode_combine_impl(shape, n_chunks, out, ws, ws_bytes,
                               reinterpret_cast<int32_t *>(step_dev), stream);
}

nosa_status nosa_host_alloc(size_t bytes, int32_t coherent, void **host, void **dev) {
    if (!host || !dev || bytes == 0) return NOSA_ERR_INVALID_ARGUMENT;
    *host = nullptr;
    *dev = nullptr;
    unsigned flags = hipHostMallocMapped | (coherent ? hipHostMallocCoherent : hipHostMallocNonCoherent);
    void *h = nullptr;
    hipError_t e = hipHostMalloc(&h, bytes, flags);
    if (e != hipSuccess) return hip_status(e);
    void *d = nullptr;
    e = hipHostGetDevicePointer(&d, h, 0);
    if (e != hipSuccess) {
        (void)hipHostFree(h);
        return hip_status(e);
    }
    *host = h;
    *dev = d;
    return NOSA_OK;
}

nosa_status nosa_host_free(void *host) {
    if (!host) return NOSA_ERR_INVALID_ARGUMENT;
    return hip_status(hipHostFree(host));
}

const char *nosa_status_string(nosa_status s) {
    switch (s) {
    case NOSA_OK: return "ok";
    case NOSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case NOSA_ERR_UNSUPPORTED: return "unsupported shape";
    case NOSA_ERR_HIP: return "HIP error";
    case NOSA_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
    }
}

const char *nosa_last_error(void) { return g_last_error.c_str(); }

nosa_status nosa_read_probe(const void *src, int64_t bytes, uint32_t *sink, int32_t workgroups,
                            void *stream) {
    if (!src || !sink || bytes <= 0 || (bytes & 15) || workgroups <= 0 ||
        (reinterpret_cast<uintptr_t>(src) & 15))
        return NOSA_ERR_INVALID_ARGUMENT;
    return hip_status(launch_read_probe(src, bytes, sink, workgroups, (hipStream_t)stream));
}

int32_t nosa_version(void) { return 100; }

}  // extern "C"
