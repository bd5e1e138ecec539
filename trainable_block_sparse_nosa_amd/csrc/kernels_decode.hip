// Sparse decode attention with the ED-DMA logit bias, split-K over blocks.
//
// NOSA technical summary, Methodology, "1. Algorithm: NOSA", bullet "ED-DMA":
// eviction scores stay pre-exponential through selection and their
// exponential happens in the attention softmax; here each token's score is
// added to its logit, z = scale * q.k + e, and softmax(z) weighs the values.
//
// Work split: one workgroup per (chunk of entries, row). A call's entries are
// the blocks of a list (the whole selection, or one part of it) plus, when
// asked, the newest block. Each workgroup
// keeps an online-softmax state (max, sum, output) per head and writes it to
// the workspace as its chunk's partial; a second kernel merges each row's
// partials in chunk order and writes the output. The merge order is fixed,
// so results do not depend on scheduling. Merging inside the first kernel
// would need device-scope fences, which on a multi-XCD part write back and
// invalidate L2 under the other workgroups' streaming reads: a merge by each
// row's last-arriving workgroup, on a 64-row, 4-chunk step, took 79.5 us with
// a fence in every wave and 29.1 us with one write-back per workgroup,
// against 24.0 us plus a 4.1 us merge launch; the kernel boundary gives the
// same ordering for free. A row served
// by a single chunk needs no merge: its workgroup can normalize and write the
// output itself.
//
// Two kernels compute the partials:
//  * MFMA (bf16): the G query heads of a row are padded to a 16-wide tile
//    and S^T = K Q^T and O^T = V^T P^T run on v_mfma_f32_16x16x32_bf16 (P
//    enters as a bf16 hi + lo pair, so the weights keep ~16 bits). The
//    K and V tiles are read straight into MFMA operand registers with 16-byte
//    loads; the V tile's token order inside each 32-token half is stored so
//    that the probabilities a lane holds after S^T are exactly the 8 k-slots
//    it feeds to O^T (no cross-lane shuffles).
//  * VALU (float32 and bf16): K and V tiles staged in LDS, fp32 FMAs.
#include "kernels.h"

#include <hip/hip_ext.h>

namespace nosa {


// MFMA kernel: 8 waves per workgroup, about one workgroup per CU (at ~230
// registers two waves share a SIMD, so 8 waves fill a CU).
constexpr int WAVES = 8;
constexpr int MFMA_TARGET_WGS = 256;

DecodePlan decode_plan(const Dims &dm, int kind, int list_len, int with_newest) {
    DecodePlan p;
    const int entries = list_len + with_newest;
    if (entries <= 0) {
        p.cb = 1;
        p.n_chunks = 0;
        return p;
    }
    if (kind == NOSA_DECODE_MFMA) {
        // Few, long chunks: each workgroup's waves walk a chunk's entries with
        // a running softmax state, so a row leaves few partials behind. The
        // partials are the kernel's only writes, and writes mixed into the
        // read stream cost far more HBM time than their bytes (measured on the
        // 64k workload: 33 chunks per row of 4 one-block waves took 202 us, a
        // chunk per row 186 us; with the partial writes dropped, 178 us).
        int nc = (MFMA_TARGET_WGS + dm.rows - 1) / dm.rows;
        const int maxc = (entries + WAVES - 1) / WAVES;  // at least a block per wave
        nc = nc < 1 ? 1 : (nc > maxc ? maxc : nc);
        // The list splits evenly over the chunks and the newest block (often
        // partly filled) joins the last one, so that it lengthens one wave of
        // one chunk rather than every chunk: 64 listed blocks over 4 chunks of
        // 8 waves are 2 blocks per wave, plus the newest in one wave of the last.
        if (list_len == 0) {
            p.cb = 1;
            p.n_chunks = 1;
        } else {
            p.cb = (list_len + nc - 1) / nc;
            p.n_chunks = (list_len + p.cb - 1) / p.cb;
        }
    } else {
        // enough workgroups to cover 256 CUs several times over
        const long total = (long)dm.rows * entries;
        int cb = 1;
        while (cb < 16 && total / (cb * 2) >= 2048) cb *= 2;
        p.cb = cb;
        p.n_chunks = (entries + p.cb - 1) / p.cb;
    }
    return p;
}

int decode_kind(const Dims &dm, int requested) {
    if (requested == NOSA_DECODE_AUTO) return dm.dtype == NOSA_BF16 ? NOSA_DECODE_MFMA : NOSA_DECODE_VALU;
    return requested;
}

// ---------------------------------------------------------------------------
// Combine: one workgroup per (row, head), one thread per dimension, merges
// the row's chunk partials in chunk order. Lane c of each wave loads chunk
// c's (max, sum); wave reductions give the row maximum and the denominator,
// and each chunk's weight is read back from its lane. The partial outputs'
// loads are issued together with those: one memory round trip, no LDS. With
// dstep_adv, the first workgroup also moves the device step record on.
// ---------------------------------------------------------------------------
template <typename T, int D, int G>
__global__ void __launch_bounds__(D)
combine_kernel(Dims dm, int n_chunks, int chunk_cap, const float *__restrict__ ws_o,
               const float *__restrict__ ws_ml, T *__restrict__ out, int32_t *dstep_adv) {
    constexpr int CREG = 33;  // chunks held in registers (every MFMA plan fits)
    const int r = blockIdx.x, h = blockIdx.y, d = threadIdx.x, lane = threadIdx.x & 63;
    const float *ml = ws_ml + ((int64_t)r * chunk_cap * G + h) * 2;  // chunk c at ml[c*G*2]
    const float *po = ws_o + ((int64_t)r * chunk_cap * G + h) * D + d;  // chunk c at po[c*G*D]
    float O = 0.f, L;
    if (n_chunks <= CREG && n_chunks <= 64) {
        float ov[CREG];
#pragma unroll
        for (int c = 0; c < CREG; ++c)
            if (c < n_chunks) ov[c] = po[(int64_t)c * G * D];
        const float mv = lane < n_chunks ? ml[lane * G * 2] : -INFINITY;
        const float lv = lane < n_chunks ? ml[lane * G * 2 + 1] : 0.f;
        const float M = wave_max(lv > 0.f ? mv : -INFINITY);
        const float wc = lv > 0.f ? __expf(mv - M) : 0.f;
        L = wave_sum(lv * wc);
#pragma unroll
        for (int c = 0; c < CREG; ++c)
            if (c < n_chunks)
                O = fmaf(ov[c], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wc), c)), O);
    } else {
        float M = -INFINITY;
        L = 0.f;
        for (int c = 0; c < n_chunks; ++c)
            if (ml[c * G * 2 + 1] > 0.f) M = fmaxf(M, ml[c * G * 2]);
        for (int c = 0; c < n_chunks; ++c) {
            const float l = ml[c * G * 2 + 1];
            const float wc = l > 0.f ? __expf(ml[c * G * 2] - M) : 0.f;
            L = fmaf(l, wc, L);
            O = fmaf(po[(int64_t)c * G * D], wc, O);
        }
    }
    const int b = r / dm.Hkv, g = r % dm.Hkv;
    out[((int64_t)b * dm.Hq + (int64_t)g * G + h) * D + d] = stf<T>(O / L);
    // the step's last kernel moves the device step record on: no workgroup of
    // this kernel reads it, and every kernel that does ran before it
    if (dstep_adv && r == 0 && h == 0 && d == 0) {
        const StepVals sv = read_step(dstep_adv, dm);
        dstep_adv[1] = sv.n_cand;
        dstep_adv[0] = sv.n_tokens + 1;
    }
}

// Resolve entry e of row r: data pointer, block id and valid tokens.
// Returns false when the entry holds no block.
template <typename T>
__device__ __forceinline__ bool resolve_entry(const DecodeArgs &a, const StepVals &sv, int e,
                                              int cnt_e, int r, int64_t BE, const T *&blk,
                                              int &bid, int &valid) {
    if (a.with_newest && e == a.list_len) {
        // the newest block: block cur_block of cur's row (n_cand when it
        // follows the device step: cur is then the full KV)
        const int64_t cb = a.cur_at_step ? sv.n_cand : 0;
        blk = static_cast<const T *>(a.cur) + ((int64_t)r * a.cur_row_blocks + cb) * BE;
        bid = sv.n_cand;
        valid = sv.n_tokens - sv.n_cand * 64;
        return true;
    }
    if (e >= a.list_len) return false;
    bid = a.list[(int64_t)r * a.list_stride + e];  // issued before the count is known
    if (e >= cnt_e || bid < 0 || bid >= sv.n_cand) return false;  // only candidates are listed
    const int64_t at = a.kv_mode == NOSA_KV_FULL ? bid : e;
    blk = static_cast<const T *>(a.kv) + ((int64_t)r * a.kv_row_blocks + at) * BE;
    valid = 64;
    return true;
}

// ---------------------------------------------------------------------------
// MFMA partial kernel (bf16). Chunk c of a row covers entries
// [c*cb, (c+1)*cb), the last chunk up to the end (the newest block
// included); wave w takes entries c*cb + w, + 8, ...,
// one block at a time with all of its loads in flight, keeping a running
// softmax state; the 8 waves merge through LDS into the chunk's partial.
// Lane l: col = l % 16 (head in S^T / O^T), grp = l / 16.
// ---------------------------------------------------------------------------
template <int D>
struct BlockRegs {
    bf16x8 k[4][D / 32];  // A operands of S^T = K Q^T, tile t = tokens 16t..16t+15
    bf16x8 v[D / 16][2];  // A operands of O^T = V^T P^T, d-tile dt, token half s
    f32x4 e[4];           // eviction scores of tokens 16t + 4grp + u
    int valid;            // tokens of this block that exist (0: no block)
};

// One 16-byte operand vector; NT marks the load non-temporal (streamed once:
// the lines are not kept in the caches).
template <bool NT>
__device__ __forceinline__ bf16x8 load_frag(const bf16_t *p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(p));
    else return *reinterpret_cast<const bf16x8 *>(p);
}

// The block's K and V^T fragments (the block layout in common.h: fragment f,
// lane l at 16 bytes (64 f + l)), so each load instruction of the wave reads
// 1 KiB of whole cache lines.
template <int D, bool NT>
__device__ __forceinline__ void load_block(BlockRegs<D> &br, const bf16_t *blk, const float *eb,
                                           int valid, int col, int grp) {
    constexpr int S = 64, KS = D / 32, DT = D / 16;
    const bf16_t *Kt = blk + 8 * (col + 16 * grp);  // K fragment t KS + s
    const bf16_t *Vt = Kt + S * D;                  // V^T fragment 2 dt + s
    // eviction scores first: the QK^T MFMAs and the softmax then wait only for
    // the K loads (waits are in issue order), not for V as well
#pragma unroll
    for (int t = 0; t < 4; ++t) br.e[t] = *reinterpret_cast<const f32x4 *>(eb + 16 * t + 4 * grp);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int s = 0; s < KS; ++s) br.k[t][s] = load_frag<NT>(Kt + 512 * (t * KS + s));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int s = 0; s < 2; ++s) br.v[dt][s] = load_frag<NT>(Vt + 512 * (2 * dt + s));
    br.valid = valid;
}

template <int D>
__device__ __forceinline__ void attend_block(const BlockRegs<D> &br, const bf16x8 (&qop)[D / 32],
                                             float scale, int grp, int lim, float &m_run,
                                             float &l_run, f32x4 (&o)[D / 16]) {
    constexpr int KS = D / 32, DT = D / 16;
    // S^T tile t: lane holds logits of tokens 16t + 4grp + u for head col
    f32x4 sc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
            sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(br.k[t][s], qop[s], sc[t], 0, 0, 0);
    }
    float z[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            // tokens of the block from lim on are masked for this lane's column
            const bool ok = 16 * t + 4 * grp + u < lim;
            z[t][u] = ok ? fmaf(sc[t][u], scale, br.e[t][u]) : -INFINITY;
            mx = fmaxf(mx, z[t][u]);
        }
    // the 64 tokens of head col live in lanes col, col+16, col+32, col+48
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
    // P as a sum of two bf16 operands (hi + lo) keeps ~16 mantissa bits
    bf16x8 phi[2], plo[2];
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float p = z[t][u] == -INFINITY ? 0.f : __expf(z[t][u] - m_new);
            const __bf16 hi = (__bf16)p;
            phi[t / 2][(t % 2) * 4 + u] = hi;
            plo[t / 2][(t % 2) * 4 + u] = (__bf16)(p - (float)hi);
            ps += p;
        }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    // O^T tile dt: lane holds dims 16dt + 4grp + u for head col
    if (lim >= 64) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            o[dt] *= alpha;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(br.v[dt][s], phi[s], o[dt], 0, 0, 0);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(br.v[dt][s], plo[s], o[dt], 0, 0, 0);
            }
        }
        return;
    }
    // a partly filled block (the newest): the value slots of tokens from lim
    // on hold whatever the buffer held before, possibly not finite, and a
    // zero weight times a NaN or an infinity is a NaN; they enter as zeros.
    // Element i of the lane's operand for token half s is stored position
    // 32s + 8grp + i; a 32-bit mask per element pair keeps the live ones.
    u32x4 keep[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p0 = 32 * s + 8 * grp + 2 * j;
            keep[s][j] = (vt_token_at(p0) < lim ? 0x0000FFFFu : 0u) |
                         (vt_token_at(p0 + 1) < lim ? 0xFFFF0000u : 0u);
        }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        o[dt] *= alpha;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const bf16x8 v = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, br.v[dt][s]) & keep[s]);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, phi[s], o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, plo[s], o[dt], 0, 0, 0);
        }
    }
}

template <int D, int G, bool NT>
__global__ void __launch_bounds__(64 * WAVES)
decode_mfma_kernel(Dims dm, DecodeArgs a) {
    static_assert(G <= 16, "the group is one 16-wide MFMA tile");
    constexpr int S = 64, KS = D / 32, DT = D / 16;
    constexpr int64_t BE = 2 * S * D;
    __shared__ float wm[WAVES][G], wl[WAVES][G];
    __shared__ float wo[WAVES][D][G];

    const int lane = threadIdx.x & 63;
    // the wave index is uniform: block ids come from scalar loads
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int r = blockIdx.y, chunk = blockIdx.x;
    const int b = r / dm.Hkv, g = r % dm.Hkv;
    const StepVals sv = a.dstep ? read_step(a.dstep, dm) : StepVals{a.n_tokens, a.n_cand, 0};
    const int cnt_e = a.n_list ? min(a.n_list[r], a.list_len) : a.list_len;
    const float *er = a.e_tok + (int64_t)r * a.e_stride;
    const int e_beg = chunk * a.cb;
    // the last chunk also takes the newest block (decode_plan)
    const int e_end = chunk == (int)gridDim.x - 1 ? a.list_len + a.with_newest : e_beg + a.cb;
    const bf16_t *q = static_cast<const bf16_t *>(a.q);

    // B operand of S^T = K Q^T: lane holds q[head col][32s + 8grp .. +7].
    // Padding columns (col >= G) repeat head G-1: their softmax reductions
    // stay within their own column and their outputs are never stored.
    bf16x8 qop[KS];
    {
        const int hc = col < G ? col : G - 1;
        const bf16_t *qh = q + ((int64_t)b * dm.Hq + (int64_t)g * G + hc) * D + 8 * grp;
#pragma unroll
        for (int s = 0; s < KS; ++s) qop[s] = *reinterpret_cast<const bf16x8 *>(qh + 32 * s);
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int e = e_beg + wave; e < e_end; e += WAVES) {
        BlockRegs<D> br;
        const bf16_t *blk;
        int bid, valid;
        if (resolve_entry<bf16_t>(a, sv, e, cnt_e, r, BE, blk, bid, valid)) {
            load_block<D, NT>(br, blk, er + (int64_t)bid * S, valid, col, grp);
            // keep every load of the block ahead of the math: without this the
            // scheduler interleaves loads with MFMAs to save registers and the
            // block is no longer in flight at once
            __builtin_amdgcn_sched_barrier(0);
            attend_block<D>(br, qop, dm.scale, grp, br.valid, m_run, l_run, o);
        }
    }

    // merge the waves' states
    if (col < G) {
        if (grp == 0) {
            wm[wave][col] = m_run;
            wl[wave][col] = l_run;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int u = 0; u < 4; ++u) wo[wave][16 * dt + 4 * grp + u][col] = o[dt][u];
    }
    __syncthreads();
    const int64_t base = ((int64_t)r * a.chunk_cap + a.chunk0 + chunk) * G;
    float *ws_o = a.ws_o, *ws_ml = a.ws_ml;
    bf16_t *out = static_cast<bf16_t *>(a.out);
    const int64_t out_row = ((int64_t)b * dm.Hq + (int64_t)g * G) * D;  // head 0 of the row's group
    const bool direct = out && gridDim.x == 1;  // the row's only chunk: normalize here
    for (int p = threadIdx.x; p < G * D; p += blockDim.x) {
        const int h = p / D, d = p % D;
        float mw[WAVES], lw[WAVES];
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            mw[w] = wm[w][h];
            lw[w] = wl[w][h];
            M = fmaxf(M, lw[w] > 0.f ? mw[w] : -INFINITY);
        }
        float O = 0.f, L = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float c = lw[w] > 0.f ? __expf(mw[w] - M) : 0.f;
            O = fmaf(wo[w][d][h], c, O);
            L = fmaf(lw[w], c, L);
        }
        if (direct) {
            out[out_row + p] = stf<bf16_t>(O / L);
            continue;
        }
        ws_o[base * D + p] = O;
        if (d == 0) {
            ws_ml[(base + h) * 2 + 0] = M;
            ws_ml[(base + h) * 2 + 1] = L;
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill (training-time forward) with the selection per query block.
//
// Pooled queries: qbar[i][b][hq][d] = mean of q[b][64 i + u][hq][d] over the
// query block's tokens, in the pooled dtype TK (exact mean rounded once).
// ---------------------------------------------------------------------------
template <typename T, typename TK, int D>
__global__ void __launch_bounds__(256)
pool_queries_kernel(Dims dm, const T *__restrict__ q, int n_tokens, TK *__restrict__ qbar) {
    // one workgroup per (query block i, sequence b); thread t owns the
    // 16-byte vectors t, t + 256, ... of a token's Hq * D elements and sums
    // each element over the block's tokens in order, in double (exact for
    // bf16 inputs), eight tokens' loads in flight; the mean is rounded once
    constexpr int EV = 16 / sizeof(T);
    const int i = blockIdx.x, b = blockIdx.y;
    const int lo = 64 * i, n = min(64, n_tokens - lo);
    const int64_t tok = (int64_t)dm.Hq * D;  // elements per token
    const int nv = (int)(tok / EV);
    const T *qb = q + ((int64_t)b * n_tokens + lo) * tok;
    TK *ob = qbar + ((int64_t)i * dm.B + b) * tok;
    for (int v = threadIdx.x; v < nv; v += blockDim.x) {
        double s[EV];
#pragma unroll
        for (int e = 0; e < EV; ++e) s[e] = 0.0;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(qb) + v;
        const int64_t stride = tok / EV;  // vectors per token
#pragma unroll 8
        for (int u = 0; u < n; ++u) {
            const u32x4 raw = src[(int64_t)u * stride];
            float x[EV];
            if constexpr (std::is_same_v<T, float>) {
                x[0] = __uint_as_float(raw.x); x[1] = __uint_as_float(raw.y);
                x[2] = __uint_as_float(raw.z); x[3] = __uint_as_float(raw.w);
            } else {
                x[0] = bf_lo(raw.x); x[1] = bf_hi(raw.x); x[2] = bf_lo(raw.y); x[3] = bf_hi(raw.y);
                x[4] = bf_lo(raw.z); x[5] = bf_hi(raw.z); x[6] = bf_lo(raw.w); x[7] = bf_hi(raw.w);
            }
#pragma unroll
            for (int e = 0; e < EV; ++e) s[e] += (double)x[e];
        }
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            const double mean = s[e] / (double)n;
            if constexpr (std::is_same_v<TK, float>) ob[(int64_t)v * EV + e] = (float)mean;
            else ob[(int64_t)v * EV + e] = bf16_rne_from_double(mean);
        }
    }
}

// Block-sparse causal attention (bf16, MFMA). A workgroup takes ROWS query
// rows of one query block i of row r (query row qr = G u + h: token u, head
// h); each of its W waves owns CT tiles of 16 query rows, the 16 columns of
// S^T = K Q^T. The workgroup walks the query block's selected blocks and then
// its own block (causal: a column sees its own block's tokens up to its own
// token). Each block is loaded once per workgroup into LDS, laid out in MFMA
// fragment order (a wave's fragment read is 1 KiB contiguous), and double
// buffered: the next block's loads are in flight while the current one is
// used. Every K and V fragment read from LDS feeds the CT tiles of the wave.
// The eviction score is an additive logit as in the decode kernel. The
// softmax runs in base 2 with a lazy base per column (moved only when a
// block's maximum passes it by more than 8), P enters P.V as bf16 and the
// denominator sums the same bf16 values on the matrix cores; the output is
// normalized and stored in bf16.
struct PrefillArgs {
    const void *q;          // [B][N][Hq][D]
    const void *kv;         // block-unit KV [rows][kv_row_blocks][2*S*D]
    int64_t kv_row_blocks;
    const float *e_tok;     // [rows][e_stride]
    int64_t e_stride;
    const int32_t *sel;     // [n_qb][rows][k], ascending
    const int32_t *n_sel;   // [n_qb][rows]
    int n_tokens;
    void *out;              // [B][N][Hq][D]
};

constexpr float LOG2E = 1.4426950408889634f;

template <int G>
struct PrefillShape {
    static constexpr int CT = G == 1 ? 1 : 2;                       // tiles per wave
    static constexpr int W = G == 1 ? 4 : (2 * G < 8 ? 2 * G : 8);  // waves per workgroup
    static constexpr int ROWS = 16 * CT * W;                        // query rows per workgroup
    static constexpr int NG = (64 * G + ROWS - 1) / ROWS;           // workgroups per query block
    static_assert((64 * G) % (16 * CT) == 0, "a wave's tiles are all live or all idle");
};

// One KV block in LDS: K fragments (t, s) at t*KS + s, then V^T fragments
// (dt, s) at 4 KS + 2 dt + s; lane l of fragment f holds the 16 bytes the
// MFMA A operand of lane l needs. Then the block's 64 eviction scores,
// multiplied by log2(e) for the base-2 softmax.
template <int D>
struct PrefillTile {
    static constexpr int KS = D / 32, DT = D / 16;
    static constexpr int NF = 4 * KS + 2 * DT;
    bf16x8 frag[NF][64];
    float e[64];
};

template <int D, int NT>
struct PrefillStage {
    static constexpr int NF = PrefillTile<D>::NF;
    static constexpr int CH = (NF * 64 + NT - 1) / NT;  // 16-byte chunks per thread
    bf16x8 v[CH];
    f32x4 e;
};

// Issue the global loads of one block (chunk x = tid + j NT is lane x % 64 of
// fragment x / 64). The stored block is in this fragment order already (the
// layout in common.h): the loads are one contiguous 16-byte vector per thread.
template <int D, int NT>
__device__ __forceinline__ void prefill_load(PrefillStage<D, NT> &st, const bf16_t *blk,
                                             const float *eb, int tid) {
    constexpr int NF = PrefillTile<D>::NF;
#pragma unroll
    for (int j = 0; j < PrefillStage<D, NT>::CH; ++j) {
        const int x = tid + j * NT;
        if (NF * 64 % NT == 0 || x < NF * 64) st.v[j] = *reinterpret_cast<const bf16x8 *>(blk + 8 * x);
    }
    if (tid < 16) st.e = *reinterpret_cast<const f32x4 *>(eb + 4 * tid);
}

// Write a staged block to LDS. Tokens from `valid` on (the tail of a
// sequence's last block) are written as zeros, so that whatever the KV
// storage holds there cannot reach the MFMA sums.
template <int D, int NT>
__device__ __forceinline__ void prefill_store(PrefillTile<D> &tl, const PrefillStage<D, NT> &st,
                                              int valid, int tid) {
    constexpr int KS = D / 32, NF = PrefillTile<D>::NF;
#pragma unroll
    for (int j = 0; j < PrefillStage<D, NT>::CH; ++j) {
        const int x = tid + j * NT;
        if (NF * 64 % NT == 0 || x < NF * 64) {
            const int f = x / 64, l = x % 64, col = l % 16, grp = l / 16;
            bf16x8 v = st.v[j];
            if (valid < 64) {
                if (f < 4 * KS) {
                    if (16 * (f / KS) + col >= valid) v = bf16x8{};
                } else {
                    const int base = 32 * ((f - 4 * KS) % 2) + 8 * grp;
#pragma unroll
                    for (int m = 0; m < 8; ++m)
                        if (vt_token_at(base + m) >= valid) v[m] = 0;
                }
            }
            tl.frag[f][l] = v;
        }
    }
    if (tid < 16) *reinterpret_cast<f32x4 *>(&tl.e[4 * tid]) = st.e * LOG2E;
}

// One block against the wave's CT tiles, with running softmax states kept in
// the base-2 domain: z2 = log2(e) (scale q.k + e). The block's eviction
// scores arrive already multiplied by log2(e). CAUSAL masks, per column, the
// tokens from lim[c] on (the own block); the other blocks are whole. P
// enters P V as a bf16 hi + lo pair (about 16 significant bits: when a few
// tokens dominate a softmax, one bf16 rounding of their weights would show
// in the output), and the denominator sums the same pair.
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

// Two floats rounded to bf16 (nearest, ties to even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Max of v over the four rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48) on
// the gfx950 row-swap instructions: with both operands holding v, each lane
// of the swapped pair holds v at its own lane and at the lane 16 (32) away.
__device__ __forceinline__ float max_over_rows(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t w = __float_as_uint(v);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int D, int CT, bool CAUSAL>
__device__ __forceinline__ void prefill_block(const PrefillTile<D> &tl,
                                              const bf16x8 (&qop)[CT][D / 32], float scale2,
                                              int lane, const int (&lim)[CT], float (&m_run)[CT],
                                              f32x4 (&l_run)[CT], f32x4 (&o)[CT][D / 16]) {
    constexpr int KS = D / 32, DT = D / 16;
    const int grp = lane >> 4;
    f32x4 sc[CT][4];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int t = 0; t < 4; ++t) sc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 kf = tl.frag[t * KS + s][lane];
#pragma unroll
            for (int c = 0; c < CT; ++c)
                sc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qop[c][s], sc[c][t], 0, 0, 0);
        }
    f32x4 ev[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) ev[t] = *reinterpret_cast<const f32x4 *>(&tl.e[16 * t + 4 * grp]);
    u32x4 ph[CT][2], pl[CT][2];  // bf16 pairs, as the MFMA B operand
    float alpha[CT];
    bool rescale = false;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        float z[4][4];
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                z[t][u] = fmaf(sc[c][t][u], scale2, ev[t][u]);
                if (CAUSAL && 16 * t + 4 * grp + u >= lim[c]) z[t][u] = -INFINITY;
                mx = fmaxf(mx, z[t][u]);
            }
        mx = max_over_rows(mx);
        // lazy base: the running base moves only when the block's maximum
        // exceeds it by more than 8 (log2 units), so probabilities stay below
        // 2^8 (exact in the fp32 sums, the same relative precision in bf16)
        // and the accumulators are rescaled only on those rare moves; the
        // softmax itself does not depend on the base
        const bool move = mx > m_run[c] + 8.f;  // also the first finite maximum
        const float m_new = move ? mx : m_run[c];
        // a column with no token yet subtracts 0: exp2(-inf - 0) = 0, no NaN
        const float m_sub = m_new == -INFINITY ? 0.f : m_new;
        alpha[c] = __builtin_amdgcn_exp2f(m_run[c] - m_sub);
        rescale |= move;
        // P as hi + lo, two weights at a time: hi is p with its low 16 bits
        // cleared (p truncated to bf16, relative error below 2^-7), two his
        // packed by one byte permute; lo = p - hi exactly in float32, two
        // los rounded to bf16 by one packed conversion: hi + lo is within
        // 2^-16 of p
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int u = 0; u < 4; u += 2) {
                const float p0 = __builtin_amdgcn_exp2f(z[t][u] - m_sub);
                const float p1 = __builtin_amdgcn_exp2f(z[t][u + 1] - m_sub);
                const uint32_t b0 = __float_as_uint(p0) & 0xFFFF0000u;
                const uint32_t b1 = __float_as_uint(p1) & 0xFFFF0000u;
                const int w = (t % 2) * 2 + u / 2;
                ph[c][t / 2][w] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
                pl[c][t / 2][w] = pack_bf16x2(p0 - __uint_as_float(b0), p1 - __uint_as_float(b1));
            }
        m_run[c] = m_new;
    }
    // most blocks move no column's maximum: skip the rescale then
    if (__any(rescale)) {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            l_run[c] *= alpha[c];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[c][dt] *= alpha[c];
        }
    }
    // the denominator on the matrix cores: an all-ones A operand sums the
    // column of P^T (the same hi + lo pair P.V uses) into every row of
    // l_run[c], rescaled with O above
    const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                         (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int c = 0; c < CT; ++c) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            l_run[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, as_bf16x8(ph[c][s2]), l_run[c], 0, 0, 0);
            l_run[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, as_bf16x8(pl[c][s2]), l_run[c], 0, 0, 0);
        }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 v0 = tl.frag[4 * KS + 2 * dt][lane];
        const bf16x8 v1 = tl.frag[4 * KS + 2 * dt + 1][lane];
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            o[c][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, as_bf16x8(ph[c][0]), o[c][dt], 0, 0, 0);
            o[c][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, as_bf16x8(pl[c][0]), o[c][dt], 0, 0, 0);
            o[c][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, as_bf16x8(ph[c][1]), o[c][dt], 0, 0, 0);
            o[c][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, as_bf16x8(pl[c][1]), o[c][dt], 0, 0, 0);
        }
    }
}

// Workgroups are handed to the 8 XCDs in turn; give each XCD a contiguous
// range of work items (the query blocks of a few rows), so that the blocks
// those query blocks share are read from one L2.
__device__ __forceinline__ int xcd_contiguous(int id, int total) {
    constexpr int X = 8;
    const int per = total / X, rem = total % X, x = id % X;
    return x * per + min(x, rem) + id / X;
}

template <int D, int G>
__global__ void __launch_bounds__(64 * PrefillShape<G>::W)
prefill_mfma_kernel(Dims dm, PrefillArgs a) {
    using Sh = PrefillShape<G>;
    constexpr int S = 64, KS = D / 32, DT = D / 16, CT = Sh::CT, NT = 64 * Sh::W;
    constexpr int64_t BE = 2 * S * D;
    __shared__ PrefillTile<D> tile[2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int nqb = (a.n_tokens + S - 1) / S;
    const int item = xcd_contiguous(blockIdx.x, gridDim.x);
    const int cg = item % Sh::NG, i = (item / Sh::NG) % nqb, r = item / (Sh::NG * nqb);
    const int b = r / dm.Hkv, g = r % dm.Hkv;
    const int row0 = Sh::ROWS * cg + 16 * CT * wave;  // first query row of the wave
    const bool active = row0 < S * G;                 // wave-uniform
    const int valid_own = min(S, a.n_tokens - S * i);
    const float scale2 = dm.scale * LOG2E;

    const bf16_t *q = static_cast<const bf16_t *>(a.q);
    bf16x8 qop[CT][KS];
    int lim[CT], u_of[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        const int qr = min(row0 + 16 * c + col, S * G - 1);
        const int u = qr / G, h = qr % G;
        const int pc = min(S * i + u, a.n_tokens - 1);
        u_of[c] = u;
        lim[c] = S;
        const bf16_t *qh = q + (((int64_t)b * a.n_tokens + pc) * dm.Hq + (int64_t)g * G + h) * D + 8 * grp;
#pragma unroll
        for (int s = 0; s < KS; ++s) qop[c][s] = *reinterpret_cast<const bf16x8 *>(qh + 32 * s);
    }
    float m_run[CT];
    f32x4 l_run[CT];  // the softmax denominator of column c, in all four entries
    f32x4 o[CT][DT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        m_run[c] = -INFINITY;
        l_run[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[c][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int64_t li = (int64_t)i * dm.rows + r;
    const int nsel = max(0, min(a.n_sel[li], dm.k));
    const int32_t *sl = a.sel + li * dm.k;
    const bf16_t *kvr = static_cast<const bf16_t *>(a.kv) + (int64_t)r * a.kv_row_blocks * BE;
    const float *er = a.e_tok + (int64_t)r * a.e_stride;
    // item e: selected block e for e < nsel (only blocks before the query
    // block are listed; anything else is skipped), then the own block
    auto block_of = [&](int e) {
        const int bid = e < nsel ? sl[e] : i;
        return (e == nsel || (bid >= 0 && bid < i)) ? bid : -1;
    };

    PrefillStage<D, NT> st;
    int bid = block_of(0);
    if (bid >= 0) {
        prefill_load<D, NT>(st, kvr + (int64_t)bid * BE, er + (int64_t)bid * S, tid);
        prefill_store<D, NT>(tile[0], st, nsel == 0 ? valid_own : S, tid);
    }
    __syncthreads();
    for (int e = 0; e < nsel; ++e) {
        const int nb = block_of(e + 1);
        if (nb >= 0)
            prefill_load<D, NT>(st, kvr + (int64_t)nb * BE, er + (int64_t)nb * S, tid);
        if (active && bid >= 0)
            prefill_block<D, CT, false>(tile[e & 1], qop, scale2, lane, lim, m_run, l_run, o);
        if (nb >= 0) prefill_store<D, NT>(tile[(e + 1) & 1], st, e + 1 == nsel ? valid_own : S, tid);
        __syncthreads();
        bid = nb;
    }
    // the own block, item nsel, causal per column
    if (active) {
#pragma unroll
        for (int c = 0; c < CT; ++c) lim[c] = u_of[c] + 1;
        prefill_block<D, CT, true>(tile[nsel & 1], qop, scale2, lane, lim, m_run, l_run, o);
    }

    if (active) {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const int qr = row0 + 16 * c + col;
            const int u = qr / G, h = qr % G, p = S * i + u;
            if (qr < S * G && p < a.n_tokens) {
                const float inv = 1.0f / l_run[c][0];
                bf16_t *out = static_cast<bf16_t *>(a.out) +
                              (((int64_t)b * a.n_tokens + p) * dm.Hq + (int64_t)g * G + h) * D;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        out[16 * dt + 4 * grp + v] = f2bf(o[c][dt][v] * inv);
            }
        }
    }
}

template <typename T, typename TK, int D>
hipError_t launch_pool_queries(const Dims &dm, const void *q, int n_tokens, void *qbar,
                               hipStream_t st) {
    const int nqb = (n_tokens + 63) / 64;
    if (nqb == 0) return hipSuccess;
    hipLaunchKernelGGL((pool_queries_kernel<T, TK, D>), dim3(nqb, dm.B), dim3(256), 0, st, dm,
                       static_cast<const T *>(q), n_tokens, static_cast<TK *>(qbar));
    return hipGetLastError();
}
#define NOSA_POOLQ_INST(T, TK, D)                                                              \
    template hipError_t launch_pool_queries<T, TK, D>(const Dims &, const void *, int, void *, \
                                                      hipStream_t);
NOSA_POOLQ_INST(float, float, 64)
NOSA_POOLQ_INST(bf16_t, float, 64)
NOSA_POOLQ_INST(bf16_t, float, 128)
NOSA_POOLQ_INST(bf16_t, bf16_t, 64)
NOSA_POOLQ_INST(bf16_t, bf16_t, 128)

template <int D, int G>
hipError_t launch_prefill(const Dims &dm, const void *q, int n_tokens, const void *kv,
                          int64_t kv_row_blocks, const float *e_tok, int64_t e_stride,
                          const int32_t *sel, const int32_t *n_sel, void *out, hipStream_t st) {
    using Sh = PrefillShape<G>;
    const int64_t nqb = (n_tokens + 63) / 64;
    const int64_t wgs = nqb * Sh::NG * dm.rows;
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    const PrefillArgs a{q, kv, kv_row_blocks, e_tok, e_stride, sel, n_sel, n_tokens, out};
    hipLaunchKernelGGL((prefill_mfma_kernel<D, G>), dim3((unsigned)wgs), dim3(64 * Sh::W), 0, st,
                       dm, a);
    return hipGetLastError();
}
#define NOSA_PREFILL_INST(D, G)                                                                \
    template hipError_t launch_prefill<D, G>(const Dims &, const void *, int, const void *,     \
                                             int64_t, const float *, int64_t, const int32_t *,  \
                                             const int32_t *, void *, hipStream_t);
#define NOSA_PREFILL_ALLG(D)                                                                   \
    NOSA_PREFILL_INST(D, 1) NOSA_PREFILL_INST(D, 2) NOSA_PREFILL_INST(D, 3)                    \
    NOSA_PREFILL_INST(D, 4) NOSA_PREFILL_INST(D, 5) NOSA_PREFILL_INST(D, 6)                    \
    NOSA_PREFILL_INST(D, 7) NOSA_PREFILL_INST(D, 8)
NOSA_PREFILL_ALLG(64)
NOSA_PREFILL_ALLG(128)

// ---------------------------------------------------------------------------
// VALU partial kernel (float32 and bf16): K and V^T tiles staged in LDS.
// ---------------------------------------------------------------------------
template <typename T, int D, int G>
__global__ void __launch_bounds__(256)
decode_valu_kernel(Dims dm, DecodeArgs a) {
    constexpr int S = 64;
    constexpr int EPV = 16 / sizeof(T);       // elements per 16-byte vector
    constexpr int KP = D + EPV;               // padded LDS row of the K tile
    constexpr int VP = S + EPV;               // padded LDS row of the V^T tile
    constexpr int NPT = (G * D + 255) / 256;  // outputs per thread
    constexpr int64_t BE = 2 * S * D;         // elements per block-unit
    __shared__ __attribute__((aligned(16))) T Ks[S * KP];
    __shared__ __attribute__((aligned(16))) T Vs[D * VP];
    __shared__ __attribute__((aligned(16))) float qs[G * D];
    __shared__ __attribute__((aligned(16))) float ps[G * S];
    __shared__ float m_sh[G], l_sh[G], a_sh[G];

    const int tid = threadIdx.x;
    const int r = blockIdx.y, chunk = blockIdx.x;
    const int b = r / dm.Hkv, g = r % dm.Hkv;
    const T *qr = static_cast<const T *>(a.q) + ((int64_t)b * dm.Hq + (int64_t)g * G) * D;
    for (int p = tid; p < G * D; p += 256) qs[p] = ldf(qr + p) * dm.scale;
    if (tid < G) { m_sh[tid] = -INFINITY; l_sh[tid] = 0.f; }
    float o[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i) o[i] = 0.f;

    const StepVals sv = a.dstep ? read_step(a.dstep, dm) : StepVals{a.n_tokens, a.n_cand, 0};
    const int cnt_e = a.n_list ? min(a.n_list[r], a.list_len) : a.list_len;
    const int e0 = chunk * a.cb, e1 = min(e0 + a.cb, a.list_len + a.with_newest);
    const float *er = a.e_tok + (int64_t)r * a.e_stride;

    for (int e = e0; e < e1; ++e) {
        const T *blk;
        int bid, valid;
        if (!resolve_entry<T>(a, sv, e, cnt_e, r, BE, blk, bid, valid))
            continue;  // uniform over the workgroup
        __syncthreads();  // the previous block's readers are done with LDS
        // the block's 16-byte vectors in stored order (coalesced), each to its
        // place in the row-major LDS tiles (the layout in common.h)
        constexpr int KV_VEC = S * D / EPV;
        for (int v = tid; v < KV_VEC; v += 256) {
            int row, c;
            kv_k_vec<T, D>(v, row, c);
            *reinterpret_cast<uint4 *>(Ks + row * KP + c) = reinterpret_cast<const uint4 *>(blk)[v];
        }
        for (int v = tid; v < KV_VEC; v += 256) {
            int row, c;
            kv_v_vec<T, D>(v, row, c);
            uint4 x = reinterpret_cast<const uint4 *>(blk + S * D)[v];
            if (valid < S) {
                // value slots of tokens from `valid` on (a partly filled
                // block) may hold anything; a zero weight times a NaN is a
                // NaN, so they enter as zeros
                T el[EPV];
                __builtin_memcpy(el, &x, sizeof(x));
#pragma unroll
                for (int m = 0; m < EPV; ++m)
                    if (vt_token_at(c + m) >= valid) el[m] = T{};
                __builtin_memcpy(&x, el, sizeof(x));
            }
            *reinterpret_cast<uint4 *>(Vs + row * VP + c) = x;
        }
        __syncthreads();

        // logits: thread <-> (head, token)
        for (int p = tid; p < G * S; p += 256) {
            const int h = p / S, t = p % S;
            float z = -INFINITY;
            if (t < valid) {
                float acc = 0.f;
#pragma unroll 4
                for (int d = 0; d < D; d += 8) {
                    float x[8];
                    Vec8<T>::load(Ks + t * KP + d, x);
                    const float4 q0 = *reinterpret_cast<const float4 *>(qs + h * D + d);
                    const float4 q1 = *reinterpret_cast<const float4 *>(qs + h * D + d + 4);
                    acc = fmaf(q0.x, x[0], acc); acc = fmaf(q0.y, x[1], acc);
                    acc = fmaf(q0.z, x[2], acc); acc = fmaf(q0.w, x[3], acc);
                    acc = fmaf(q1.x, x[4], acc); acc = fmaf(q1.y, x[5], acc);
                    acc = fmaf(q1.z, x[6], acc); acc = fmaf(q1.w, x[7], acc);
                }
                z = acc + er[(int64_t)bid * S + t];
            }
            ps[p] = z;
        }
        __syncthreads();

        // online softmax: wave <-> head, lane <-> token
        {
            const int wave = tid >> 6, lane = tid & 63;
            for (int h = wave; h < G; h += 4) {
                const float z = ps[h * S + lane];
                const float m_old = m_sh[h];
                const float m_new = fmaxf(m_old, wave_max(z));
                const float p = z == -INFINITY ? 0.f : __expf(z - m_new);
                const float sum = wave_sum(p);
                ps[h * S + lane] = p;
                if (lane == 0) {
                    const float alpha = m_old == -INFINITY ? 0.f : __expf(m_old - m_new);
                    a_sh[h] = alpha;
                    l_sh[h] = l_sh[h] * alpha + sum;
                    m_sh[h] = m_new;
                }
            }
        }
        __syncthreads();

        // P.V: thread <-> (head, dim); V^T positions 8j..8j+7 of half s hold
        // tokens 32s+4j..+3 and 32s+16+4j..+3
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int p = tid + i * 256;
            if (p < G * D) {
                const int h = p / D, d = p % D;
                float acc = o[i] * a_sh[h];
#pragma unroll 2
                for (int t = 0; t < S; t += 8) {
                    float x[8];
                    Vec8<T>::load(Vs + d * VP + t, x);
                    const int t0 = vt_token_at(t);
                    const float4 p0 = *reinterpret_cast<const float4 *>(ps + h * S + t0);
                    const float4 p1 = *reinterpret_cast<const float4 *>(ps + h * S + t0 + 16);
                    acc = fmaf(p0.x, x[0], acc); acc = fmaf(p0.y, x[1], acc);
                    acc = fmaf(p0.z, x[2], acc); acc = fmaf(p0.w, x[3], acc);
                    acc = fmaf(p1.x, x[4], acc); acc = fmaf(p1.y, x[5], acc);
                    acc = fmaf(p1.z, x[6], acc); acc = fmaf(p1.w, x[7], acc);
                }
                o[i] = acc;
            }
        }
    }
    __syncthreads();
    const int64_t base = ((int64_t)r * a.chunk_cap + a.chunk0 + chunk) * G;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const int p = tid + i * 256;
        if (p < G * D) a.ws_o[base * D + p] = o[i];
    }
    if (tid < G) {
        a.ws_ml[(base + tid) * 2 + 0] = m_sh[tid];
        a.ws_ml[(base + tid) * 2 + 1] = l_sh[tid];
    }
}

// With ev0 / ev1 (timing events), the launch goes through
// hipExtLaunchKernelGGL, which records them at the kernel's own start and end.
template <typename T, int D, int G>
hipError_t launch_decode_valu(const Dims &dm, const DecodePlan &pl, const DecodeArgs &a,
                              hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if (pl.n_chunks == 0) return hipSuccess;
    const dim3 grid(pl.n_chunks, dm.rows), block(256);
    if (ev0 || ev1)
        hipExtLaunchKernelGGL((decode_valu_kernel<T, D, G>), grid, block, 0, st, ev0, ev1, 0, dm, a);
    else
        hipLaunchKernelGGL((decode_valu_kernel<T, D, G>), grid, block, 0, st, dm, a);
    return hipGetLastError();
}

// Non-temporal K/V loads when a launch reads more KV than the 256 MB
// Infinity Cache holds: nothing it reads survives to the next step there
// anyway, and streamed whole-line fragments then arrive faster. Measured on
// the 64k workload (256 rows x 129 blocks, 1.08 GB per launch): 162 against
// 182 us; on the 32-layer offload step (512 rows x 65 cache slots per layer):
// 158 against 187 us. On the 32k workload (64 rows x 65 blocks, 136 MB, which
// the Infinity Cache keeps from step to step) the cached loads are faster:
// 23.0 against 24.2 us.
constexpr int64_t NT_MIN_BYTES = (int64_t)256 << 20;

template <int D, int G, bool NT>
hipError_t launch_decode_mfma_nt(const Dims &dm, const DecodePlan &pl, const DecodeArgs &a,
                                 hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    const dim3 grid(pl.n_chunks, dm.rows), block(64 * WAVES);
    if (ev0 || ev1)
        hipExtLaunchKernelGGL((decode_mfma_kernel<D, G, NT>), grid, block, 0, st, ev0, ev1, 0, dm, a);
    else
        hipLaunchKernelGGL((decode_mfma_kernel<D, G, NT>), grid, block, 0, st, dm, a);
    return hipGetLastError();
}

template <int D, int G>
hipError_t launch_decode_mfma(const Dims &dm, const DecodePlan &pl, const DecodeArgs &a,
                              hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
    if (pl.n_chunks == 0) return hipSuccess;
    const int64_t kv_bytes = (int64_t)dm.rows * (a.list_len + a.with_newest) * (2 * 64 * D) * 2;
    return kv_bytes > NT_MIN_BYTES ? launch_decode_mfma_nt<D, G, true>(dm, pl, a, st, ev0, ev1)
                                   : launch_decode_mfma_nt<D, G, false>(dm, pl, a, st, ev0, ev1);
}

template <typename T, int D, int G>
hipError_t launch_combine(const Dims &dm, int n_chunks, int chunk_cap, const float *ws_o,
                          const float *ws_ml, void *out, hipStream_t st, int32_t *dstep_adv) {
    hipLaunchKernelGGL((combine_kernel<T, D, G>), dim3(dm.rows, G), dim3(D), 0, st, dm, n_chunks,
                       chunk_cap, ws_o, ws_ml, static_cast<T *>(out), dstep_adv);
    return hipGetLastError();
}

#define NOSA_DEC_INST(T, D, G)                                                                 \
    template hipError_t launch_decode_valu<T, D, G>(const Dims &, const DecodePlan &,          \
                                                    const DecodeArgs &, hipStream_t,           \
                                                    hipEvent_t, hipEvent_t);                   \
    template hipError_t launch_combine<T, D, G>(const Dims &, int, int, const float *,         \
                                                const float *, void *, hipStream_t, int32_t *);
#define NOSA_DEC_ALLG(T, D)                                                                    \
    NOSA_DEC_INST(T, D, 1) NOSA_DEC_INST(T, D, 2) NOSA_DEC_INST(T, D, 3)                       \
    NOSA_DEC_INST(T, D, 4) NOSA_DEC_INST(T, D, 5) NOSA_DEC_INST(T, D, 6)                       \
    NOSA_DEC_INST(T, D, 7) NOSA_DEC_INST(T, D, 8)
NOSA_DEC_ALLG(float, 64)
NOSA_DEC_ALLG(bf16_t, 64)
NOSA_DEC_ALLG(bf16_t, 128)

#define NOSA_MFMA_INST(D, G)                                                                   \
    template hipError_t launch_decode_mfma<D, G>(const Dims &, const DecodePlan &,             \
                                                 const DecodeArgs &, hipStream_t, hipEvent_t,  \
                                                 hipEvent_t);
#define NOSA_MFMA_ALLG(D)                                                                      \
    NOSA_MFMA_INST(D, 1) NOSA_MFMA_INST(D, 2) NOSA_MFMA_INST(D, 3) NOSA_MFMA_INST(D, 4)        \
    NOSA_MFMA_INST(D, 5) NOSA_MFMA_INST(D, 6) NOSA_MFMA_INST(D, 7) NOSA_MFMA_INST(D, 8)
NOSA_MFMA_ALLG(64)
NOSA_MFMA_ALLG(128)

}  // namespace nosa
