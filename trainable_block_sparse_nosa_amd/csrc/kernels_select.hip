// Pooling, block scoring, dual selection, set difference and block fetch.
//
// NOSA technical summary, Methodology: "1. Algorithm: NOSA" (two-stage
// pooling, Gamma_e / Gamma_q dual selection, strict eviction, ED-DMA
// selection on pre-exponential scores) and "2. System: NOSI" (block-unit
// cache, set difference for block swapping, host-to-device copy kernels).
#include "kernels.h"

namespace nosa {

// ---------------------------------------------------------------------------
// Pooled keys are stored in the KV dtype T, V = 16 / sizeof(T) dimensions per
// 16-byte vector: kbar[row][D/V][m * max_blocks][V] (dimension vectors
// outermost, so a wave whose lanes hold consecutive sub-blocks reads 1 KiB
// contiguous per load).
// ---------------------------------------------------------------------------
template <typename T> struct KbarVec;
template <> struct KbarVec<float> {
    static constexpr int V = 4;
    __device__ __forceinline__ static void load(const float *p, float (&x)[4]) {
        const float4 v = *reinterpret_cast<const float4 *>(p);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
};
template <> struct KbarVec<bf16_t> {
    static constexpr int V = 8;
    __device__ __forceinline__ static void load(const bf16_t *p, float (&x)[8]) {
        const uint4 v = *reinterpret_cast<const uint4 *>(p);
        x[0] = bf_lo(v.x); x[1] = bf_hi(v.x); x[2] = bf_lo(v.y); x[3] = bf_hi(v.y);
        x[4] = bf_lo(v.z); x[5] = bf_hi(v.z); x[6] = bf_lo(v.w); x[7] = bf_hi(v.w);
    }
};

// x (double) rounded to the nearest bfloat16, ties to even, with one
// rounding: x is first rounded to float32 by rounding to odd (truncate, then
// set the last bit if anything was dropped), which float32's 16 extra bits
// make innocuous for the final round-to-nearest-even (Boldo and Melquiond,
// "Emulation of FMA and correctly rounded sums: proved algorithms using
// rounding to odd", IEEE Trans. Computers 57(4), 2008).
__device__ __forceinline__ bf16_t bf16_rne_from_double(double x) {
    float f = (float)x;
    if ((double)f != x) {
        uint32_t u = __float_as_uint(f);
        if (fabs((double)f) > fabs(x)) u -= 1u;  // rounded away from zero: step back
        f = __uint_as_float(u | 1u);
    }
    return f2bf(f);
}

// Sub-block mean of 16 keys in the storage type: float32 keys sum in float32;
// bfloat16 keys sum exactly in double (16 values with 8 significant bits) and
// the exact mean is rounded once to bfloat16.
template <typename T> __device__ __forceinline__ T pooled_mean(const T *k, int stride);
template <> __device__ __forceinline__ float pooled_mean<float>(const float *k, int stride) {
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) s += k[u * stride];
    return s * (1.0f / 16);
}
template <> __device__ __forceinline__ bf16_t pooled_mean<bf16_t>(const bf16_t *k, int stride) {
    double s = 0.0;
#pragma unroll
    for (int u = 0; u < 16; ++u) s += (double)bf2f(k[u * stride]);
    return bf16_rne_from_double(s * (1.0 / 16));
}

// ---------------------------------------------------------------------------
// Pool: one workgroup per (block, row). Sub-block means of the keys go to the
// kbar layout above; the eviction scores get mean-then-max pooling.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256)
pool_kernel(Dims dm, const T *__restrict__ kv, int64_t kv_row_blocks, int kv_first,
            const float *__restrict__ e_tok, int64_t e_stride, int blk_begin,
            T *__restrict__ kbar, float *__restrict__ e_blk) {
    constexpr int S = 64, SUB = 16, M = S / SUB, V = KbarVec<T>::V;
    static_assert(SUB == 16, "pooled_mean sums 16 tokens");
    __shared__ float emean[M];
    const int r = blockIdx.y;
    const int j = blk_begin + blockIdx.x;
    const T *K = kv + ((int64_t)r * kv_row_blocks + kv_first + blockIdx.x) * (int64_t)(2 * S * D);
    const int64_t ld_sb = (int64_t)M * dm.max_blocks;  // sub-blocks per dimension-vector plane
    T *kb = kbar + (int64_t)r * D * ld_sb;
    for (int p = threadIdx.x; p < M * D; p += blockDim.x) {
        const int i = p / D, d = p % D;
        kb[((int64_t)(d / V) * ld_sb + (int64_t)(M * j + i)) * V + (d % V)] =
            pooled_mean<T>(K + (i * SUB) * D + d, D);
    }
    if (threadIdx.x < M) {
        const float *e = e_tok + (int64_t)r * e_stride + (int64_t)j * S + threadIdx.x * SUB;
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < SUB; ++u) s += e[u];
        emean[threadIdx.x] = s * (1.0f / SUB);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float mx = emean[0];
#pragma unroll
        for (int i = 1; i < M; ++i) mx = fmaxf(mx, emean[i]);
        e_blk[(int64_t)r * dm.max_blocks + j] = mx;
    }
}

// ---------------------------------------------------------------------------
// Score: lane <-> sub-block. Each lane walks the head dimension one 16-byte
// vector at a time; a wave's loads cover 64 consecutive sub-blocks (1 KiB).
// The group's G dot products stay in registers; the block max over the 4
// sub-blocks is a DPP quad reduction, then the heads are summed.
// ---------------------------------------------------------------------------
template <typename T, int D, int G>
__global__ void __launch_bounds__(256)
score_kernel(Dims dm, const T *__restrict__ q, const T *__restrict__ kbar, int n_cand,
             float *__restrict__ s_q) {
    constexpr int M = 4, V = KbarVec<T>::V;
    __shared__ float qs[G][D];
    const int r = blockIdx.y;
    const int b = r / dm.Hkv, g = r % dm.Hkv;
    const T *qr = q + ((int64_t)b * dm.Hq + (int64_t)g * G) * D;
    for (int p = threadIdx.x; p < G * D; p += blockDim.x)
        (&qs[0][0])[p] = ldf(qr + p) * dm.scale;
    __syncthreads();

    const int nsb = M * n_cand;
    const int sb = blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t ld_sb = (int64_t)M * dm.max_blocks;
    const T *kb = kbar + (int64_t)r * D * ld_sb;
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
    if (sb < nsb) {
#pragma unroll 8
        for (int dv = 0; dv < D / V; ++dv) {
            float x[V];
            KbarVec<T>::load(kb + ((int64_t)dv * ld_sb + sb) * V, x);
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int u = 0; u < V; ++u) acc[h] = fmaf(qs[h][dv * V + u], x[u], acc[h]);
        }
    }
    // every lane takes part in the quad reductions (n_cand*4 keeps quads whole)
    float s = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) s += quad_max(acc[h]);
    if (sb < nsb && (sb & (M - 1)) == 0) s_q[(int64_t)r * dm.max_blocks + sb / M] = s;
}

// ---------------------------------------------------------------------------
// Select: one workgroup (8 waves) per row. Keys are 64-bit rank keys
// (orderable score << 32 | ~index), so a larger key ranks first and no two
// keys are equal; 0 marks "not a candidate".
//  * top-k with k <= 64: every thread holds its candidates' keys in registers
//    (candidate j = tid + 512 i). Each wave finds the smallest key T of its own
//    top-k by a most-significant-bit-first search with ballots and popcounts
//    (stopping as soon as exactly k of its keys are >= the prefix); its keys
//    >= T go to LDS; each of these <= 8k survivors then counts how many
//    survivors are larger, and the ones with fewer than k above them are the
//    row's top-k. No sorting, two barriers.
//  * top-k with k > 64 (an eviction budget above 64 at initialisation, or a
//    query budget above 64): bitonic sort of all keys in LDS.
//  * Gamma_e after initialisation: each new candidate in turn replaces the
//    lowest-ranked member if it ranks above it, else it is evicted.
//  * the ascending selection list comes from a popcount prefix scan.
//  * optionally the set difference against the block cache runs in the same
//    workgroup (wave 0), from the selection bitmap and the slot table alone.
// ---------------------------------------------------------------------------
constexpr int SELECT_THREADS = 512;
constexpr int SELECT_WAVES = SELECT_THREADS / 64;
constexpr int MAX_W = 128;   // 4096 blocks
constexpr int MAX_K = 128;
constexpr int WAVE_TOPK = 64;
constexpr int KEYS_PER_THREAD = 4096 / SELECT_THREADS;

__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Smallest key of the wave's top-k among the keys held in x[0..m) of every
// lane (0 = no key). Returns 0 when the wave holds at most k keys (then all
// of its non-zero keys qualify).
template <int M>
__device__ uint64_t wave_kth_key(const uint64_t (&x)[M], int k) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < M; ++i) n += __popcll(__ballot(x[i] != 0ull));
    if (n <= k) return 0ull;
    uint64_t t = 0ull;
    for (int b = 63; b >= 0; --b) {
        const uint64_t cand = t | (1ull << b);
        int c = 0;
#pragma unroll
        for (int i = 0; i < M; ++i) c += __popcll(__ballot(x[i] >= cand));
        if (c >= k) {
            t = cand;
            if (c == k) break;  // exactly the top-k are >= t
        }
    }
    return t;
}

// Top-k (k <= 64) of the keys x[0..M) held by every thread of the block:
// sets the selected indices' bits in `bits` (LDS). Returns nothing; the
// caller synchronises before reading `bits`.
template <int M>
__device__ void block_topk(const uint64_t (&x)[M], int k, uint64_t *surv, int *n_surv,
                           uint32_t *bits) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x == 0) *n_surv = 0;
    __syncthreads();
    const uint64_t t = wave_kth_key<M>(x, k);
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const bool keep = x[i] != 0ull && x[i] >= t;
        const uint64_t m = __ballot(keep);
        int base = 0;
        if (lane == 0 && m) base = atomicAdd(n_surv, __popcll(m));
        base = __shfl(base, 0, 64);
        if (keep) surv[base + __popcll(m & lt)] = x[i];
    }
    __syncthreads();
    // four threads per survivor, each counting the larger survivors in a
    // quarter of the list (two keys per 16-byte LDS read), quad-summed
    const int ns = *n_surv;
    const int q4 = ((ns + 7) / 8) * 2;  // keys per quarter, even
    for (int base = 0; base < ns * 4; base += blockDim.x) {
        const int i = (base + threadIdx.x) >> 2, part = threadIdx.x & 3;
        const uint64_t me = i < ns ? surv[i] : ~0ull;
        int above = 0;
        const int j0 = part * q4, j1 = min(j0 + q4, ns);
        int j = j0;
        for (; j + 1 < j1; j += 2) {
            const ulonglong2 two = *reinterpret_cast<const ulonglong2 *>(surv + j);
            above += (two.x > me) + (two.y > me);
        }
        if (j < j1) above += surv[j] > me;
        above += __shfl_xor(above, 1, 64);
        above += __shfl_xor(above, 2, 64);
        if (i < ns && part == 0 && above < k) {
            const int idx = key_index(me);
            atomicOr(&bits[idx >> 5], 1u << (idx & 31));
        }
    }
}

// Keys of candidates tid + 512 i (i < M) from key_of(j, i); then block_topk.
template <int M, typename KeyFn>
__device__ void topk_m(int n, int k, KeyFn key_of, uint64_t *surv, int *n_surv, uint32_t *bits) {
    uint64_t x[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int j = threadIdx.x + SELECT_THREADS * i;
        x[i] = j < n ? key_of(j, i) : 0ull;
    }
    block_topk<M>(x, k, surv, n_surv, bits);
}

// Dispatch on how many keys each thread holds (uniform over the block).
template <typename KeyFn>
__device__ void topk_dispatch(int n, int k, KeyFn key_of, uint64_t *surv, int *n_surv,
                              uint32_t *bits) {
    if (n <= SELECT_THREADS) topk_m<1>(n, k, key_of, surv, n_surv, bits);
    else if (n <= 2 * SELECT_THREADS) topk_m<2>(n, k, key_of, surv, n_surv, bits);
    else if (n <= 4 * SELECT_THREADS) topk_m<4>(n, k, key_of, surv, n_surv, bits);
    else topk_m<8>(n, k, key_of, surv, n_surv, bits);
}

__device__ void bitonic_desc(uint64_t *keys, int P) {
    for (int k2 = 2; k2 <= P; k2 <<= 1) {
        for (int j2 = k2 >> 1; j2 > 0; j2 >>= 1) {
            for (int i = threadIdx.x; i < P / 2; i += blockDim.x) {
                const int lo = 2 * i - (i & (j2 - 1));
                const int hi = lo + j2;
                const bool desc = (lo & k2) == 0;
                const uint64_t a = keys[lo], b = keys[hi];
                if ((a < b) == desc) {
                    keys[lo] = b;
                    keys[hi] = a;
                }
            }
            __syncthreads();
        }
    }
}

__device__ uint64_t block_min_u64(uint64_t v, uint64_t *red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = umin64(v, __shfl_xor(v, o, 64));
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    uint64_t m = red[0];
    for (int i = 1; i < nw; ++i) m = umin64(m, red[i]);
    __syncthreads();
    return m;
}

__device__ int block_sum_int(int v, int *red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    int s = 0;
    for (int i = 0; i < nw; ++i) s += red[i];
    __syncthreads();
    return s;
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

struct SwapArgs {
    int32_t *slot_block, *block_slot, *fetch_block, *fetch_slot, *n_fetch;
    uint64_t *counters;
};

struct ListArgs {
    int32_t *ge_list, *n_ge, *gq_list, *n_gq;  // n_ge null: not requested
};

// Set difference of one row, run by one wave. `bits` (LDS or global) is the
// selection bitmap; slot l of the cache holds slots[l] (lane l and l + 64,
// already loaded). `res` is an LDS bitmap of W words for the cached set.
// Fetch list = selected and not cached, ascending; free slots = empty or
// holding an unselected block, ascending; fetched block i goes to free slot
// i, leftover free slots become empty. Every output address is written once.
__device__ void swap_row(const Dims &dm, int r, const uint32_t *bits, int s0, int s1, uint64_t cnt,
                         uint32_t *res, int *fb, int *fs, int *fo, const SwapArgs &sw) {
    const int lane = threadIdx.x & 63, k = dm.k, W = dm.W;
    const uint64_t lt = lanemask_lt();
    for (int w = lane; w < W; w += 64) res[w] = 0u;
    wave_sync_lds();
    if (lane < k && s0 >= 0 && s0 < dm.max_blocks) atomicOr(&res[s0 >> 5], 1u << (s0 & 31));
    if (lane + 64 < k && s1 >= 0 && s1 < dm.max_blocks) atomicOr(&res[s1 >> 5], 1u << (s1 & 31));
    wave_sync_lds();
    // fetch list: set bits of (selected & ~cached), two words per lane, ascending
    int nf = 0, kept = 0;
    for (int base = 0; base < W; base += 128) {
        const int w0 = base + 2 * lane, w1 = w0 + 1;
        const uint32_t b0 = w0 < W ? bits[w0] : 0u, b1 = w1 < W ? bits[w1] : 0u;
        const uint32_t f0 = b0 & ~(w0 < W ? res[w0] : 0u);
        const uint32_t f1 = b1 & ~(w1 < W ? res[w1] : 0u);
        kept += __popc(b0 & ~f0) + __popc(b1 & ~f1);
        const int cnt = __popc(f0) + __popc(f1);
        int inc = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
        }
        int pos = nf + inc - cnt;
        uint32_t m = f0;
        while (m && pos < MAX_K) { fb[pos++] = w0 * 32 + __ffs(m) - 1; m &= m - 1u; }
        m = f1;
        while (m && pos < MAX_K) { fb[pos++] = w1 * 32 + __ffs(m) - 1; m &= m - 1u; }
        nf += __shfl(inc, 63, 64);
    }
    for (int o = 32; o > 0; o >>= 1) kept += __shfl_xor(kept, o, 64);
    nf = min(nf, k);
    // free slots, ascending
    int nfree = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int sl = lane + 64 * h;
        const int blk = h ? s1 : s0;
        bool fr = false;
        if (sl < k) fr = blk < 0 || blk >= dm.max_blocks || !((bits[blk >> 5] >> (blk & 31)) & 1u);
        const uint64_t m = __ballot(fr);
        if (fr) {
            const int at = nfree + __popcll(m & lt);
            fs[at] = sl;
            fo[at] = blk;
        }
        nfree += __popcll(m);
    }
    wave_sync_lds();
    int32_t *sbk = sw.slot_block + (int64_t)r * k;
    int32_t *bsl = sw.block_slot + (int64_t)r * dm.max_blocks;
    for (int i = lane; i < nfree; i += 64) {
        const int sl = fs[i], old = fo[i];
        if (old >= 0 && old < dm.max_blocks) bsl[old] = -1;
        if (i < nf) {
            sbk[sl] = fb[i];
            bsl[fb[i]] = sl;
        } else {
            sbk[sl] = -1;
        }
    }
    int32_t *fbo = sw.fetch_block + (int64_t)r * k;
    int32_t *fso = sw.fetch_slot + (int64_t)r * k;
    for (int i = lane; i < k; i += 64) {
        fbo[i] = i < nf ? fb[i] : -1;
        fso[i] = i < nf ? fs[i] : -1;
    }
    // cnt: lane 0 holds the running fetch count, lane 1 the running kept count
    if (lane == 0) {
        sw.n_fetch[r] = nf;
        sw.counters[2 * r] = cnt + (uint64_t)nf;
    } else if (lane == 1) {
        sw.counters[2 * r + 1] = cnt + (uint64_t)kept;
    }
}

__global__ void __launch_bounds__(SELECT_THREADS)
select_kernel(Dims dm, const float *__restrict__ s_q, const float *__restrict__ e_blk, int n_cand,
              int n_prev, int P, uint32_t *__restrict__ ge_bits, uint32_t *__restrict__ ev_bits,
              int32_t *__restrict__ sel, int32_t *__restrict__ n_sel,
              uint32_t *__restrict__ sel_bits, SwapArgs sw, ListArgs lists) {
    extern __shared__ uint64_t keys[];  // P keys, only when a budget exceeds 64
    __shared__ uint32_t ge[MAX_W], ev[MAX_W], sb[MAX_W], res[MAX_W];
    __shared__ __attribute__((aligned(16))) uint64_t surv[SELECT_WAVES * WAVE_TOPK + 2];
    __shared__ int n_surv;
    __shared__ uint64_t red64[SELECT_WAVES];
    __shared__ int red32[SELECT_WAVES];
    __shared__ int fb[MAX_K], fs[MAX_K], fo[MAX_K];
    __shared__ int woff[3 * (MAX_W + 1)];
    const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int W = dm.W;
    const float *E = e_blk + (int64_t)r * dm.max_blocks;
    const float *Sq = s_q + (int64_t)r * dm.max_blocks;
    uint32_t *ge_g = ge_bits + (int64_t)r * W;
    uint32_t *ev_g = ev_bits + (int64_t)r * W;

    // independent loads first: this thread's scores, the cache's slot table
    float sv[KEYS_PER_THREAD];
#pragma unroll
    for (int i = 0; i < KEYS_PER_THREAD; ++i) {
        const int j = tid + SELECT_THREADS * i;
        sv[i] = j < n_cand ? Sq[j] : 0.f;
    }
    int s0 = -1, s1 = -1;
    uint64_t cnt = 0ull;
    if (sw.slot_block && wave == 0) {
        if (lane < dm.k) s0 = sw.slot_block[(int64_t)r * dm.k + lane];
        if (lane + 64 < dm.k) s1 = sw.slot_block[(int64_t)r * dm.k + lane + 64];
        if (lane < 2) cnt = sw.counters[2 * r + lane];
    }

    // ---- Gamma_e ----
    if (n_prev < 0) {
        for (int w = tid; w < W; w += nt) { ge[w] = 0u; ev[w] = 0u; }
        __syncthreads();
        const int ke = min(dm.k_e, n_cand);
        if (ke > 0 && dm.k_e <= WAVE_TOPK) {
            topk_dispatch(n_cand, ke, [&](int j, int) { return rank_key(E[j], j); }, surv,
                          &n_surv, ge);
        } else if (ke > 0) {
            for (int i = tid; i < P; i += nt) keys[i] = i < n_cand ? rank_key(E[i], i) : 0ull;
            __syncthreads();
            bitonic_desc(keys, P);
            for (int i = tid; i < ke; i += nt) {
                const int j = key_index(keys[i]);
                atomicOr(&ge[j >> 5], 1u << (j & 31));
            }
        }
        __syncthreads();
        for (int w = tid; w < W; w += nt) {
            const int lo = w * 32;
            const uint32_t cand = lo + 32 <= n_cand ? 0xFFFFFFFFu
                                : (lo >= n_cand ? 0u : ((1u << (n_cand - lo)) - 1u));
            ev[w] = cand & ~ge[w];
        }
        __syncthreads();
    } else {
        // state only ever holds blocks that were candidates at the previous step
        for (int w = tid; w < W; w += nt) {
            const int lo = w * 32;
            const uint32_t prev = lo + 32 <= n_prev ? 0xFFFFFFFFu
                                : (lo >= n_prev ? 0u : ((1u << (n_prev - lo)) - 1u));
            ge[w] = ge_g[w] & prev;
            ev[w] = ev_g[w] & prev;
        }
        __syncthreads();
        for (int x = n_prev; x < n_cand; ++x) {
            int c = 0;
            for (int w = tid; w < W; w += nt) c += __popc(ge[w]);
            const int count = block_sum_int(c, red32);
            if (count < dm.k_e) {
                if (tid == 0) ge[x >> 5] |= 1u << (x & 31);
            } else if (dm.k_e > 0) {
                uint64_t mn = ~0ull;
                for (int w = tid; w < W; w += nt) {
                    uint32_t bits = ge[w];
                    while (bits) {
                        const int j = w * 32 + __ffs(bits) - 1;
                        bits &= bits - 1u;
                        mn = umin64(mn, rank_key(E[j], j));
                    }
                }
                mn = block_min_u64(mn, red64);
                if (tid == 0) {
                    if (rank_key(E[x], x) > mn) {
                        const int j = key_index(mn);
                        ge[j >> 5] &= ~(1u << (j & 31));
                        ev[j >> 5] |= 1u << (j & 31);
                        ge[x >> 5] |= 1u << (x & 31);
                    } else {
                        ev[x >> 5] |= 1u << (x & 31);
                    }
                }
            } else if (tid == 0) {
                ev[x >> 5] |= 1u << (x & 31);
            }
            __syncthreads();
        }
    }

    // ---- Gamma_q: best k_q of the candidates outside Gamma_e ----
    int ne_loc = 0;
    for (int w = tid; w < W; w += nt) {
        sb[w] = ge[w];
        ne_loc += __popc(ge[w]);
    }
    const int n_e = block_sum_int(ne_loc, red32);  // also orders the sb copies
    const int kq = min(dm.k_q, n_cand - n_e);
    if (kq > 0 && dm.k_q <= WAVE_TOPK) {
        topk_dispatch(n_cand, kq, [&](int j, int i) -> uint64_t {
            return ((ge[j >> 5] >> (j & 31)) & 1u) ? 0ull : rank_key(sv[i], j);
        }, surv, &n_surv, sb);
    } else if (kq > 0) {
        for (int i = tid; i < P; i += nt) {
            const bool ok = i < n_cand && !((ge[i >> 5] >> (i & 31)) & 1u);
            keys[i] = ok ? rank_key(Sq[i], i) : 0ull;
        }
        __syncthreads();
        bitonic_desc(keys, P);
        for (int i = tid; i < kq; i += nt) {
            const int j = key_index(keys[i]);
            atomicOr(&sb[j >> 5], 1u << (j & 31));
        }
    }
    __syncthreads();

    // ---- state and the ascending selection ----
    for (int w = tid; w < W; w += nt) {
        ge_g[w] = ge[w];
        ev_g[w] = ev[w];
        sel_bits[(int64_t)r * W + w] = sb[w];
    }
    // word offsets of the selection, of Gamma_e and of Gamma_q (one wave scans
    // <= 128 words, two per lane)
    if (wave == 0) {
#pragma unroll
        for (int li = 0; li < 3; ++li) {
            auto word = [&](int w) -> uint32_t {
                if (w >= W) return 0u;
                return li == 0 ? sb[w] : (li == 1 ? ge[w] : (sb[w] & ~ge[w]));
            };
            const uint32_t w0 = word(2 * lane), w1 = word(2 * lane + 1);
            const int cnt = __popc(w0) + __popc(w1);
            int inc = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(inc, o, 64);
                if (lane >= o) inc += y;
            }
            int *wo = woff + li * (MAX_W + 1);
            if (2 * lane < W) wo[2 * lane] = inc - cnt;
            if (2 * lane + 1 < W) wo[2 * lane + 1] = inc - cnt + __popc(w0);
            if (lane == 63) wo[MAX_W] = inc;
        }
    }
    __syncthreads();
    // every thread places its own selected candidates (union, and each part
    // when asked for)
    int32_t *out = sel + (int64_t)r * dm.k;
    const int total = min(woff[MAX_W], dm.k);
    const int *wo_e = woff + (MAX_W + 1), *wo_q = woff + 2 * (MAX_W + 1);
    for (int j = tid; j < n_cand; j += nt) {
        const uint32_t word = sb[j >> 5];
        const uint32_t bit = 1u << (j & 31), below = bit - 1u;
        if (word & bit) {
            const int pos = woff[j >> 5] + __popc(word & below);
            if (pos < dm.k) out[pos] = j;
            if (lists.n_ge) {
                const uint32_t we = ge[j >> 5];
                if (we & bit) {
                    const int pe = wo_e[j >> 5] + __popc(we & below);
                    if (pe < dm.k_e) lists.ge_list[(int64_t)r * dm.k_e + pe] = j;
                } else {
                    const uint32_t wq = word & ~we;
                    const int pq = wo_q[j >> 5] + __popc(wq & below);
                    if (pq < dm.k_q) lists.gq_list[(int64_t)r * dm.k_q + pq] = j;
                }
            }
        }
    }
    for (int i = total + tid; i < dm.k; i += nt) out[i] = -1;
    if (lists.n_ge) {
        const int ne = min(wo_e[MAX_W], dm.k_e), nq = min(wo_q[MAX_W], dm.k_q);
        for (int i = ne + tid; i < dm.k_e; i += nt) lists.ge_list[(int64_t)r * dm.k_e + i] = -1;
        for (int i = nq + tid; i < dm.k_q; i += nt) lists.gq_list[(int64_t)r * dm.k_q + i] = -1;
        if (tid == 0) {
            lists.n_ge[r] = ne;
            lists.n_gq[r] = nq;
        }
    }
    if (tid == 0) n_sel[r] = total;
    if (sw.slot_block && wave == 0) swap_row(dm, r, sb, s0, s1, cnt, res, fb, fs, fo, sw);
}

// Stand-alone set difference: one wave per row, selection bitmap and slot
// table from global memory.
__global__ void __launch_bounds__(64)
swap_kernel(Dims dm, const uint32_t *__restrict__ sel_bits, SwapArgs sw) {
    __shared__ uint32_t res[MAX_W];
    __shared__ int fb[MAX_K], fs[MAX_K], fo[MAX_K];
    const int r = blockIdx.x, lane = threadIdx.x;
    const int s0 = lane < dm.k ? sw.slot_block[(int64_t)r * dm.k + lane] : -1;
    const int s1 = lane + 64 < dm.k ? sw.slot_block[(int64_t)r * dm.k + lane + 64] : -1;
    const uint64_t cnt = lane < 2 ? sw.counters[2 * r + lane] : 0ull;
    swap_row(dm, r, sel_bits + (int64_t)r * dm.W, s0, s1, cnt, res, fb, fs, fo, sw);
}

// ---------------------------------------------------------------------------
// Fetch: one workgroup per (list entry, row); entries past n_fetch exit.
// Each thread keeps eight 16-byte loads in flight before storing them.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
fetch_kernel(const u32x4 *__restrict__ src, int64_t src_row_blocks, const int32_t *__restrict__ fblk,
             const int32_t *__restrict__ fslot, const int32_t *__restrict__ nfetch, int k,
             u32x4 *__restrict__ dst, int64_t dst_row_blocks, int vec_per_block) {
    const int r = blockIdx.y, i = blockIdx.x;
    if (i >= nfetch[r]) return;
    const int b = fblk[(int64_t)r * k + i];
    const int s = fslot[(int64_t)r * k + i];
    const u32x4 *sp = src + ((int64_t)r * src_row_blocks + b) * vec_per_block;
    u32x4 *dp = dst + ((int64_t)r * dst_row_blocks + s) * vec_per_block;
    for (int base = 0; base < vec_per_block; base += 8 * 256) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int idx = base + u * 256 + threadIdx.x;
            if (idx < vec_per_block) v[u] = __builtin_nontemporal_load(sp + idx);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int idx = base + u * 256 + threadIdx.x;
            if (idx < vec_per_block) dp[idx] = v[u];
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename T, int D>
hipError_t launch_pool(const Dims &dm, const void *kv, int64_t kv_row_blocks, int kv_first,
                       const float *e_tok, int64_t e_stride, int blk_begin, int blk_end,
                       void *kbar, float *e_blk, hipStream_t st) {
    dim3 grid(blk_end - blk_begin, dm.rows);
    hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(256), 0, st, dm,
                       static_cast<const T *>(kv), kv_row_blocks, kv_first, e_tok, e_stride,
                       blk_begin, static_cast<T *>(kbar), e_blk);
    return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t launch_score(const Dims &dm, const void *q, const void *kbar, int n_cand, float *s_q,
                        hipStream_t st) {
    dim3 grid((4 * n_cand + 255) / 256, dm.rows);
    hipLaunchKernelGGL((score_kernel<T, D, G>), grid, dim3(256), 0, st, dm,
                       static_cast<const T *>(q), static_cast<const T *>(kbar), n_cand, s_q);
    return hipGetLastError();
}

hipError_t launch_select(const Dims &dm, const float *s_q, const float *e_blk, int n_cand,
                         int n_prev, uint32_t *ge, uint32_t *ev, int32_t *sel, int32_t *n_sel,
                         uint32_t *sel_bits, const SwapPtrs *swap, const SelectLists *parts,
                         hipStream_t st) {
    // LDS keys only when a budget is above what the register top-k holds
    int P = 0;
    if ((n_prev < 0 && dm.k_e > WAVE_TOPK) || dm.k_q > WAVE_TOPK) {
        P = 2;
        while (P < n_cand) P <<= 1;
    }
    SwapArgs sw{};
    if (swap) {
        sw.slot_block = swap->slot_block;
        sw.block_slot = swap->block_slot;
        sw.fetch_block = swap->fetch_block;
        sw.fetch_slot = swap->fetch_slot;
        sw.n_fetch = swap->n_fetch;
        sw.counters = swap->counters;
    }
    ListArgs li{};
    if (parts) li = ListArgs{parts->ge_list, parts->n_ge, parts->gq_list, parts->n_gq};
    hipLaunchKernelGGL(select_kernel, dim3(dm.rows), dim3(SELECT_THREADS), P * sizeof(uint64_t),
                       st, dm, s_q, e_blk, n_cand, n_prev, P, ge, ev, sel, n_sel, sel_bits, sw, li);
    return hipGetLastError();
}

hipError_t launch_swap(const Dims &dm, const int32_t *sel, const int32_t *n_sel,
                       const uint32_t *sel_bits, const SwapPtrs &swap, hipStream_t st) {
    (void)sel;
    (void)n_sel;  // the bitmap carries the same selection
    SwapArgs sw{swap.slot_block, swap.block_slot, swap.fetch_block, swap.fetch_slot, swap.n_fetch,
                swap.counters};
    hipLaunchKernelGGL(swap_kernel, dim3(dm.rows), dim3(64), 0, st, dm, sel_bits, sw);
    return hipGetLastError();
}

hipError_t launch_fetch(const Dims &dm, const void *src, int64_t src_row_blocks,
                        const int32_t *fblk, const int32_t *fslot, const int32_t *nfetch,
                        int max_fetch, void *dst, int64_t dst_row_blocks, hipStream_t st) {
    const int elem = dm.dtype == NOSA_BF16 ? 2 : 4;
    const int vec = 2 * dm.S * dm.D * elem / 16;
    dim3 grid(max_fetch, dm.rows);
    hipLaunchKernelGGL(fetch_kernel, grid, dim3(256), 0, st, static_cast<const u32x4 *>(src),
                       src_row_blocks, fblk, fslot, nfetch, dm.k, static_cast<u32x4 *>(dst),
                       dst_row_blocks, vec);
    return hipGetLastError();
}

#define NOSA_POOL_INST(T, D)                                                                   \
    template hipError_t launch_pool<T, D>(const Dims &, const void *, int64_t, int,            \
                                          const float *, int64_t, int, int, void *, float *,   \
                                          hipStream_t);
NOSA_POOL_INST(float, 64)
NOSA_POOL_INST(float, 128)
NOSA_POOL_INST(bf16_t, 64)
NOSA_POOL_INST(bf16_t, 128)

#define NOSA_SCORE_INST(T, D, G)                                                               \
    template hipError_t launch_score<T, D, G>(const Dims &, const void *, const void *, int,   \
                                              float *, hipStream_t);
#define NOSA_SCORE_ALLG(T, D)                                                                  \
    NOSA_SCORE_INST(T, D, 1) NOSA_SCORE_INST(T, D, 2) NOSA_SCORE_INST(T, D, 3)                 \
    NOSA_SCORE_INST(T, D, 4) NOSA_SCORE_INST(T, D, 5) NOSA_SCORE_INST(T, D, 6)                 \
    NOSA_SCORE_INST(T, D, 7) NOSA_SCORE_INST(T, D, 8)
NOSA_SCORE_ALLG(float, 64)
NOSA_SCORE_ALLG(float, 128)
NOSA_SCORE_ALLG(bf16_t, 64)
NOSA_SCORE_ALLG(bf16_t, 128)

}  // namespace nosa
