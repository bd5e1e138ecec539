// Pooling, block scoring, dual selection, set difference and block fetch.
//
// NOSA technical summary, Methodology: "1. Algorithm: NOSA" (two-stage
// pooling, Gamma_e / Gamma_q dual selection, strict eviction, ED-DMA
// selection on pre-exponential scores) and "2. System: NOSI" (block-unit
// cache, set difference for block swapping, host-to-device copy kernels).
#include "kernels.h"

#include <algorithm>

namespace nosa {

// ---------------------------------------------------------------------------
// Pooled keys are stored in the pooled dtype TK (float32 by default: the
// exact sub-block means rounded once; bfloat16 for the model-dtype variant),
// V = 16 / sizeof(TK) dimensions per 16-byte vector, grouped by quads of
// blocks (16 sub-blocks): kbar[row][Q][D/V][16][V], Q = ceil(max_blocks / 4);
// sub-block sb = 4 j + i of block j is slot sb % 16 of quad sb / 16. A quad is
// 16 * D elements in one piece: for bfloat16 laid out as the A operand tiles
// of a 16 x 16 x 32 MFMA want them (one load instruction of a wave, 16
// sub-blocks x 4 dimension vectors, reads 1 KiB contiguous); for float32 a
// wave's 64 lanes (one sub-block each) read 4 pieces of 256 B per load.
// ---------------------------------------------------------------------------
template <typename T> struct KbarVec;
template <> struct KbarVec<float> {
    static constexpr int V = 4;
    __device__ __forceinline__ static void unpack(const uint4 &v, float (&x)[4]) {
        x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
        x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
    }
    __device__ __forceinline__ static void load(const float *p, float (&x)[4]) {
        unpack(*reinterpret_cast<const uint4 *>(p), x);
    }
};
template <> struct KbarVec<bf16_t> {
    static constexpr int V = 8;
    __device__ __forceinline__ static void unpack(const uint4 &v, float (&x)[8]) {
        x[0] = bf_lo(v.x); x[1] = bf_hi(v.x); x[2] = bf_lo(v.y); x[3] = bf_hi(v.y);
        x[4] = bf_lo(v.z); x[5] = bf_hi(v.z); x[6] = bf_lo(v.w); x[7] = bf_hi(v.w);
    }
    __device__ __forceinline__ static void load(const bf16_t *p, float (&x)[8]) {
        unpack(*reinterpret_cast<const uint4 *>(p), x);
    }
};

// A 16-byte vector as floats (4 float32 or 8 bfloat16).
template <typename T>
__device__ __forceinline__ void unpack16(const u32x4 &v, float (&x)[16 / sizeof(T)]) {
    KbarVec<T>::unpack(uint4{v.x, v.y, v.z, v.w}, x);
}

// Element offset of dimension vector dv of sub-block sb in row r.
template <typename T, int D>
__device__ __forceinline__ int64_t kbar_vec(const Dims &dm, int r, int sb, int dv) {
    constexpr int V = KbarVec<T>::V;
    const int64_t quads = (dm.max_blocks + 3) / 4;
    return (((int64_t)r * quads + (sb >> 4)) * (D / V) + dv) * (16 * V) + (int64_t)(sb & 15) * V;
}

// Sub-block mean of 16 keys of type T (key u from get(u)) in the pooled type
// TK: the keys are summed in order in double (exact for bfloat16 keys, 16
// values with 8 significant bits; for float32 keys within one rounding of
// double) and the mean is rounded once, to the nearest float32 or to the
// nearest bfloat16. Every caller gets identical bits.
template <typename T> __device__ __forceinline__ double dbl(T v);
template <> __device__ __forceinline__ double dbl<float>(float v) { return (double)v; }
template <> __device__ __forceinline__ double dbl<bf16_t>(bf16_t v) { return (double)bf2f(v); }

template <typename T, typename TK, typename Get>
__device__ __forceinline__ TK pooled_mean_of(Get get) {
    double s = 0.0;
#pragma unroll
    for (int u = 0; u < 16; ++u) s += dbl<T>(get(u));
    const double mean = s * (1.0 / 16);
    if constexpr (std::is_same_v<TK, float>) return (float)mean;
    else return bf16_rne_from_double(mean);
}

// Write the pooled keys of block j of row r, run by a whole workgroup of 256
// threads: mean_at(i, d) gives dimension d of sub-block i's mean in the pooled
// type. With certified scoring (bfloat16 KV, float32 pooled keys; kbar's
// regions in common.h) each mean's bfloat16 rounding goes to the shadow and
// the block's radius r = max over its sub-blocks of ||shadow - mean||_2 +
// 2^-14 ||mean||_2, enlarged by 2^-10 for the float32 sums behind it. For any
// query q, the score of a sub-block from the shadow then differs from the
// float32 score by at most scale * ||q||_2 * r: the first term bounds
// q . (shadow - mean) (Cauchy-Schwarz), the second the rounding of the two
// float32 dot products of D <= 128 terms ((2 D + 19) 2^-24 < 2^-14 of
// ||q|| ||mean||, head sum included). Sums of squares reduce in a fixed
// order, so the radius is the same bits on every run.
template <typename T, typename TK, int D, typename MeanAt>
__device__ __forceinline__ void pool_write(const Dims &dm, TK *kbar, int r, int j, MeanAt mean_at) {
    constexpr int M = 4, V = KbarVec<TK>::V, NW = 256 / 64;
    constexpr bool CERT = std::is_same_v<T, bf16_t> && std::is_same_v<TK, float>;
    float dd[M], xx[M];
#pragma unroll
    for (int i = 0; i < M; ++i) dd[i] = xx[i] = 0.f;
#pragma unroll
    for (int k = 0; k < M * D / 256; ++k) {
        const int p = threadIdx.x + 256 * k;
        const int i = p / D, d = p % D;
        const TK x = mean_at(i, d);
        kbar[kbar_vec<TK, D>(dm, r, M * j + i, d / V) + (d % V)] = x;
        if constexpr (CERT) {
            bf16_t *shadow = reinterpret_cast<bf16_t *>(reinterpret_cast<char *>(kbar) +
                                                        kbar_shadow_offset(dm));
            const bf16_t xb = f2bf(x);
            shadow[kbar_vec<bf16_t, D>(dm, r, M * j + i, d / 8) + (d % 8)] = xb;
            const float dl = bf2f(xb) - x;  // exact: x minus its rounding
#pragma unroll
            for (int ii = 0; ii < M; ++ii)
                if (ii == i) {
                    dd[ii] = fmaf(dl, dl, dd[ii]);
                    xx[ii] = fmaf(x, x, xx[ii]);
                }
        }
    }
    if constexpr (CERT) {
        __shared__ float red[2 * M][NW];
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int i = 0; i < M; ++i) {
            const float a = wave_sum(dd[i]), b = wave_sum(xx[i]);
            if (lane == 0) {
                red[i][wave] = a;
                red[M + i][wave] = b;
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            float rad = 0.f;
#pragma unroll
            for (int i = 0; i < M; ++i) {
                float a = 0.f, b = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    a += red[i][w];
                    b += red[M + i][w];
                }
                rad = fmaxf(rad, sqrtf(a) + sqrtf(b) * (1.0f / 16384.0f));
            }
            float *radius = reinterpret_cast<float *>(reinterpret_cast<char *>(kbar) +
                                                      kbar_radius_offset(dm));
            radius[(int64_t)r * dm.max_blocks + j] = rad * (1.0f + 1.0f / 1024.0f);
        }
    }
}

// ---------------------------------------------------------------------------
// Pool: one workgroup per (block, row). Sub-block means of the keys go to the
// kbar layout above; the eviction scores get mean-then-max pooling.
// ---------------------------------------------------------------------------
template <typename T, typename TK, int D>
__global__ void __launch_bounds__(256)
pool_kernel(Dims dm, const T *__restrict__ kv, int64_t kv_row_blocks, int kv_first,
            const float *__restrict__ e_tok, int64_t e_stride, int blk_begin,
            TK *__restrict__ kbar, float *__restrict__ e_blk, const int32_t *__restrict__ dstep) {
    constexpr int S = 64, SUB = 16, M = S / SUB, V = KbarVec<TK>::V;
    static_assert(SUB == 16, "pooled_mean sums 16 tokens");
    __shared__ float emean[M];
    const int r = blockIdx.y;
    int j = blk_begin + blockIdx.x, src = kv_first + blockIdx.x;
    if (dstep) {
        // the blocks completed since the previous step: n_cand_prev .. n_cand - 1
        const StepVals sv = read_step(dstep, dm);
        if (sv.n_prev < 0 || sv.n_prev + (int)blockIdx.x >= sv.n_cand) return;
        j = src = sv.n_prev + blockIdx.x;
    }
    const T *K = kv + ((int64_t)r * kv_row_blocks + src) * (int64_t)(2 * S * D);
    static_assert(V > 0, "pooled-key vector width");
    pool_write<T, TK, D>(dm, kbar, r, j, [&](int i, int d) {
        return pooled_mean_of<T, TK>([&](int u) { return K[kv_k_off<T, D>(i * SUB + u, d)]; });
    });
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
// Score on the VALU (float32 pooled keys): lane <-> sub-block. Each lane walks
// the head dimension one 16-byte vector at a time; a wave's loads cover 64
// consecutive sub-blocks. The group's G dot products stay in registers
// (float32 FMAs of the queries, of type TQ, and the pooled keys, of type TK);
// the block max over the 4 sub-blocks is a DPP quad reduction, then the heads
// are summed. With dstep, n_cand comes from the step record (the grid covers
// the capacity; workgroups past the candidates exit at once).
// ---------------------------------------------------------------------------
template <typename TQ, typename TK, int D, int G>
__global__ void __launch_bounds__(256)
score_kernel(Dims dm, const TQ *__restrict__ q, const TK *__restrict__ kbar, int n_cand,
             float *__restrict__ s_q, const int32_t *__restrict__ dstep) {
    constexpr int M = 4, V = KbarVec<TK>::V;
    if (dstep) n_cand = read_step(dstep, dm).n_cand;
    const int nsb = M * n_cand;
    if ((int)(blockIdx.x * blockDim.x) >= nsb) return;
    __shared__ float qs[G][D];
    const int r = blockIdx.y;
    const int b = r / dm.Hkv, g = r % dm.Hkv;
    const TQ *qr = q + ((int64_t)b * dm.Hq + (int64_t)g * G) * D;
    for (int p = threadIdx.x; p < G * D; p += blockDim.x)
        (&qs[0][0])[p] = ldf(qr + p) * dm.scale;
    __syncthreads();

    const int sb = blockIdx.x * blockDim.x + threadIdx.x;
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
    if (sb < nsb) {
#pragma unroll 8
        for (int dv = 0; dv < D / V; ++dv) {
            float x[V];
            KbarVec<TK>::load(kbar + kbar_vec<TK, D>(dm, r, sb, dv), x);
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
//    top-k by a most-significant-bit-first search with ballots and popcounts,
//    two bits per step with one or two keys per lane, one bit with more
//    (stopping as soon as exactly k of its keys are >= the prefix); its keys
//    >= T go to LDS; then the survivors' ranks among themselves are counted
//    by all threads at once (up to 8 per survivor), and the ones with fewer
//    than k above them are the row's top-k. No sorting, two barriers.
//  * top-k with k > 64 (an eviction budget above 64 at initialisation, or a
//    query budget above 64): bitonic sort of all keys in LDS.
//  * Gamma_e after initialisation: each new candidate in turn replaces the
//    lowest-ranked member if it ranks above it, else it is evicted.
//  * the ascending selection list comes from a popcount prefix scan (DPP).
//  * optionally the set difference against the block cache runs in the same
//    workgroup (wave 1, beside wave 0's lists), from the selection bitmap and
//    the slot table alone.
// ---------------------------------------------------------------------------
constexpr int SELECT_THREADS = 512;
constexpr int SELECT_WAVES = SELECT_THREADS / 64;
constexpr int MAX_W = 128;   // 4096 blocks
constexpr int MAX_K = 128;
constexpr int WAVE_TOPK = 64;
constexpr int KEYS_PER_THREAD = 4096 / SELECT_THREADS;
static_assert(MAX_W <= SELECT_THREADS, "one bitmap word per thread");
static_assert(SELECT_WAVES >= 2, "the set difference runs on wave 1 beside wave 0's lists");

__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Inclusive prefix sum over the 64 lanes of a wave on DPP: a log-step scan
// inside each row of 16 lanes (row_shr 1, 2, 4, 8; lanes shifted in from
// outside the row read 0), then the row totals carried across rows with the
// GFX9 row broadcasts (lane 15 of rows 0 and 2 into rows 1 and 3, then lane
// 31 into rows 2 and 3). Every lane must be active.
__device__ __forceinline__ int wave_incl_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Smallest key of the wave's top-k among the keys held in x[0..M) of every
// lane (0 = no key). When the wave holds at most k keys, all of them qualify
// and the smallest is returned. Otherwise a most-significant-bit-first search
// builds the largest prefix value t with at least k keys >= t and stops early
// once exactly k keys are >= t. With one or two keys per lane it takes two
// bits per step (the three candidate extensions are counted independently, so
// their ballots overlap); with more keys per lane the three-fold ballots cost
// more than the halved chain saves, and it takes one bit per step.
template <int M>
__device__ uint64_t wave_kth_key(const uint64_t (&x)[M], int k) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < M; ++i) n += __popcll(__ballot(x[i] != 0ull));
    if (n <= k) {
        // every key qualifies: the smallest one (~0 when there is none)
        uint64_t mn = ~0ull;
#pragma unroll
        for (int i = 0; i < M; ++i)
            if (x[i] != 0ull) mn = umin64(mn, x[i]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mn = umin64(mn, __shfl_xor(mn, o, 64));
        return mn;
    }
    uint64_t t = 0ull;
    if constexpr (M > 2) {
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
    for (int b = 62; b >= 0; b -= 2) {
        const uint64_t c3 = t | (3ull << b), c2 = t | (2ull << b), c1 = t | (1ull << b);
        int n3 = 0, n2 = 0, n1 = 0;
#pragma unroll
        for (int i = 0; i < M; ++i) {
            n3 += __popcll(__ballot(x[i] >= c3));
            n2 += __popcll(__ballot(x[i] >= c2));
            n1 += __popcll(__ballot(x[i] >= c1));
        }
        // n3 <= n2 <= n1: extend by the largest pair of bits that keeps k keys
        int c;
        if (n3 >= k) { t = c3; c = n3; }
        else if (n2 >= k) { t = c2; c = n2; }
        else if (n1 >= k) { t = c1; c = n1; }
        else c = -1;
        if (c == k) break;  // exactly the top-k are >= t
    }
    return t;
}

// Top-k (k <= 64) of the keys x[0..M) held by every thread of the block:
// sets the selected indices' bits in `bits` (LDS). Returns nothing; the
// caller synchronises before reading `bits`.
// Each wave keeps its own top k as survivors (at most 8k): every key of the
// row's top k is among them, since it has fewer than k keys of the row, so
// of its wave, above it. A survivor is then selected iff fewer than k
// survivors exceed it: a row top-k key has fewer than k keys of the row above
// it at all, and any other survivor has the k row top-k keys, all survivors,
// above it. Keys are unique (the index is part of the key), so the count is
// exact. The counts run in parallel: P threads per survivor (P = 8, 4, 2 or
// 1 as the survivors fill 64, 128, 256 or 512), each over every P-th run of
// 8 survivors (two 16-byte LDS reads per 4 keys; the array is zero-filled
// first, and a zero key exceeds nothing), summed across the P adjacent lanes.
template <int M>
__device__ void block_topk(const uint64_t (&x)[M], int k, uint64_t *surv, int *n_surv,
                           uint32_t *bits) {
    const int lane = threadIdx.x & 63;
    static_assert(SELECT_THREADS <= SELECT_WAVES * WAVE_TOPK, "one zero per thread covers surv");
    surv[threadIdx.x] = 0ull;
    if (threadIdx.x == 0) *n_surv = 0;
    __syncthreads();
    // each wave's own top-k go to LDS: together they hold the row's top-k
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
    const int ns = *n_surv;  // <= SELECT_WAVES * k <= SELECT_THREADS
    const int lp = ns <= 64 ? 3 : ns <= 128 ? 2 : ns <= 256 ? 1 : 0;  // log2 P
    const int s = threadIdx.x >> lp, part = threadIdx.x & ((1 << lp) - 1);
    const uint64_t mine = s < ns ? surv[s] : ~0ull;
    // runs of 8 keys up to a whole number of rounds over the P parts (<= 512)
    const int runs = ((ns + (8 << lp) - 1) >> (3 + lp)) << lp;
    const ulonglong2 *sv2 = reinterpret_cast<const ulonglong2 *>(surv);
    int above = 0;
    for (int c = part; c < runs; c += 1 << lp) {
        ulonglong2 y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) y[u] = sv2[4 * c + u];
#pragma unroll
        for (int u = 0; u < 4; ++u) above += (y[u].x > mine ? 1 : 0) + (y[u].y > mine ? 1 : 0);
    }
    // sum over the P lanes of this survivor (aligned groups of P lanes)
    if (lp >= 1) above += __shfl_xor(above, 1, 64);
    if (lp >= 2) above += __shfl_xor(above, 2, 64);
    if (lp >= 3) above += __shfl_xor(above, 4, 64);
    if (s < ns && part == 0 && above < k) {
        const int idx = key_index(mine);
        atomicOr(&bits[idx >> 5], 1u << (idx & 31));
    }
}

// Keys of candidates tid + 512 i (i < M) from key_of(j, i); then block_topk.
template <int M, typename KeyFn>
__device__ void topk_m(int n, int k, KeyFn key_of, uint64_t *surv, int *n_surv,
                       uint32_t *bits) {
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
        const int inc = wave_incl_sum(cnt);
        int pos = nf + inc - cnt;
        uint32_t m = f0;
        while (m && pos < MAX_K) { fb[pos++] = w0 * 32 + __ffs(m) - 1; m &= m - 1u; }
        m = f1;
        while (m && pos < MAX_K) { fb[pos++] = w1 * 32 + __ffs(m) - 1; m &= m - 1u; }
        nf += __builtin_amdgcn_readlane(inc, 63);
    }
    kept = __builtin_amdgcn_readlane(wave_incl_sum(kept), 63);
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

// Where a row's query-aware scores come from.
// ScoresGlobal: s_q as written by score_kernel.
struct ScoresGlobal {
    static constexpr bool kCert = false;
    const float *s_q;
    __device__ __forceinline__ const float *row(const Dims &dm, int r, int) const {
        return s_q + (int64_t)r * dm.max_blocks;
    }
};

// ScoresFused: computed by the selecting workgroup itself into LDS (and
// written to s_q as well), with the same arithmetic as score_kernel: lane <->
// sub-block, U sub-blocks per thread per pass, DPP quad max over a block's
// sub-blocks, then the head sum. Needs the whole workgroup (barriers inside).
template <typename TQ, typename TK, int D, int G>
struct ScoresFused {
    static constexpr bool kCert = false;
    const TQ *q;
    const TK *kbar;
    float *s_q;          // may be null: scores stay in LDS
    int64_t q_step = 0;  // query offset per workgroup row y (batched selections)
    __device__ const float *row(const Dims &dm, int r, int n_cand) const {
        constexpr int M = 4, V = KbarVec<TK>::V, NV = D / V, U = sizeof(TK) == 2 ? 2 : 1;
        __shared__ float qs[G][D];
        __shared__ float sc[MAX_W * 32];
        const int tid = threadIdx.x, nt = blockDim.x;
        const int b = r / dm.Hkv, g = r % dm.Hkv;
        const TQ *qr = q + blockIdx.y * q_step + ((int64_t)b * dm.Hq + (int64_t)g * G) * D;
        for (int p = tid; p < G * D; p += nt) (&qs[0][0])[p] = ldf(qr + p) * dm.scale;
        __syncthreads();
        const int nsb = M * n_cand;
        float *out = s_q ? s_q + (int64_t)r * dm.max_blocks : nullptr;
        // With a whole sub-block per thread at D = 128 the loads of a pass
        // would take 128 registers, which leaves one 512-thread workgroup per
        // CU: the dimension vectors are taken in halves instead (each half's
        // loads in flight together), the sums running on in the same order.
        constexpr int HV = U * NV > 16 ? 2 : 1, NVH = NV / HV;
        for (int base = 0; base < nsb; base += U * nt) {
            // compiler-only memory barrier: keeps the LDS reads of q inside the
            // pass (hoisted out of it, G * D floats would not fit in registers)
            __asm__ volatile("" ::: "memory");
            float acc[U][G];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int h = 0; h < G; ++h) acc[u][h] = 0.f;
#pragma unroll
            for (int hv = 0; hv < HV; ++hv) {
                uint4 raw[U][NVH];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int sb = base + u * nt + tid;
                    if (sb < nsb) {
#pragma unroll
                        for (int i = 0; i < NVH; ++i)
                            raw[u][i] = *reinterpret_cast<const uint4 *>(
                                kbar + kbar_vec<TK, D>(dm, r, sb, hv * NVH + i));
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int sb = base + u * nt + tid;
                    if (sb < nsb) {
#pragma unroll
                        for (int i = 0; i < NVH; ++i) {
                            const int dv = hv * NVH + i;
                            float x[V];
                            KbarVec<TK>::unpack(raw[u][i], x);
#pragma unroll
                            for (int h = 0; h < G; ++h)
#pragma unroll
                                for (int e = 0; e < V; ++e)
                                    acc[u][h] = fmaf(qs[h][dv * V + e], x[e], acc[u][h]);
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int sb = base + u * nt + tid;
                // every lane takes part in the quad reductions (nt keeps quads whole)
                float sum = 0.f;
#pragma unroll
                for (int h = 0; h < G; ++h) sum += quad_max(acc[u][h]);
                if (sb < nsb && (sb & (M - 1)) == 0) {
                    sc[sb / M] = sum;
                    if (out) out[sb / M] = sum;
                }
            }
        }
        __syncthreads();
        return sc;
    }
};

// Block scores of a row on the matrix cores (bf16). A wave takes tiles of 16
// sub-blocks (a quad of blocks): S = K̄ Q^T on v_mfma_f32_16x16x32_bf16, the
// A operand being one 16-byte vector of the pooled keys per lane (sub-block
// 16 tile + l % 16, dimensions 32 s + 8 (l / 16) .. + 7: the quad's vectors as
// stored), B the group's queries with the heads padded to 16 by zeros. The
// output tile puts a block's 4 sub-blocks in one lane's 4 accumulators (rows
// 4 (l / 16) + r), so the block max is in-lane, and the head sum a reduction
// over the 16 lanes of a row group. The scale multiplies the fp32 dot
// product. The wave takes the TPI tiles from t0 on in each of its passes
// (t0 = t_first, t_first + t_stride, ... below t_end), all their loads in
// flight together; block j's score goes to lds[j] and/or out[j] (either may
// be null). NT makes the pooled-key loads non-temporal.
template <int D, int G, int TPI, bool NT = false>
__device__ __forceinline__ void mfma_block_scores(const Dims &dm, const bf16_t *qg,
                                                  const bf16_t *kbar, int r, int n_cand,
                                                  int t_first, int t_stride, int t_end,
                                                  float *lds, float *out) {
    constexpr int KS = D / 32;  // k-steps
    static_assert(G <= 16, "the group is one 16-wide MFMA tile");
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, grp = lane >> 4;
    // B operand: lane holds q[head col][32 s + 8 grp .. + 7]; zero past G
    bf16x8 qop[KS];
    {
        const bf16_t *qh = qg + (int64_t)(col < G ? col : 0) * D + 8 * grp;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qop[s] = *reinterpret_cast<const bf16x8 *>(qh + 32 * s);
            if (col >= G) qop[s] = bf16x8{};
        }
    }
    const int nsb = 4 * n_cand;
    // row r's quads of 16 sub-blocks, in bf16x8 vectors: [Q][D/8][16]
    const bf16x8 *kb = reinterpret_cast<const bf16x8 *>(kbar + kbar_vec<bf16_t, D>(dm, r, 0, 0));
    for (int t0 = t_first; t0 < t_end; t0 += t_stride) {
        bf16x8 a[TPI][KS];
#pragma unroll
        for (int u = 0; u < TPI; ++u) {
            const int sb = 16 * (t0 + u) + col;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8 *p = kb + ((int64_t)(t0 + u) * (D / 8) + 4 * s + grp) * 16 + col;
                a[u][s] = sb >= nsb ? bf16x8{} : (NT ? __builtin_nontemporal_load(p) : *p);
            }
        }
#pragma unroll
        for (int u = 0; u < TPI; ++u) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][s], qop[s], acc, 0, 0, 0);
            // rows 4 grp .. 4 grp + 3 = the sub-blocks of block 4 (t0 + u) + grp
            const float sc4 = dm.scale;
            float m = fmaxf(fmaxf(acc[0] * sc4, acc[1] * sc4), fmaxf(acc[2] * sc4, acc[3] * sc4));
            m = col < G ? m : 0.f;
            m += __shfl_xor(m, 8, 16);
            m += __shfl_xor(m, 4, 16);
            m += __shfl_xor(m, 2, 16);
            m += __shfl_xor(m, 1, 16);
            const int blk = 4 * (t0 + u) + grp;
            if (col == 0 && blk < n_cand) {
                if (lds) lds[blk] = m;
                if (out) out[blk] = m;
            }
        }
    }
}

// ScoresFusedMfma (bf16): the selecting workgroup computes its row's scores
// itself, its waves taking turns over the row's tiles, into LDS.
template <int D, int G>
struct ScoresFusedMfma {
    static constexpr bool kCert = false;
    const bf16_t *q;
    const bf16_t *kbar;
    float *s_q;          // may be null: scores stay in LDS
    int64_t q_step = 0;  // query offset per workgroup row y (batched selections)
    __device__ const float *row(const Dims &dm, int r, int n_cand) const {
        constexpr int TPI = 4;  // tiles per pass per wave
        __shared__ float sc[MAX_W * 32];
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int nw = blockDim.x >> 6;
        const int b = r / dm.Hkv, g = r % dm.Hkv;
        const bf16_t *qg = q + blockIdx.y * q_step + ((int64_t)b * dm.Hq + (int64_t)g * G) * D;
        float *out = s_q ? s_q + (int64_t)r * dm.max_blocks : nullptr;
        mfma_block_scores<D, G, TPI>(dm, qg, kbar, r, n_cand, wave * TPI, nw * TPI,
                                     (n_cand + 3) / 4, sc, out);
        __syncthreads();
        return sc;
    }
};

// Certified scoring (bfloat16 KV, float32 pooled keys; kbar's regions in
// common.h). The selection first ranks scores taken from the pooled keys'
// bfloat16 shadow, each within eps_j = scale * sum_h ||q_h||_2 * radius_j of
// any float32 evaluation of its score (pool_write). cert_refine then takes
// every candidate whose interval reaches the lowest lower bound of that first
// top-k_q, scores it again from the float32 means, and keeps the top k_q of
// those: every other candidate has k_q candidates certainly above it, so the
// selection is the top k_q by float32 scores while the scoring reads half the
// bytes.
struct CertArgs {
    const bf16_t *q;      // [B][Hq][D], the step's queries
    const float *kbar32;  // region 0: the float32 means
    const float *radius;  // region 2: [rows][max_blocks]
    int64_t q_step;       // query offset per workgroup row y (batched selections)
};

// Shadow scores from s_q (written by the split scoring grid on the shadow).
template <int D_, int G_>
struct ScoresCert {
    static constexpr bool kCert = true;
    static constexpr int D = D_, G = G_;
    const float *s_q;
    CertArgs c;
    __device__ __forceinline__ const float *row(const Dims &dm, int r, int) const {
        return s_q + (int64_t)r * dm.max_blocks;
    }
};

// Shadow scores computed by the selecting workgroup on the matrix cores, into
// LDS (and s_q).
template <int D_, int G_>
struct ScoresCertFused {
    static constexpr bool kCert = true;
    static constexpr int D = D_, G = G_;
    const bf16_t *shadow;
    float *s_q;
    CertArgs c;
    __device__ const float *row(const Dims &dm, int r, int n_cand) const {
        const ScoresFusedMfma<D, G> f{c.q, shadow, s_q, c.q_step};
        return f.row(dm, r, n_cand);
    }
};

// What cert_refine reads that depends on nothing before it: the row's
// queries (raw bfloat16) and its candidates' radii, loaded at the start of
// the selection so that their latency hides behind the scoring and top-k.
// The loads are unconditional (indexes clamped into the arrays), so that
// nothing waits for them before cert_refine; entries past the queries or
// the candidates are never used.
template <int D, int G>
struct CertPre {
    static constexpr int QPT = (G * D + SELECT_THREADS - 1) / SELECT_THREADS;
    bf16_t q[QPT];                // query element tid + SELECT_THREADS u of the group
    float rad[KEYS_PER_THREAD];   // radius of candidate tid + SELECT_THREADS i
};
template <int D, int G>
__device__ __forceinline__ void cert_prefetch(const Dims &dm, const CertArgs &ca, int r,
                                              int n_cand, CertPre<D, G> &p) {
    const int b = r / dm.Hkv, g = r % dm.Hkv;
    const bf16_t *qr = ca.q + blockIdx.y * ca.q_step + ((int64_t)b * dm.Hq + (int64_t)g * G) * D;
#pragma unroll
    for (int u = 0; u < CertPre<D, G>::QPT; ++u)
        p.q[u] = qr[min((int)threadIdx.x + SELECT_THREADS * u, G * D - 1)];
    const float *rad = ca.radius + (int64_t)r * dm.max_blocks;
    const int last = max(n_cand - 1, 0);
#pragma unroll
    for (int i = 0; i < KEYS_PER_THREAD; ++i)
        p.rad[i] = rad[min((int)threadIdx.x + SELECT_THREADS * i, last)];
}

template <typename Src, bool = Src::kCert> struct CertPreOf { struct type {}; };
template <typename Src> struct CertPreOf<Src, true> { using type = CertPre<Src::D, Src::G>; };

// DPP rotations inside each row of 16 lanes.
constexpr int DPP_ROW_ROR4 = 0x124, DPP_ROW_ROR8 = 0x128;

// Gamma_q from certified scores, by the whole selecting workgroup, after the
// top-k_q of the shadow scores sv (in sb, beside Gamma_e in ge): see
// CertArgs. Rewrites sb's Gamma_q bits; the caller synchronises after.
template <int D, int G>
__device__ void cert_refine(const Dims &dm, const CertArgs &ca, int r, int n_cand, int kq,
                            const uint32_t *ge, uint32_t *sb,
                            const float (&sv)[KEYS_PER_THREAD], const CertPre<D, G> &pre) {
    constexpr int M = 4, V = 4, NQ = D / V / 4;  // float4 vectors per quarter of D
    static_assert(D % 64 == 0, "a wave's query elements lie in one head");
    __shared__ float qs[G * D];
    __shared__ float qn[G * D / 64];
    __shared__ float red[SELECT_WAVES];
    __shared__ int rl[MAX_W * 32];
    __shared__ uint64_t rk[MAX_W * 32 + 8];  // R's rank keys by float32 score, 0-padded
    __shared__ int n_r;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the queries as the scoring takes them (q * scale), and per wave the sum
    // of squares of its 64 elements, all of one head
#pragma unroll
    for (int u = 0; u < CertPre<D, G>::QPT; ++u) {
        const int e = tid + SELECT_THREADS * u;
        if ((e & ~63) < G * D) {  // the whole wave
            const float x = bf2f(pre.q[u]) * dm.scale;
            qs[e] = x;
            const float s2 = wave_sum(x * x);
            if (lane == 0) qn[e >> 6] = s2;
        }
    }
    if (tid == 0) n_r = 0;
    __syncthreads();
    // scale * sum_h ||q_h||_2, enlarged by 2^-10
    float cq = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float s2 = 0.f;
#pragma unroll
        for (int c = 0; c < D / 64; ++c) s2 += qn[h * (D / 64) + c];
        cq += sqrtf(s2);
    }
    cq *= 1.0f + 1.0f / 1024.0f;
    // the lowest lower bound over the shadow's top k_q
    float eps[KEYS_PER_THREAD];
    float lbmin = INFINITY;
#pragma unroll
    for (int i = 0; i < KEYS_PER_THREAD; ++i) {
        const int j = tid + SELECT_THREADS * i;
        eps[i] = 0.f;
        if (j < n_cand && !((ge[j >> 5] >> (j & 31)) & 1u)) {
            eps[i] = cq * pre.rad[i];
            if ((sb[j >> 5] >> (j & 31)) & 1u) lbmin = fminf(lbmin, sv[i] - eps[i]);
        }
    }
    lbmin = -wave_max(-lbmin);
    if (lane == 0) red[wave] = lbmin;
    __syncthreads();
    float T = red[0];
#pragma unroll
    for (int w = 1; w < SELECT_WAVES; ++w) T = fminf(T, red[w]);
    // R: the candidates outside Gamma_e whose upper bound reaches T
#pragma unroll
    for (int i = 0; i < KEYS_PER_THREAD; ++i) {
        const int j = tid + SELECT_THREADS * i;
        if (j < n_cand && !((ge[j >> 5] >> (j & 31)) & 1u) && sv[i] + eps[i] >= T)
            rl[atomicAdd(&n_r, 1)] = j;
    }
    __syncthreads();
    const int nr = n_r;
    // their float32 scores: 16 lanes per block, lane 4 i + c holding sub-block
    // i and the c-th quarter of D (all 8 of its 16-byte loads in flight at
    // once); a head's dot product is the sum of the four quarters' float32
    // partial sums, in a fixed order, and the block takes the max over its
    // sub-blocks per head and sums the heads in order
    constexpr int TPB = 16, BPP = SELECT_THREADS / TPB;
    const int c = tid & 3, i = (tid >> 2) & 3;
    for (int base = 0; base < nr; base += BPP) {
        const int m = base + tid / TPB;
        const int blk = rl[m < nr ? m : nr - 1];
        const int sbk = M * blk + i;
        float x[NQ][V];
#pragma unroll
        for (int v = 0; v < NQ; ++v)
            KbarVec<float>::load(ca.kbar32 + kbar_vec<float, D>(dm, r, sbk, c * NQ + v), x[v]);
        float sc = 0.f;
#pragma unroll 1
        for (int h = 0; h < G; ++h) {
            float a = 0.f;
#pragma unroll
            for (int v = 0; v < NQ; ++v)
#pragma unroll
                for (int u = 0; u < V; ++u) a = fmaf(qs[h * D + (c * NQ + v) * V + u], x[v][u], a);
            a += dpp_f<QUAD_SWAP1>(a);
            a += dpp_f<QUAD_SWAP2>(a);
            a = fmaxf(a, dpp_f<DPP_ROW_ROR4>(a));
            a = fmaxf(a, dpp_f<DPP_ROW_ROR8>(a));
            sc += a;
        }
        if (m < nr && (tid & (TPB - 1)) == 0) rk[m] = rank_key(sc, blk);
    }
    if (tid < 8) rk[nr + tid] = 0ull;
    // Gamma_q anew: the k_q best of R by float32 score, lower id first on ties
    for (int w = tid; w < dm.W; w += SELECT_THREADS) sb[w] = ge[w];
    __syncthreads();
    for (int m = tid; m < nr; m += SELECT_THREADS) {
        const uint64_t km = rk[m];
        int above = 0;
        for (int m2 = 0; m2 < nr; m2 += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u) above += rk[m2 + u] > km ? 1 : 0;
        }
        if (above < kq) {
            const int j = key_index(km);
            atomicOr(&sb[j >> 5], 1u << (j & 31));
        }
    }
}

// Block scores on the matrix cores with the row split over workgroups
// (blockIdx.x = chunk of SCORE_TILES_PER_WG tiles, blockIdx.y = row), so that
// a launch has many more workgroups than rows: each wave loads its tile (16
// sub-blocks x D: 4 KiB of bf16 pooled keys at D = 128) at once, and the
// grid covers the row in one pass. Swept on the 32k workload (64 rows x 512
// candidates): 8 waves of one tile 7.3 us, 4 waves of two 7.5, 4 of four
// 7.9, 4 of eight 9.5, 8 of two 7.7, 16 of one 7.9, 16 of two 8.4. At 256
// rows x 1024 candidates it streams the pooled keys at 6.7 TB/s.
// With dstep, n_cand comes from the step record and the grid is sized for the
// capacity; chunks past the candidates exit at once.
constexpr int SCORE_WAVES = 8;
constexpr int SCORE_TPI = 1;
constexpr int SCORE_TILES_PER_WG = SCORE_WAVES * SCORE_TPI;
// Non-temporal pooled-key loads once a launch reads more than half of the
// 256 MB Infinity Cache, which the step's attention reads compete for: at
// 256 rows x 1024 candidates (268 MB) 4,505-4,513 against 4,465-4,470
// steps/s; at 64 rows x 512 (34 MB, kept in the cache from step to step) the
// cached loads are faster.
constexpr int64_t SCORE_NT_MIN_BYTES = (int64_t)128 << 20;
template <int D, int G, bool NT>
__global__ void __launch_bounds__(64 * SCORE_WAVES)
score_mfma_kernel(Dims dm, const bf16_t *__restrict__ q, const bf16_t *__restrict__ kbar,
                  int n_cand, float *__restrict__ s_q, const int32_t *__restrict__ dstep) {
    if (dstep) n_cand = read_step(dstep, dm).n_cand;
    const int n_tiles = (n_cand + 3) / 4;
    const int t_begin = blockIdx.x * SCORE_TILES_PER_WG;
    if (t_begin >= n_tiles) return;
    const int r = blockIdx.y;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b = r / dm.Hkv, g = r % dm.Hkv;
    const bf16_t *qg = q + ((int64_t)b * dm.Hq + (int64_t)g * G) * D;
    const int t0 = t_begin + wave * SCORE_TPI;
    mfma_block_scores<D, G, SCORE_TPI, NT>(dm, qg, kbar, r, n_cand, t0, n_tiles,
                                           min(t0 + 1, n_tiles), nullptr,
                                           s_q + (int64_t)r * dm.max_blocks);
}

// Independent selections in one launch (workgroup row y = blockIdx.y): y
// has n_cand + y * cand_step candidates and writes sel / n_sel shifted by y
// steps. A single selection has gridDim.y = 1.
struct BatchArgs {
    int cand_step;
    int64_t sel_step, nsel_step;
    const int32_t *dstep;  // device step record: n_cand and n_prev from it
};

// Four waves per SIMD at most 128 registers each: two selecting workgroups
// share a CU, so that one's selection (latency-bound) runs beside the other's
// scoring. The batched prefill selection over float32 pooled keys went from
// 2.57-2.61 to 1.16-1.17 ms on the 32k context when it reached that (its
// scoring's loads had taken 162 registers).
template <typename Src>
__global__ void __launch_bounds__(SELECT_THREADS, 4)
select_kernel(Dims dm, Src src, const float *__restrict__ e_blk, int n_cand0,
              int n_prev_arg, int P, uint32_t *__restrict__ ge_bits, uint32_t *__restrict__ ev_bits,
              int32_t *__restrict__ sel, int32_t *__restrict__ n_sel,
              uint32_t *__restrict__ sel_bits, SwapArgs sw, ListArgs lists, BatchArgs bt) {
    extern __shared__ uint64_t keys[];  // P keys, only when a budget exceeds 64
    __shared__ uint32_t ge[MAX_W], ev[MAX_W], sb[MAX_W], res[MAX_W];
    __shared__ __attribute__((aligned(16))) uint64_t surv[SELECT_WAVES * WAVE_TOPK + 2];
    __shared__ int n_surv;
    __shared__ uint64_t red64[SELECT_WAVES];
    __shared__ int red32[SELECT_WAVES];
    __shared__ int fb[MAX_K], fs[MAX_K], fo[MAX_K];
    const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int W = dm.W;
    StepVals stp{0, n_cand0 + (int)blockIdx.y * bt.cand_step, n_prev_arg};
    if (bt.dstep) stp = read_step(bt.dstep, dm);
    const int n_cand = stp.n_cand, n_prev = stp.n_prev;
    sel += blockIdx.y * bt.sel_step;
    n_sel += blockIdx.y * bt.nsel_step;
    const float *E = e_blk + (int64_t)r * dm.max_blocks;
    // eviction state and selection bitmap: absent (null) for batched selections
    uint32_t *ge_g = ge_bits ? ge_bits + (int64_t)r * W : nullptr;
    uint32_t *ev_g = ev_bits ? ev_bits + (int64_t)r * W : nullptr;

    // independent loads first: the cache's slot table and counters (for wave
    // 1, which runs the set difference), then this thread's scores
    int s0 = -1, s1 = -1;
    uint64_t cnt = 0ull;
    if (sw.slot_block && wave == 1) {
        if (lane < dm.k) s0 = sw.slot_block[(int64_t)r * dm.k + lane];
        if (lane + 64 < dm.k) s1 = sw.slot_block[(int64_t)r * dm.k + lane + 64];
        if (lane < 2) cnt = sw.counters[2 * r + lane];
    }
    // the eviction state: word tid (W <= MAX_W <= the workgroup size)
    uint32_t ge_w = 0u, ev_w = 0u;
    if (n_prev >= 0 && ge_g && tid < W) {
        ge_w = ge_g[tid];
        ev_w = ev_g[tid];
    }
    [[maybe_unused]] typename CertPreOf<Src>::type cpre;
    if constexpr (Src::kCert) cert_prefetch(dm, src.c, r, n_cand, cpre);
    const float *Sq = src.row(dm, r, n_cand);
    float sv[KEYS_PER_THREAD];
#pragma unroll
    for (int i = 0; i < KEYS_PER_THREAD; ++i) {
        const int j = tid + SELECT_THREADS * i;
        sv[i] = j < n_cand ? Sq[j] : 0.f;
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
        if (tid < W) {
            const int lo = tid * 32;
            const uint32_t prev = lo + 32 <= n_prev ? 0xFFFFFFFFu
                                : (lo >= n_prev ? 0u : ((1u << (n_prev - lo)) - 1u));
            ge[tid] = ge_w & prev;
            ev[tid] = ev_w & prev;
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
    // every wave counts Gamma_e itself (no barrier); the copies into sb are
    // ordered before the top-k's updates by the top-k's first barrier
    for (int w = tid; w < W; w += nt) sb[w] = ge[w];
    const int ne_loc = (lane < W ? __popc(ge[lane]) : 0) + (lane + 64 < W ? __popc(ge[lane + 64]) : 0);
    const int n_e = __builtin_amdgcn_readlane(wave_incl_sum(ne_loc), 63);
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
    if constexpr (Src::kCert) {
        // the top k_q above ranks shadow scores: settle it on float32 scores
        if (kq > 0 && n_cand - n_e > kq) {
            cert_refine<Src::D, Src::G>(dm, src.c, r, n_cand, kq, ge, sb, sv, cpre);
            __syncthreads();
        }
    }

    // ---- state and the ascending selection ----
    if (ge_g) {
        for (int w = tid; w < W; w += nt) {
            ge_g[w] = ge[w];
            ev_g[w] = ev[w];
            sel_bits[(int64_t)r * W + w] = sb[w];
        }
    }
    // the set difference (wave 1) and the ascending lists (wave 0) both work
    // from the selection bitmap in LDS alone, so they run side by side
    if (wave == 1) {
        if (sw.slot_block) swap_row(dm, r, sb, s0, s1, cnt, res, fb, fs, fo, sw);
        return;
    }
    if (wave != 0) return;
    // wave 0 writes the ascending lists: the union, and each part when asked
    // for. Lane l holds bitmap words 2l and 2l+1 (<= 128 words); a prefix sum
    // of their popcounts places each lane's candidates.
    const int w0 = 2 * lane, w1 = 2 * lane + 1;
    auto place = [&](uint32_t a0, uint32_t a1, int32_t *dst, int cap) -> int {
        const int cnt = __popc(a0) + __popc(a1);
        const int inc = wave_incl_sum(cnt);
        int pos = inc - cnt;
        for (uint32_t m = a0; m; m &= m - 1u, ++pos)
            if (pos < cap) dst[pos] = 32 * w0 + __ffs(m) - 1;
        for (uint32_t m = a1; m; m &= m - 1u, ++pos)
            if (pos < cap) dst[pos] = 32 * w1 + __ffs(m) - 1;
        const int n = __builtin_amdgcn_readlane(inc, 63);
        for (int i = min(n, cap) + lane; i < cap; i += 64) dst[i] = -1;
        return min(n, cap);
    };
    const uint32_t s0w = w0 < W ? sb[w0] : 0u, s1w = w1 < W ? sb[w1] : 0u;
    const int total = place(s0w, s1w, sel + (int64_t)r * dm.k, dm.k);
    if (lists.n_ge) {
        const uint32_t e0w = w0 < W ? ge[w0] : 0u, e1w = w1 < W ? ge[w1] : 0u;
        const int ne = place(e0w, e1w, lists.ge_list + (int64_t)r * dm.k_e, dm.k_e);
        const int nq = place(s0w & ~e0w, s1w & ~e1w, lists.gq_list + (int64_t)r * dm.k_q, dm.k_q);
        if (lane == 0) {
            lists.n_ge[r] = ne;
            lists.n_gq[r] = nq;
        }
    }
    if (lane == 0) n_sel[r] = total;
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
// Fetch: a bounded grid of workgroups walks the work items (list entry i, row
// r) = item, item + gridDim.x, ... in entry-major order, so the valid ones
// (i < n_fetch[r]) come first and spread over every workgroup; a workgroup
// copies one block at a time, each thread keeping eight 16-byte loads in
// flight before storing them. FETCH_WGS workgroups keep far more reads in
// flight than the PCIe link needs (128 x 32 KiB), while a grid of one
// workgroup per item filled every CU with copies waiting on PCIe, so that
// attention workgroups launched beside the copy (another half of the batch)
// found no room until it drained.
// ---------------------------------------------------------------------------
constexpr int FETCH_WGS = 128;
__global__ void __launch_bounds__(256)
fetch_kernel(const u32x4 *__restrict__ src, int64_t src_row_blocks, const int32_t *__restrict__ fblk,
             const int32_t *__restrict__ fslot, const int32_t *__restrict__ nfetch, int k,
             int max_fetch, int rows, u32x4 *__restrict__ dst, int64_t dst_row_blocks,
             int vec_per_block) {
    const int total = max_fetch * rows;
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        const int i = item / rows, r = item % rows;
        if (i >= nfetch[r]) continue;
        const int b = fblk[(int64_t)r * k + i];
        const int s = fslot[(int64_t)r * k + i];
        if (b < 0 || b >= src_row_blocks || s < 0 || s >= dst_row_blocks) continue;  // not a block
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
}

// ---------------------------------------------------------------------------
// Ingest: the step before the path, fused (NOSI's kernel-fusion bullet: the
// eviction head, the QKV split and pooling in one launch). One workgroup per
// row, for the token `tok` of every row:
//  * split: the row's G query heads of the fused projection output go to
//    q_out; its key and value heads go into token slot tok % 64 of a block of
//    the block-unit KV buffer (the layout in common.h);
//  * eviction head: e = x . w_g + b_g (float32 sum), written to e_tok;
//  * when the token completes its block: the block's sub-block key means
//    (pooled_mean_of, the same arithmetic and order as pool_kernel) and its
//    max-of-means eviction score, with the new token taken from LDS and the
//    block's other 63 tokens from memory.
// ---------------------------------------------------------------------------
template <typename T, typename TK, int D, int G>
__global__ void __launch_bounds__(256)
ingest_kernel(Dims dm, const T *__restrict__ qkv, const T *__restrict__ x,
              const T *__restrict__ w_e, const float *__restrict__ b_e, int hidden, int tok,
              T *__restrict__ q_out, T *__restrict__ kv, int64_t kv_row_blocks, int block,
              float *__restrict__ e_tok, int64_t e_stride, TK *__restrict__ kbar,
              float *__restrict__ e_blk) {
    constexpr int S = 64, M = 4, V = KbarVec<TK>::V, NW = 256 / 64;
    __shared__ T knew[D];
    __shared__ float red[NW];
    __shared__ float e_new, emean[M];
    const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = r / dm.Hkv, g = r % dm.Hkv;
    const int pos = tok % S, j = tok / S;
    const T *src = qkv + (int64_t)b * (dm.Hq + 2 * dm.Hkv) * D;
    T *qo = q_out + ((int64_t)b * dm.Hq + (int64_t)g * G) * D;
    {
        // the row's G query heads: G * D elements, 16-byte vectors (D * sizeof(T)
        // is a multiple of 16, and so are the row and head offsets)
        constexpr int EV = 16 / sizeof(T);
        const u32x4 *qs = reinterpret_cast<const u32x4 *>(src + (int64_t)g * G * D);
        u32x4 *qd = reinterpret_cast<u32x4 *>(qo);
        for (int p = tid; p < G * D / EV; p += blockDim.x) qd[p] = qs[p];
    }
    T *blk = kv + ((int64_t)r * kv_row_blocks + block) * (int64_t)(2 * S * D);
    for (int d = tid; d < D; d += blockDim.x) {
        const T kval = src[(int64_t)(dm.Hq + g) * D + d];
        const T vval = src[(int64_t)(dm.Hq + dm.Hkv + g) * D + d];
        blk[kv_k_off<T, D>(pos, d)] = kval;
        blk[kv_v_off<T, D>(pos, d)] = vval;
        knew[d] = kval;
    }
    // eviction head: 16-byte vectors when the rows allow them, else elements
    const T *xr = x + (int64_t)b * hidden;
    const T *wr = w_e + (int64_t)g * hidden;
    float acc = 0.f;
    constexpr int EV = 16 / sizeof(T);
    if (hidden % EV == 0 && ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w_e)) & 15) == 0) {
        const u32x4 *xv = reinterpret_cast<const u32x4 *>(xr);
        const u32x4 *wv = reinterpret_cast<const u32x4 *>(wr);
        for (int i = tid; i < hidden / EV; i += blockDim.x) {
            const u32x4 a = xv[i], c = wv[i];
            float fa[EV], fc[EV];
            unpack16<T>(a, fa);
            unpack16<T>(c, fc);
#pragma unroll
            for (int u = 0; u < EV; ++u) acc = fmaf(fa[u], fc[u], acc);
        }
    } else {
        for (int i = tid; i < hidden; i += blockDim.x) acc = fmaf(ldf(xr + i), ldf(wr + i), acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) red[wave] = acc;
    __syncthreads();
    if (tid == 0) {
        float e = b_e ? b_e[g] : 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) e += red[w];
        e_tok[(int64_t)r * e_stride + tok] = e;
        e_new = e;
    }
    if (pos != S - 1) return;
    __syncthreads();
    // the block is complete: pool it
    static_assert(V > 0, "pooled-key vector width");
    pool_write<T, TK, D>(dm, kbar, r, j, [&](int i, int d) {
        return pooled_mean_of<T, TK>([&](int u) {
            const int t = 16 * i + u;
            return t == S - 1 ? knew[d] : blk[kv_k_off<T, D>(t, d)];
        });
    });
    if (tid < M) {
        const float *er = e_tok + (int64_t)r * e_stride + (int64_t)j * S + tid * 16;
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) s += (16 * tid + u == S - 1) ? e_new : er[u];
        emean[tid] = s * (1.0f / 16);
    }
    __syncthreads();
    if (tid == 0) {
        float mx = emean[0];
#pragma unroll
        for (int i = 1; i < M; ++i) mx = fmaxf(mx, emean[i]);
        e_blk[(int64_t)r * dm.max_blocks + j] = mx;
    }
}

// ---------------------------------------------------------------------------
// Append: the newest token of every row enters token slot `pos` of block
// `block` of a KV buffer: its key as token pos of the K tile, its value as
// column vt_pos_of(pos) of the V^T tile (the layout in common.h). One
// workgroup per row, thread d writes dimension d.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(D)
append_kernel(Dims dm, const T *__restrict__ k_new, const T *__restrict__ v_new, int pos,
              T *__restrict__ kv, int64_t kv_row_blocks, int block,
              const int32_t *__restrict__ dstep) {
    constexpr int S = 64;
    const int r = blockIdx.x, d = threadIdx.x;
    if (dstep) {
        const StepVals sv = read_step(dstep, dm);
        pos = (sv.n_tokens - 1) % S;
        block = sv.n_cand;
    }
    T *blk = kv + ((int64_t)r * kv_row_blocks + block) * (int64_t)(2 * S * D);
    blk[kv_k_off<T, D>(pos, d)] = k_new[(int64_t)r * D + d];
    blk[kv_v_off<T, D>(pos, d)] = v_new[(int64_t)r * D + d];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename T, typename TK, int D>
hipError_t launch_pool(const Dims &dm, const void *kv, int64_t kv_row_blocks, int kv_first,
                       const float *e_tok, int64_t e_stride, int blk_begin, int blk_end,
                       void *kbar, float *e_blk, hipStream_t st) {
    dim3 grid(blk_end - blk_begin, dm.rows);
    hipLaunchKernelGGL((pool_kernel<T, TK, D>), grid, dim3(256), 0, st, dm,
                       static_cast<const T *>(kv), kv_row_blocks, kv_first, e_tok, e_stride,
                       blk_begin, static_cast<TK *>(kbar), e_blk, nullptr);
    return hipGetLastError();
}

template <typename T, typename TK, int D>
hipError_t launch_pool_step(const Dims &dm, const void *kv, int64_t kv_row_blocks,
                            const float *e_tok, int64_t e_stride, const int32_t *dstep,
                            void *kbar, float *e_blk, hipStream_t st) {
    // one token per step completes at most one block
    hipLaunchKernelGGL((pool_kernel<T, TK, D>), dim3(1, dm.rows), dim3(256), 0, st, dm,
                       static_cast<const T *>(kv), kv_row_blocks, 0, e_tok, e_stride, 0,
                       static_cast<TK *>(kbar), e_blk, dstep);
    return hipGetLastError();
}

// The step record moves to the next step: the candidates of this step become
// the previous ones, one more token.
__global__ void step_advance_kernel(Dims dm, int32_t *dstep) {
    if (threadIdx.x == 0) {
        const StepVals sv = read_step(dstep, dm);
        dstep[1] = sv.n_cand;
        dstep[0] = sv.n_tokens + 1;
    }
}

hipError_t launch_step_advance(const Dims &dm, int32_t *dstep, hipStream_t st) {
    hipLaunchKernelGGL(step_advance_kernel, dim3(1), dim3(64), 0, st, dm, dstep);
    return hipGetLastError();
}

// With a device step record the grid covers the capacity.
template <typename T, typename TK, int D, int G>
hipError_t launch_score(const Dims &dm, const void *q, const void *kbar, int n_cand, float *s_q,
                        hipStream_t st, const int32_t *dstep) {
    const int cand = dstep ? dm.max_blocks : n_cand;
    if (cand == 0) return hipSuccess;  // no candidates: nothing to score
    if constexpr (std::is_same_v<TK, bf16_t>) {
        // bfloat16 pooled keys (and queries): the matrix cores
        const int n_tiles = (cand + 3) / 4;
        dim3 grid((n_tiles + SCORE_TILES_PER_WG - 1) / SCORE_TILES_PER_WG, dm.rows);
        const bool nt = (int64_t)dm.rows * cand * 4 * D * 2 > SCORE_NT_MIN_BYTES;
        const bf16_t *qb = static_cast<const bf16_t *>(q), *kb = static_cast<const bf16_t *>(kbar);
        if (nt)
            hipLaunchKernelGGL((score_mfma_kernel<D, G, true>), grid, dim3(64 * SCORE_WAVES), 0,
                               st, dm, qb, kb, n_cand, s_q, dstep);
        else
            hipLaunchKernelGGL((score_mfma_kernel<D, G, false>), grid, dim3(64 * SCORE_WAVES), 0,
                               st, dm, qb, kb, n_cand, s_q, dstep);
    } else {
        dim3 grid((4 * cand + 255) / 256, dm.rows);
        hipLaunchKernelGGL((score_kernel<T, TK, D, G>), grid, dim3(256), 0, st, dm,
                           static_cast<const T *>(q), static_cast<const TK *>(kbar), n_cand, s_q,
                           dstep);
    }
    return hipGetLastError();
}

template <typename Src>
static hipError_t launch_select_from(const Dims &dm, const Src &src, const float *e_blk,
                                     int n_cand, int n_prev, uint32_t *ge, uint32_t *ev,
                                     int32_t *sel, int32_t *n_sel, uint32_t *sel_bits,
                                     const SwapPtrs *swap, const SelectLists *parts,
                                     hipStream_t st, int batch = 1,
                                     const int32_t *dstep = nullptr) {
    // LDS keys only when a budget is above what the register top-k holds
    // (batch > 1: selections y = 0..batch-1 with y candidates each; a device
    // step: up to the capacity)
    const int max_cand = dstep ? dm.max_blocks : batch > 1 ? batch - 1 : n_cand;
    int P = 0;
    if (((n_prev < 0 || dstep) && dm.k_e > WAVE_TOPK) || dm.k_q > WAVE_TOPK) {
        P = 2;
        while (P < max_cand) P <<= 1;
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
    const BatchArgs bt = batch > 1 ? BatchArgs{1, (int64_t)dm.rows * dm.k, dm.rows, nullptr}
                                   : BatchArgs{0, 0, 0, dstep};
    hipLaunchKernelGGL(select_kernel<Src>, dim3(dm.rows, batch), dim3(SELECT_THREADS),
                       P * sizeof(uint64_t), st, dm, src, e_blk, batch > 1 ? 0 : n_cand, n_prev, P,
                       ge, ev, sel, n_sel, sel_bits, sw, li, bt);
    return hipGetLastError();
}

hipError_t launch_select(const Dims &dm, const float *s_q, const float *e_blk, int n_cand,
                         int n_prev, uint32_t *ge, uint32_t *ev, int32_t *sel, int32_t *n_sel,
                         uint32_t *sel_bits, const SwapPtrs *swap, const SelectLists *parts,
                         hipStream_t st) {
    return launch_select_from(dm, ScoresGlobal{s_q}, e_blk, n_cand, n_prev, ge, ev, sel, n_sel,
                              sel_bits, swap, parts, st);
}

// Rows up to which nosa_score_select scores on the split grid and selects in
// a second launch (bf16); above it one workgroup per row does both. Measured
// with HIP events on 256 CUs, score + select vs one launch: 64 rows x 512
// candidates 8.8 + 8.7 vs 19.3 us; 128 rows x 2048 51 + 10.4 vs 72 us; 256
// rows x 1024 53 + 10.8 vs 59-62 us (with a workgroup per CU the fused form
// hides each row's selection behind other rows' scoring).
constexpr int SPLIT_SCORE_MAX_ROWS = 128;
// The same for certified scoring, whose selection also rescores the rows'
// near ties: at 256 rows x 1024 candidates the split form took 65.5-66.0 us
// against 70.5-70.6 (whole score + select stage), at 512 rows x 512 the two
// are level (rocprof: 44.1 + 18.3 against 63.8 us).
constexpr int CERT_SPLIT_MAX_ROWS = 256;

template <typename T, typename TK, int D, int G>
hipError_t launch_score_select(const Dims &dm, const void *q, const void *kbar, float *s_q,
                               const float *e_blk, int n_cand, int n_prev, uint32_t *ge,
                               uint32_t *ev, int32_t *sel, int32_t *n_sel, uint32_t *sel_bits,
                               const SwapPtrs *swap, hipStream_t st, const int32_t *dstep) {
    if constexpr (std::is_same_v<T, bf16_t> && std::is_same_v<TK, float>) {
        // certified scoring: shadow scores on the matrix cores, settled on
        // float32 scores inside the selection (s_q receives the shadow scores)
        const char *kb = static_cast<const char *>(kbar);
        const bf16_t *shadow = reinterpret_cast<const bf16_t *>(kb + kbar_shadow_offset(dm));
        const CertArgs ca{static_cast<const bf16_t *>(q), static_cast<const float *>(kbar),
                          reinterpret_cast<const float *>(kb + kbar_radius_offset(dm)), 0};
        if (dm.rows <= CERT_SPLIT_MAX_ROWS) {
            const hipError_t e =
                launch_score<bf16_t, bf16_t, D, G>(dm, q, shadow, n_cand, s_q, st, dstep);
            if (e != hipSuccess) return e;
            return launch_select_from(dm, ScoresCert<D, G>{s_q, ca}, e_blk, n_cand, n_prev, ge,
                                      ev, sel, n_sel, sel_bits, swap, nullptr, st, 1, dstep);
        }
        return launch_select_from(dm, ScoresCertFused<D, G>{shadow, s_q, ca}, e_blk, n_cand,
                                  n_prev, ge, ev, sel, n_sel, sel_bits, swap, nullptr, st, 1,
                                  dstep);
    }
    if (std::is_same_v<T, bf16_t> && dm.rows <= SPLIT_SCORE_MAX_ROWS) {
        // too few rows to fill the chip with one workgroup each: score on a
        // grid split over the row's candidates, then select from s_q
        const hipError_t e = launch_score<T, TK, D, G>(dm, q, kbar, n_cand, s_q, st, dstep);
        if (e != hipSuccess) return e;
        return launch_select_from(dm, ScoresGlobal{s_q}, e_blk, n_cand, n_prev, ge, ev, sel,
                                  n_sel, sel_bits, swap, nullptr, st, 1, dstep);
    }
    if constexpr (std::is_same_v<TK, bf16_t>) {
        const ScoresFusedMfma<D, G> src{static_cast<const bf16_t *>(q),
                                        static_cast<const bf16_t *>(kbar), s_q};
        return launch_select_from(dm, src, e_blk, n_cand, n_prev, ge, ev, sel, n_sel, sel_bits,
                                  swap, nullptr, st, 1, dstep);
    } else {
        const ScoresFused<T, TK, D, G> src{static_cast<const T *>(q),
                                           static_cast<const TK *>(kbar), s_q};
        return launch_select_from(dm, src, e_blk, n_cand, n_prev, ge, ev, sel, n_sel, sel_bits,
                                  swap, nullptr, st, 1, dstep);
    }
}

// The pooled queries qbar have the pooled dtype TK, like the pooled keys.
template <typename T, typename TK, int D, int G>
hipError_t launch_prefill_select(const Dims &dm, const void *qbar, const void *kbar,
                                 const float *e_blk, int n_qb, int32_t *sel, int32_t *n_sel,
                                 hipStream_t st) {
    const int64_t q_step = (int64_t)dm.B * dm.Hq * D;
    if constexpr (std::is_same_v<TK, bf16_t>) {
        const ScoresFusedMfma<D, G> src{static_cast<const bf16_t *>(qbar),
                                        static_cast<const bf16_t *>(kbar), nullptr, q_step};
        return launch_select_from(dm, src, e_blk, 0, -1, nullptr, nullptr, sel, n_sel, nullptr,
                                  nullptr, nullptr, st, n_qb);
    } else {
        const ScoresFused<TK, TK, D, G> src{static_cast<const TK *>(qbar),
                                            static_cast<const TK *>(kbar), nullptr, q_step};
        return launch_select_from(dm, src, e_blk, 0, -1, nullptr, nullptr, sel, n_sel, nullptr,
                                  nullptr, nullptr, st, n_qb);
    }
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

template <typename T, typename TK, int D, int G>
hipError_t launch_ingest(const Dims &dm, const void *qkv, const void *x, const void *w_e,
                         const float *b_e, int hidden, int tok, void *q_out, void *kv,
                         int64_t kv_row_blocks, int block, float *e_tok, int64_t e_stride,
                         void *kbar, float *e_blk, hipStream_t st) {
    hipLaunchKernelGGL((ingest_kernel<T, TK, D, G>), dim3(dm.rows), dim3(256), 0, st, dm,
                       static_cast<const T *>(qkv), static_cast<const T *>(x),
                       static_cast<const T *>(w_e), b_e, hidden, tok, static_cast<T *>(q_out),
                       static_cast<T *>(kv), kv_row_blocks, block, e_tok, e_stride,
                       static_cast<TK *>(kbar), e_blk);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_append(const Dims &dm, const void *k_new, const void *v_new, int pos, void *kv,
                         int64_t kv_row_blocks, int block, hipStream_t st, const int32_t *dstep) {
    hipLaunchKernelGGL((append_kernel<T, D>), dim3(dm.rows), dim3(D), 0, st, dm,
                       static_cast<const T *>(k_new), static_cast<const T *>(v_new), pos,
                       static_cast<T *>(kv), kv_row_blocks, block, dstep);
    return hipGetLastError();
}
template hipError_t launch_append<float, 64>(const Dims &, const void *, const void *, int, void *,
                                            int64_t, int, hipStream_t, const int32_t *);
template hipError_t launch_append<bf16_t, 64>(const Dims &, const void *, const void *, int,
                                             void *, int64_t, int, hipStream_t, const int32_t *);
template hipError_t launch_append<bf16_t, 128>(const Dims &, const void *, const void *, int,
                                              void *, int64_t, int, hipStream_t, const int32_t *);

hipError_t launch_fetch(const Dims &dm, const void *src, int64_t src_row_blocks,
                        const int32_t *fblk, const int32_t *fslot, const int32_t *nfetch,
                        int max_fetch, void *dst, int64_t dst_row_blocks, hipStream_t st) {
    const int elem = dm.dtype == NOSA_BF16 ? 2 : 4;
    const int vec = 2 * dm.S * dm.D * elem / 16;
    const int64_t items = (int64_t)max_fetch * dm.rows;
    if (items <= 0) return hipSuccess;
    const int wgs = (int)std::min<int64_t>(items, FETCH_WGS);
    hipLaunchKernelGGL(fetch_kernel, dim3(wgs), dim3(256), 0, st, static_cast<const u32x4 *>(src),
                       src_row_blocks, fblk, fslot, nfetch, dm.k, max_fetch, dm.rows,
                       static_cast<u32x4 *>(dst), dst_row_blocks, vec);
    return hipGetLastError();
}

// (KV dtype, pooled dtype, D): float32 keys pool to float32; bfloat16 keys to
// float32 (the default) or to bfloat16 (the model-dtype variant).
#define NOSA_POOL_INST(T, TK, D)                                                               \
    template hipError_t launch_pool<T, TK, D>(const Dims &, const void *, int64_t, int,        \
                                              const float *, int64_t, int, int, void *,        \
                                              float *, hipStream_t);                           \
    template hipError_t launch_pool_step<T, TK, D>(const Dims &, const void *, int64_t,        \
                                                   const float *, int64_t, const int32_t *,    \
                                                   void *, float *, hipStream_t);
NOSA_POOL_INST(float, float, 64)
NOSA_POOL_INST(bf16_t, float, 64)
NOSA_POOL_INST(bf16_t, float, 128)
NOSA_POOL_INST(bf16_t, bf16_t, 64)
NOSA_POOL_INST(bf16_t, bf16_t, 128)

#define NOSA_SCORE_INST(T, TK, D, G)                                                           \
    template hipError_t launch_score<T, TK, D, G>(const Dims &, const void *, const void *,    \
                                                  int, float *, hipStream_t, const int32_t *); \
    template hipError_t launch_ingest<T, TK, D, G>(const Dims &, const void *, const void *,   \
                                                   const void *, const float *, int, int,      \
                                                   void *, void *, int64_t, int, float *,      \
                                                   int64_t, void *, float *, hipStream_t);     \
    template hipError_t launch_score_select<T, TK, D, G>(                                      \
        const Dims &, const void *, const void *, float *, const float *, int, int, uint32_t *, \
        uint32_t *, int32_t *, int32_t *, uint32_t *, const SwapPtrs *, hipStream_t,           \
        const int32_t *);                                                                      \
    template hipError_t launch_prefill_select<T, TK, D, G>(                                    \
        const Dims &, const void *, const void *, const float *, int, int32_t *, int32_t *,    \
        hipStream_t);
#define NOSA_SCORE_ALLG(T, TK, D)                                                              \
    NOSA_SCORE_INST(T, TK, D, 1) NOSA_SCORE_INST(T, TK, D, 2) NOSA_SCORE_INST(T, TK, D, 3)     \
    NOSA_SCORE_INST(T, TK, D, 4) NOSA_SCORE_INST(T, TK, D, 5) NOSA_SCORE_INST(T, TK, D, 6)     \
    NOSA_SCORE_INST(T, TK, D, 7) NOSA_SCORE_INST(T, TK, D, 8)
NOSA_SCORE_ALLG(float, float, 64)
NOSA_SCORE_ALLG(bf16_t, float, 64)
NOSA_SCORE_ALLG(bf16_t, float, 128)
NOSA_SCORE_ALLG(bf16_t, bf16_t, 64)
NOSA_SCORE_ALLG(bf16_t, bf16_t, 128)

}  // namespace nosa
