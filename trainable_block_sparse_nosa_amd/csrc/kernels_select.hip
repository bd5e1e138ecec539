// Pooling, block scoring, dual selection, set difference and block fetch.
//
// NOSA technical summary, Methodology: "1. Algorithm: NOSA" (two-stage
// pooling, Gamma_e / Gamma_q dual selection, strict eviction, ED-DMA
// selection on pre-exponential scores) and "2. System: NOSI" (block-unit
// cache, set difference for block swapping, host-to-device copy kernels).
#include "kernels.h"

namespace nosa {

// ---------------------------------------------------------------------------
// Pool: one workgroup per (block, row). Sub-block means of the keys go to the
// dim-quad-major kbar layout; the eviction scores get mean-then-max pooling.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256)
pool_kernel(Dims dm, const T *__restrict__ kv, int64_t kv_row_blocks, int kv_first,
            const float *__restrict__ e_tok, int64_t e_stride, int blk_begin,
            float *__restrict__ kbar, float *__restrict__ e_blk) {
    constexpr int S = 64, SUB = 16, M = S / SUB;
    __shared__ float emean[M];
    const int r = blockIdx.y;
    const int j = blk_begin + blockIdx.x;
    const T *K = kv + ((int64_t)r * kv_row_blocks + kv_first + blockIdx.x) * (int64_t)(2 * S * D);
    const int64_t ld_sb = (int64_t)M * dm.max_blocks;  // sub-blocks per dim-quad plane
    float *kb = kbar + (int64_t)r * (D / 4) * ld_sb * 4;
    for (int p = threadIdx.x; p < M * D; p += blockDim.x) {
        const int i = p / D, d = p % D;
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < SUB; ++u) s += ldf(K + (i * SUB + u) * D + d);
        kb[((int64_t)(d / 4) * ld_sb + (int64_t)(M * j + i)) * 4 + (d % 4)] = s * (1.0f / SUB);
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
// Score: lane <-> sub-block. Each lane walks the head dimension four floats
// at a time; a wave's loads cover 64 consecutive sub-blocks (1 KiB). The
// group's G dot products stay in registers; the block max over the 4
// sub-blocks is a DPP quad reduction, then the heads are summed.
// ---------------------------------------------------------------------------
template <typename T, int D, int G>
__global__ void __launch_bounds__(256)
score_kernel(Dims dm, const T *__restrict__ q, const float *__restrict__ kbar, int n_cand,
             float *__restrict__ s_q) {
    constexpr int M = 4;
    __shared__ float4 qs[G][D / 4];
    const int r = blockIdx.y;
    const int b = r / dm.Hkv, g = r % dm.Hkv;
    const T *qr = q + ((int64_t)b * dm.Hq + (int64_t)g * G) * D;
    for (int p = threadIdx.x; p < G * D; p += blockDim.x)
        reinterpret_cast<float *>(qs)[p] = ldf(qr + p) * dm.scale;
    __syncthreads();

    const int nsb = M * n_cand;
    const int sb = blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t ld_sb = (int64_t)M * dm.max_blocks;
    const float4 *kb = reinterpret_cast<const float4 *>(kbar) + (int64_t)r * (D / 4) * ld_sb;
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
    if (sb < nsb) {
#pragma unroll 8
        for (int dq = 0; dq < D / 4; ++dq) {
            const float4 v = kb[(int64_t)dq * ld_sb + sb];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float4 w = qs[h][dq];
                acc[h] = fmaf(w.x, v.x, acc[h]);
                acc[h] = fmaf(w.y, v.y, acc[h]);
                acc[h] = fmaf(w.z, v.z, acc[h]);
                acc[h] = fmaf(w.w, v.w, acc[h]);
            }
        }
    }
    // every lane takes part in the quad reductions (n_cand*4 keeps quads whole)
    float s = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) s += quad_max(acc[h]);
    if (sb < nsb && (sb & (M - 1)) == 0) s_q[(int64_t)r * dm.max_blocks + sb / M] = s;
}

// ---------------------------------------------------------------------------
// Select: one workgroup per row. Bitonic sort of 64-bit rank keys in LDS for
// the full top-k (initial Gamma_e, and Gamma_q every step); incremental
// eviction for new candidates.
// ---------------------------------------------------------------------------
constexpr int SELECT_THREADS = 512;
constexpr int MAX_W = 128;  // 4096 blocks

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
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t w = __shfl_xor(v, o, 64);
        v = w < v ? w : v;
    }
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    uint64_t m = red[0];
    for (int i = 1; i < nw; ++i) m = red[i] < m ? red[i] : m;
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

__global__ void __launch_bounds__(SELECT_THREADS)
select_kernel(Dims dm, const float *__restrict__ s_q, const float *__restrict__ e_blk, int n_cand,
              int n_prev, int P, uint32_t *__restrict__ ge_bits, uint32_t *__restrict__ ev_bits,
              int32_t *__restrict__ sel, int32_t *__restrict__ n_sel,
              uint32_t *__restrict__ sel_bits) {
    extern __shared__ uint64_t keys[];
    __shared__ uint32_t ge[MAX_W], ev[MAX_W], sb[MAX_W];
    __shared__ int woff[MAX_W + 1];
    __shared__ uint64_t red64[SELECT_THREADS / 64];
    __shared__ int red32[SELECT_THREADS / 64];
    const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
    const int W = dm.W;
    const float *E = e_blk + (int64_t)r * dm.max_blocks;
    const float *Sq = s_q + (int64_t)r * dm.max_blocks;
    uint32_t *ge_g = ge_bits + (int64_t)r * W;
    uint32_t *ev_g = ev_bits + (int64_t)r * W;

    // ---- Gamma_e ----
    if (n_prev < 0) {
        for (int w = tid; w < W; w += nt) { ge[w] = 0u; ev[w] = 0u; }
        if (dm.k_e > 0) {
            for (int i = tid; i < P; i += nt) keys[i] = i < n_cand ? rank_key(E[i], i) : 0ull;
            __syncthreads();
            bitonic_desc(keys, P);
            const int ke = min(dm.k_e, n_cand);
            for (int i = tid; i < ke; i += nt) {
                const int j = key_index(keys[i]);
                atomicOr(&ge[j >> 5], 1u << (j & 31));
            }
        }
        __syncthreads();
        for (int w = tid; w < W; w += nt) {
            const int lo = w * 32;
            uint32_t cand = lo + 32 <= n_cand ? 0xFFFFFFFFu
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
                        const uint64_t kj = rank_key(E[j], j);
                        mn = kj < mn ? kj : mn;
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
    for (int w = tid; w < W; w += nt) sb[w] = ge[w];
    int ne_loc = 0;
    for (int w = tid; w < W; w += nt) ne_loc += __popc(ge[w]);
    const int n_e = block_sum_int(ne_loc, red32);
    const int kq = min(dm.k_q, n_cand - n_e);
    if (kq > 0) {
        for (int i = tid; i < P; i += nt) {
            const bool in_e = i < n_cand && ((ge[i >> 5] >> (i & 31)) & 1u);
            keys[i] = (i < n_cand && !in_e) ? rank_key(Sq[i], i) : 0ull;
        }
        __syncthreads();
        bitonic_desc(keys, P);
        for (int i = tid; i < kq; i += nt) {
            const int j = key_index(keys[i]);
            atomicOr(&sb[j >> 5], 1u << (j & 31));
        }
    }
    __syncthreads();

    // ---- write state and the ascending selection ----
    for (int w = tid; w < W; w += nt) {
        ge_g[w] = ge[w];
        ev_g[w] = ev[w];
        sel_bits[(int64_t)r * W + w] = sb[w];
    }
    if (tid == 0) {
        int acc = 0;
        for (int w = 0; w < W; ++w) { woff[w] = acc; acc += __popc(sb[w]); }
        woff[W] = acc;
    }
    __syncthreads();
    int32_t *out = sel + (int64_t)r * dm.k;
    for (int w = tid; w < W; w += nt) {
        uint32_t bits = sb[w];
        int pos = woff[w];
        while (bits && pos < dm.k) {
            out[pos++] = w * 32 + __ffs(bits) - 1;
            bits &= bits - 1u;
        }
    }
    const int total = min(woff[W], dm.k);
    for (int i = total + tid; i < dm.k; i += nt) out[i] = -1;
    if (tid == 0) n_sel[r] = total;
}

// ---------------------------------------------------------------------------
// Set difference: one wave per row. Ballot + popcount prefixes compact the
// fetch list (ascending block id) and the free slots (ascending slot id).
// ---------------------------------------------------------------------------
constexpr int MAX_K = 128;

__global__ void __launch_bounds__(64)
swap_kernel(Dims dm, const int32_t *__restrict__ sel, const int32_t *__restrict__ n_sel,
            const uint32_t *__restrict__ sel_bits, int32_t *__restrict__ slot_block,
            int32_t *__restrict__ block_slot, int32_t *__restrict__ fetch_block,
            int32_t *__restrict__ fetch_slot, int32_t *__restrict__ n_fetch,
            uint64_t *__restrict__ counters) {
    __shared__ int fb[MAX_K], fs[MAX_K];
    const int r = blockIdx.x, lane = threadIdx.x, k = dm.k;
    const int32_t *s = sel + (int64_t)r * k;
    const int ns = min(max(n_sel[r], 0), k);
    int32_t *sbk = slot_block + (int64_t)r * k;
    int32_t *bsl = block_slot + (int64_t)r * dm.max_blocks;
    const uint32_t *bits = sel_bits + (int64_t)r * dm.W;
    const uint64_t lt = lanemask_lt();

    int nf = 0, kept = 0;
    for (int base = 0; base < ns; base += 64) {
        const int i = base + lane;
        const int blk = i < ns ? s[i] : -1;
        const bool ok = blk >= 0 && blk < dm.max_blocks;
        const bool need = ok && bsl[blk] < 0;
        const uint64_t m = __ballot(need);
        if (need) fb[nf + __popcll(m & lt)] = blk;
        nf += __popcll(m);
        kept += __popcll(__ballot(ok && !need));
    }
    int nfree = 0;
    for (int base = 0; base < k; base += 64) {
        const int sl = base + lane;
        bool fr = false;
        if (sl < k) {
            const int blk = sbk[sl];
            fr = blk < 0 || blk >= dm.max_blocks || !((bits[blk >> 5] >> (blk & 31)) & 1u);
        }
        const uint64_t m = __ballot(fr);
        if (fr) fs[nfree + __popcll(m & lt)] = sl;
        nfree += __popcll(m);
    }
    __syncthreads();
    for (int i = lane; i < nfree; i += 64) {
        const int sl = fs[i];
        const int old = sbk[sl];
        if (old >= 0 && old < dm.max_blocks) bsl[old] = -1;
        sbk[sl] = -1;
    }
    __syncthreads();
    int32_t *fbo = fetch_block + (int64_t)r * k;
    int32_t *fso = fetch_slot + (int64_t)r * k;
    for (int i = lane; i < k; i += 64) {
        if (i < nf) {
            const int blk = fb[i], sl = fs[i];
            sbk[sl] = blk;
            bsl[blk] = sl;
            fbo[i] = blk;
            fso[i] = sl;
        } else {
            fbo[i] = -1;
            fso[i] = -1;
        }
    }
    if (lane == 0) {
        n_fetch[r] = nf;
        counters[2 * r] += (uint64_t)nf;
        counters[2 * r + 1] += (uint64_t)kept;
    }
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
                       float *kbar, float *e_blk, hipStream_t st) {
    dim3 grid(blk_end - blk_begin, dm.rows);
    hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(256), 0, st, dm,
                       static_cast<const T *>(kv), kv_row_blocks, kv_first, e_tok, e_stride,
                       blk_begin, kbar, e_blk);
    return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t launch_score(const Dims &dm, const void *q, const float *kbar, int n_cand, float *s_q,
                        hipStream_t st) {
    dim3 grid((4 * n_cand + 255) / 256, dm.rows);
    hipLaunchKernelGGL((score_kernel<T, D, G>), grid, dim3(256), 0, st, dm,
                       static_cast<const T *>(q), kbar, n_cand, s_q);
    return hipGetLastError();
}

hipError_t launch_select(const Dims &dm, const float *s_q, const float *e_blk, int n_cand,
                         int n_prev, uint32_t *ge, uint32_t *ev, int32_t *sel, int32_t *n_sel,
                         uint32_t *sel_bits, hipStream_t st) {
    int P = 2;
    while (P < n_cand) P <<= 1;
    hipLaunchKernelGGL(select_kernel, dim3(dm.rows), dim3(SELECT_THREADS), P * sizeof(uint64_t),
                       st, dm, s_q, e_blk, n_cand, n_prev, P, ge, ev, sel, n_sel, sel_bits);
    return hipGetLastError();
}

hipError_t launch_swap(const Dims &dm, const int32_t *sel, const int32_t *n_sel,
                       const uint32_t *sel_bits, int32_t *slot_block, int32_t *block_slot,
                       int32_t *fetch_block, int32_t *fetch_slot, int32_t *n_fetch,
                       uint64_t *counters, hipStream_t st) {
    hipLaunchKernelGGL(swap_kernel, dim3(dm.rows), dim3(64), 0, st, dm, sel, n_sel, sel_bits,
                       slot_block, block_slot, fetch_block, fetch_slot, n_fetch, counters);
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
                                          const float *, int64_t, int, int, float *, float *,  \
                                          hipStream_t);
NOSA_POOL_INST(float, 64)
NOSA_POOL_INST(float, 128)
NOSA_POOL_INST(bf16_t, 64)
NOSA_POOL_INST(bf16_t, 128)

#define NOSA_SCORE_INST(T, D, G)                                                               \
    template hipError_t launch_score<T, D, G>(const Dims &, const void *, const float *, int,  \
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
