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
// Select: one workgroup (8 waves) per row.
//  * top-k with k <= 64: each wave sorts 64 rank keys at a time across its
//    lanes (bitonic network on lane shuffles, no barriers) and keeps a
//    running sorted top-64; wave 0 then merges the 8 waves' lists.
//  * top-k with k > 64 (an eviction budget above 64 at initialisation):
//    bitonic sort of all keys in LDS.
//  * Gamma_e after initialisation: each new candidate in turn replaces the
//    lowest-ranked member if it ranks above it, else it is evicted.
//  * the ascending selection list comes from a popcount prefix scan.
//  * optionally the set difference against the block cache runs in the same
//    workgroup (wave 0), saving a launch and a round trip per step.
// ---------------------------------------------------------------------------
constexpr int SELECT_THREADS = 512;
constexpr int SELECT_WAVES = SELECT_THREADS / 64;
constexpr int MAX_W = 128;   // 4096 blocks
constexpr int MAX_K = 128;
constexpr int WAVE_TOPK = 64;

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Sort the wave's 64 keys (one per lane) descending: lane 0 holds the largest.
__device__ uint64_t wave_sort_desc(uint64_t x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k2 = 2; k2 <= 64; k2 <<= 1) {
#pragma unroll
        for (int j2 = k2 >> 1; j2 > 0; j2 >>= 1) {
            const uint64_t y = __shfl_xor(x, j2, 64);
            const bool desc = (lane & k2) == 0;
            const bool lower = (lane & j2) == 0;
            x = (lower == desc) ? umax64(x, y) : umin64(x, y);
        }
    }
    return x;
}

// a and b sorted descending across the wave -> the 64 largest of both,
// sorted descending (max against the reversed list gives a bitonic
// sequence holding them, which a half-cleaner cascade sorts).
__device__ uint64_t wave_merge_top(uint64_t a, uint64_t b) {
    const int lane = threadIdx.x & 63;
    uint64_t x = umax64(a, __shfl(b, 63 - lane, 64));
#pragma unroll
    for (int j2 = 32; j2 > 0; j2 >>= 1) {
        const uint64_t y = __shfl_xor(x, j2, 64);
        x = (lane & j2) == 0 ? umax64(x, y) : umin64(x, y);
    }
    return x;
}

// The 64 largest keys of key_of(0..n-1) (0 = not a candidate), sorted
// descending, into top[0..64) in LDS.
template <typename KeyFn>
__device__ void topk_waves(int n, KeyFn key_of, uint64_t *lists, uint64_t *top) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint64_t best = 0ull;
    for (int base = wave * 64; base < n; base += SELECT_WAVES * 64) {
        const int j = base + lane;
        uint64_t x = j < n ? key_of(j) : 0ull;
        if (__ballot(x != 0ull) == 0ull) continue;
        best = wave_merge_top(best, wave_sort_desc(x));
    }
    lists[wave * 64 + lane] = best;
    __syncthreads();
    if (wave == 0) {
        uint64_t acc = lists[lane];
        for (int w = 1; w < SELECT_WAVES; ++w) acc = wave_merge_top(acc, lists[w * 64 + lane]);
        top[lane] = acc;
    }
    __syncthreads();
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

// Set difference of one row, run by one wave. sel (ascending, ns entries)
// and bits may live in LDS or global memory. Every output address is written
// once: free slot i receives fetched block i (or becomes empty), the blocks
// they held lose their slot, the fetched blocks gain one.
__device__ void swap_row(const Dims &dm, int r, const int32_t *sel, int ns, const uint32_t *bits,
                         int32_t *__restrict__ slot_block, int32_t *__restrict__ block_slot,
                         int32_t *__restrict__ fetch_block, int32_t *__restrict__ fetch_slot,
                         int32_t *__restrict__ n_fetch, uint64_t *__restrict__ counters,
                         int *fb, int *fs, int *fo) {
    const int lane = threadIdx.x & 63, k = dm.k;
    int32_t *sbk = slot_block + (int64_t)r * k;
    int32_t *bsl = block_slot + (int64_t)r * dm.max_blocks;
    const uint64_t lt = lanemask_lt();
    ns = min(max(ns, 0), k);
    int nf = 0, kept = 0;
    for (int base = 0; base < ns; base += 64) {
        const int i = base + lane;
        const int blk = i < ns ? sel[i] : -1;
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
        int blk = -1;
        bool fr = false;
        if (sl < k) {
            blk = sbk[sl];
            fr = blk < 0 || blk >= dm.max_blocks || !((bits[blk >> 5] >> (blk & 31)) & 1u);
        }
        const uint64_t m = __ballot(fr);
        if (fr) {
            const int at = nfree + __popcll(m & lt);
            fs[at] = sl;
            fo[at] = blk;
        }
        nfree += __popcll(m);
    }
    wave_sync_lds();
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
    int32_t *fbo = fetch_block + (int64_t)r * k;
    int32_t *fso = fetch_slot + (int64_t)r * k;
    for (int i = lane; i < k; i += 64) {
        fbo[i] = i < nf ? fb[i] : -1;
        fso[i] = i < nf ? fs[i] : -1;
    }
    if (lane == 0) {
        n_fetch[r] = nf;
        counters[2 * r] += (uint64_t)nf;
        counters[2 * r + 1] += (uint64_t)kept;
    }
}

struct SwapArgs {
    int32_t *slot_block, *block_slot, *fetch_block, *fetch_slot, *n_fetch;
    uint64_t *counters;
};

__global__ void __launch_bounds__(SELECT_THREADS)
select_kernel(Dims dm, const float *__restrict__ s_q, const float *__restrict__ e_blk, int n_cand,
              int n_prev, int P, uint32_t *__restrict__ ge_bits, uint32_t *__restrict__ ev_bits,
              int32_t *__restrict__ sel, int32_t *__restrict__ n_sel,
              uint32_t *__restrict__ sel_bits, SwapArgs sw) {
    extern __shared__ uint64_t keys[];  // P keys, only when a budget exceeds 64
    __shared__ uint32_t ge[MAX_W], ev[MAX_W], sb[MAX_W];
    __shared__ uint64_t lists[SELECT_WAVES * 64], top[64];
    __shared__ uint64_t red64[SELECT_WAVES];
    __shared__ int red32[SELECT_WAVES];
    __shared__ int sel_l[MAX_K], fb[MAX_K], fs[MAX_K], fo[MAX_K];
    __shared__ int n_sel_l;
    const int r = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int W = dm.W;
    const float *E = e_blk + (int64_t)r * dm.max_blocks;
    const float *Sq = s_q + (int64_t)r * dm.max_blocks;
    uint32_t *ge_g = ge_bits + (int64_t)r * W;
    uint32_t *ev_g = ev_bits + (int64_t)r * W;

    // ---- Gamma_e ----
    if (n_prev < 0) {
        for (int w = tid; w < W; w += nt) { ge[w] = 0u; ev[w] = 0u; }
        __syncthreads();
        const int ke = min(dm.k_e, n_cand);
        if (ke > 0 && dm.k_e <= WAVE_TOPK) {
            topk_waves(n_cand, [&](int j) { return rank_key(E[j], j); }, lists, top);
            if (tid < ke) {
                const int j = key_index(top[tid]);
                atomicOr(&ge[j >> 5], 1u << (j & 31));
            }
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
    for (int w = tid; w < W; w += nt) sb[w] = ge[w];
    int ne_loc = 0;
    for (int w = tid; w < W; w += nt) ne_loc += __popc(ge[w]);
    const int n_e = block_sum_int(ne_loc, red32);
    const int kq = min(dm.k_q, n_cand - n_e);
    auto q_key = [&](int j) -> uint64_t {
        return ((ge[j >> 5] >> (j & 31)) & 1u) ? 0ull : rank_key(Sq[j], j);
    };
    if (kq > 0 && dm.k_q <= WAVE_TOPK) {
        topk_waves(n_cand, q_key, lists, top);
        if (tid < kq) {
            const int j = key_index(top[tid]);
            atomicOr(&sb[j >> 5], 1u << (j & 31));
        }
    } else if (kq > 0) {
        for (int i = tid; i < P; i += nt) keys[i] = i < n_cand ? q_key(i) : 0ull;
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
    if (wave == 0) {
        // lane l holds words 2l and 2l+1; exclusive prefix of their popcounts
        const uint32_t w0 = 2 * lane < W ? sb[2 * lane] : 0u;
        const uint32_t w1 = 2 * lane + 1 < W ? sb[2 * lane + 1] : 0u;
        const int cnt = __popc(w0) + __popc(w1);
        int inc = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
        }
        int pos = inc - cnt;
        int32_t *out = sel + (int64_t)r * dm.k;
        uint32_t bits = w0;
        while (bits && pos < dm.k) {
            const int j = 2 * lane * 32 + __ffs(bits) - 1;
            bits &= bits - 1u;
            out[pos] = j;
            sel_l[pos++] = j;
        }
        bits = w1;
        while (bits && pos < dm.k) {
            const int j = (2 * lane + 1) * 32 + __ffs(bits) - 1;
            bits &= bits - 1u;
            out[pos] = j;
            sel_l[pos++] = j;
        }
        const int total = min(__shfl(inc, 63, 64), dm.k);
        for (int i = total + lane; i < dm.k; i += 64) out[i] = -1;
        if (lane == 0) {
            n_sel[r] = total;
            n_sel_l = total;
        }
        if (sw.slot_block) {
            wave_sync_lds();
            swap_row(dm, r, sel_l, n_sel_l, sb, sw.slot_block, sw.block_slot, sw.fetch_block,
                     sw.fetch_slot, sw.n_fetch, sw.counters, fb, fs, fo);
        }
    }
}

// Stand-alone set difference: one wave per row, inputs from global memory.
__global__ void __launch_bounds__(64)
swap_kernel(Dims dm, const int32_t *__restrict__ sel, const int32_t *__restrict__ n_sel,
            const uint32_t *__restrict__ sel_bits, SwapArgs sw) {
    __shared__ int fb[MAX_K], fs[MAX_K], fo[MAX_K];
    const int r = blockIdx.x;
    swap_row(dm, r, sel + (int64_t)r * dm.k, n_sel[r], sel_bits + (int64_t)r * dm.W,
             sw.slot_block, sw.block_slot, sw.fetch_block, sw.fetch_slot, sw.n_fetch,
             sw.counters, fb, fs, fo);
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
                         uint32_t *sel_bits, const SwapPtrs *swap, hipStream_t st) {
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
    hipLaunchKernelGGL(select_kernel, dim3(dm.rows), dim3(SELECT_THREADS), P * sizeof(uint64_t),
                       st, dm, s_q, e_blk, n_cand, n_prev, P, ge, ev, sel, n_sel, sel_bits, sw);
    return hipGetLastError();
}

hipError_t launch_swap(const Dims &dm, const int32_t *sel, const int32_t *n_sel,
                       const uint32_t *sel_bits, const SwapPtrs &swap, hipStream_t st) {
    SwapArgs sw{swap.slot_block, swap.block_slot, swap.fetch_block, swap.fetch_slot, swap.n_fetch,
                swap.counters};
    hipLaunchKernelGGL(swap_kernel, dim3(dm.rows), dim3(64), 0, st, dm, sel, n_sel, sel_bits, sw);
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
