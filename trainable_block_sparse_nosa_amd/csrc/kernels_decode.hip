// Sparse decode attention with the ED-DMA logit bias, split-K over blocks.
//
// NOSA technical summary, Methodology, "1. Algorithm: NOSA", bullet "ED-DMA":
// eviction scores are kept pre-exponential through selection and their
// exponential happens in the attention softmax; here each token's score is
// added to its logit, z = scale * q.k + e, and softmax(z) weighs the values.
//
// Work split: one workgroup per (chunk of list entries, row). For every
// block of its chunk a workgroup stages the K tile [64][D] and the V^T tile
// [D][64] in LDS with coalesced 16-byte loads, computes the G x 64 logits,
// updates a running (max, sum, output) per head (online softmax) and keeps
// its partial in a workspace. A second kernel merges the partials of a row in
// chunk order, so results do not depend on scheduling.
#include "kernels.h"

namespace nosa {

DecodePlan decode_plan(const Dims &dm) {
    // Enough workgroups to cover 256 CUs several times over, and no fewer
    // than one block per chunk.
    const int entries = dm.k + 1;
    const long total = (long)dm.rows * entries;
    int cb = 1;
    while (cb < 16 && total / (cb * 2) >= 2048) cb *= 2;
    DecodePlan p;
    p.cb = cb;
    p.n_chunks = (entries + cb - 1) / cb;
    return p;
}

template <typename T, int D, int G>
__global__ void __launch_bounds__(256)
decode_valu_kernel(Dims dm, int cb, int n_chunks, const T *__restrict__ q,
                   const T *__restrict__ kv, int64_t kv_row_blocks, int kv_mode,
                   const int32_t *__restrict__ list, const int32_t *__restrict__ n_list,
                   const T *__restrict__ cur, int64_t cur_row_blocks, int n_tokens, int n_cand,
                   const float *__restrict__ e_tok, int64_t e_stride, float *__restrict__ ws_o,
                   float *__restrict__ ws_ml) {
    constexpr int S = 64;
    constexpr int EPV = 16 / sizeof(T);     // elements per 16-byte vector
    constexpr int KP = D + EPV;             // padded LDS row of the K tile
    constexpr int VP = S + EPV;             // padded LDS row of the V^T tile
    constexpr int NPT = (G * D + 255) / 256;  // outputs per thread
    constexpr int64_t BE = 2 * S * D;       // elements per block-unit
    __shared__ __attribute__((aligned(16))) T Ks[S * KP];
    __shared__ __attribute__((aligned(16))) T Vs[D * VP];
    __shared__ __attribute__((aligned(16))) float qs[G * D];
    __shared__ __attribute__((aligned(16))) float ps[G * S];
    __shared__ float m_sh[G], l_sh[G], a_sh[G];

    const int tid = threadIdx.x;
    const int r = blockIdx.y, chunk = blockIdx.x;
    const int b = r / dm.Hkv, g = r % dm.Hkv;
    const T *qr = q + ((int64_t)b * dm.Hq + (int64_t)g * G) * D;
    for (int p = tid; p < G * D; p += 256) qs[p] = ldf(qr + p) * dm.scale;
    if (tid < G) { m_sh[tid] = -INFINITY; l_sh[tid] = 0.f; }
    float o[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i) o[i] = 0.f;

    const int k = dm.k;
    const int cnt = kv_mode == NOSA_KV_FULL ? n_list[r] : k;
    const int e0 = chunk * cb, e1 = min(e0 + cb, k + 1);
    const float *er = e_tok + (int64_t)r * e_stride;

    for (int e = e0; e < e1; ++e) {
        const T *blk;
        int bid, valid;
        if (e == k) {
            blk = cur + (int64_t)r * cur_row_blocks * BE;
            bid = n_cand;
            valid = n_tokens - n_cand * S;
        } else {
            if (e >= cnt) continue;
            bid = list[(int64_t)r * k + e];
            if (bid < 0 || bid >= n_cand) continue;  // only candidates are ever listed
            const int64_t at = kv_mode == NOSA_KV_FULL ? bid : e;
            blk = kv + ((int64_t)r * kv_row_blocks + at) * BE;
            valid = S;
        }
        __syncthreads();  // the previous block's readers are done with LDS
        // stage K [S][D] and V^T [D][S]: 16-byte vectors, consecutive threads
        // take consecutive vectors of the block
        constexpr int KV_VEC = S * D / EPV;
        for (int v = tid; v < KV_VEC; v += 256) {
            const int row = v / (D / EPV), col = (v % (D / EPV)) * EPV;
            *reinterpret_cast<uint4 *>(Ks + row * KP + col) =
                reinterpret_cast<const uint4 *>(blk)[v];
        }
        for (int v = tid; v < KV_VEC; v += 256) {
            const int row = v / (S / EPV), col = (v % (S / EPV)) * EPV;
            *reinterpret_cast<uint4 *>(Vs + row * VP + col) =
                reinterpret_cast<const uint4 *>(blk + S * D)[v];
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

        // P.V: thread <-> (head, dim)
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
                    const float4 p0 = *reinterpret_cast<const float4 *>(ps + h * S + t);
                    const float4 p1 = *reinterpret_cast<const float4 *>(ps + h * S + t + 4);
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
    const int64_t base = ((int64_t)r * n_chunks + chunk) * G;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const int p = tid + i * 256;
        if (p < G * D) ws_o[base * D + p] = o[i];
    }
    if (tid < G) {
        ws_ml[(base + tid) * 2 + 0] = m_sh[tid];
        ws_ml[(base + tid) * 2 + 1] = l_sh[tid];
    }
}

// Merge a row's chunk partials in chunk order.
template <typename T, int D, int G>
__global__ void __launch_bounds__(256)
combine_kernel(Dims dm, int n_chunks, const float *__restrict__ ws_o,
               const float *__restrict__ ws_ml, T *__restrict__ out) {
    const int r = blockIdx.x;
    const int b = r / dm.Hkv, g = r % dm.Hkv;
    for (int p = threadIdx.x; p < G * D; p += blockDim.x) {
        const int h = p / D, d = p % D;
        float M = -INFINITY;
        for (int c = 0; c < n_chunks; ++c) {
            const int64_t at = (((int64_t)r * n_chunks + c) * G + h) * 2;
            if (ws_ml[at + 1] > 0.f) M = fmaxf(M, ws_ml[at]);
        }
        float L = 0.f, O = 0.f;
        for (int c = 0; c < n_chunks; ++c) {
            const int64_t at = ((int64_t)r * n_chunks + c) * G + h;
            const float l = ws_ml[at * 2 + 1];
            if (l > 0.f) {
                const float w = __expf(ws_ml[at * 2] - M);
                L = fmaf(l, w, L);
                O = fmaf(ws_o[at * D + d], w, O);
            }
        }
        out[((int64_t)b * dm.Hq + (int64_t)g * G + h) * D + d] = stf<T>(O / L);
    }
}

template <typename T, int D, int G>
hipError_t launch_decode_valu(const Dims &dm, const DecodePlan &pl, const DecodeArgs &a,
                              hipStream_t st) {
    dim3 grid(pl.n_chunks, dm.rows);
    hipLaunchKernelGGL((decode_valu_kernel<T, D, G>), grid, dim3(256), 0, st, dm, pl.cb,
                       pl.n_chunks, static_cast<const T *>(a.q), static_cast<const T *>(a.kv),
                       a.kv_row_blocks, a.kv_mode, a.list, a.n_list,
                       static_cast<const T *>(a.cur), a.cur_row_blocks, a.n_tokens, a.n_cand,
                       a.e_tok, a.e_stride, a.ws_o, a.ws_ml);
    return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t launch_combine(const Dims &dm, const DecodePlan &pl, const DecodeArgs &a,
                          hipStream_t st) {
    hipLaunchKernelGGL((combine_kernel<T, D, G>), dim3(dm.rows), dim3(256), 0, st, dm,
                       pl.n_chunks, a.ws_o, a.ws_ml, static_cast<T *>(a.out));
    return hipGetLastError();
}

#define NOSA_DEC_INST(T, D, G)                                                                 \
    template hipError_t launch_decode_valu<T, D, G>(const Dims &, const DecodePlan &,          \
                                                    const DecodeArgs &, hipStream_t);          \
    template hipError_t launch_combine<T, D, G>(const Dims &, const DecodePlan &,              \
                                                const DecodeArgs &, hipStream_t);
#define NOSA_DEC_ALLG(T, D)                                                                    \
    NOSA_DEC_INST(T, D, 1) NOSA_DEC_INST(T, D, 2) NOSA_DEC_INST(T, D, 3)                       \
    NOSA_DEC_INST(T, D, 4) NOSA_DEC_INST(T, D, 5) NOSA_DEC_INST(T, D, 6)                       \
    NOSA_DEC_INST(T, D, 7) NOSA_DEC_INST(T, D, 8)
NOSA_DEC_ALLG(float, 64)
NOSA_DEC_ALLG(float, 128)
NOSA_DEC_ALLG(bf16_t, 64)
NOSA_DEC_ALLG(bf16_t, 128)

}  // namespace nosa
