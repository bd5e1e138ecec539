// Device helpers shared by the NOSA gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "nosa.h"

namespace nosa {

// Host-validated, derived shape passed by value to every kernel.
struct Dims {
    int B, Hq, Hkv, G, D, S, sub, m;
    int k_e, k_q, k;
    int max_blocks, W;  // per-row block capacity, bitmap words per row
    int rows;
    int dtype;
    int pdtype;  // pooled dtype (kbar, qbar): NOSA_F32 or NOSA_BF16
    float scale;
};

// The step record in device memory ({n_tokens, n_cand_prev}, nosa_step's
// layout) for steps replayed from a captured graph: kernels read it instead
// of taking the values as launch arguments. n_tokens is clamped to the
// shape's capacity so that no index derived from it leaves the buffers.
struct StepVals {
    int n_tokens, n_cand, n_prev;
};
__device__ __forceinline__ StepVals read_step(const int32_t *dstep, const struct Dims &dm);

using bf16_t = uint16_t;  // bfloat16 storage
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// MFMA operand types: eight bf16 (A/B of 16x16x32 bf16), four fp32 (C/D)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Pooled keys of bfloat16 KV kept in float32 (pooled dtype NOSA_F32) are
// scored in certified form: the kbar buffer holds, after the float32 means
// (region 0, [rows][Q][D/4][16][4]), their bfloat16 roundings (region 1, the
// bfloat16 pooled-key layout [rows][Q][D/8][16][8]) and a float32 radius per
// block (region 2, [rows][max_blocks]). Element counts and byte offsets:
__host__ __device__ inline int64_t kbar_elems(const Dims &dm) {
    return (int64_t)dm.rows * ((dm.max_blocks + 3) / 4) * 16 * dm.D;
}
__host__ __device__ inline bool kbar_certified(const Dims &dm) {
    return dm.dtype == NOSA_BF16 && dm.pdtype == NOSA_F32;
}
__host__ __device__ inline int64_t kbar_shadow_offset(const Dims &dm) { return kbar_elems(dm) * 4; }
__host__ __device__ inline int64_t kbar_radius_offset(const Dims &dm) { return kbar_elems(dm) * 6; }
__host__ __device__ inline int64_t kbar_bytes(const Dims &dm) {
    if (!kbar_certified(dm)) return kbar_elems(dm) * (dm.pdtype == NOSA_F32 ? 4 : 2);
    return kbar_radius_offset(dm) + (int64_t)dm.rows * dm.max_blocks * 4;
}

__device__ __forceinline__ StepVals read_step(const int32_t *dstep, const Dims &dm) {
    const int n = min(max(dstep[0], 1), dm.max_blocks * dm.S);
    const int c = (n - 1) / dm.S;
    return StepVals{n, c, min(max(dstep[1], -1), c)};
}

__device__ __forceinline__ float bf2f(uint32_t h16) { return __uint_as_float(h16 << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bfloat16, round to nearest even (inputs are finite).
__device__ __forceinline__ bf16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

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

template <typename T> __device__ __forceinline__ float ldf(const T *p);
template <> __device__ __forceinline__ float ldf<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float ldf<bf16_t>(const bf16_t *p) { return bf2f(*p); }

template <typename T> __device__ __forceinline__ T stf(float v);
template <> __device__ __forceinline__ float stf<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t stf<bf16_t>(float v) { return f2bf(v); }

// Eight consecutive elements as floats from a 16-byte-aligned address (bf16)
// or two 16-byte loads (fp32).
template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
    __device__ __forceinline__ static void load(const bf16_t *p, float (&x)[8]) {
        uint4 v = *reinterpret_cast<const uint4 *>(p);
        x[0] = bf_lo(v.x); x[1] = bf_hi(v.x); x[2] = bf_lo(v.y); x[3] = bf_hi(v.y);
        x[4] = bf_lo(v.z); x[5] = bf_hi(v.z); x[6] = bf_lo(v.w); x[7] = bf_hi(v.w);
    }
};
template <> struct Vec8<float> {
    __device__ __forceinline__ static void load(const float *p, float (&x)[8]) {
        float4 a = reinterpret_cast<const float4 *>(p)[0];
        float4 b = reinterpret_cast<const float4 *>(p)[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
};

// Token order of the stored V^T tile: position pos (0..63) of a V^T row
// holds token vt_token_at(pos); within each 32-token half, positions
// 8g..8g+7 hold tokens 4g..4g+3 and 16+4g..16+4g+3. vt_pos_of is the inverse.
__host__ __device__ constexpr int vt_token_at(int pos) {
    return 32 * (pos / 32) + 16 * ((pos % 8) / 4) + 4 * ((pos % 32) / 8) + pos % 4;
}
__host__ __device__ constexpr int vt_pos_of(int tok) {
    return 32 * (tok / 32) + 8 * ((tok % 16) / 4) + 4 * ((tok % 32) / 16) + tok % 4;
}
constexpr bool vt_order_is_inverse() {
    for (int p = 0; p < 64; ++p)
        if (vt_pos_of(vt_token_at(p)) != p) return false;
    return true;
}
static_assert(vt_order_is_inverse(), "vt_pos_of inverts vt_token_at");

// Block-unit KV layout: a block of 64 tokens is the K tile, S * D elements,
// then the V^T tile, D * S elements, each stored as 1 KiB fragments of 64
// 16-byte vectors (E = 16 / sizeof(T) elements each). Vector l of a fragment
// holds what lane l of a wave loads for a matrix-core operand, with col =
// l % 16 and grp = l / 16:
//  K fragment t * NS + s (NS = D / 4E): token 16 t + col, dimensions
//    (4 s + grp) E .. + E - 1;
//  V^T fragment dt * NP + s (NP = 64 / 4E): dimension 16 dt + col, stored
//    positions (4 s + grp) E .. + E - 1 of the V^T row, whose tokens are
//    vt_token_at(position).
// For bfloat16 a fragment is exactly one A operand of v_mfma_f32_16x16x32_bf16,
// so each load instruction of a wave reads 1 KiB of consecutive whole cache
// lines. Element offsets within the block:
template <typename T, int D>
__host__ __device__ constexpr int kv_k_off(int tok, int d) {
    constexpr int E = 16 / sizeof(T), NS = D / (4 * E);
    return (((tok / 16) * NS + d / (4 * E)) * 64 + tok % 16 + 16 * ((d / E) % 4)) * E + d % E;
}
template <typename T, int D>
__host__ __device__ constexpr int kv_v_off(int tok, int d) {
    constexpr int E = 16 / sizeof(T), NP = 64 / (4 * E);
    const int pos = vt_pos_of(tok);
    return 64 * D +
           (((d / 16) * NP + pos / (4 * E)) * 64 + d % 16 + 16 * ((pos / E) % 4)) * E + pos % E;
}
// The inverse for the VALU kernel's staging: 16-byte vector v of the K (or
// V^T) tile holds token (dimension) row and dimensions (positions) col0 ..
template <typename T, int D>
__host__ __device__ constexpr void kv_k_vec(int v, int &tok, int &d0) {
    constexpr int E = 16 / sizeof(T), NS = D / (4 * E);
    const int f = v / 64, l = v % 64;
    tok = 16 * (f / NS) + l % 16;
    d0 = (4 * (f % NS) + l / 16) * E;
}
template <typename T, int D>
__host__ __device__ constexpr void kv_v_vec(int v, int &d, int &pos0) {
    constexpr int E = 16 / sizeof(T), NP = 64 / (4 * E);
    const int f = v / 64, l = v % 64;
    d = 16 * (f / NP) + l % 16;
    pos0 = (4 * (f % NP) + l / 16) * E;
}
template <typename T, int D>
constexpr bool kv_layout_is_bijective() {
    // every element lands once, and the vector inverses agree
    constexpr int E = 16 / sizeof(T);
    bool seen[2 * 64 * D] = {};
    for (int t = 0; t < 64; ++t)
        for (int d = 0; d < D; ++d) {
            const int a = kv_k_off<T, D>(t, d), b = kv_v_off<T, D>(t, d);
            if (a < 0 || a >= 64 * D || b < 64 * D || b >= 128 * D || seen[a] || seen[b]) return false;
            seen[a] = seen[b] = true;
        }
    for (int v = 0; v < 64 * D / E; ++v) {
        int t = 0, d0 = 0, dd = 0, p0 = 0;
        kv_k_vec<T, D>(v, t, d0);
        kv_v_vec<T, D>(v, dd, p0);
        if (kv_k_off<T, D>(t, d0) != v * E) return false;
        if (kv_v_off<T, D>(vt_token_at(p0), dd) != 64 * D + v * E) return false;
    }
    return true;
}
static_assert(kv_layout_is_bijective<uint16_t, 64>() && kv_layout_is_bijective<uint16_t, 128>() &&
                  kv_layout_is_bijective<float, 64>() && kv_layout_is_bijective<float, 128>(),
              "block layout");

// Total order used by every selection: a higher score ranks first, an equal
// score ranks the lower block id first. Keys compare as unsigned integers.
// -0 and +0 are equal scores, so -0 is mapped to +0 first (the id decides).
__device__ __forceinline__ uint32_t orderable(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t rank_key(float score, int j) {
    return ((uint64_t)orderable(score) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}
__device__ __forceinline__ int key_index(uint64_t key) {
    return (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull));
}

// DPP lane permutations inside groups of four lanes (quad_perm controls).
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int QUAD_SWAP1 = 0xB1;  // [1,0,3,2]
constexpr int QUAD_SWAP2 = 0x4E;  // [2,3,0,1]

__device__ __forceinline__ float quad_max(float v) {
    v = fmaxf(v, dpp_f<QUAD_SWAP1>(v));
    v = fmaxf(v, dpp_f<QUAD_SWAP2>(v));
    return v;
}

// One DPP move of v (lanes without a source, or in rows outside ROWS, get
// `old`, or 0 with BOUND_ZERO).
template <int CTRL, int ROWS, bool BOUND_ZERO>
__device__ __forceinline__ float dpp_move(float old, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL,
                                                      ROWS, 0xF, BOUND_ZERO));
}
constexpr int DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114,
              DPP_ROW_SHR8 = 0x118, DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;

// Max / sum over the 64 lanes of a wave on DPP: a log-step scan inside each
// row of 16 lanes (row_shr 1, 2, 4, 8), the row results carried across rows
// by the GFX9 row broadcasts (lane 15 of rows 0 and 2 into rows 1 and 3,
// then lane 31 into rows 2 and 3), so lane 63 ends with the whole wave's;
// every lane gets that value. Every lane must be active.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_move<DPP_ROW_SHR1, 0xF, false>(v, v));
    v = fmaxf(v, dpp_move<DPP_ROW_SHR2, 0xF, false>(v, v));
    v = fmaxf(v, dpp_move<DPP_ROW_SHR4, 0xF, false>(v, v));
    v = fmaxf(v, dpp_move<DPP_ROW_SHR8, 0xF, false>(v, v));
    v = fmaxf(v, dpp_move<DPP_ROW_BCAST15, 0xA, false>(v, v));
    v = fmaxf(v, dpp_move<DPP_ROW_BCAST31, 0xC, false>(v, v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_move<DPP_ROW_SHR1, 0xF, true>(0.f, v);
    v += dpp_move<DPP_ROW_SHR2, 0xF, true>(0.f, v);
    v += dpp_move<DPP_ROW_SHR4, 0xF, true>(0.f, v);
    v += dpp_move<DPP_ROW_SHR8, 0xF, true>(0.f, v);
    v += dpp_move<DPP_ROW_BCAST15, 0xA, false>(0.f, v);
    v += dpp_move<DPP_ROW_BCAST31, 0xC, false>(0.f, v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const unsigned lane = threadIdx.x & 63u;
    return lane ? (~0ull >> (64u - lane)) : 0ull;
}

}  // namespace nosa
