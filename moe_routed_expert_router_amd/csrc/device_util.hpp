// Device building blocks shared by the routing and grouping kernels.
#pragma once

#include "common.hpp"

namespace moe {

// ---- wave-level primitives on DPP lane moves (VALU, no LDS round trip) ----
// DPP controls: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// row_half_mirror (i <-> 7-i in each 8 lanes), row_mirror (i <-> 15-i in each
// row of 16), row_shr:n (from lane - n in the row).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_movf(float v) {
    return __int_as_float(dpp_mov<CTRL>(__float_as_int(v)));
}
__device__ __forceinline__ float readlanef(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Arg-max order: the larger value wins, equal values go to the lower index.
__device__ __forceinline__ bool beats(float av, int ae, float bv, int be) {
    return av > bv || (av == bv && ae < be);
}

template <int CTRL>
__device__ __forceinline__ void argmax_step(float &v, int &e) {
    const float ov = dpp_movf<CTRL>(v);
    const int oe = dpp_mov<CTRL>(e);
    const bool win = (ov > v) | ((ov == v) & (oe < e));
    v = win ? ov : v;
    e = win ? oe : e;
}

// All-reduce arg-max over the wave: every lane ends with the winning pair.
// Exchanges inside each row of 16 lanes, then the four row winners (lanes 0,
// 16, 32, 48) are read as uniform values.  The order is a total order on
// (value, index) pairs with distinct indices, so the result is unique.
__device__ __forceinline__ void wave_argmax(float &v, int &e) {
    argmax_step<kDppXor1>(v, e);
    argmax_step<kDppXor2>(v, e);
    argmax_step<kDppHalfMirror>(v, e);
    argmax_step<kDppMirror>(v, e);
    float bv = readlanef(v, 0);
    int be = __builtin_amdgcn_readlane(e, 0);
#pragma unroll
    for (int r = 16; r < 64; r += 16) {
        const float cv = readlanef(v, r);
        const int ce = __builtin_amdgcn_readlane(e, r);
        if (beats(cv, ce, bv, be)) {
            bv = cv;
            be = ce;
        }
    }
    v = bv;
    e = be;
}

// Sum over the wave, the same bits in every lane (fixed pairing order).
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_movf<kDppXor1>(v);
    v += dpp_movf<kDppXor2>(v);
    v += dpp_movf<kDppHalfMirror>(v);
    v += dpp_movf<kDppMirror>(v);
    return (readlanef(v, 0) + readlanef(v, 16)) + (readlanef(v, 32) + readlanef(v, 48));
}

__device__ __forceinline__ int wave_sum_int(int v) {
    v += dpp_mov<kDppXor1>(v);
    v += dpp_mov<kDppXor2>(v);
    v += dpp_mov<kDppHalfMirror>(v);
    v += dpp_mov<kDppMirror>(v);
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// Exclusive prefix sum over the 64 lanes; *total gets the wave total.
__device__ __forceinline__ int wave_exscan(int v, int *total) {
    const int lane = threadIdx.x & 63;
    int s = v;
    s += __builtin_amdgcn_update_dpp(0, s, 0x111, 0xf, 0xf, false);   // row_shr:1
    s += __builtin_amdgcn_update_dpp(0, s, 0x112, 0xf, 0xf, false);   // row_shr:2
    s += __builtin_amdgcn_update_dpp(0, s, 0x114, 0xf, 0xf, false);   // row_shr:4
    s += __builtin_amdgcn_update_dpp(0, s, 0x118, 0xf, 0xf, false);   // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(s, 15), r1 = __builtin_amdgcn_readlane(s, 31);
    const int r2 = __builtin_amdgcn_readlane(s, 47), r3 = __builtin_amdgcn_readlane(s, 63);
    const int row = lane >> 4;
    s += (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
    *total = r0 + r1 + r2 + r3;
    return s - v;
}

// Exclusive scan of one int per thread across a 1024-thread block (16 waves);
// *tot receives the block total.  Every thread of the block must call it.
// lds: at least 40 ints of shared memory.
__device__ __forceinline__ int block_exscan1024(int v, int *lds, int *tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int wt;
    const int ex = wave_exscan(v, &wt);
    if (lane == 0) lds[wave] = wt;
    __syncthreads();
    if (wave == 0) {
        int all;
        const int wex = wave_exscan(lane < 16 ? lds[lane] : 0, &all);
        if (lane < 16) lds[16 + lane] = wex;
        if (lane == 0) lds[32] = all;
    }
    __syncthreads();
    const int r = lds[16 + wave] + ex;
    *tot = lds[32];
    __syncthreads();
    return r;
}

constexpr int kPerLane = kMaxExperts / kWave;

// Order-preserving map of a float to uint32 (larger float -> larger key).
// -0 and +0 get one key (they compare equal, so they tie and the lower
// index goes first); NaN gets key 1, below every number including -inf
// (key 0x007fffff), so a NaN logit is picked last, after -inf.
// key_to_float inverts it (+0 for both zeros, a NaN for key 1).
__device__ __forceinline__ uint32_t float_key(float v) {
    if (v != v) return 1u;
    const uint32_t u = (v == 0.0f) ? 0u : __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// One step of the wave-wide maximum of 64-bit keys: lanes the DPP control
// (with row mask RM) does not write keep their own key.
template <int CTRL, int RM>
__device__ __forceinline__ uint64_t kmax_step(uint64_t key) {
    const uint32_t hi = (uint32_t)(key >> 32), lo = (uint32_t)key;
    const uint32_t oh = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, RM, 0xf, false);
    const uint32_t ol = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, RM, 0xf, false);
    const uint64_t o = ((uint64_t)oh << 32) | ol;
    return o > key ? o : key;
}

// Maximum key over the wave, in every lane: butterflies inside each row of
// 16 lanes, then row 0 -> 1 and 2 -> 3 (row_bcast:15), then rows 0..1 -> 3
// (row_bcast:31); lane 63 ends with the maximum and is read back uniformly.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t key) {
    key = kmax_step<kDppXor1, 0xf>(key);
    key = kmax_step<kDppXor2, 0xf>(key);
    key = kmax_step<kDppHalfMirror, 0xf>(key);
    key = kmax_step<kDppMirror, 0xf>(key);
    key = kmax_step<0x142, 0xa>(key);
    key = kmax_step<0x143, 0xc>(key);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(key >> 32), 63);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)key, 63);
    return ((uint64_t)hi << 32) | lo;
}

// Top-k of one token's E logits by one wave (NPL >= E / 64 values per lane).
// Each logit becomes the 64-bit key (float_key(z), E - 1 - e), so the key
// order is: larger logit first, equal logits (+0 and -0 included) by lower
// expert index, NaN after -inf.  k rounds take the wave maximum and clear it
// (key 0 is below every real key; a NaN's is (1, .) > 0).  Pick j (k <= 32)
// ends in lane j, which returns its expert and softmax weight (renormalised
// over the k picks, or over all E; a picked NaN logit gives a NaN weight).
template <int NPL>
__device__ __forceinline__ void topk_wave(const float *__restrict__ zr, int E, int k, int renorm, int *pick_e,
                                          float *pick_w) {
    const int lane = threadIdx.x & 63;
    float v[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {   // every load before any use (the guard is wave-uniform)
        const int e = lane + 64 * i;
        v[i] = (64 * i < E) ? zr[e < E ? e : 0] : -INFINITY;
    }
    uint64_t key[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < E ? (((uint64_t)float_key(v[i]) << 32) | (uint32_t)(E - 1 - e)) : 0;
        v[i] = (e < E && v[i] == v[i]) ? v[i] : -INFINITY;   // the all-E softmax sum skips NaN
    }
    uint64_t mine = 0;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < NPL; ++i) best = key[i] > best ? key[i] : best;
        const uint64_t win = wave_max_key(best);
#pragma unroll
        for (int i = 0; i < NPL; ++i) key[i] = key[i] == win ? 0 : key[i];
        mine = lane == j ? win : mine;
    }
    const float my_v = key_to_float((uint32_t)(mine >> 32));
    const int my_e = E - 1 - (int)(uint32_t)mine;
    const float m = readlanef(my_v, 0);
    const float p = (lane < k) ? expf(my_v - m) : 0.0f;
    float s;
    if (renorm) {
        s = wave_sum(p);
    } else {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (lane + 64 * i < E) a += expf(v[i] - m);
        s = wave_sum(a);
    }
    *pick_e = lane < k ? my_e : 0;
    *pick_w = p / s;
}

// Values per lane for E experts: ceil(E / 64) rounded up to 1, 2, 4, 8 or 16.
inline int topk_npl(int E) {
    const int n = (E + 63) / 64;
    return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : n <= 8 ? 8 : 16;
}

// Blob address of expert e per the residency table, or 0 when its entry does
// not point inside [0, n_hot) / [0, n_cold).
__device__ __forceinline__ uint64_t expert_address(int s, int n_hot, int n_cold, const uint8_t *hot_base,
                                                   const uint8_t *scratch, size_t blob_bytes, bool *ok,
                                                   bool *cold) {
    *cold = s < 0;
    if (s >= 0) {
        *ok = s < n_hot && hot_base != nullptr;
        return *ok ? (uint64_t)(hot_base + (size_t)s * blob_bytes) : 0;
    }
    const int c = -(s + 1);
    *ok = c < n_cold && scratch != nullptr;
    return *ok ? (uint64_t)(scratch + (size_t)c * blob_bytes) : 0;
}

}  // namespace moe
