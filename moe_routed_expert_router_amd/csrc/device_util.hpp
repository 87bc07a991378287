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

// Top-k of one token's E logits by one wave: k rounds of a wave arg-max whose
// order is (larger value, then lower index), so the picks are the k largest
// logits with ties to the lower expert index, in decreasing order; NaN orders
// as -inf.  Pick j ends in lane j (k <= 32), which returns its expert and
// softmax weight (renormalised over the k picks, or over all E).
__device__ __forceinline__ void topk_wave(const float *__restrict__ zr, int E, int k, int renorm,
                                          int *pick_e, float *pick_w) {
    const int lane = threadIdx.x & 63;
    float v[kPerLane];
    uint32_t taken = 0;
    // issue every load before looking at any value (the guard is wave-uniform)
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int e = lane + 64 * i;
        v[i] = (64 * i < E) ? zr[e < E ? e : 0] : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int e = lane + 64 * i;
        const float a = v[i];
        v[i] = (e < E && a == a) ? a : -INFINITY;
        taken |= (e < E ? 0u : 1u) << i;
    }
    float my_v = -INFINITY;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {   // branch-free local arg-max
            const int e = lane + 64 * i;
            const bool free_ = ((taken >> i) & 1u) == 0u;
            const bool win = free_ & ((v[i] > bv) | ((v[i] == bv) & (e < be)));
            bv = win ? v[i] : bv;
            be = win ? e : be;
        }
        wave_argmax(bv, be);
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == j) {
            my_v = bv;
            my_e = be;
        }
    }
    const float m = readlanef(my_v, 0);
    const float p = (lane < k) ? expf(my_v - m) : 0.0f;
    float s;
    if (renorm) {
        s = wave_sum(p);
    } else {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i)
            if (lane + 64 * i < E) a += expf(v[i] - m);
        s = wave_sum(a);
    }
    *pick_e = my_e;
    *pick_w = p / s;
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
