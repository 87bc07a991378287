// Router: logits (a1) and top-k softmax selection (a2).
//
// The pages: a tiny router picks the 6 most relevant of 384 experts per token
// (GB300 inference write-up, mixture-of-experts paragraph).  Scores are a
// softmax over z[t,e] = x_t . Wr_e + b_e; the k largest logits are kept, equal
// logits going to the lower expert index, and the kept weights renormalised.
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Decode-size logits (T <= 32): one wave per expert row.  The row (16 KB at
// H = 4096) is streamed once per group of 8 tokens with 128-bit loads; the
// tokens come from L2.  HBM-bound on the router matrix (E*H*4 bytes).
// ---------------------------------------------------------------------------
constexpr int kGemvTok = 8;

__global__ __launch_bounds__(256) void route_logits_gemv(
    const uint16_t *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    int T, int H, int E, float *__restrict__ z) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    const float4 *wrow = reinterpret_cast<const float4 *>(wr + (size_t)e * H);
    const float b = bias ? bias[e] : 0.0f;
    const int nq = H / 4;
    for (int t0 = 0; t0 < T; t0 += kGemvTok) {
        float acc[kGemvTok];
#pragma unroll
        for (int i = 0; i < kGemvTok; ++i) acc[i] = 0.0f;
        for (int c = lane; c < nq; c += 64) {
            const float4 w4 = wrow[c];
#pragma unroll
            for (int i = 0; i < kGemvTok; ++i) {
                if (t0 + i < T) {
                    const uint2 xv = *reinterpret_cast<const uint2 *>(x + (size_t)(t0 + i) * H + 4 * c);
                    float a = acc[i];
                    a = fmaf(w4.x, bf16_bits_to_f32(xv.x & 0xffffu), a);
                    a = fmaf(w4.y, bf16_bits_to_f32(xv.x >> 16), a);
                    a = fmaf(w4.z, bf16_bits_to_f32(xv.y & 0xffffu), a);
                    a = fmaf(w4.w, bf16_bits_to_f32(xv.y >> 16), a);
                    acc[i] = a;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kGemvTok; ++i) {
            float v = acc[i];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
            if (lane == 0 && t0 + i < T) z[(size_t)(t0 + i) * E + e] = v + b;
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill-size logits (T > 32): MFMA GEMM on 16x16x32 bf16 tiles.  x is bf16
// already; each fp32 router weight is split exactly-enough into three bf16
// terms (hi + mid + lo carry 24 significant bits), so the three products per
// term are exact in fp32 and only the fp32 accumulation rounds.  A wave owns a
// 32-token x 32-expert tile; a 256-thread block 64 x 64.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split3(const float *v, bf16x8 &hi, bf16x8 &mid, bf16x8 &lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float a = v[i];
        const uint32_t h = f32_to_bf16_bits(a);
        const float r1 = a - __uint_as_float(h << 16);
        const uint32_t m = f32_to_bf16_bits(r1);
        const float r2 = r1 - __uint_as_float(m << 16);
        const uint32_t l = f32_to_bf16_bits(r2);
        hi[i] = __builtin_bit_cast(__bf16, (uint16_t)h);
        mid[i] = __builtin_bit_cast(__bf16, (uint16_t)m);
        lo[i] = __builtin_bit_cast(__bf16, (uint16_t)l);
    }
}

__global__ __launch_bounds__(256) void route_logits_mfma(
    const uint16_t *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    int T, int H, int E, float *__restrict__ z) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int tok0 = blockIdx.y * 64 + (wave >> 1) * 32;
    const int ex0 = blockIdx.x * 64 + (wave & 1) * 32;
    const bool tv[2] = {tok0 + r < T, tok0 + 16 + r < T};
    const bool ev[2] = {ex0 + r < E, ex0 + 16 + r < E};
    const uint16_t *xr[2] = {x + (size_t)(tv[0] ? tok0 + r : 0) * H,
                             x + (size_t)(tv[1] ? tok0 + 16 + r : 0) * H};
    const float *wrr[2] = {wr + (size_t)(ev[0] ? ex0 + r : 0) * H,
                           wr + (size_t)(ev[1] ? ex0 + 16 + r : 0) * H};
    f32x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint4 zero4 = {0u, 0u, 0u, 0u};
    for (int k0 = 0; k0 < H; k0 += 32) {
        const int kk = k0 + 8 * g;
        bf16x8 A[2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
            A[a] = as_bf16x8(tv[a] ? *reinterpret_cast<const uint4 *>(xr[a] + kk) : zero4);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            float wv[8];
            if (ev[b]) {
                const float4 w0 = *reinterpret_cast<const float4 *>(wrr[b] + kk);
                const float4 w1 = *reinterpret_cast<const float4 *>(wrr[b] + kk + 4);
                wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w;
                wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) wv[i] = 0.f;
            }
            bf16x8 hi, mid, lo;
            split3(wv, hi, mid, lo);
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                acc[a][b] = mfma16x16x32(A[a], hi, acc[a][b]);
                acc[a][b] = mfma16x16x32(A[a], mid, acc[a][b]);
                acc[a][b] = mfma16x16x32(A[a], lo, acc[a][b]);
            }
        }
    }
    // D[row = token 4*g + i][col = expert r] in lane (r, g), element i
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int e = ex0 + 16 * b + r;
        if (e >= E) continue;
        const float bb = bias ? bias[e] : 0.0f;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = tok0 + 16 * a + 4 * g + i;
                if (t < T) z[(size_t)t * E + e] = acc[a][b][i] + bb;
            }
    }
}

hipError_t launch_route_logits(const uint16_t *x, const float *wr, const float *bias,
                               int T, int H, int E, float *z, hipStream_t st) {
    if (T <= 32) {
        hipLaunchKernelGGL(route_logits_gemv, dim3((E + 3) / 4), dim3(256), 0, st,
                           x, wr, bias, T, H, E, z);
    } else {
        hipLaunchKernelGGL(route_logits_mfma, dim3((E + 63) / 64, (T + 63) / 64), dim3(256), 0, st,
                           x, wr, bias, T, H, E, z);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token.  Lane l holds logits l, l+64, ...; k rounds of a
// wave arg-max whose order is (larger value, then lower index), so the result
// is the k largest logits with ties to the lower expert index.  NaN logits
// order as -inf.  Pick j ends in lane j, which computes its weight.
// ---------------------------------------------------------------------------
constexpr int kPerLane = kMaxExperts / kWave;

__global__ __launch_bounds__(256) void route_topk(const float *__restrict__ z, int T, int E, int k,
                                                  int renorm, int32_t *__restrict__ ids,
                                                  float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float *zr = z + (size_t)t * E;
    float v[kPerLane];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int e = lane + 64 * i;
        float a = -INFINITY;
        if (e < E) {
            a = zr[e];
            if (a != a) a = -INFINITY;
        } else {
            taken |= 1u << i;
        }
        v[i] = a;
    }
    float my_v = -INFINITY;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int e = lane + 64 * i;
            const bool better = (v[i] > bv) || (v[i] == bv && e < be);
            if (!((taken >> i) & 1u) && better) {
                bv = v[i];
                be = e;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oe = __shfl_xor(be, off);
            if (ov > bv || (ov == bv && oe < be)) {
                bv = ov;
                be = oe;
            }
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == j) {
            my_v = bv;
            my_e = be;
        }
    }
    const float m = __shfl(my_v, 0);
    float p = (lane < k) ? expf(my_v - m) : 0.0f;
    float s;
    if (renorm) {
        s = p;
    } else {
        s = 0.0f;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i)
            if (lane + 64 * i < E) s += expf(v[i] - m);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_e;
        w[(size_t)t * k + lane] = p / s;
    }
}

hipError_t launch_topk(const float *z, int T, int E, int k, int renorm, int32_t *ids, float *w,
                       hipStream_t st) {
    hipLaunchKernelGGL(route_topk, dim3((T + 3) / 4), dim3(256), 0, st, z, T, E, k, renorm, ids, w);
    return hipGetLastError();
}

}  // namespace moe
