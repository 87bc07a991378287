// Router: logits and top-k softmax selection, plus the fused select-and-group
// kernel of the decode path.
//
// The pages: a tiny router picks the 6 most relevant of 384 experts per token
// (GB300 inference write-up, mixture-of-experts paragraph).  Scores are a
// softmax over z[t,e] = x_t . Wr_e + b_e; the k largest logits are kept, equal
// logits going to the lower expert index, and the kept weights renormalised.
#include "kernels.hpp"
#include "select.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits for few tokens (T <= 32).  One block per expert row; its
// four waves take a quarter of the row each (lane l: the float4 chunks
// l + 64 i of its quarter), issue every weight and token load before using
// any, and accumulate fp32 products per token.  Per token, a wave sum and
// then the four wave partials added in wave order give the logit, so the
// result is reproducible.  Tokens go in passes of kRtTok.  NC >= H / 1024
// chunks per lane.
constexpr int kRtTok = 8;

template <int NC>
__global__ __launch_bounds__(256) void route_logits_small(const uint16_t *__restrict__ x, const float *__restrict__ wr,
                                                          const float *__restrict__ bias, int T, int H, int E,
                                                          float *__restrict__ z) {
    __shared__ float part[4][kRtTok];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = blockIdx.x;
    const int nch = H / 4;   // float4 chunks of the row
    const float4 *wrow = reinterpret_cast<const float4 *>(wr + (size_t)e * H);
    float4 w4[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = wave * 64 + lane + 256 * i;
        w4[i] = c < nch ? wrow[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float b = bias ? bias[e] : 0.0f;
    for (int t0 = 0; t0 < T; t0 += kRtTok) {
        const int nt = (T - t0) < kRtTok ? (T - t0) : kRtTok;
        uint2 xv[kRtTok][NC];
#pragma unroll
        for (int tt = 0; tt < kRtTok; ++tt)
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const int c = wave * 64 + lane + 256 * i;
                xv[tt][i] = (tt < nt && c < nch)
                                ? *reinterpret_cast<const uint2 *>(x + (size_t)(t0 + tt) * H + 4 * c)
                                : make_uint2(0u, 0u);
            }
#pragma unroll
        for (int tt = 0; tt < kRtTok; ++tt) {
            float a = 0.0f;
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                a = fmaf(w4[i].x, bf16_bits_to_f32(xv[tt][i].x & 0xffffu), a);
                a = fmaf(w4[i].y, bf16_bits_to_f32(xv[tt][i].x >> 16), a);
                a = fmaf(w4[i].z, bf16_bits_to_f32(xv[tt][i].y & 0xffffu), a);
                a = fmaf(w4[i].w, bf16_bits_to_f32(xv[tt][i].y >> 16), a);
            }
            if (tt < nt) {
                const float v = wave_sum(a);
                if (lane == 0) part[wave][tt] = v;
            }
        }
        __syncthreads();
        if (threadIdx.x < nt)
            z[(size_t)(t0 + threadIdx.x) * E + e] =
                ((part[0][threadIdx.x] + part[1][threadIdx.x]) + (part[2][threadIdx.x] + part[3][threadIdx.x])) + b;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Prefill-size logits (T > 32): MFMA GEMM on 16x16x32 bf16 tiles.  x is bf16
// already; each fp32 router weight is split into three bf16 terms (hi + mid +
// lo carry 24 significant bits), so the three products per term are exact in
// fp32 and only the fp32 accumulation rounds.  A wave owns a 32-token x
// 32-expert tile; a 256-thread block 64 x 64.
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

// One K step (32 elements) of a wave's operands: the token rows for its two
// 16-token halves and the router rows for its two 16-expert halves.
struct RtStep {
    uint4 xa[2];
    float4 w[2][2];
};

__device__ __forceinline__ void rt_load(RtStep &s, const uint16_t *const xr[2], const float *const wrr[2], int kk) {
#pragma unroll
    for (int a = 0; a < 2; ++a) s.xa[a] = *reinterpret_cast<const uint4 *>(xr[a] + kk);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        s.w[b][0] = *reinterpret_cast<const float4 *>(wrr[b] + kk);
        s.w[b][1] = *reinterpret_cast<const float4 *>(wrr[b] + kk + 4);
    }
}

__device__ __forceinline__ void rt_compute(const RtStep &s, const bool tv[2], const bool ev[2], f32x4 acc[2][2]) {
    const uint4 zero4 = {0u, 0u, 0u, 0u};
    bf16x8 A[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) A[a] = as_bf16x8(tv[a] ? s.xa[a] : zero4);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const float wv[8] = {s.w[b][0].x, s.w[b][0].y, s.w[b][0].z, s.w[b][0].w,
                             s.w[b][1].x, s.w[b][1].y, s.w[b][1].z, s.w[b][1].w};
        float wz[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) wz[i] = ev[b] ? wv[i] : 0.f;
        bf16x8 hi, mid, lo;
        split3(wz, hi, mid, lo);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            acc[a][b] = mfma16x16x32(A[a], hi, acc[a][b]);
            acc[a][b] = mfma16x16x32(A[a], mid, acc[a][b]);
            acc[a][b] = mfma16x16x32(A[a], lo, acc[a][b]);
        }
    }
}

// The loads run four K steps ahead of the MFMAs (a register ring of four
// steps, issued unconditionally with the last step repeated at the end), so
// each wave keeps several round trips in flight instead of one.  (The kernel
// is still bound by L2 / Infinity Cache traffic: a 64 x 64 block tile reads
// each router row once per 64 tokens.)
__global__ __launch_bounds__(256) void route_logits_mfma(
    const uint16_t *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    int T, int H, int E, float *__restrict__ z) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int tok0 = blockIdx.y * 64 + (wave >> 1) * 32;
    const int ex0 = blockIdx.x * 64 + (wave & 1) * 32;
    const bool tv[2] = {tok0 + r < T, tok0 + 16 + r < T};
    const bool ev[2] = {ex0 + r < E, ex0 + 16 + r < E};
    const uint16_t *const xr[2] = {x + (size_t)(tv[0] ? tok0 + r : 0) * H + 8 * g,
                                   x + (size_t)(tv[1] ? tok0 + 16 + r : 0) * H + 8 * g};
    const float *const wrr[2] = {wr + (size_t)(ev[0] ? ex0 + r : 0) * H + 8 * g,
                                 wr + (size_t)(ev[1] ? ex0 + 16 + r : 0) * H + 8 * g};
    f32x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int last = H - 32;   // H is a multiple of 128
    RtStep s0, s1, s2, s3;
    rt_load(s0, xr, wrr, 0);
    rt_load(s1, xr, wrr, 32);
    rt_load(s2, xr, wrr, 64);
    rt_load(s3, xr, wrr, 96);
    for (int k0 = 0; k0 < H; k0 += 128) {
        const int nk = k0 + 128;
        rt_compute(s0, tv, ev, acc);
        rt_load(s0, xr, wrr, nk < H ? nk : last);
        rt_compute(s1, tv, ev, acc);
        rt_load(s1, xr, wrr, nk + 32 < H ? nk + 32 : last);
        rt_compute(s2, tv, ev, acc);
        rt_load(s2, xr, wrr, nk + 64 < H ? nk + 64 : last);
        rt_compute(s3, tv, ev, acc);
        rt_load(s3, xr, wrr, nk + 96 < H ? nk + 96 : last);
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
        const int nc = (H + 1023) / 1024;   // float4 chunks per lane
        const dim3 g(E), b(256);
        if (nc <= 1)
            MOE_LAUNCH("route_logits_small", route_logits_small<1>, g, b, 0, st, x, wr, bias, T, H, E, z);
        else if (nc <= 2)
            MOE_LAUNCH("route_logits_small", route_logits_small<2>, g, b, 0, st, x, wr, bias, T, H, E, z);
        else if (nc <= 4)
            MOE_LAUNCH("route_logits_small", route_logits_small<4>, g, b, 0, st, x, wr, bias, T, H, E, z);
        else if (nc <= 8)
            MOE_LAUNCH("route_logits_small", route_logits_small<8>, g, b, 0, st, x, wr, bias, T, H, E, z);
        else if (nc <= 16)
            MOE_LAUNCH("route_logits_small", route_logits_small<16>, g, b, 0, st, x, wr, bias, T, H, E, z);
        else
            MOE_LAUNCH("route_logits_mfma", route_logits_mfma, dim3((E + 63) / 64, (T + 63) / 64), dim3(256), 0,
                       st, x, wr, bias, T, H, E, z);
    } else {
        MOE_LAUNCH("route_logits_mfma", route_logits_mfma, dim3((E + 63) / 64, (T + 63) / 64), dim3(256), 0, st,
                   x, wr, bias, T, H, E, z);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k for any T: one wave per token.
// ---------------------------------------------------------------------------
template <int NPL>
__global__ __launch_bounds__(256) void route_topk(const float *__restrict__ z, int T, int E, int k,
                                                  int renorm, int32_t *__restrict__ ids,
                                                  float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int pe;
    float pw;
    topk_wave<NPL>(z + (size_t)t * E, E, k, renorm, &pe, &pw);
    if (lane < k) {
        ids[(size_t)t * k + lane] = pe;
        w[(size_t)t * k + lane] = pw;
    }
}

hipError_t launch_topk(const float *z, int T, int E, int k, int renorm, int32_t *ids, float *w,
                       hipStream_t st) {
    const dim3 g((T + 3) / 4), b(256);
    switch (topk_npl(E)) {
        case 1: MOE_LAUNCH("route_topk", route_topk<1>, g, b, 0, st, z, T, E, k, renorm, ids, w); break;
        case 2: MOE_LAUNCH("route_topk", route_topk<2>, g, b, 0, st, z, T, E, k, renorm, ids, w); break;
        case 4: MOE_LAUNCH("route_topk", route_topk<4>, g, b, 0, st, z, T, E, k, renorm, ids, w); break;
        case 8: MOE_LAUNCH("route_topk", route_topk<8>, g, b, 0, st, z, T, E, k, renorm, ids, w); break;
        default: MOE_LAUNCH("route_topk", route_topk<16>, g, b, 0, st, z, T, E, k, renorm, ids, w); break;
    }
    return hipGetLastError();
}

// Decode path (T * k <= 1024 pairs): top-k of every token and the whole pick
// set in one single-block launch (the selection itself is shared with the
// decode gate/up kernel, which recomputes it per block when no expert is cold).
template <int NPL>
__global__ __launch_bounds__(1024) void select_group_small(SelectArgs a, GroupOut o) {
    __shared__ int sid[1024], sflag[1024], spl[64], sinfo[4], sslot[kMaxExperts];
    select_group_block<NPL>(a, o, true, -1, SelectLds{sid, sflag, spl, sinfo, sslot});
}

SelectArgs select_args(const float *z, int T, int k, int renorm, int32_t *ids, float *w, const GroupArgs &a) {
    SelectArgs s;
    s.z = z;
    s.T = T;
    s.E = a.E;
    s.k = k;
    s.renorm = renorm;
    s.ids = ids;
    s.w = w;
    s.slot = a.slot;
    s.n_hot = a.n_hot;
    s.n_cold = a.n_cold;
    s.hot_base = a.hot_base;
    s.scratch = a.scratch;
    s.blob_bytes = a.blob_bytes;
    return s;
}

hipError_t launch_select_group_small(const float *z, int T, int k, int renorm, int32_t *ids, float *w,
                                     const GroupArgs &a, char *ws, const WsLayout &L, hipStream_t st) {
    const GroupOut o = GroupOut::at(ws, L);
    const SelectArgs sa = select_args(z, T, k, renorm, ids, w, a);
    switch (topk_npl(a.E)) {
        case 1: MOE_LAUNCH("select_group_small", select_group_small<1>, dim3(1), dim3(1024), 0, st, sa, o); break;
        case 2: MOE_LAUNCH("select_group_small", select_group_small<2>, dim3(1), dim3(1024), 0, st, sa, o); break;
        case 4: MOE_LAUNCH("select_group_small", select_group_small<4>, dim3(1), dim3(1024), 0, st, sa, o); break;
        case 8: MOE_LAUNCH("select_group_small", select_group_small<8>, dim3(1), dim3(1024), 0, st, sa, o); break;
        default: MOE_LAUNCH("select_group_small", select_group_small<16>, dim3(1), dim3(1024), 0, st, sa, o); break;
    }
    return hipGetLastError();
}

}  // namespace moe
