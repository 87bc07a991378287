// Grouped SwiGLU expert FFN and weighted combine (a5-a8), decode path.
//
// The gracetier write-up (section 1) runs every picked expert "in a single
// call, as if they had been in HBM all along": here a blob-address table from
// the grouping points each distinct expert at its HBM home or its scratch
// slot, and the kernels never look at residency again, so an all-hot run and a
// mixed hot/cold run execute identical instructions on identical bytes.
//
// At decode an expert sees a handful of tokens and the work is a bandwidth-
// bound grouped GEMV over MXFP4 weights.  It still runs on the matrix cores:
// a wave owns 16 weight rows and streams them with 128-bit loads (per 128-
// element K step a lane loads one 16-byte run of 32 codes, i.e. exactly one
// MX block, plus the dword holding that row's four block scales), turns codes
// into exact bf16 with the gfx950 scaled fp4 converts, and feeds 16x16x32 bf16
// MFMAs whose other operand holds up to 16 tokens.  The K order inside a step
// is permuted identically in both operands (lane group g takes block 4s+g), so
// every MFMA is an exact partial dot product.  Compared with a VALU dot, the
// converts are the only per-element vector work (a fifth of the issue slots
// at the HBM rate), and 1 to 16 tokens per expert cost the same.
//
//   gate/up: A = gate and up rows (two accumulators share the token operand);
//            epilogue h = silu(g) * u, stored as bf16 hi + lo parts (h - hi
//            rounded again), which carry ~16 significant bits into the down
//            projection's bf16 MFMAs.
//   down:    A = w2 rows, B = h hi and h lo (two MFMAs per K slice), output
//            y[pair][row] in fp32.
//   combine: out[t] = sum_j w[t,j] * y[t*k+j] in j order, no atomics.
#include "kernels.hpp"

namespace moe {

namespace {

GroupView group_view(const char *ws, const WsLayout &L) {
    GroupView v;
    v.nuniq = reinterpret_cast<const int32_t *>(ws + L.nuniq);
    v.uniq = reinterpret_cast<const int32_t *>(ws + L.uniq);
    v.ucnt = reinterpret_cast<const int32_t *>(ws + L.ucnt);
    v.uoff = reinterpret_cast<const int32_t *>(ws + L.uoff);
    v.uptr = reinterpret_cast<const uint64_t *>(ws + L.uptr);
    v.plist = reinterpret_cast<const int32_t *>(ws + L.plist);
    v.cold = reinterpret_cast<const int32_t *>(ws + L.cold);
    return v;
}

}  // namespace

// ------------------------------- gate / up ---------------------------------
template <int D>
struct GateUpStage {
    uint4 gq[D], uq[D];      // 32 codes of a gate row / an up row per step
    uint32_t gs[D], us[D];   // the four block scales of that step
    uint4 xb[D][4];          // token operand: 4 x 8 bf16 per step
};

template <int D>
__device__ __forceinline__ void gate_up_load(GateUpStage<D> &st, const uint8_t *gq, const uint8_t *uq,
                                             const uint32_t *gs, const uint32_t *us, const uint16_t *xr,
                                             bool tv, int s0) {
    const uint4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const int s = s0 + d;
        st.gq[d] = *reinterpret_cast<const uint4 *>(gq + (size_t)s * 64);
        st.uq[d] = *reinterpret_cast<const uint4 *>(uq + (size_t)s * 64);
        st.gs[d] = gs[s];
        st.us[d] = us[s];
#pragma unroll
        for (int m = 0; m < 4; ++m)
            st.xb[d][m] = tv ? *reinterpret_cast<const uint4 *>(xr + (size_t)s * 128 + 8 * m) : z4;
    }
}

template <int D>
__device__ __forceinline__ void gate_up_compute(const GateUpStage<D> &st, int g, f32x4 &ag, f32x4 &au) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const float sg = e8m0_to_f32((st.gs[d] >> (8 * g)) & 0xffu);
        const float su = e8m0_to_f32((st.us[d] >> (8 * g)) & 0xffu);
        const uint32_t gw[4] = {st.gq[d].x, st.gq[d].y, st.gq[d].z, st.gq[d].w};
        const uint32_t uw[4] = {st.uq[d].x, st.uq[d].y, st.uq[d].z, st.uq[d].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const bf16x8 b = as_bf16x8(st.xb[d][m]);
            ag = mfma16x16x32(fp4x8_to_bf16x8(gw[m], sg), b, ag);
            au = mfma16x16x32(fp4x8_to_bf16x8(uw[m], su), b, au);
        }
    }
}

// grid (I/16, max distinct experts), one wave per block.
template <int D>
__global__ __launch_bounds__(64) void ffn_gate_up(const uint16_t *__restrict__ x, int H, int I, int k,
                                                  GroupView gv, uint16_t *__restrict__ hhi,
                                                  uint16_t *__restrict__ hlo) {
    const int u = blockIdx.y;
    if (u >= gv.nuniq[0]) return;
    const uint8_t *base = reinterpret_cast<const uint8_t *>(gv.uptr[u]);
    if (base == nullptr) return;
    const int n = gv.ucnt[u], q0 = gv.uoff[u];
    const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
    const int row = blockIdx.x * 16 + r;
    const BlobLayout L = BlobLayout::make(H, I);
    const size_t rb = (size_t)H / 2, sb = (size_t)H / 32;
    const uint8_t *gq = base + L.w13_codes + (size_t)row * rb + 16 * g;
    const uint8_t *uq = gq + (size_t)I * rb;
    const uint32_t *gs = reinterpret_cast<const uint32_t *>(base + L.w13_scales + (size_t)row * sb);
    const uint32_t *us = reinterpret_cast<const uint32_t *>(base + L.w13_scales + (size_t)(I + row) * sb);
    const int nsteps = H / 128;
    for (int tb = 0; tb < n; tb += 16) {
        const bool tv = tb + r < n;   // this lane's token column is r
        const int p = tv ? gv.plist[q0 + tb + r] : 0;
        const uint16_t *xr = x + (size_t)(p / k) * H + 32 * g;
        f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
        GateUpStage<D> sa, sbuf;
        gate_up_load<D>(sa, gq, uq, gs, us, xr, tv, 0);
        for (int s0 = 0; s0 < nsteps; s0 += 2 * D) {
            if (s0 + D < nsteps) gate_up_load<D>(sbuf, gq, uq, gs, us, xr, tv, s0 + D);
            gate_up_compute<D>(sa, g, ag, au);
            if (s0 + D >= nsteps) break;
            if (s0 + 2 * D < nsteps) gate_up_load<D>(sa, gq, uq, gs, us, xr, tv, s0 + 2 * D);
            gate_up_compute<D>(sbuf, g, ag, au);
        }
        // lane (r, g) holds rows 4g..4g+3 of the tile for token column r
        if (tv) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float h = silu(ag[i]) * au[i];
                hi[i] = f32_to_bf16_bits(h);
                lo[i] = f32_to_bf16_bits(h - __uint_as_float(hi[i] << 16));
            }
            const size_t off = (size_t)(q0 + tb + r) * I + (size_t)blockIdx.x * 16 + 4 * g;
            *reinterpret_cast<uint2 *>(hhi + off) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
            *reinterpret_cast<uint2 *>(hlo + off) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
        }
    }
}

// --------------------------------- down ------------------------------------
template <int D>
struct DownStage {
    uint4 wq[D];
    uint32_t ws[D];
    uint4 hh[D][4], hl[D][4];
};

template <int D>
__device__ __forceinline__ void down_load(DownStage<D> &st, const uint8_t *wq, const uint32_t *ws,
                                          const uint16_t *hh, const uint16_t *hl, bool tv, int s0) {
    const uint4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const int s = s0 + d;
        st.wq[d] = *reinterpret_cast<const uint4 *>(wq + (size_t)s * 64);
        st.ws[d] = ws[s];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            st.hh[d][m] = tv ? *reinterpret_cast<const uint4 *>(hh + (size_t)s * 128 + 8 * m) : z4;
            st.hl[d][m] = tv ? *reinterpret_cast<const uint4 *>(hl + (size_t)s * 128 + 8 * m) : z4;
        }
    }
}

template <int D>
__device__ __forceinline__ void down_compute(const DownStage<D> &st, int g, f32x4 &acc) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const float sc = e8m0_to_f32((st.ws[d] >> (8 * g)) & 0xffu);
        const uint32_t w4[4] = {st.wq[d].x, st.wq[d].y, st.wq[d].z, st.wq[d].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const bf16x8 a = fp4x8_to_bf16x8(w4[m], sc);
            acc = mfma16x16x32(a, as_bf16x8(st.hh[d][m]), acc);
            acc = mfma16x16x32(a, as_bf16x8(st.hl[d][m]), acc);
        }
    }
}

// grid (H/16, max distinct experts), one wave per block.
template <int D>
__global__ __launch_bounds__(64) void ffn_down(int H, int I, GroupView gv, const uint16_t *__restrict__ hhi,
                                               const uint16_t *__restrict__ hlo, float *__restrict__ y) {
    const int u = blockIdx.y;
    if (u >= gv.nuniq[0]) return;
    const uint8_t *base = reinterpret_cast<const uint8_t *>(gv.uptr[u]);
    const int n = gv.ucnt[u], q0 = gv.uoff[u];
    const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
    const int row0 = blockIdx.x * 16;
    if (base == nullptr) {   // unusable residency entry: its pairs contribute zero
        for (int tb = 0; tb < n; tb += 16)
            if (tb + r < n) {
                const int p = gv.plist[q0 + tb + r];
                *reinterpret_cast<float4 *>(y + (size_t)p * H + row0 + 4 * g) = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        return;
    }
    const BlobLayout L = BlobLayout::make(H, I);
    const int row = row0 + r;
    const uint8_t *wq = base + L.w2_codes + (size_t)row * (I / 2) + 16 * g;
    const uint32_t *ws = reinterpret_cast<const uint32_t *>(base + L.w2_scales + (size_t)row * (I / 32));
    const int nsteps = I / 128;
    for (int tb = 0; tb < n; tb += 16) {
        const bool tv = tb + r < n;
        const size_t hoff = (size_t)(q0 + tb + (tv ? r : 0)) * I + 32 * g;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        DownStage<D> sa, sbuf;
        down_load<D>(sa, wq, ws, hhi + hoff, hlo + hoff, tv, 0);
        for (int s0 = 0; s0 < nsteps; s0 += 2 * D) {
            if (s0 + D < nsteps) down_load<D>(sbuf, wq, ws, hhi + hoff, hlo + hoff, tv, s0 + D);
            down_compute<D>(sa, g, acc);
            if (s0 + D >= nsteps) break;
            if (s0 + 2 * D < nsteps) down_load<D>(sa, wq, ws, hhi + hoff, hlo + hoff, tv, s0 + 2 * D);
            down_compute<D>(sbuf, g, acc);
        }
        if (tv) {
            const int p = gv.plist[q0 + tb + r];
            *reinterpret_cast<float4 *>(y + (size_t)p * H + row0 + 4 * g) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    }
}

// -------------------------------- combine ----------------------------------
__global__ __launch_bounds__(256) void ffn_combine(const float *__restrict__ y, const int32_t *__restrict__ ids,
                                                   const float *__restrict__ w, int T, int H, int E, int k,
                                                   int out_bf16, void *__restrict__ out) {
    const int c4 = blockIdx.x * blockDim.x + threadIdx.x;
    if (c4 * 4 >= H) return;
    for (int t = blockIdx.y; t < T; t += gridDim.y) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < k; ++j) {
            const int id = ids[(size_t)t * k + j];
            if (id < 0 || id >= E) continue;
            const float wj = w[(size_t)t * k + j];
            const float4 v = reinterpret_cast<const float4 *>(y + ((size_t)t * k + j) * H)[c4];
            acc.x += wj * v.x;
            acc.y += wj * v.y;
            acc.z += wj * v.z;
            acc.w += wj * v.w;
        }
        if (out_bf16) {
            const uint32_t b0 = f32_to_bf16_bits(acc.x), b1 = f32_to_bf16_bits(acc.y);
            const uint32_t b2 = f32_to_bf16_bits(acc.z), b3 = f32_to_bf16_bits(acc.w);
            reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + (size_t)t * H)[c4] =
                make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
        } else {
            reinterpret_cast<float4 *>(static_cast<float *>(out) + (size_t)t * H)[c4] = acc;
        }
    }
}

hipError_t launch_ffn(const FfnArgs &a, char *ws, const WsLayout &L, hipStream_t st) {
    const GroupView gv = group_view(ws, L);
    const size_t P = (size_t)a.T * a.k;
    const int umax = (int)((size_t)a.E < P ? (size_t)a.E : P);
    uint16_t *hhi = reinterpret_cast<uint16_t *>(ws + L.hbuf);
    uint16_t *hlo = hhi + P * (size_t)a.I;
    float *y = reinterpret_cast<float *>(ws + L.ybuf);

    const int sgu = a.H / 128;
    const dim3 ggu(a.I / 16, umax);
    if (sgu % 4 == 0)
        hipLaunchKernelGGL(ffn_gate_up<4>, ggu, dim3(64), 0, st, a.x, a.H, a.I, a.k, gv, hhi, hlo);
    else if (sgu % 2 == 0)
        hipLaunchKernelGGL(ffn_gate_up<2>, ggu, dim3(64), 0, st, a.x, a.H, a.I, a.k, gv, hhi, hlo);
    else
        hipLaunchKernelGGL(ffn_gate_up<1>, ggu, dim3(64), 0, st, a.x, a.H, a.I, a.k, gv, hhi, hlo);

    const int sd = a.I / 128;
    const dim3 gd(a.H / 16, umax);
    if (sd % 2 == 0)
        hipLaunchKernelGGL(ffn_down<2>, gd, dim3(64), 0, st, a.H, a.I, gv, hhi, hlo, y);
    else
        hipLaunchKernelGGL(ffn_down<1>, gd, dim3(64), 0, st, a.H, a.I, gv, hhi, hlo, y);

    const int n4 = a.H / 4;
    const int ty = a.T < 65535 ? a.T : 65535;
    hipLaunchKernelGGL(ffn_combine, dim3((n4 + 255) / 256, ty), dim3(256), 0, st, y, a.ids, a.w, a.T, a.H,
                       a.E, a.k, a.out_bf16, a.out);
    return hipGetLastError();
}

}  // namespace moe
