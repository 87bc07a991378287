// Router: logits and top-k softmax selection, plus the fused select-and-group
// kernel of the decode path.
//
// The pages: per token a small router chooses 6 of the 384 experts (the
// inference-engineering write-up, mixture-of-experts paragraph).  Scores are a
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
// An fp32 value as three bf16 terms hi + mid + lo (24 significant bits, so
// hi + mid + lo == v for normal v): a product with a bf16 value is then three
// products that are exact in fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split3(const float *v, bf16x8 &hi, bf16x8 &mid, bf16x8 &lo) {
    // native round-to-nearest-even conversions (one instruction per two
    // values); each remainder is exact in fp32, whatever the rounding
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const __bf16 h = (__bf16)v[i];
        const float r1 = v[i] - (float)h;
        const __bf16 m = (__bf16)r1;
        const float r2 = r1 - (float)m;
        hi[i] = h;
        mid[i] = m;
        lo[i] = (__bf16)r2;
    }
}

// ---------------------------------------------------------------------------
// Prefill-size logits as an LDS-tiled GEMM on 32x32x16 bf16 MFMAs (on gfx950
// the 32x32 form issues twice the flops per cycle of the 16x16 one).  Same
// exact-product scheme: x is bf16, each fp32 router weight is split into
// three bf16 terms and only the fp32 accumulation rounds.  A block computes
// BT tokens (128, or 64 for at most kRgSmallT tokens, giving more blocks) x
// 64 experts.  Per K step of 32 it copies the token rows and the fp32 router
// rows straight into LDS (a ring of four stages, three steps ahead: one
// step's compute is far shorter than an L2 round trip), then each wave runs a
// 32-expert x BT/2-token tile from LDS, splitting its router values into the
// three bf16 terms in registers as it reads them (native bf16 converts).
// Every block of a token tile sits on the same XCD (consecutive blocks go to
// consecutive XCDs), so the tile's token rows come into that XCD's L2 once
// for all the expert tiles.  (A wave that reads its operands from global
// memory and splits the router rows itself re-reads every router row once
// per 64 tokens and repeats each split 256 times: L2 / Infinity Cache
// traffic and VALU work that this layout removes.)
constexpr int kRgE = 64, kRgK = 32;               // experts per block, K step
constexpr int kRgW = kRgE * kRgK * 4;             // fp32 router rows per stage: 128 B each
constexpr int kRgSmallT = 4096;                   // up to this many tokens, 64-token blocks (more of them)

// LDS rows of 64 bytes (token rows) hold their four 16-byte chunks swizzled:
// chunk k of row c sits in slot k ^ (c & 3).
__device__ __forceinline__ int rg_slot(int c, int k) { return c * 64 + 16 * (k ^ (c & 3)); }
// Router rows of 128 bytes: chunk k of row e sits in slot k ^ ((e >> 1) & 7),
// so 16 lanes reading one chunk of 16 consecutive rows hit 16 distinct bank
// groups (row e's slots start at bank 32 (e & 1)).
__device__ __forceinline__ int rg_wslot(int e, int k) { return e * 128 + 16 * (k ^ ((e >> 1) & 7)); }

// grid 8 * expert tiles * ceil(token tiles / 8); 256 threads.  H % 32 == 0,
// T * H * 2 and E * H * 4 below 2^32 (32-bit fill offsets).
template <int BT>
__global__ __launch_bounds__(256) void route_logits_gemm(const uint16_t *__restrict__ x, const float *__restrict__ wr,
                                                         const float *__restrict__ bias, int T, int H, int E,
                                                         float *__restrict__ z) {
    // four separate stage arrays, used with fixed roles per unrolled step,
    // so the compiler can tell a fill's destination from the stage being read
    // (a computed stage index would make it drain every fill before each read)
    constexpr int kRgX = BT * kRgK * 2;   // token rows per stage: 64 B each
    constexpr int kRgStage = kRgX + kRgW;
    __shared__ __align__(16) uint8_t st0[kRgStage];
    __shared__ __align__(16) uint8_t st1[kRgStage];
    __shared__ __align__(16) uint8_t st2[kRgStage];
    __shared__ __align__(16) uint8_t st3[kRgStage];
    const int net = (E + kRgE - 1) / kRgE, ntt = (T + BT - 1) / BT;
    const int b = blockIdx.x, xcd = b & 7, rest = b >> 3;
    const int et = rest % net, tt = (rest / net) * 8 + xcd;
    if (tt >= ntt) return;
    const int tok0 = tt * BT, ex0 = et * kRgE;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lc = lane & 31, h = lane >> 5;

    // fills of this wave (byte offsets; a step adds its K offset): token rows
    // 16 f .. +15 and router rows 8 f .. +7 for f = 2 wave, 2 wave + 1; rows
    // past T or E repeat a valid row (their results are never stored)
    const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(x, (uint32_t)((size_t)T * H * 2));
    const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(wr, (uint32_t)((size_t)E * H * 4));
    constexpr int XF = BT / 64;   // token-row fills per wave and step
    uint32_t xsrc[XF], wsrc[2];
#pragma unroll
    for (int j = 0; j < XF; ++j) {
        const int f = XF * wave + j;
        const int c = 16 * f + (lane >> 2), k = (lane & 3) ^ (c & 3);
        const int t = tok0 + c < T ? tok0 + c : T - 1;
        xsrc[j] = ((uint32_t)t * (uint32_t)H + 8 * k) * 2;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {   // lane: row er, slot lane & 7, which holds chunk (lane & 7) ^ ((er >> 1) & 7)
        const int f = 2 * wave + j;
        const int er = 8 * f + (lane >> 3), e = ex0 + er < E ? ex0 + er : E - 1;
        wsrc[j] = ((uint32_t)e * (uint32_t)H + 4 * ((lane & 7) ^ ((er >> 1) & 7))) * 4;
    }
    auto fill = [&](uint8_t *st, int k0) {
#pragma unroll
        for (int j = 0; j < XF; ++j) lds_fill<16>(xrs, xsrc[j] + k0 * 2, st + (XF * wave + j) * 1024);
#pragma unroll
        for (int j = 0; j < 2; ++j) lds_fill<16>(wrs, wsrc[j] + k0 * 4, st + kRgX + (2 * wave + j) * 1024);
    };

    // operand reads of this wave: experts 32 (wave & 1) + lc, tokens
    // (BT / 2) (wave >> 1) + 32 b + lc for its NB column tiles b; MFMA q
    // takes K [16q, 16q+16) of the step, lane half h its elements 8h..8h+7
    // (router: the fp32 chunks 2 (2q + h) and 2 (2q + h) + 1)
    constexpr int NB = BT / 64;
    const int ea = 32 * (wave & 1) + lc, tb0 = (BT / 2) * (wave >> 1) + lc;
    int aoff[2][2], boff[NB][2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int p = 0; p < 2; ++p) aoff[q][p] = kRgX + rg_wslot(ea, 2 * (2 * q + h) + p);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) boff[bb][q] = rg_slot(tb0 + 32 * bb, 2 * q + h);
    }
    f32x16 acc[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[bb][i] = 0.f;

    // the bias of this lane's 16 experts, requested now and used after the K loop
    float bv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = ex0 + 32 * (wave & 1) + 8 * (i / 4) + 4 * h + i % 4;
        bv[i] = (bias != nullptr && e < E) ? bias[e] : 0.0f;
    }
    const int S = H / kRgK;   // a multiple of 4 (H % 128 == 0)
    // Step s computes from stage s % 4 and fills step s + 3 into the stage of
    // step s - 1 (steps past the end refill the last one into a stage that
    // nothing reads).
    auto step = [&](const uint8_t *cur, uint8_t *nxt, int s) {
        // this wave's fills of step s are in (the later two steps' 4 fills
        // each may stay in flight); after the barrier everyone's are, and
        // every wave is done with step s - 1, whose stage `nxt` is
        fill_barrier<2 * (XF + 2)>();
        fill(nxt, (s + 3 < S ? s + 3 : S - 1) * kRgK);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            bf16x8 a[3], bt[NB];
            {
                const float4 v0 = *reinterpret_cast<const float4 *>(cur + aoff[q][0]);
                const float4 v1 = *reinterpret_cast<const float4 *>(cur + aoff[q][1]);
                const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                split3(v, a[0], a[1], a[2]);
            }
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) bt[bb] = *reinterpret_cast<const bf16x8 *>(cur + boff[bb][q]);
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                for (int pl = 0; pl < 3; ++pl) acc[bb] = mfma32x32x16(a[pl], bt[bb], acc[bb]);
        }
    };
    fill(st0, 0);
    fill(st1, (1 < S ? 1 : S - 1) * kRgK);
    fill(st2, (2 < S ? 2 : S - 1) * kRgK);
    for (int s = 0; s < S; s += 4) {
        step(st0, st3, s);
        step(st1, st0, s + 1);
        step(st2, st1, s + 2);
        step(st3, st2, s + 3);
    }

    // lane (lc, h), element i: expert 8 (i / 4) + 4 h + i % 4 of the wave's 32,
    // token lc of its column tile bb
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
        const int t = tok0 + tb0 + 32 * bb;
        if (t >= T) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = ex0 + 32 * (wave & 1) + 8 * (i / 4) + 4 * h + i % 4;
            if (e < E) z[(size_t)t * E + e] = acc[bb][i] + bv[i];
        }
    }
}

hipError_t launch_route_logits_gemm(const uint16_t *x, const float *wr, const float *bias, int T, int H, int E,
                                    float *z, hipStream_t st) {
    const int net = (E + kRgE - 1) / kRgE;
    if (T <= kRgSmallT) {
        const int ntt = (T + 63) / 64;
        MOE_LAUNCH("route_logits_gemm", route_logits_gemm<64>, dim3(8 * net * ((ntt + 7) / 8)), dim3(256), 0, st, x,
                   wr, bias, T, H, E, z);
    } else {
        const int ntt = (T + 127) / 128;
        MOE_LAUNCH("route_logits_gemm", route_logits_gemm<128>, dim3(8 * net * ((ntt + 7) / 8)), dim3(256), 0, st, x,
                   wr, bias, T, H, E, z);
    }
    return hipGetLastError();
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
            return launch_route_logits_gemm(x, wr, bias, T, H, E, z, st);
    } else {
        return launch_route_logits_gemm(x, wr, bias, T, H, E, z, st);
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
    s.nsync = WsLayout::kSyncWords;
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
