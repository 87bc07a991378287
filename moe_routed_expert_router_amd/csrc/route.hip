// Router: logits and top-k softmax selection, plus the fused select-and-group
// kernel of the decode path.
//
// The pages: a tiny router picks the 6 most relevant of 384 experts per token
// (GB300 inference write-up, mixture-of-experts paragraph).  Scores are a
// softmax over z[t,e] = x_t . Wr_e + b_e; the k largest logits are kept, equal
// logits going to the lower expert index, and the kept weights renormalised.
#include "device_util.hpp"
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Decode-size logits (T <= 32): a block of 4 waves owns 4 expert rows; tokens
// are staged in LDS 8 at a time and each wave issues its whole row (up to
// 4096 columns, 16 x 128-bit loads per lane) before the first FMA, so the
// router matrix (E*H*4 bytes, the only HBM traffic) streams with every load
// in flight at once.
// ---------------------------------------------------------------------------
constexpr int kGemvTok = 8;
constexpr int kGemvCols = 4096;   // columns per register pass

__global__ __launch_bounds__(256) void route_logits_gemv(
    const uint16_t *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    int T, int H, int E, float *__restrict__ z) {
    extern __shared__ __align__(16) uint16_t xs[];   // [kGemvTok][min(H, kGemvCols)]
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    const bool ve = e < E;
    const float4 *wrow = reinterpret_cast<const float4 *>(wr + (size_t)(ve ? e : 0) * H);
    const float b = (ve && bias) ? bias[e] : 0.0f;
    const int W = H < kGemvCols ? H : kGemvCols;   // staged columns per pass
    for (int t0 = 0; t0 < T; t0 += kGemvTok) {
        const int nt = (T - t0) < kGemvTok ? (T - t0) : kGemvTok;
        float acc[kGemvTok];
#pragma unroll
        for (int i = 0; i < kGemvTok; ++i) acc[i] = 0.0f;
        for (int h0 = 0; h0 < H; h0 += W) {
            __syncthreads();
            const int n16 = nt * (W / 8);   // 16-byte chunks of the token tile
            for (int i = threadIdx.x; i < n16; i += 256) {
                const int tt = i / (W / 8), c = i - tt * (W / 8);
                reinterpret_cast<uint4 *>(xs)[i] =
                    *reinterpret_cast<const uint4 *>(x + (size_t)(t0 + tt) * H + h0 + 8 * c);
            }
            __syncthreads();
            if (ve) {
                float4 w4[kGemvCols / 256];
#pragma unroll
                for (int i = 0; i < kGemvCols / 256; ++i) {
                    const int c = lane + 64 * i;
                    w4[i] = (4 * c < W) ? wrow[h0 / 4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int tt = 0; tt < kGemvTok; ++tt) {
                    if (tt < nt) {
                        float a = acc[tt];
#pragma unroll
                        for (int i = 0; i < kGemvCols / 256; ++i) {
                            const int c = lane + 64 * i;
                            if (4 * c < W) {
                                const uint2 xv = reinterpret_cast<const uint2 *>(xs + tt * W)[c];
                                a = fmaf(w4[i].x, bf16_bits_to_f32(xv.x & 0xffffu), a);
                                a = fmaf(w4[i].y, bf16_bits_to_f32(xv.x >> 16), a);
                                a = fmaf(w4[i].z, bf16_bits_to_f32(xv.y & 0xffffu), a);
                                a = fmaf(w4[i].w, bf16_bits_to_f32(xv.y >> 16), a);
                            }
                        }
                        acc[tt] = a;
                    }
                }
            }
        }
#pragma unroll
        for (int tt = 0; tt < kGemvTok; ++tt) {
            const float v = wave_sum(acc[tt]);
            if (ve && lane == 0 && tt < nt) z[(size_t)(t0 + tt) * E + e] = v + b;
        }
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
        const int W = H < kGemvCols ? H : kGemvCols;
        const size_t lds = (size_t)kGemvTok * W * 2;
        MOE_LAUNCH("route_logits_gemv", route_logits_gemv, dim3((E + 3) / 4), dim3(256), lds, st,
                   x, wr, bias, T, H, E, z);
    } else {
        MOE_LAUNCH("route_logits_mfma", route_logits_mfma, dim3((E + 63) / 64, (T + 63) / 64), dim3(256), 0, st,
                   x, wr, bias, T, H, E, z);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k for any T: one wave per token.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_topk(const float *__restrict__ z, int T, int E, int k,
                                                  int renorm, int32_t *__restrict__ ids,
                                                  float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int pe;
    float pw;
    topk_wave(z + (size_t)t * E, E, k, renorm, &pe, &pw);
    if (lane < k) {
        ids[(size_t)t * k + lane] = pe;
        w[(size_t)t * k + lane] = pw;
    }
}

hipError_t launch_topk(const float *z, int T, int E, int k, int renorm, int32_t *ids, float *w,
                       hipStream_t st) {
    MOE_LAUNCH("route_topk", route_topk, dim3((T + 3) / 4), dim3(256), 0, st, z, T, E, k, renorm, ids, w);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode path: top-k of every token and the whole pick set in ONE block, so
// routing and grouping cost one launch.  16 waves take the tokens and count
// each pick into its expert (LDS integer atomics: only the counts are used).
// Wave 0 then walks the experts in increasing order — lane l owns a
// contiguous run of E/64 experts — and with three wave scans turns the counts
// into each expert's pair run, the distinct-expert list with blob addresses,
// and the picked-cold list.  Finally one thread per pair ranks it among the
// earlier pairs of its expert, so every run lists pairs in increasing order.
// It also zeroes the FFN's completion counters.  Needs T*k <= 1024.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void select_group_small(
    const float *__restrict__ z, int T, int E, int k, int renorm, int32_t *__restrict__ ids,
    float *__restrict__ w, const int32_t *__restrict__ slot, int n_hot, int n_cold, const uint8_t *hot_base,
    const uint8_t *scratch, size_t blob_bytes, GroupOut o) {
    __shared__ int sid[1024];
    __shared__ int cnt[kMaxExperts];
    __shared__ int offs[kMaxExperts];
    __shared__ int sslot[kMaxExperts];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < E) {
        sslot[tid] = slot[tid];
        cnt[tid] = 0;
    }
    for (int i = tid; i < WsLayout::kSyncWords; i += 1024) o.sync[i] = 0;
    __syncthreads();
    for (int t = wave; t < T; t += 16) {
        int pe;
        float pw;
        topk_wave(z + (size_t)t * E, E, k, renorm, &pe, &pw);
        if (lane < k) {
            ids[(size_t)t * k + lane] = pe;
            w[(size_t)t * k + lane] = pw;
            sid[t * k + lane] = pe;
            atomicAdd(&cnt[pe], 1);
        }
    }
    __syncthreads();
    const int P = T * k;
    if (wave == 0) {
        const int per = (E + 63) >> 6;   // experts per lane, <= 16
        const int e0 = lane * per;
        int c[kPerLane];
        int tot = 0, npick = 0, ncold = 0, nbad = 0;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int e = e0 + i;
            c[i] = (i < per && e < E) ? cnt[e] : 0;
            if (c[i] > 0) {
                bool ok, cold;
                (void)expert_address(sslot[e], n_hot, n_cold, hot_base, scratch, blob_bytes, &ok, &cold);
                npick += 1;
                ncold += (ok && cold) ? 1 : 0;
                nbad += ok ? 0 : 1;
            }
            tot += c[i];
        }
        int ptot, nu, nc;
        int off = wave_exscan(tot, &ptot);
        int ui = wave_exscan(npick, &nu);
        int ci = wave_exscan(ncold, &nc);
        const int nb = wave_sum_int(nbad);
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int e = e0 + i;
            if (i < per && e < E) {
                offs[e] = off;
                o.counts[e] = c[i];
                if (c[i] > 0) {
                    bool ok, cold;
                    const uint64_t addr =
                        expert_address(sslot[e], n_hot, n_cold, hot_base, scratch, blob_bytes, &ok, &cold);
                    o.uniq[ui] = e;
                    o.ucnt[ui] = c[i];
                    o.uoff[ui] = off;
                    o.uptr[ui] = addr;
                    ++ui;
                    if (ok && cold) o.cold[ci++] = e;
                }
                off += c[i];
            }
        }
        if (lane == 0) {
            o.nuniq[0] = nu;
            o.nuniq[1] = nc;
            o.status[0] = 0;
            o.status[1] = nb;
            o.uoff[nu] = ptot;
        }
    }
    __syncthreads();
    if (tid < P) {
        const int e = sid[tid];
        int rank = 0;
        for (int q = 0; q < tid; ++q) rank += (sid[q] == e);
        o.plist[offs[e] + rank] = tid;
    }
}

hipError_t launch_select_group_small(const float *z, int T, int k, int renorm, int32_t *ids, float *w,
                                     const GroupArgs &a, char *ws, const WsLayout &L, hipStream_t st) {
    MOE_LAUNCH("select_group_small", select_group_small, dim3(1), dim3(1024), 0, st, z, T, a.E, k, renorm, ids, w,
               a.slot, a.n_hot, a.n_cold, a.hot_base, a.scratch, a.blob_bytes, GroupOut::at(ws, L));
    return hipGetLastError();
}

}  // namespace moe
