// Grouped SwiGLU expert FFN, prefill path (many tokens per expert).
//
// With ~128 tokens per expert the FFN is a real dense contraction, so it runs
// as a grouped GEMM on 16x16x32 bf16 MFMAs.  The MXFP4 weights are converted
// in registers to exact bf16 (scaled fp4 converts), so the tokens enter the
// MFMA unchanged.  A work tile is (expert, up to kPT tokens of it, a block of
// weight rows); the grouping lists the (expert, token tile) pairs on the
// device.  Per K step:
//   * each wave loads its 64 weight rows' MXFP4 codes straight into registers
//     (one MX block or half of one per lane and row) and converts them once;
//   * the block stages the tile's token rows (gate/up) or h rows (down) for
//     that K step in LDS, double-buffered, prefetching the next step through
//     registers;
//   * each converted weight operand meets all kPT / 16 token column tiles, and
//     each token operand read from LDS meets four weight operands.
// gate/up: a wave owns 32 gate + 32 up rows (a block, 128 rows of h); the
// epilogue stores h = silu(g) * u as bf16 hi + lo parts.  down: a wave owns 64
// rows (a block, 256 rows of y); h hi and lo both feed the same accumulators.
//
// K permutation: inside one K step, lane group g (lanes 16g..16g+15) covers a
// contiguous run of K that lies in one MX block, and MFMA sub-step m takes the
// m-th 8 elements of that run.  The token operand is read with the same
// permutation, so each MFMA is an exact partial dot product and every lane
// needs one scale byte per row and step.
//
// Blocks are numbered so that all row blocks of one token tile land on the
// same XCD (consecutive blocks go to consecutive XCDs) and share the tile's
// tokens in that XCD's L2; token tiles alternate over the eight XCDs.
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kPT = WsLayout::kPrefillTokens;   // tokens per tile
constexpr int kNB = kPT / 16;                    // MFMA token column tiles
constexpr int kThreads = 256;

struct Tile {
    int u, q0, nt, rb;
    const uint8_t *base;
};

// The block's (row block, token tile); false when the block has no tile.
// t.base is null when the expert's residency entry is unusable.
__device__ __forceinline__ bool tile_of_block(const GroupView &gv, int rowblocks, Tile &t) {
    const int b = blockIdx.x;
    const int xcd = b & 7, rest = b >> 3;
    t.rb = rest % rowblocks;
    const int ti = (rest / rowblocks) * 8 + xcd;
    if (ti >= gv.nuniq[2]) return false;
    const int te = gv.tlist[ti];
    t.u = te & 1023;
    const int part = te >> 10;
    t.base = reinterpret_cast<const uint8_t *>(gv.uptr[t.u]);
    const int n = gv.ucnt[t.u] - part * kPT;
    t.q0 = gv.uoff[t.u] + part * kPT;
    t.nt = n < kPT ? n : kPT;
    return t.nt > 0;
}

__device__ __forceinline__ uint4 lds16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

}  // namespace

// ---------------------------------------------------------------------------
// gate/up: K step 128 (lane group g covers MX block g of the step).
// grid: 8-aligned (I/128 row blocks x token tiles); 256 threads.
constexpr int kGuRow = 136;                          // LDS row: 128 bf16 + 8 pad (bank spread)
constexpr int kGuChunks = kPT * 16 / kThreads;       // 16-byte chunks staged per thread and step

__global__ __launch_bounds__(kThreads) void ffn_gate_up_gemm(const uint16_t *__restrict__ x, int H, int I, int k,
                                                             GroupView gv,
                                                             uint16_t *__restrict__ hhi, uint16_t *__restrict__ hlo) {
    __shared__ __align__(16) uint16_t xs[2][kPT * kGuRow];
    Tile t;
    if (!tile_of_block(gv, I / 128, t) || t.base == nullptr) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int nbt = (t.nt + 15) >> 4;   // active column tiles (block-uniform)
    const BlobLayout L = BlobLayout::make(H, I);
    const size_t hrow = (size_t)t.rb * 128 + wave * 32 + r;   // h row of frag 0; frag 1 is +16
    // operand f: 0,1 gate rows hrow, hrow+16; 2,3 up rows I+hrow, I+hrow+16
    const uint8_t *cp[4], *sp[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const size_t row = hrow + (f & 1) * 16 + (f >> 1) * (size_t)I;
        cp[f] = t.base + L.w13_codes + row * (H / 2) + 16 * g;
        sp[f] = t.base + L.w13_scales + row * (H / 32);
    }
    const uint16_t *src[kGuChunks];
    int dst[kGuChunks];
#pragma unroll
    for (int j = 0; j < kGuChunks; ++j) {
        const int i = tid + kThreads * j, c = i >> 4, col = i & 15;
        src[j] = (c < t.nt) ? x + (size_t)(gv.plist[t.q0 + c] / k) * H + col * 8 : nullptr;
        dst[j] = c * kGuRow + col * 8;
    }
    const int S = H / 128;
    u32x4 st[kGuChunks];
    uint4 w[4];
    uint32_t sc[4];
#pragma unroll
    for (int j = 0; j < kGuChunks; ++j)
        if (src[j]) st[j] = gload<u32x4>(src[j]);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        w[f] = gload16(cp[f]);
        sc[f] = gload<uint32_t>(sp[f]);
    }
#pragma unroll
    for (int j = 0; j < kGuChunks; ++j)
        if (src[j]) *reinterpret_cast<u32x4 *>(&xs[0][dst[j]]) = st[j];

    f32x4 acc[4][kNB];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int b = 0; b < kNB; ++b) acc[f][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s = 0; s < S; ++s) {
        __syncthreads();   // step s staged in xs[s & 1]; xs[(s+1) & 1] free
        uint4 wn[4];
        uint32_t scn[4];
        const bool more = s + 1 < S;
        if (more) {
#pragma unroll
            for (int j = 0; j < kGuChunks; ++j)
                if (src[j]) st[j] = gload<u32x4>(src[j] + (s + 1) * 128);
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                wn[f] = gload16(cp[f] + (size_t)(s + 1) * 64);
                scn[f] = gload<uint32_t>(sp[f] + 4 * (s + 1));
            }
        }
        float fs[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) fs[f] = e8m0_to_f32((sc[f] >> (8 * g)) & 0xffu);
        const uint16_t *xb = &xs[s & 1][r * kGuRow + 32 * g];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            bf16x8 a[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const uint32_t word = m == 0 ? w[f].x : m == 1 ? w[f].y : m == 2 ? w[f].z : w[f].w;
                a[f] = fp4x8_to_bf16x8(word, fs[f]);
            }
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
                if (b < nbt) {
                    const bf16x8 bv = as_bf16x8(lds16(xb + b * 16 * kGuRow + 8 * m));
#pragma unroll
                    for (int f = 0; f < 4; ++f) acc[f][b] = mfma16x16x32(a[f], bv, acc[f][b]);
                }
            }
        }
        if (more) {
#pragma unroll
            for (int j = 0; j < kGuChunks; ++j)
                if (src[j]) *reinterpret_cast<u32x4 *>(&xs[(s + 1) & 1][dst[j]]) = st[j];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                w[f] = wn[f];
                sc[f] = scn[f];
            }
        }
    }
    // lane (r, g) holds rows 4g..4g+3 of each 16-row operand for token column r
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
        const int c = b * 16 + r;
        if (c < t.nt) {
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float h = silu(acc[f][b][i]) * acc[f + 2][b][i];
                    hi[i] = f32_to_bf16_bits(h);
                    lo[i] = f32_to_bf16_bits(h - __uint_as_float(hi[i] << 16));
                }
                const size_t off = (size_t)(t.q0 + c) * I + hrow - r + f * 16 + 4 * g;
                *reinterpret_cast<uint2 *>(hhi + off) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
                *reinterpret_cast<uint2 *>(hlo + off) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// down: K step 64 (lane group g covers K [16g, 16g+16) of the step, half of MX
// block g/2); h hi and lo staged side by side.
// grid: 8-aligned (H/256 row blocks x token tiles); 256 threads.
constexpr int kDnRow = 72;                            // LDS row: 64 bf16 + 8 pad
constexpr int kDnPlane = kPT * kDnRow;
constexpr int kDnChunks = 2 * kPT * 8 / kThreads;     // 16-byte chunks staged per thread and step

__global__ __launch_bounds__(kThreads) void ffn_down_gemm(int H, int I, GroupView gv, const uint16_t *__restrict__ hhi,
                                                          const uint16_t *__restrict__ hlo, float *__restrict__ y) {
    __shared__ __align__(16) uint16_t hs[2][2 * kDnPlane];
    Tile t;
    if (!tile_of_block(gv, H / 256, t)) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
    if (t.base == nullptr) {   // unusable residency entry: its pairs contribute zero
        for (int i = tid; i < t.nt * 64; i += kThreads) {
            const int c = i >> 6, col = i & 63;
            reinterpret_cast<float4 *>(y + (size_t)gv.plist[t.q0 + c] * H + (size_t)t.rb * 256)[col] =
                make_float4(0.f, 0.f, 0.f, 0.f);
        }
        return;
    }
    const int nbt = (t.nt + 15) >> 4;
    const BlobLayout L = BlobLayout::make(H, I);
    const size_t row0 = (size_t)t.rb * 256 + wave * 64 + r;   // operand f: rows row0 + 16f
    const uint8_t *cp[4], *sp[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const size_t row = row0 + 16 * f;
        cp[f] = t.base + L.w2_codes + row * (I / 2) + 8 * g;
        sp[f] = t.base + L.w2_scales + row * (I / 32) + (g >> 1);
    }
    const uint16_t *src[kDnChunks];
    int dst[kDnChunks];
#pragma unroll
    for (int j = 0; j < kDnChunks; ++j) {
        const int i = tid + kThreads * j, plane = i / (kPT * 8), rem = i - plane * (kPT * 8);
        const int c = rem >> 3, col = rem & 7;
        src[j] = (c < t.nt) ? (plane ? hlo : hhi) + (size_t)(t.q0 + c) * I + col * 8 : nullptr;
        dst[j] = plane * kDnPlane + c * kDnRow + col * 8;
    }
    const int S = I / 64;
    u32x4 st[kDnChunks];
    uint2 w[4];
    uint32_t sc[4];
#pragma unroll
    for (int j = 0; j < kDnChunks; ++j)
        if (src[j]) st[j] = gload<u32x4>(src[j]);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        w[f] = gload<uint2>(cp[f]);
        sc[f] = gload<uint8_t>(sp[f]);
    }
#pragma unroll
    for (int j = 0; j < kDnChunks; ++j)
        if (src[j]) *reinterpret_cast<u32x4 *>(&hs[0][dst[j]]) = st[j];

    f32x4 acc[4][kNB];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int b = 0; b < kNB; ++b) acc[f][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s = 0; s < S; ++s) {
        __syncthreads();
        uint2 wn[4];
        uint32_t scn[4];
        const bool more = s + 1 < S;
        if (more) {
#pragma unroll
            for (int j = 0; j < kDnChunks; ++j)
                if (src[j]) st[j] = gload<u32x4>(src[j] + (s + 1) * 64);
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                wn[f] = gload<uint2>(cp[f] + (size_t)(s + 1) * 32);
                scn[f] = gload<uint8_t>(sp[f] + 2 * (s + 1));
            }
        }
        const uint16_t *hb = &hs[s & 1][r * kDnRow + 16 * g];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            bf16x8 a[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) a[f] = fp4x8_to_bf16x8(m == 0 ? w[f].x : w[f].y, e8m0_to_f32(sc[f]));
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
                if (b < nbt) {
                    const bf16x8 bh = as_bf16x8(lds16(hb + b * 16 * kDnRow + 8 * m));
                    const bf16x8 bl = as_bf16x8(lds16(hb + kDnPlane + b * 16 * kDnRow + 8 * m));
#pragma unroll
                    for (int f = 0; f < 4; ++f) acc[f][b] = mfma16x16x32(a[f], bh, acc[f][b]);
#pragma unroll
                    for (int f = 0; f < 4; ++f) acc[f][b] = mfma16x16x32(a[f], bl, acc[f][b]);
                }
            }
        }
        if (more) {
#pragma unroll
            for (int j = 0; j < kDnChunks; ++j)
                if (src[j]) *reinterpret_cast<u32x4 *>(&hs[(s + 1) & 1][dst[j]]) = st[j];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                w[f] = wn[f];
                sc[f] = scn[f];
            }
        }
    }
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
        const int c = b * 16 + r;
        if (c < t.nt) {
            float *yp = y + (size_t)gv.plist[t.q0 + c] * H + row0 - r + 4 * g;
#pragma unroll
            for (int f = 0; f < 4; ++f)
                *reinterpret_cast<float4 *>(yp + 16 * f) =
                    make_float4(acc[f][b][0], acc[f][b][1], acc[f][b][2], acc[f][b][3]);
        }
    }
}

bool ffn_gemm_path(int T, int H, int I) { return T > kSmallRouteTokens && H % 256 == 0 && I % 128 == 0; }

hipError_t launch_ffn_gemm(const FfnArgs &a, const GroupView &gv, int max_tiles, uint16_t *hhi, uint16_t *hlo, float *y, hipStream_t st) {
    const int tiles8 = (max_tiles + 7) / 8 * 8;
    MOE_LAUNCH("ffn_gate_up_gemm", ffn_gate_up_gemm, dim3((a.I / 128) * tiles8), dim3(kThreads), 0, st, a.x, a.H,
               a.I, a.k, gv, hhi, hlo);
    MOE_LAUNCH("ffn_down_gemm", ffn_down_gemm, dim3((a.H / 256) * tiles8), dim3(kThreads), 0, st, a.H, a.I, gv, hhi,
               hlo, y);
    return hipGetLastError();
}

}  // namespace moe
