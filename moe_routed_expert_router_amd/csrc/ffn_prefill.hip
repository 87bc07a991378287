// Grouped SwiGLU expert FFN, prefill path (many tokens per expert).
//
// With ~128 tokens per expert the FFN is a real dense contraction, so it runs
// as a grouped GEMM on 32x32x16 bf16 MFMAs (on gfx950 the 32x32 form issues
// twice the flops per cycle of the 16x16x32 form).  The MXFP4 weights are
// converted in registers to exact bf16 (scaled fp4 converts), so the tokens
// enter the MFMA unchanged.  A work tile is (expert, up to kPT = 160 of its
// tokens, a block of weight rows); the grouping lists the (expert, token
// tile) pairs on the device.
//
// A block has 8 waves, each owning two 32-row weight operands and all of the
// tile's (up to five) 32-token column tiles.  Every K step, the block copies
// the next step's token (h) tile, weight codes and scales from global memory
// straight into LDS (buffer loads with an LDS destination, double-buffered);
// the global traffic per step is the block's unique bytes, once.  Each wave
// then reads its weight codes from LDS, converts them once per MFMA sub-step
// and runs the MFMAs, with the token operand reads issued a few MFMAs ahead.
// gate/up: operand 0 = 32 gate rows, operand 1 = the matching 32 up rows (a
// block covers 256 columns of h); the epilogue stores h = silu(g) * u as bf16
// hi + lo parts.  down: two 32-row operands of W2 (a block covers 512 output
// rows); h hi and lo both feed the same accumulators.
//
// K permutation: inside one K step, lane half h (lanes 32h..32h+31) covers a
// contiguous run of K made of whole MX blocks, and MFMA sub-step m takes the
// m-th 8 elements of that run.  The token operand is read with the same
// permutation, so each MFMA is an exact partial dot product.
//
// Blocks are numbered so that all row blocks of one token tile land on the
// same XCD (consecutive blocks go to consecutive XCDs) and share the tile's
// tokens in that XCD's L2; token tiles alternate over the eight XCDs.
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kPT = WsLayout::kPrefillTokens;   // tokens per tile
constexpr int kCT = kPT / 32;                   // 32-token column tiles per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kAhead = 2;                       // units of LDS operand reads issued ahead of the MFMAs

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

template <typename T>
__device__ __forceinline__ T lds_ld(const uint8_t *p) {
    return *reinterpret_cast<const T *>(p);
}

}  // namespace

// ---------------------------------------------------------------------------
// LDS stages.  Each kernel keeps two stages, as two separate arrays, in fixed
// roles per unrolled step (compute from one, fill the other).
//
// Token (h) tile: up to kPT rows of 256 bytes (16 chunks of 16 bytes); chunk
// k of row c sits in slot k ^ (c & 15), so 16 consecutive lanes reading one
// chunk of 16 consecutive rows hit 16 distinct slots.  A wave-wide 16-byte
// fill writes 64 consecutive slots (4 rows), lane l into slot l & 15 of row
// l >> 4, so each lane fetches the chunk its slot holds.  Weight tiles use
// the same idea with 64-byte (gate/up) or 32-byte (down) rows.
constexpr int kXBytes = kPT * 256;

// Double-buffered K loop over S (even) steps: step(cur, nxt, s, nx) computes
// step s from stage `cur` and starts the fills of step nx into `nxt`.  The
// last step refills step S - 1 into the idle stage, which nothing reads.
template <typename F>
__device__ __forceinline__ void k_loop2(int S, uint8_t *sa, uint8_t *sb, F &&step) {
    for (int s = 0; s < S; s += 2) {
        wait_vmem();
        __syncthreads();
        step(sa, sb, s, s + 1);
        wait_vmem();
        __syncthreads();
        step(sb, sa, s + 1, s + 2 < S ? s + 2 : S - 1);
    }
}

// Scheduling of one K step: its NV global fills first, then the NW weight
// reads and the LDS operand reads of the first kAhead units, then per unit
// its MPU MFMAs followed by its RPU operand reads kAhead units ahead.  The
// step is fenced on both sides so nothing moves across steps.
template <int U, int NV, int NW, int RPU, int MPU>
__device__ __forceinline__ void pipeline_order() {
    __builtin_amdgcn_sched_group_barrier(0x020, NV, 0);   // VMEM (LDS fills)
    __builtin_amdgcn_sched_group_barrier(0x100, NW + RPU * (kAhead < U ? kAhead : U), 0);   // DS reads
#pragma unroll
    for (int u = 0; u < U; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, MPU, 0);                       // MFMA
        if (u + kAhead < U) __builtin_amdgcn_sched_group_barrier(0x100, RPU, 0);   // DS read
    }
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void zero(f32x16 &a) {
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = 0.f;
}

// ---------------------------------------------------------------------------
// gate/up: K step 128.  Lane half h covers K [64h, 64h+64) of the step (MX
// blocks 2h, 2h+1); sub-step m = 0..7 takes its elements 8m..8m+7.
// Stage: token tile | weight codes [512 rows][64 B] | scales [512 rows][4 B];
// weight row r = 256 f + 32 w + c (f: 0 gate, 1 up) holds its 4 chunks in
// slots k ^ ((r >> 2) & 3).
// grid: 8-aligned (I/256 row blocks x token tiles); 512 threads.
constexpr int kGuRows = 2 * 32 * kWaves;
constexpr int kGuW = kXBytes;
constexpr int kGuS = kGuW + kGuRows * 64;
constexpr int kGuStage = kGuS + kGuRows * 4;

template <int T5>
__device__ __forceinline__ void gate_up_tile(__amdgpu_buffer_rsrc_t xrs, int H, int I, int k, const GroupView &gv,
                                             const Tile &t, uint8_t *sa, uint8_t *sb, uint16_t *__restrict__ hhi,
                                             uint16_t *__restrict__ hlo) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lc = lane & 31, h = lane >> 5;
    const BlobLayout L = BlobLayout::make(H, I);
    const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(t.base, (uint32_t)L.bytes);
    // fills of this wave (byte offsets; the step adds its K offset)
    uint32_t xsrc[T5], wsrc[4];
#pragma unroll
    for (int j = 0; j < T5; ++j) {   // token rows 4 (w T5 + j) .. +3; rows past the tile repeat its first token
        const int c = 4 * (wave * T5 + j) + (lane >> 4), chunk = (lane & 15) ^ (c & 15);
        xsrc[j] = ((uint32_t)(gv.plist[t.q0 + (c < t.nt ? c : 0)] / k) * (uint32_t)H + chunk * 8) * 2;
    }
    const size_t nst = H / 128;   // tiled blob: one 16-row group's step is 1 KB of codes, 64 B of scales
#pragma unroll
    for (int j = 0; j < 4; ++j) {    // weight rows 16 (4w + j) .. +15 (one tile: 1 KB contiguous), four lanes per row
        const int r = 16 * (4 * wave + j) + (lane >> 2), chunk = (lane & 3) ^ ((r >> 2) & 3);
        const size_t row = (size_t)((r >> 8) * I + t.rb * 256 + (r & 255));
        wsrc[j] = (uint32_t)(L.w13_codes + tiled_code_row(row, nst)) + 16 * chunk;
    }
    uint32_t ssrc;
    {                                // scales of weight rows 64 w .. +63, one per lane
        const int r = 64 * wave + lane;
        const size_t row = (size_t)((r >> 8) * I + t.rb * 256 + (r & 255));
        ssrc = (uint32_t)(L.w13_scales + tiled_scale_row(row, nst));
    }
    // reads of this wave: operand f row r_f = 256 f + 32 w + lc
    int wro[2][2], sro[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int r = 256 * f + 32 * wave + lc;
#pragma unroll
        for (int q = 0; q < 2; ++q) wro[f][q] = kGuW + r * 64 + 16 * ((2 * h + q) ^ ((r >> 2) & 3));
        sro[f] = kGuS + 4 * r;
    }
    // sub-step m reads chunk 8h + m of token row lc (column tile b adds 32
    // rows): slot (8h + m) ^ (lc & 15) = (8h ^ (lc & 8)) + (m ^ (lc & 7)), so
    // two registers give all eight offsets (eight would spill a fill address,
    // and its reload in the K loop would wait for that step's fills)
    const int rbase = lc * 256 + 16 * ((8 * h) ^ (lc & 8)), rx = lc & 7;

    auto fill = [&](uint8_t *st, int nx) {
#pragma unroll
        for (int j = 0; j < T5; ++j) lds_fill<16>(xrs, xsrc[j] + nx * 256, st + (wave * T5 + j) * 1024);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            lds_fill<16>(wrs, wsrc[j] + nx * (uint32_t)kCodeStep, st + kGuW + (4 * wave + j) * 1024);
        lds_fill<4>(wrs, ssrc + nx * (uint32_t)kScaleStep, st + kGuS + wave * 256);
    };

    f32x16 acc[2][kCT];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int b = 0; b < kCT; ++b) zero(acc[f][b]);

    fill(sa, 0);
    k_loop2(H / 128, sa, sb, [&](const uint8_t *cur, uint8_t *nxt, int, int nx) {
        __builtin_amdgcn_sched_barrier(0);
        fill(nxt, nx);
        u32x4 wc[2][2];
        float fs[2][2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const uint32_t sc = lds_ld<uint32_t>(cur + sro[f]);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                wc[f][q] = lds_ld<u32x4>(cur + wro[f][q]);
                fs[f][q] = e8m0_to_f32((sc >> (8 * (2 * h + q))) & 0xffu);
            }
        }
        constexpr int U = 8 * T5;    // units (m, b): m = u / T5, b = u % T5
        int rxs = rx;                // opaque per step, so the eight offsets are not hoisted into registers
        asm volatile("" : "+v"(rxs));
        bf16x8 bq[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            bq[u] = __builtin_bit_cast(bf16x8,
                                       lds_ld<u32x4>(cur + rbase + 16 * ((u / T5) ^ rxs) + (u % T5) * 32 * 256));
        bf16x8 a[2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int m = u / T5, b = u % T5;
            if (b == 0) {
#pragma unroll
                for (int f = 0; f < 2; ++f) a[f] = fp4x8_to_bf16x8(wc[f][m >> 2][m & 3], fs[f][m >> 2]);
            }
#pragma unroll
            for (int f = 0; f < 2; ++f) acc[f][b] = mfma32x32x16(a[f], bq[u], acc[f][b]);
        }
        pipeline_order<U, T5 + 5, 6, 1, 2>();
    });

    // lane (lc, h), element i: h column hcol + 8 (i / 4) + 4h + i % 4, token column 32 b + lc
    const size_t hcol = (size_t)t.rb * 256 + 32 * wave;
#pragma unroll
    for (int b = 0; b < T5; ++b) {
        const int c = 32 * b + lc;
        if (c < t.nt) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = silu(acc[0][b][4 * j + i]) * acc[1][b][4 * j + i];
                    hi[i] = f32_to_bf16_bits(v);
                    lo[i] = f32_to_bf16_bits(v - __uint_as_float(hi[i] << 16));
                }
                const size_t off = (size_t)(t.q0 + c) * I + hcol + 8 * j + 4 * h;
                *reinterpret_cast<uint2 *>(hhi + off) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
                *reinterpret_cast<uint2 *>(hlo + off) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
            }
        }
    }
}

// x_bytes = T * H * 2 < 2^31 (the fills address x with 32-bit byte offsets).
__global__ __launch_bounds__(kThreads) void ffn_gate_up_gemm(const uint16_t *__restrict__ x, uint32_t x_bytes, int H,
                                                             int I, int k, GroupView gv, uint16_t *__restrict__ hhi,
                                                             uint16_t *__restrict__ hlo) {
    __shared__ __align__(16) uint8_t sa[kGuStage];
    __shared__ __align__(16) uint8_t sb[kGuStage];
    Tile t;
    if (!tile_of_block(gv, I / 256, t) || t.base == nullptr) return;
    const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(x, x_bytes);
    switch ((t.nt + 31) >> 5) {   // 32-token column tiles of the tile
        case 1: gate_up_tile<1>(xrs, H, I, k, gv, t, sa, sb, hhi, hlo); break;
        case 2: gate_up_tile<2>(xrs, H, I, k, gv, t, sa, sb, hhi, hlo); break;
        case 3: gate_up_tile<3>(xrs, H, I, k, gv, t, sa, sb, hhi, hlo); break;
        case 4: gate_up_tile<4>(xrs, H, I, k, gv, t, sa, sb, hhi, hlo); break;
        default: gate_up_tile<5>(xrs, H, I, k, gv, t, sa, sb, hhi, hlo); break;
    }
}

// ---------------------------------------------------------------------------
// down: K step 64.  Lane half h covers K [32h, 32h+32) of the step (MX block
// h); sub-step m = 0..3 takes its elements 8m..8m+7.
// Stage: h tile (a row holds h hi in chunks 0..7 and h lo in chunks 8..15 for
// the step's 64 K) | W2 codes [512 rows][32 B] | scales [512 rows][4 B] (the
// aligned dword holding the step's two scale bytes and those of its pair
// step); weight row r = 64 w + 32 f + c holds its 2 chunks in slots
// k ^ ((r >> 3) & 1).
// grid: 8-aligned (H/512 row blocks x token tiles); 512 threads.
constexpr int kDnRows = 64 * kWaves;
constexpr int kDnW = kXBytes;
constexpr int kDnS = kDnW + kDnRows * 32;
constexpr int kDnStage = kDnS + kDnRows * 4;

template <int T5>
__device__ __forceinline__ void down_tile(int H, int I, uint32_t plane, const GroupView &gv, const Tile &t,
                                          uint8_t *sa, uint8_t *sb, __amdgpu_buffer_rsrc_t hrs,
                                          float *__restrict__ y) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lc = lane & 31, h = lane >> 5;
    const BlobLayout L = BlobLayout::make(H, I);
    const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(t.base, (uint32_t)L.bytes);
    const uint32_t orow0 = (uint32_t)t.rb * 512;
    uint32_t xsrc[T5], wsrc[2];
#pragma unroll
    for (int j = 0; j < T5; ++j) {   // h rows 4 (w T5 + j) .. +3 (lo plane `plane` elements after hi)
        const int c = 4 * (wave * T5 + j) + (lane >> 4), chunk = (lane & 15) ^ (c & 15);
        xsrc[j] = ((chunk < 8 ? 0u : plane) + (uint32_t)(t.q0 + (c < t.nt ? c : 0)) * (uint32_t)I + (chunk & 7) * 8) * 2;
    }
    const size_t nst = I / 128;   // tiled blob: a 64-K step is one half of each row's 64 bytes of a tile
#pragma unroll
    for (int j = 0; j < 2; ++j) {    // weight rows 32 (2w + j) .. +31, two lanes per row
        const int r = 32 * (2 * wave + j) + (lane >> 1), chunk = (lane & 1) ^ ((r >> 3) & 1);
        wsrc[j] = (uint32_t)(L.w2_codes + tiled_code_row(orow0 + r, nst)) + 16 * chunk;
    }
    const uint32_t ssrc = (uint32_t)(L.w2_scales + tiled_scale_row(orow0 + 64 * wave + lane, nst));
    int wro[2], sro[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int r = 64 * wave + 32 * f + lc;
        wro[f] = kDnW + r * 32 + 16 * (h ^ ((r >> 3) & 1));
        sro[f] = kDnS + 4 * r + h;   // + 2 for odd steps
    }
    int roff[8];   // hi: chunk 4h + m (roff[m]); lo: chunk 8 + 4h + m (roff[4 + m])
#pragma unroll
    for (int i = 0; i < 8; ++i) roff[i] = lc * 256 + 16 * ((8 * (i >> 2) + 4 * h + (i & 3)) ^ (lc & 15));

    auto fill = [&](uint8_t *st, int nx) {
#pragma unroll
        for (int j = 0; j < T5; ++j) lds_fill<16>(hrs, xsrc[j] + nx * 128, st + (wave * T5 + j) * 1024);
        const uint32_t wstep = (uint32_t)(nx >> 1) * (uint32_t)kCodeStep + (uint32_t)(nx & 1) * 32;
#pragma unroll
        for (int j = 0; j < 2; ++j) lds_fill<16>(wrs, wsrc[j] + wstep, st + kDnW + (2 * wave + j) * 1024);
        lds_fill<4>(wrs, ssrc + (uint32_t)(nx >> 1) * (uint32_t)kScaleStep, st + kDnS + wave * 256);
    };

    f32x16 acc[2][kCT];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int b = 0; b < kCT; ++b) zero(acc[f][b]);

    fill(sa, 0);
    k_loop2(I / 64, sa, sb, [&](const uint8_t *cur, uint8_t *nxt, int sc, int nx) {
        __builtin_amdgcn_sched_barrier(0);
        fill(nxt, nx);
        u32x4 wc[2];
        float fs[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            wc[f] = lds_ld<u32x4>(cur + wro[f]);
            fs[f] = e8m0_to_f32(lds_ld<uint8_t>(cur + sro[f] + 2 * (sc & 1)));
        }
        constexpr int U = 4 * T5;    // units (m, b); a unit reads the hi and lo operands of column tile b
        bf16x8 bh[U], bl[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            bh[u] = __builtin_bit_cast(bf16x8, lds_ld<u32x4>(cur + roff[u / T5] + (u % T5) * 32 * 256));
            bl[u] = __builtin_bit_cast(bf16x8, lds_ld<u32x4>(cur + roff[4 + u / T5] + (u % T5) * 32 * 256));
        }
        bf16x8 a[2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int m = u / T5, b = u % T5;
            if (b == 0) {
#pragma unroll
                for (int f = 0; f < 2; ++f) a[f] = fp4x8_to_bf16x8(wc[f][m], fs[f]);
            }
#pragma unroll
            for (int f = 0; f < 2; ++f) acc[f][b] = mfma32x32x16(a[f], bh[u], acc[f][b]);
#pragma unroll
            for (int f = 0; f < 2; ++f) acc[f][b] = mfma32x32x16(a[f], bl[u], acc[f][b]);
        }
        pipeline_order<U, T5 + 3, 4, 2, 4>();
    });

    // lane (lc, h), element i: row orow0 + 64 w + 32 f + 8 (i / 4) + 4h + i % 4, token column 32 b + lc
#pragma unroll
    for (int b = 0; b < T5; ++b) {
        const int c = 32 * b + lc;
        if (c < t.nt) {
            float *yp = y + (size_t)gv.plist[t.q0 + c] * H + orow0 + 64 * wave + 4 * h;
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<float4 *>(yp + 32 * f + 8 * j) =
                        make_float4(acc[f][b][4 * j], acc[f][b][4 * j + 1], acc[f][b][4 * j + 2], acc[f][b][4 * j + 3]);
        }
    }
}

// hbuf: the h hi plane followed by the lo plane, `plane` = P * I elements
// each; 2 * plane * 2 < 2^31 bytes.
__global__ __launch_bounds__(kThreads) void ffn_down_gemm(int H, int I, GroupView gv,
                                                          const uint16_t *__restrict__ hbuf, uint32_t plane,
                                                          float *__restrict__ y) {
    __shared__ __align__(16) uint8_t sa[kDnStage];
    __shared__ __align__(16) uint8_t sb[kDnStage];
    Tile t;
    if (!tile_of_block(gv, H / 512, t)) return;
    if (t.base == nullptr) {   // unusable residency entry: its pairs contribute zero
        for (int i = threadIdx.x; i < t.nt * 128; i += kThreads) {
            const int c = i >> 7, col = i & 127;
            reinterpret_cast<float4 *>(y + (size_t)gv.plist[t.q0 + c] * H + (size_t)t.rb * 512)[col] =
                make_float4(0.f, 0.f, 0.f, 0.f);
        }
        return;
    }
    const __amdgpu_buffer_rsrc_t hrs = buffer_rsrc(hbuf, 4 * plane);
    switch ((t.nt + 31) >> 5) {
        case 1: down_tile<1>(H, I, plane, gv, t, sa, sb, hrs, y); break;
        case 2: down_tile<2>(H, I, plane, gv, t, sa, sb, hrs, y); break;
        case 3: down_tile<3>(H, I, plane, gv, t, sa, sb, hrs, y); break;
        case 4: down_tile<4>(H, I, plane, gv, t, sa, sb, hrs, y); break;
        default: down_tile<5>(H, I, plane, gv, t, sa, sb, hrs, y); break;
    }
}

bool ffn_gemm_path(int T, int H, int I, int k) {
    const size_t P = (size_t)T * k;
    return T > kSmallRouteTokens && H % 512 == 0 && I % 256 == 0 && (size_t)T * H * 2 < ((size_t)1 << 31) &&
           P * I * 4 < ((size_t)1 << 31) && BlobLayout::make(H, I).bytes < ((size_t)1 << 31);
}

hipError_t launch_ffn_gemm(const FfnArgs &a, const GroupView &gv, int max_tiles, uint16_t *hhi, uint16_t *hlo,
                           float *y, hipStream_t st) {
    const int tiles8 = (max_tiles + 7) / 8 * 8;
    const uint32_t plane = (uint32_t)(hlo - hhi);
    MOE_LAUNCH("ffn_gate_up_gemm", ffn_gate_up_gemm, dim3((a.I / 256) * tiles8), dim3(kThreads), 0, st, a.x,
               (uint32_t)((size_t)a.T * a.H * 2), a.H, a.I, a.k, gv, hhi, hlo);
    MOE_LAUNCH("ffn_down_gemm", ffn_down_gemm, dim3((a.H / 512) * tiles8), dim3(kThreads), 0, st, a.H, a.I, gv, hhi,
               plane, y);
    return hipGetLastError();
}

}  // namespace moe
