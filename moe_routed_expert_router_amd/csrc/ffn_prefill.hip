// Grouped SwiGLU expert FFN, prefill path (many tokens per expert).
//
// With ~128 tokens per expert the FFN is a real dense contraction, so it runs
// as a grouped GEMM on the matrix cores.  gate/up: 32x32x16 bf16 MFMAs (on
// gfx950 the 32x32 form issues twice the flops per cycle of the 16x16x32
// form), the MXFP4 weights converted in registers to exact bf16 (scaled fp4
// converts), so the bf16 tokens enter unchanged.  down: the scaled 32x32x64
// fp4 x fp8 MFMA on the W2 codes as stored, h entering as three MXFP8 terms
// (2.3 times the bf16 rate per flop).  A work tile is (expert, up to kPT =
// 160 of its tokens, a block of weight rows); the grouping lists the
// (expert, token tile) pairs on the device.
//
// A block has 8 waves, each owning two 32-row weight operands and all of the
// tile's (up to five) 32-token column tiles.  Every K step, the block copies
// the next step's token (x or h) tile, weight codes and scales from global
// memory straight into LDS (buffer loads with an LDS destination,
// double-buffered); the global traffic per step is the block's unique bytes,
// once.  Each wave then reads its weight codes from LDS (the gate/up converts
// them once per MFMA sub-step) and runs the MFMAs, with the token operand
// reads issued a few MFMAs ahead.
// gate/up: operand 0 = 32 gate rows, operand 1 = the matching 32 up rows (a
// block covers 256 columns of h); the epilogue stores h = silu(g) * u as three
// MXFP8 terms (e4m3 codes, one e8m0 scale per 32 columns each), the second
// and third holding what the terms before leave.  down: two 32-row operands
// of W2 (a block covers 512 output rows); per K step each h term enters one
// scaled fp4 x fp8 MFMA that takes the W2 codes and scales as stored.
//
// K permutation (gate/up): inside one K step, lane half h (lanes
// 32h..32h+31) covers a contiguous run of K made of whole MX blocks, and MFMA
// sub-step m takes the m-th 8 elements of that run.  The token operand is
// read with the same permutation, so each MFMA is an exact partial dot
// product.  (The down GEMM's scaled MFMA takes K in its own operand order.)
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

// Least e with amax <= 448 * 2^e (448: the largest e4m3 value), clamped to
// e8m0's [-127, 127]; -127 for amax = 0.
__device__ __forceinline__ int e8m0_for(float amax) {
    if (!(amax > 0.f)) return -127;
    int e = (int)((__float_as_uint(amax) >> 23) & 255u) - 127 - 8;   // amax / 2^e in [256, 512)
    if (amax > ldexpf(448.f, e)) ++e;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Four values as e4m3 codes (round to nearest even), a in the low byte.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    const uint32_t v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)v, true);
}

// silu(g) = g / (1 + e^-g) with the reciprocal instruction (about 1 ulp) in
// place of an IEEE division (a ten-instruction sequence): the epilogue runs
// it on every h element of a tile.  g << 0 gives -0, as the division does.
__device__ __forceinline__ float silu_rcp(float g) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// D += W x H over one 64-K step on the scaled 32x32x64 MFMA: A = 32 weight
// rows as fp4 codes (lane half h: K [32h, 32h+32), element order) with their
// e8m0 scale bytes, B = 32 token columns as e4m3 codes (lane half h: K [16h,
// 16h+16) in xa, [32+16h, 32+16h+16) in xb) with theirs; lane half h's
// scale covers K block h for both operands.
__device__ __forceinline__ f32x16 mfma_f4_f8(const u32x4 &w, const u32x4 &xa, const u32x4 &xb, uint32_t ws,
                                             uint32_t xs, f32x16 c) {
    const i32x8 a = {(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
    const i32x8 b = {(int)xa[0], (int)xa[1], (int)xa[2], (int)xa[3], (int)xb[0], (int)xb[1], (int)xb[2], (int)xb[3]};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 0, 0, (int)ws, 0, (int)xs);
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
    // the wave index as a scalar, so the fills' LDS destinations stay in
    // scalar registers
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lc = lane & 31,
              h = lane >> 5;
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

    // lane (lc, h), element i: h column hcol + 8 (i / 4) + 4h + i % 4, token
    // column 32 b + lc.  The wave's 32 columns are one MX block of h along I,
    // half in each lane half.  h ~ q0 2^e0 + q1 2^e1 + q2 2^e2: term t holds
    // the e4m3 codes of the remainder r_t (r_0 = h, r_t+1 = r_t - q_t 2^e_t,
    // exact in fp32) under the e8m0 scale e_t.  e0 is the least power of two
    // that puts the block's largest |h| at or below 448; a remainder is at
    // most half an e4m3 step of the term before (16 at the top, [256, 448)
    // binade), so e_t = e0 - 4t keeps term 1's codes at or below 256 and term
    // 2's at or below 128 (no code saturates; clamped at e8m0's -127, the
    // codes only shrink).  hbuf bytes: term t's codes [P][I] from t * plane, then
    // scale slots [P][I/64][16] from 3 plane; byte 4 b2 + t of a slot is term
    // t's scale for block b2 (0, 1) of the 64-column step.
    const size_t hcol = (size_t)t.rb * 256 + 32 * wave;
    const size_t plane = (size_t)(hlo - hhi);
    uint8_t *hq = reinterpret_cast<uint8_t *>(hhi);
    uint8_t *hs = hq + 3 * plane;
#pragma unroll
    for (int b = 0; b < T5; ++b) {
        const int c = 32 * b + lc;
        float r[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) r[i] = silu_rcp(acc[0][b][i]) * acc[1][b][i];
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(r[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 32));   // the block's other 16 columns
        const int e0 = e8m0_for(amax);
        uint32_t q[3][4], sc = 0;
#pragma unroll
        for (int tm = 0; tm < 3; ++tm) {
            const int e = e0 - 4 * tm < -127 ? -127 : e0 - 4 * tm;
            const float inv = ldexpf(1.f, -e), sv = ldexpf(1.f, e);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                q[tm][j] = e4m3x4(r[4 * j] * inv, r[4 * j + 1] * inv, r[4 * j + 2] * inv, r[4 * j + 3] * inv);
                if (tm < 2) {   // codes times 2^e, two per convert (low, high half)
                    const f32x2 d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q[tm][j], sv, false);
                    const f32x2 d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(q[tm][j], sv, true);
                    r[4 * j] -= d0[0];
                    r[4 * j + 1] -= d0[1];
                    r[4 * j + 2] -= d1[0];
                    r[4 * j + 3] -= d1[1];
                }
            }
            sc |= (uint32_t)(e + 127) << (8 * tm);
        }
        if (c < t.nt) {
            const size_t row = (size_t)(t.q0 + c);
#pragma unroll
            for (int tm = 0; tm < 3; ++tm)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<uint32_t *>(hq + tm * plane + row * I + hcol + 8 * j + 4 * h) = q[tm][j];
            if (h == 0)
                *reinterpret_cast<uint32_t *>(hs + (row * (I / 64) + hcol / 64) * 16 + 4 * (wave & 1)) = sc;
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
// down: K step 64.  Lane half h holds K [32h, 32h+32) of the step (MX block
// h) of its W2 row as stored (16 code bytes, one scale byte); each of h's
// three e4m3 terms enters one scaled fp4 x fp8 MFMA per column tile.
// Stage: h tile (a row holds, for the step's 64 K, term t's codes in chunks
// 4t..4t+3 and the scale slot in chunk 12; chunks 13..15 are not filled) |
// W2 codes [512 rows][32 B] | scales [512 rows][4 B]
// (the aligned dword holding the step's two scale bytes and those of its pair
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
    // the wave index as a scalar, so the fills' LDS destinations stay in
    // scalar registers
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lc = lane & 31,
              h = lane >> 5;
    const BlobLayout L = BlobLayout::make(H, I);
    const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(t.base, (uint32_t)L.bytes);
    const uint32_t orow0 = (uint32_t)t.rb * 512;
    // h rows 4 (w T5 + j) .. +3.  hbuf bytes: term t's codes [P][I] from t *
    // plane, scale slots [P][I/64][16] from 3 plane.  A fill's step offset is
    // 64 nx for the codes, 16 nx for the scale slot (xsl: one bit per fill).
    // Chunks 13..15 take an offset past the buffer's end (kNoFill + at most
    // 16 I / 64 < 2^32), where a buffer load reads nothing and returns zeros:
    // no branch in the K loop.
    constexpr uint32_t kNoFill = 0x80000000u;
    uint32_t xsrc[T5], xsl = 0;
#pragma unroll
    for (int j = 0; j < T5; ++j) {
        const int c = 4 * (wave * T5 + j) + (lane >> 4), chunk = (lane & 15) ^ (c & 15);
        const uint32_t row = (uint32_t)(t.q0 + (c < t.nt ? c : 0));
        if (chunk < 12) {
            xsrc[j] = (uint32_t)(chunk >> 2) * plane + row * (uint32_t)I + (chunk & 3) * 16;
        } else {
            xsrc[j] = chunk == 12 ? 3 * plane + row * (uint32_t)(I / 4) : kNoFill;
            xsl |= 1u << j;
        }
    }
    uint32_t wsrc[2];
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
    // token row lc (column tile b adds 32 rows): term t's bytes [16h, 16h+16)
    // and [32+16h, 32+16h+16) of the step are chunks 4t + 2q + h (q = 0, 1),
    // in slot ((4t + 2q) ^ (lc & 14)) + (h ^ (lc & 1)); the three scale bytes
    // of block h are the dword at byte 4h of chunk 12.  Two registers give
    // the six offsets (made opaque per step, so they are not hoisted).
    const int xbase = lc * 256 + 16 * (h ^ (lc & 1)), xx = lc & 14;
    const int soff = lc * 256 + 16 * (12 ^ (lc & 15)) + 4 * h;

    auto fill = [&](uint8_t *st, int nx) {
#pragma unroll
        for (int j = 0; j < T5; ++j)
            lds_fill<16>(hrs, xsrc[j] + ((uint32_t)nx << (((xsl >> j) & 1u) ? 4 : 6)), st + (wave * T5 + j) * 1024);
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
        uint32_t ws[2], xs[T5];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            wc[f] = lds_ld<u32x4>(cur + wro[f]);
            ws[f] = lds_ld<uint8_t>(cur + sro[f] + 2 * (sc & 1));
        }
#pragma unroll
        for (int b = 0; b < T5; ++b) xs[b] = lds_ld<uint32_t>(cur + soff + b * 32 * 256);
        // units (t, b) = (u / T5, u % T5): two reads of term t, two MFMAs
        constexpr int U = 3 * T5;
        int xxs = xx;
        asm volatile("" : "+v"(xxs));
        u32x4 bx[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                bx[u][q] = lds_ld<u32x4>(cur + xbase + 16 * ((4 * (u / T5) + 2 * q) ^ xxs) + (u % T5) * 32 * 256);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tm = u / T5, b = u % T5;
            const uint32_t s = (xs[b] >> (8 * tm)) & 0xffu;
#pragma unroll
            for (int f = 0; f < 2; ++f) acc[f][b] = mfma_f4_f8(wc[f], bx[u][0], bx[u][1], ws[f], s, acc[f][b]);
        }
        pipeline_order<U, T5 + 3, 4 + T5, 2, 2>();
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

// hbuf: h as the gate/up GEMM stores it (three planes of P * I = `plane`
// e4m3 codes, then the scale slots); 4 * plane < 2^31 bytes.
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
