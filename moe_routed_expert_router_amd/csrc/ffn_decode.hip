// Grouped SwiGLU expert FFN and weighted combine.
//
// The gracetier write-up (section 1) runs every picked expert in one call,
// as though all of them were resident in HBM: a blob-address table from the
// grouping points each distinct expert at its HBM home or its scratch slot,
// and the kernels never look at residency again, so an all-hot run and a
// mixed hot/cold run execute identical instructions on identical bytes.
//
// At decode an expert sees a handful of tokens and the work is a bandwidth-
// bound grouped GEMV over MXFP4 weights.  It still runs on the matrix cores:
// a wave owns 16 weight rows; per 128-element K step a lane loads one 16-byte
// run of 32 codes (exactly one MX block) and that row's block scale (the
// tiled blob layout makes the wave's 16 rows of one step a contiguous 1 KB,
// read with streaming loads), turns the
// codes into exact bf16 with the gfx950 scaled fp4 converts, and feeds 16x16x32
// bf16 MFMAs whose other operand holds up to 16 tokens.  The K order inside a
// step is permuted identically in both operands (lane group g takes block
// 4s+g), so every MFMA is an exact partial dot product.  The converts are the
// only per-element vector work (about a fifth of the issue slots at the HBM
// rate), and 1 to 16 tokens per expert cost the same.
//
// Decode kernels (T <= 32), one 512-thread block per (row block, expert):
//   gate/up: 8 waves = {gate, up} x RT row tiles x K slices (RT = 1 below 12
//            tokens, 2 from 12 tokens on, so that one staging of the token
//            rows serves twice the weight rows); each wave issues all of its
//            slice's weight loads at once, before the token rows (memory-
//            level parallelism comes from many small independent waves, not
//            deep per-wave pipelines);
//            tokens are staged once per block in LDS; the slice partials are
//            added in a fixed order in LDS; h = silu(g) * u is stored as bf16
//            hi + lo parts (h - hi rounded again), ~16 significant bits.
//   down:    8 waves = RT row tiles x K slices (RT = 2 below 8 tokens, else
//            4 with the first h units requested ahead of the weights), B = h
//            hi and h lo of up to 8 token rows as the 16 columns of one MFMA,
//            y[pair][row] in fp32.
// The block shapes depend only on T and the layer shape, never on where the
// experts live, so all-resident and mixed runs still add in the same order.
//   down + combine (T*k <= 8, one decode token): one block per 16-row tile
//            runs every distinct expert, keeps the pairs' outputs in LDS and
//            writes out[t] itself — no y round trip, no combine launch; an
//            expert's h hi and h lo rows sit in different columns of one
//            MFMA (at most 8 pairs each), so one MFMA per K chunk, not two.
// General kernels (any T): one wave per 16 rows.
// Otherwise the combine kernel follows: out[t] = sum_j w[t,j] * y[t*k+j] in j
// order, no float atomics.  (Folding the combine into a down kernel whose
// blocks each hold one expert needs a last-arriver counter and an
// agent-scope release per block, which on this GPU writes the XCD's L2 back
// each time and costs more than the launch it saves.)
#include "kernels.hpp"
#include "select.hpp"

namespace moe {

namespace {

__device__ __forceinline__ uint2 pack_bf16x4(const uint32_t v[4]) {
    return make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
}

__device__ __forceinline__ void split_store_h(const f32x4 &g, const f32x4 &u, uint16_t *hi_dst, uint16_t *lo_dst) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float h = silu(g[i]) * u[i];
        hi[i] = f32_to_bf16_bits(h);
        lo[i] = f32_to_bf16_bits(h - __uint_as_float(hi[i] << 16));
    }
    *reinterpret_cast<uint2 *>(hi_dst) = pack_bf16x4(hi);
    *reinterpret_cast<uint2 *>(lo_dst) = pack_bf16x4(lo);
}

}  // namespace

// ============================ decode block kernels ==========================
constexpr int kStageBytes = 49152;   // LDS budget for staged tokens / h rows (3 blocks per CU)
constexpr int kStageBytesWide = 67584;   // two-tile gate/up blocks (2 per CU by registers): 8 rows of H = 4096
constexpr int kWideTokens = 8;       // tokens from which down blocks take more weight rows
// Tokens from which gate/up blocks take two row tiles (two blocks per CU by
// registers) instead of one (three per CU).  Measured per batch-size (FFN
// alone, Zipf routing): one tile is 3% faster at 8 tokens, even at 12, and
// two are 3-10% faster from 16 to 32.
constexpr int kGateUpWideTokens = 12;
constexpr int kDmaRows = 8;          // first-pass token rows staged by LDS DMA
constexpr int kFusedCombineTokens = 16;   // tokens below which the down blocks combine

// The distinct expert of this block for an FFN part (kPartAll / Hot / Cold)
// and its blob address, pair count and run start; false when the block has
// none.  Every distinct expert belongs to exactly one of the hot and cold
// parts, so the hot and cold launches together equal one kPartAll launch.
// All reads are issued in one round (each round trip to what the grouping
// just wrote costs about a microsecond); only the cold part needs a second,
// through its list of picked cold experts.
struct PartExpert {
    const uint8_t *base;
    int n, q0;
};
__device__ __forceinline__ bool part_expert(const GroupView &gv, int part, PartExpert &pe) {
    const int b = blockIdx.y;   // < grid rows <= min(E, T*k): every read below is in bounds
    const int nu0 = gv.nuniq[0], nu1 = gv.nuniq[1], cold_b = gv.ucold[b];
    uint64_t ptr = gv.uptr[b];
    int n = gv.ucnt[b], q0 = gv.uoff[b];
    // use every value at one point, so the compiler cannot sink a load into
    // the branch that needs it and chain the round trips
    asm volatile("" ::"s"(nu0), "s"(nu1), "s"(cold_b), "s"(n), "s"(q0), "s"((uint32_t)ptr),
                 "s"((uint32_t)(ptr >> 32)));
    if (part == kPartCold) {
        if (b >= nu1) return false;
        const int u = gv.cu[b];
        ptr = gv.uptr[u];
        n = gv.ucnt[u];
        q0 = gv.uoff[u];
    } else if (b >= nu0 || (part == kPartHot && cold_b)) {
        return false;
    }
    pe.base = reinterpret_cast<const uint8_t *>(ptr);
    pe.n = n;
    pe.q0 = q0;
    return true;
}

// ---------------------------- weighted combine ------------------------------
// out[t] = sum over the token's valid picks j, in pick order, of w[t][j] *
// y[t*k+j] (the output of the token's j-th pair), accumulated in fp32.  Picks
// with an id outside [0, E) are skipped.
struct CombineOut {
    const int32_t *ids;
    const float *w;
    int T, k, E, out_bf16;
    void *out;
    int fuse;   // the down blocks combine (else a combine launch follows them)
};

// y stores and loads that are coherent across the XCDs' L2s (device scope):
// the combine of a row tile reads pairs written by blocks on other XCDs.
__device__ __forceinline__ void store4_dev(float *p, float4 v) {
    uint64_t *q = reinterpret_cast<uint64_t *>(p);
    const uint64_t lo = (uint64_t)__float_as_uint(v.x) | ((uint64_t)__float_as_uint(v.y) << 32);
    const uint64_t hi = (uint64_t)__float_as_uint(v.z) | ((uint64_t)__float_as_uint(v.w) << 32);
    __hip_atomic_store(q, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 load4_dev(const float *p) {
    const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float4(__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                       __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32)));
}

// Combined columns [4*c4, 4*c4 + 4) of token t.  The ids, weights and y
// columns of up to 8 picks are loaded together with no branch between them
// (picks past k re-read pick k-1, and an invalid pick's row, never written,
// is read and dropped), so one wait covers them all; the sums are added in
// pick order.
template <bool kDev>
__device__ __forceinline__ float4 combine4(const float *__restrict__ y, const CombineOut &co, int H, int t,
                                           int c4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < co.k; j0 += 8) {
        float4 v[8];
        float wv[8];
        int id[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const size_t q = (size_t)t * co.k + (j0 + u < co.k ? j0 + u : co.k - 1);
            id[u] = co.ids[q];
            wv[u] = co.w[q];
            const float *src = y + q * H + 4 * (size_t)c4;
            v[u] = kDev ? load4_dev(src) : *reinterpret_cast<const float4 *>(src);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u >= co.k || id[u] < 0 || id[u] >= co.E) continue;
            acc.x += wv[u] * v[u].x;
            acc.y += wv[u] * v[u].y;
            acc.z += wv[u] * v[u].z;
            acc.w += wv[u] * v[u].w;
        }
    }
    return acc;
}

__device__ __forceinline__ void store_out4(const CombineOut &co, int H, int t, int c4, float4 acc) {
    if (co.out_bf16) {
        const uint32_t b[4] = {f32_to_bf16_bits(acc.x), f32_to_bf16_bits(acc.y), f32_to_bf16_bits(acc.z),
                               f32_to_bf16_bits(acc.w)};
        reinterpret_cast<uint2 *>(static_cast<uint16_t *>(co.out) + (size_t)t * H)[c4] = pack_bf16x4(b);
    } else {
        reinterpret_cast<float4 *>(static_cast<float *>(co.out) + (size_t)t * H)[c4] = acc;
    }
}

// Output rows [row0, row0 + nrows) of every token, by the whole block.
__device__ __forceinline__ void combine_rows(const float *__restrict__ y, const CombineOut &co, int H, int row0,
                                             int nrows) {
    const int per_t = nrows / 4;
    for (int i = threadIdx.x; i < co.T * per_t; i += blockDim.x) {
        const int t = i / per_t, c4 = row0 / 4 + i % per_t;
        store_out4(co, H, t, c4, combine4<true>(y, co, H, t, c4));
    }
}

// Called by every thread of a down block once its y stores are issued (with
// store4_dev): counts the block in its row tile's counter and, in the block
// that completes the tile (one per distinct expert), combines the tile.  Each
// thread waits for its own stores to be acknowledged at device scope before
// the block counts itself, so the last block sees every pair's rows.  `flag`:
// one int of LDS that no thread reads any more.
__device__ __forceinline__ void arrive_combine(const GroupView &gv, const CombineOut &co, const float *y, int H,
                                               int row0, int nrows, int *flag) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const int done = __hip_atomic_fetch_add(gv.sync + blockIdx.x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = done == gv.nuniq[0] - 1;
    }
    __syncthreads();
    if (*flag) combine_rows(y, co, H, row0, nrows);
}

// RT 16-row tiles of one expert in the decode gate/up: the expert's blob at
// `base`, its n pairs starting at grouped position q0, pair_of(c) the pair id
// of its c-th pair.  Waves: {gate, up} x RT tiles x K slices.  LDS: NT rows of
// x (staged once for all RT tiles) and the per-wave partial sums.
template <int SPW, typename PairOf>
__device__ __forceinline__ void gate_up_tile_blk(const uint16_t *__restrict__ x, int H, int I, int k, int NT,
                                                 int RT, const uint8_t *base, int n, int q0, PairOf pair_of, char *smem,
                                                 uint16_t *__restrict__ hhi, uint16_t *__restrict__ hlo) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int nw = blockDim.x >> 6;
    const int role = wave & 1;   // role 0: gate rows, 1: up rows
    const int rt = (wave >> 1) % RT, slice = (wave >> 1) / RT;
    const int col0 = blockIdx.x * 16 * RT + rt * 16;   // first h column of this wave's tile
    const BlobLayout L = BlobLayout::make(H, I);
    const size_t row = (size_t)role * I + col0 + r, nst = H / 128;
    const uint8_t *qp = base + L.w13_codes + tiled_code_row(row, nst) + (size_t)slice * SPW * kCodeStep + 16 * g;
    const uint8_t *sp = base + L.w13_scales + tiled_scale_row(row, nst) + (size_t)slice * SPW * kScaleStep;

    // LDS rows in 16-byte units, padded by one unit: conflict-free token reads
    const int nch = H / 8, stride = nch + 1;
    uint4 *xs = reinterpret_cast<uint4 *>(smem);
    f32x4 *red = reinterpret_cast<f32x4 *>(smem + (size_t)NT * stride * 16);

    // Weights first: every weight load of this wave's slice goes out as soon
    // as the expert is known, preceded only by the read of the first pass's
    // pair ids (the oldest load, so using them waits for no weight).  The
    // token rows then go to LDS by DMA (one 1 KB fill per wave and row, no
    // registers held); the vector memory counter retires in issue order, so
    // the MFMAs start once the fills, and with them every weight, are in.
    // Against fills first and weights after, this sends the weights one
    // round trip (the pair ids) earlier.
    const bool dma = nch % 64 == 0 && nch / 64 <= nw;
    const int ndma = (n < NT ? n : NT) < kDmaRows ? (n < NT ? n : NT) : kDmaRows;
    uint4 q[SPW];
    uint32_t sc[SPW];
    int my_tok = 0;   // lane c < ndma: pair id of token row c
    if (dma && wave < nch / 64) my_tok = pair_of(lane < ndma ? lane : ndma - 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < SPW; ++i) q[i] = gload16_nt(qp + (size_t)i * kCodeStep);
#pragma unroll
    for (int i = 0; i < SPW; ++i) sc[i] = gload_nt<uint32_t>(sp + (size_t)i * kScaleStep);
    __builtin_amdgcn_sched_barrier(0);
    if (dma && wave < nch / 64) {
        const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(x, 0xFFFFFFF0u);
        my_tok /= k;
#pragma unroll
        for (int c = 0; c < kDmaRows; ++c)
            if (c < ndma) {
                const int tok = __builtin_amdgcn_readlane(my_tok, c);
                lds_fill<16>(xrs, (uint32_t)((size_t)tok * H + (wave * 64 + lane) * 8) * 2u,
                             reinterpret_cast<uint8_t *>(xs + c * stride) + wave * 1024);
            }
    }
    __builtin_amdgcn_sched_barrier(0);

    for (int tb = 0; tb < n; tb += NT) {
        const int nt = (n - tb) < NT ? (n - tb) : NT;
        if (tb == 0 && dma) {
            for (int c = ndma; c < nt; ++c) {   // rows past kDmaRows (small H only): copied
                const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)(pair_of(c) / k) * H);
                for (int j = tid; j < nch; j += blockDim.x) xs[c * stride + j] = src[j];
            }
            fill_barrier<0>();   // fills and weights
        } else {
            __syncthreads();
            for (int c = 0; c < nt; ++c) {
                const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)(pair_of(tb + c) / k) * H);
                for (int j = tid; j < nch; j += blockDim.x) xs[c * stride + j] = src[j];
            }
            __syncthreads();
        }
        // MFMA output columns are independent, so a lane whose token column is
        // empty reads row 0 and its column is never stored: no masked reads
        const bool tv = r < nt;   // this lane's token column
        const uint4 *xr = xs + (tv ? r : 0) * stride + slice * SPW * 16 + 4 * g;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            // the scale is read here, at its step (its load was issued last;
            // a convert hoisted above the fill barrier would wait for it)
            uint32_t scv = sc[i];
            asm volatile("" : "+v"(scv));
            float s = e8m0_to_f32((scv >> (8 * g)) & 0xffu);
            // converted weights are loop-invariant across token passes; keep
            // the converts at their step instead of holding 4x the registers
            asm volatile("" : "+v"(s));
            const uint32_t w4[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                acc = mfma16x16x32(fp4x8_to_bf16x8(w4[m], s), as_bf16x8(xr[i * 16 + m]), acc);
            }
            // one step's operands live at a time (keeps three blocks per CU)
            __builtin_amdgcn_sched_barrier(0);
        }
        red[wave * 64 + lane] = acc;
        __syncthreads();
        if (role == 0 && slice == 0) {   // the tile's gate wave adds its slices in a fixed order
            f32x4 gs = red[wave * 64 + lane], us = red[(wave + 1) * 64 + lane];
            for (int w = wave + 2 * RT; w < nw; w += 2 * RT) {
                gs += red[w * 64 + lane];
                us += red[(w + 1) * 64 + lane];
            }
            if (tv) {
                const size_t off = (size_t)(q0 + tb + r) * I + col0 + 4 * g;
                split_store_h(gs, us, hhi + off, hlo + off);
            }
        }
    }
}

// grid (I/(16*RT), max distinct experts of the part), 128 * RT * slices threads.
template <int SPW>
__global__ __launch_bounds__(512) void ffn_gate_up_blk(const uint16_t *__restrict__ x, int H, int I, int k,
                                                       int NT, int RT, GroupView gv, int part, uint16_t *__restrict__ hhi,
                                                       uint16_t *__restrict__ hlo) {
    extern __shared__ __align__(16) char smem[];
    PartExpert pe;
    if (!part_expert(gv, part, pe) || pe.base == nullptr) return;
    const int q0 = pe.q0;
    gate_up_tile_blk<SPW>(x, H, I, k, NT, RT, pe.base, pe.n, q0, [&](int c) { return gv.plist[q0 + c]; }, smem,
                          hhi, hlo);
}

// The same with the top-k and grouping recomputed in every block (no cold
// expert, T*k <= kFusedSelectPairs): block (0, 0) publishes ids, w and the
// pick set for the down and combine kernels; block (., u) works on distinct
// expert u.  grid (I/(16*RT), min(E, T*k)), 128 * RT * slices threads.
template <int SPW, int NPL>
__global__ __launch_bounds__(512) void ffn_gate_up_sel(const uint16_t *__restrict__ x, int H, int I, int k, int NT,
                                                       int RT, SelectArgs sa, GroupOut o, int hot_only,
                                                       uint16_t *__restrict__ hhi, uint16_t *__restrict__ hlo) {
    extern __shared__ __align__(16) char smem[];
    __shared__ int sid[kFusedSelectPairs], sflag[kFusedSelectPairs], spl[kSmallRouteTokens], sinfo[4];
    // the residency table borrows the start of the token staging area, which
    // the selection is done with before any token row arrives
    select_group_block<NPL>(sa, o, blockIdx.x == 0 && blockIdx.y == 0, blockIdx.y,
                            SelectLds{sid, sflag, spl, sinfo, reinterpret_cast<int *>(smem)});
    const int n = sinfo[0];
    const uint8_t *base = reinterpret_cast<const uint8_t *>(((uint64_t)(uint32_t)sinfo[3] << 32) | (uint32_t)sinfo[2]);
    if (n == 0 || base == nullptr) return;
    // hot_only: an expert read from a scratch slot is left to the cold part
    if (hot_only && base >= sa.scratch && base < sa.scratch + (size_t)sa.n_cold * sa.blob_bytes) return;
    gate_up_tile_blk<SPW>(x, H, I, k, NT, RT, base, n, sinfo[1], [&](int c) { return spl[c]; }, smem, hhi, hlo);
}

// grid (H/(16*RT), max distinct experts of the part), 64 * RT * slices
// threads: RT row tiles of 16 rows x slices of K.  LDS: NT rows of h hi and
// lo and the per-wave partial sums.
// Up to 8 steps per wave, registers are held to 80 per lane (six waves per
// SIMD): with the LDS of 5 staged rows that is three blocks per CU instead of
// the two that 81 registers allowed (with the shared hi / lo MFMA, the
// batch-32 down went from 76 to 68 us).
// With co.fuse, the block that completes a row tile (the last of the distinct
// experts, over the hot and cold launches together) also writes the tile's
// combined output rows, so no combine launch follows.
template <int SPW, int RT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(SPW <= 8 ? 6 : 4))) void ffn_down_blk(int H, int I, int NT, GroupView gv, int part,
                                                    const uint16_t *__restrict__ hhi,
                                                    const uint16_t *__restrict__ hlo, float *__restrict__ y,
                                                    CombineOut co) {
    extern __shared__ __align__(16) char smem[];
    const int row0 = blockIdx.x * (16 * RT);
    PartExpert pe;
    if (!part_expert(gv, part, pe)) {
        // no valid pick at all: no block arrives below, so the first row of
        // blocks writes the (zero) output
        if (co.fuse && blockIdx.y == 0 && gv.nuniq[0] == 0) combine_rows(y, co, H, row0, 16 * RT);
        return;
    }
    const uint8_t *base = pe.base;
    const int n = pe.n, q0 = pe.q0;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int nw = blockDim.x >> 6;
    const int rt = wave % RT, slice = wave / RT;
    const BlobLayout L = BlobLayout::make(H, I);

    if (base == nullptr) {   // unusable residency entry: its pairs contribute zero
        for (int i = tid; i < n * 4 * RT; i += blockDim.x) {
            const int p = gv.plist[q0 + i / (4 * RT)];
            float *dst = y + (size_t)p * H + row0 + 4 * (i % (4 * RT));
            if (co.fuse)
                store4_dev(dst, make_float4(0.f, 0.f, 0.f, 0.f));
            else
                *reinterpret_cast<float4 *>(dst) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (co.fuse) arrive_combine(gv, co, y, H, row0, 16 * RT, reinterpret_cast<int *>(smem));
        return;
    }
    const size_t row = (size_t)row0 + rt * 16 + r, nst = I / 128;
    const uint8_t *qp = base + L.w2_codes + tiled_code_row(row, nst) + (size_t)slice * SPW * kCodeStep + 16 * g;
    const uint8_t *sp = base + L.w2_scales + tiled_scale_row(row, nst) + (size_t)slice * SPW * kScaleStep;
    const int nch = I / 8, stride = nch + 1;   // 16-byte units per row; LDS rows padded
    uint4 *hs = reinterpret_cast<uint4 *>(smem);
    uint4 *ls = hs + (size_t)NT * stride;
    f32x4 *red = reinterpret_cast<f32x4 *>(smem + (size_t)2 * NT * stride * 16);

    // The first pass's h rows (contiguous in grouped order, hi and lo
    // planes) go to LDS by DMA ahead of the weight loads, as in the gate/up
    // tile: one 1 KB fill per wave and chunk, no registers held, and the
    // fills' wait leaves the weights in flight.
    const int ncp = nch / 64;   // 1 KB chunks per row and plane
    const bool dma = nch % 64 == 0;
    const int ndma = n < NT ? n : NT;
    if (dma) {
        const __amdgpu_buffer_rsrc_t hrs = buffer_rsrc(hhi, 0xFFFFFFF0u);
        const uint32_t lo_off = (uint32_t)((hlo - hhi) * 2);   // the lo plane, in bytes past hhi
        for (int ch = wave; ch < 2 * ncp; ch += nw) {
            const int pl = ch / ncp, cc = ch % ncp;
            for (int c = 0; c < ndma; ++c)
                lds_fill<16>(hrs, (pl ? lo_off : 0u) + (uint32_t)(((size_t)(q0 + c) * I + (cc * 64 + lane) * 8) * 2),
                             reinterpret_cast<uint8_t *>((pl ? ls : hs) + c * stride) + cc * 1024);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    uint4 q[SPW];   // codes, then scales (the fills' wait counts both as outstanding)
#pragma unroll
    for (int i = 0; i < SPW; ++i) q[i] = gload16_nt(qp + (size_t)i * kCodeStep);
    uint32_t sc[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) sc[i] = gload_nt<uint32_t>(sp + (size_t)i * kScaleStep);
    __builtin_amdgcn_sched_barrier(0);

    for (int tb = 0; tb < n; tb += NT) {
        const int nt = (n - tb) < NT ? (n - tb) : NT;
        if (tb == 0 && dma) {
            fill_barrier<SPW + (SPW + 3) / 4>();
        } else {   // copied (later passes of experts with more than NT tokens)
            __syncthreads();
            const int total = nt * nch;
            const uint4 *sh = reinterpret_cast<const uint4 *>(hhi + (size_t)(q0 + tb) * I);
            const uint4 *sl = reinterpret_cast<const uint4 *>(hlo + (size_t)(q0 + tb) * I);
            for (int i0 = tid; i0 < total; i0 += 2 * blockDim.x) {
                const int i1 = i0 + (int)blockDim.x < total ? i0 + (int)blockDim.x : i0;
                const uint4 a = sh[i0], b = sl[i0], c = sh[i1], d = sl[i1];
                const int o0 = (i0 / nch) * stride + i0 % nch, o1 = (i1 / nch) * stride + i1 % nch;
                hs[o0] = a;
                ls[o0] = b;
                hs[o1] = c;
                ls[o1] = d;
            }
            __syncthreads();
        }
        const bool tv = r < nt;
        // nt <= 8: column c < nt takes row c's h hi, column nt + c its h lo,
        // so each K chunk is one MFMA (the other columns read row 0 and are
        // never used)
        const int pr = tv ? r : (r < 2 * nt ? r - nt : 0);
        const uint4 *hp = (tv ? hs : ls) + pr * stride + slice * SPW * 16 + 4 * g;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            uint32_t scv = sc[i];   // read at its step (the scales were issued last)
            asm volatile("" : "+v"(scv));
            float s = e8m0_to_f32((scv >> (8 * g)) & 0xffu);
            asm volatile("" : "+v"(s));   // keep the converts at their step
            const uint32_t w4[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) acc = mfma16x16x32(fp4x8_to_bf16x8(w4[m], s), as_bf16x8(hp[i * 16 + m]), acc);
            __builtin_amdgcn_sched_barrier(0);
        }
        red[wave * 64 + lane] = acc;
        __syncthreads();
        if (wave < RT && tv) {   // wave rt adds its row tile's slices in a fixed order, hi then lo
            f32x4 sh = red[wave * 64 + lane], sl = red[wave * 64 + lane + nt];
            for (int w2 = wave + RT; w2 < nw; w2 += RT) {
                sh += red[w2 * 64 + lane];
                sl += red[w2 * 64 + lane + nt];
            }
            const f32x4 s = sh + sl;
            const int p = gv.plist[q0 + tb + r];
            float *dst = y + (size_t)p * H + row0 + wave * 16 + 4 * g;
            if (co.fuse)
                store4_dev(dst, make_float4(s[0], s[1], s[2], s[3]));
            else
                *reinterpret_cast<float4 *>(dst) = make_float4(s[0], s[1], s[2], s[3]);
        }
    }
    if (co.fuse) arrive_combine(gv, co, y, H, row0, 16 * RT, reinterpret_cast<int *>(smem));
}

// ====================== down + combine for a few pairs =======================
constexpr int kDcMaxPairs = 8;   // pairs (T*k) up to which down and combine run as one kernel
constexpr int kDcHUnits = 4;     // h units (16 B) per thread and plane requested ahead of the weights
constexpr size_t kMaxLdsBytes = 160 * 1024;   // LDS per workgroup on gfx950

// Down projection and weighted combine for at most kDcMaxPairs pairs (one
// decode token): one block per 16-row tile runs every distinct expert of the
// batch, with all their weight loads in flight together, keeps the pairs'
// outputs for its 16 rows in LDS and writes out[t][rows] itself, adding the
// k picks of each token in j order.  This saves the combine launch and the
// y round trip through HBM.  grid H/16; 64 * slices threads (K slices of
// SPW steps).  LDS: the h hi and lo rows of every grouped pair, the
// (expert, wave) partial sums and the grouped position of each pair.
template <int SPW, int P>
__global__ __launch_bounds__(512) void ffn_down_combine(int H, int I, int T, int k, int E, GroupView gv,
                                                        const uint16_t *__restrict__ hhi,
                                                        const uint16_t *__restrict__ hlo,
                                                        const int32_t *__restrict__ ids, const float *__restrict__ w,
                                                        int out_bf16, void *__restrict__ out) {
    // P == T * k: one expert slot per pair (at most P distinct experts)
    static_assert(P <= 8, "an expert's hi and lo columns must fit one 16-column MFMA");
    extern __shared__ __align__(16) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int nw = blockDim.x >> 6, bd = blockDim.x;
    const int row0 = blockIdx.x * 16;
    const int nch = I / 8, stride = nch + 1, total = P * nch;
    const BlobLayout L = BlobLayout::make(H, I);

    // One round of reads of what the grouping published, none waiting for
    // another (each round trip to data the previous kernel wrote costs about
    // a microsecond): the distinct count, every slot's run start and blob
    // address (slots past the count hold stale values and are masked below),
    // the pairs' ids, weights and grouped order, and the h rows of all P
    // grouped positions (rows past the valid pairs feed only output columns
    // that are never read).  Per-pair values by unconditional clamped vector
    // loads: a value loaded under a branch gets consumed inside it, which
    // would wait for it at once.
    const int U = gv.nuniq[0];
    int uo_raw[P + 1];
    uint64_t up_raw[P];
#pragma unroll
    for (int u = 0; u <= P; ++u) uo_raw[u] = gv.uoff[u < E ? u : E];
#pragma unroll
    for (int u = 0; u < P; ++u) up_raw[u] = gv.uptr[u < E ? u : E - 1];
    const int tp = tid < P ? tid : P - 1;
    const int m_id = ids[tp];
    const float m_w = w[tp];
    const int m_pl = gv.plist[tp];
    const u32x4 *sh = reinterpret_cast<const u32x4 *>(hhi);
    const u32x4 *sl = reinterpret_cast<const u32x4 *>(hlo);
    u32x4 ph[kDcHUnits], pl[kDcHUnits];
#pragma unroll
    for (int v = 0; v < kDcHUnits; ++v) {
        const int i = tid + v * bd;
        const int ic = i < total ? i : total - 1;
        ph[v] = sh[ic];
        pl[v] = sl[ic];
    }
    int nq = 0;   // grouped (valid) pairs
#pragma unroll
    for (int u = 0; u <= P; ++u)
        if (u == U) nq = uo_raw[u];
    int uo[P + 1];
    uint32_t okmask = 0;   // bit u: slot u is a distinct expert with a usable blob
#pragma unroll
    for (int u = 0; u <= P; ++u) uo[u] = u <= U ? uo_raw[u] : nq;
#pragma unroll
    for (int u = 0; u < P; ++u)
        if (u < U && up_raw[u] != 0) okmask |= 1u << u;

    // every slot loads unconditionally (a masked slot gets a zero-size
    // resource whose reads return 0), so the compiler knows how many loads
    // are in flight at every wait; scales before codes
    const uint32_t row = (uint32_t)(row0 + r);
    const size_t nst = I / 128;
    const uint32_t soff = (uint32_t)(L.w2_scales + tiled_scale_row(row, nst) + (size_t)wave * SPW * kScaleStep);
    const uint32_t qoff = (uint32_t)(L.w2_codes + tiled_code_row(row, nst) + (size_t)wave * SPW * kCodeStep + 16 * g);
    __amdgpu_buffer_rsrc_t rs[P];
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const bool ok = (okmask >> u) & 1u;
        rs[u] = buffer_rsrc(ok ? reinterpret_cast<const void *>(up_raw[u]) : nullptr, ok ? (uint32_t)L.bytes : 0u);
    }
    uint32_t sc[P][SPW];
    u32x4 q[P][SPW];
#pragma unroll
    for (int u = 0; u < P; ++u)
#pragma unroll
        for (int i = 0; i < SPW; ++i) sc[u][i] = __builtin_amdgcn_raw_buffer_load_b32(rs[u], soff + (uint32_t)kScaleStep * i, 0, kLoadNT);
#pragma unroll
    for (int u = 0; u < P; ++u)
#pragma unroll
        for (int i = 0; i < SPW; ++i)
            q[u][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs[u], qoff + (uint32_t)kCodeStep * i, 0, kLoadNT));
    __builtin_amdgcn_sched_barrier(0);

    uint4 *hs = reinterpret_cast<uint4 *>(smem);
    uint4 *ls = hs + (size_t)P * stride;
    f32x4 *red = reinterpret_cast<f32x4 *>(ls + (size_t)P * stride);   // [P][nw][64]
    int *pu = reinterpret_cast<int *>(red + (size_t)P * nw * 64);      // [P] slot of pair p (-1: none)
    int *pc = pu + P;                                                   // [P] its column in that slot's run
    int *pn = pc + P;                                                   // [P] that slot's pair count
    float *sw = reinterpret_cast<float *>(pn + P);                      // [P] weights (0: invalid id)
    float *ys = sw + P;                                                 // [P][16] pair outputs of the rows
#pragma unroll
    for (int v = 0; v < kDcHUnits; ++v) {   // clamped units rewrite their own bytes
        const int i = tid + v * bd;
        const int ic = i < total ? i : total - 1;
        const int o = (ic / nch) * stride + ic % nch;
        reinterpret_cast<u32x4 *>(hs)[o] = ph[v];
        reinterpret_cast<u32x4 *>(ls)[o] = pl[v];
    }
    for (int i = tid + kDcHUnits * bd; i < total; i += bd) {
        const int o = (i / nch) * stride + i % nch;
        hs[o] = reinterpret_cast<const uint4 *>(hhi)[i];
        ls[o] = reinterpret_cast<const uint4 *>(hlo)[i];
    }
    if (tid < P) {
        pu[tid] = -1;
        sw[tid] = (m_id >= 0 && m_id < E) ? m_w : 0.f;
    }
    __syncthreads();
    if (tid < nq) {   // grouped position tid holds pair m_pl of run u
        int u = 0, start = uo[0], end = uo[1];
#pragma unroll
        for (int v = 1; v < P; ++v)
            if (uo[v] <= tid && v < U) {
                u = v;
                start = uo[v];
                end = uo[v + 1];
            }
        pu[m_pl] = u;
        pc[m_pl] = tid - start;
        pn[m_pl] = end - start;
    }

    // Every slot computes, branch-free (a masked slot multiplies zeros and
    // its sums are never read): per-slot branches let the compiler merge the
    // slots' bodies, and the merged body waits for all weights at once.
    // A slot has n <= P <= 8 pairs, so its h hi and h lo rows share one MFMA:
    // column c < n takes pair c's hi part, column n + c its lo part (the
    // columns are independent; the rest read row 0 and are never used), and
    // the two columns' sums are added after the K slices.
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int n = uo[u + 1] - uo[u];
        const bool hic = r < n;
        const int pr = hic ? r : (r < 2 * n ? r - n : 0);
        const uint4 *hp = (hic ? hs : ls) + (n > 0 ? uo[u] + pr : 0) * stride + wave * SPW * 16 + 4 * g;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            float s = e8m0_to_f32((sc[u][i] >> (8 * g)) & 0xffu);
            asm volatile("" : "+v"(s));
#pragma unroll
            for (int m = 0; m < 4; ++m)
                acc = mfma16x16x32(fp4x8_to_bf16x8(q[u][i][m], s), as_bf16x8(hp[i * 16 + m]), acc);
        }
        red[(u * nw + wave) * 64 + lane] = acc;
    }
    __syncthreads();

    // y of pair p for row rr: its slot's K-slice partials of the hi column,
    // then of the lo column, each in slice order (an invalid id or an
    // unusable residency entry gives 0)
    for (int idx = tid; idx < P * 16; idx += bd) {
        const int p = idx >> 4, rr = idx & 15, u = pu[p];
        float y = 0.f;
        if (u >= 0 && ((okmask >> u) & 1u)) {
            const int ln = pc[p] + 16 * (rr >> 2), ll = ln + pn[p];
            float yh = 0.f, yl = 0.f;
            for (int s2 = 0; s2 < nw; ++s2) {
                yh += red[(u * nw + s2) * 64 + ln][rr & 3];
                yl += red[(u * nw + s2) * 64 + ll][rr & 3];
            }
            y = yh + yl;
        }
        ys[idx] = y;
    }
    __syncthreads();
    // out[t][row0 + rr]: the k picks of token t added in j order
    for (int idx = tid; idx < T * 16; idx += bd) {
        const int t = idx >> 4, rr = idx & 15;
        float acc = 0.f;
        for (int j = 0; j < k; ++j) acc += sw[t * k + j] * ys[(t * k + j) * 16 + rr];
        if (out_bf16)
            static_cast<uint16_t *>(out)[(size_t)t * H + row0 + rr] = (uint16_t)f32_to_bf16_bits(acc);
        else
            static_cast<float *>(out)[(size_t)t * H + row0 + rr] = acc;
    }
}

// ========================= general one-wave kernels =========================
template <int D>
struct GateUpStage {
    uint4 gq[D], uq[D];      // 32 codes of a gate row / an up row per step
    uint32_t gs[D], us[D];   // the four block scales of that step
    uint4 xb[D][4];          // token operand: 4 x 8 bf16 per step
};

template <int D>
__device__ __forceinline__ void gate_up_load(GateUpStage<D> &st, const uint8_t *gq, const uint8_t *uq,
                                             const uint8_t *gs, const uint8_t *us, const uint16_t *xr,
                                             bool tv, int s0) {
    const uint4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const int s = s0 + d;
        st.gq[d] = *reinterpret_cast<const uint4 *>(gq + (size_t)s * kCodeStep);
        st.uq[d] = *reinterpret_cast<const uint4 *>(uq + (size_t)s * kCodeStep);
        st.gs[d] = *reinterpret_cast<const uint32_t *>(gs + (size_t)s * kScaleStep);
        st.us[d] = *reinterpret_cast<const uint32_t *>(us + (size_t)s * kScaleStep);
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
__global__ __launch_bounds__(64) void ffn_gate_up_wave(const uint16_t *__restrict__ x, int H, int I, int k,
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
    const size_t nst = H / 128;
    const uint8_t *gq = base + L.w13_codes + tiled_code_row(row, nst) + 16 * g;
    const uint8_t *uq = base + L.w13_codes + tiled_code_row((size_t)I + row, nst) + 16 * g;
    const uint8_t *gs = base + L.w13_scales + tiled_scale_row(row, nst);
    const uint8_t *us = base + L.w13_scales + tiled_scale_row((size_t)I + row, nst);
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
            const size_t off = (size_t)(q0 + tb + r) * I + (size_t)blockIdx.x * 16 + 4 * g;
            split_store_h(ag, au, hhi + off, hlo + off);
        }
    }
}

template <int D>
struct DownStage {
    uint4 wq[D];
    uint32_t ws[D];
    uint4 hh[D][4], hl[D][4];
};

template <int D>
__device__ __forceinline__ void down_load(DownStage<D> &st, const uint8_t *wq, const uint8_t *ws,
                                          const uint16_t *hh, const uint16_t *hl, bool tv, int s0) {
    const uint4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const int s = s0 + d;
        st.wq[d] = *reinterpret_cast<const uint4 *>(wq + (size_t)s * kCodeStep);
        st.ws[d] = *reinterpret_cast<const uint32_t *>(ws + (size_t)s * kScaleStep);
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
__global__ __launch_bounds__(64) void ffn_down_wave(int H, int I, GroupView gv, const uint16_t *__restrict__ hhi,
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
    const size_t nst = I / 128;
    const uint8_t *wq = base + L.w2_codes + tiled_code_row(row, nst) + 16 * g;
    const uint8_t *ws = base + L.w2_scales + tiled_scale_row(row, nst);
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

__global__ __launch_bounds__(256) void ffn_combine(const float *__restrict__ y, CombineOut co, int H) {
    const int c4 = blockIdx.x * blockDim.x + threadIdx.x;
    if (c4 * 4 >= H) return;
    for (int t = blockIdx.y; t < co.T; t += gridDim.y) store_out4(co, H, t, c4, combine4<false>(y, co, H, t, c4));
}

// ================================ launchers =================================
namespace {

// Whether the decode down blocks combine (the block completing a row tile
// adds it up) rather than a combine launch following them.  Each block then
// waits for its y stores and a counter round trip before it ends: measured
// (FFN alone, Zipf routing), 8 tokens 72.2 against 73.9 us; 16, 24 and 32
// tokens 114.2, 147.9 and 174.1 against 113.1, 145.8 and 171.4 us (with
// thousands of blocks the tails cost more than the launch).
bool down_combines(int T) { return T < kFusedCombineTokens; }

size_t down_combine_lds(int T, int k, int H, int I);

// Completion counter words the down blocks of a decode FFN use (one per row
// tile of at least 32 rows), 0 when they do not combine.
int down_counter_words(const FfnArgs &a) {
    return !down_combine_lds(a.T, a.k, a.H, a.I) && down_combines(a.T) ? a.H / 32 : 0;
}

CombineOut combine_out(const FfnArgs &a) {
    CombineOut c;
    c.ids = a.ids;
    c.w = a.w;
    c.T = a.T;
    c.k = a.k;
    c.E = a.E;
    c.out_bf16 = a.out_bf16;
    c.out = a.out;
    c.fuse = down_combines(a.T);
    return c;
}

// Smallest steps-per-wave in {1,2,4,8,16} dividing `steps` with at most
// max_slices slices; 0 if none.
int pick_spw(int steps, int max_slices) {
    for (int spw = 1; spw <= 16; spw *= 2)
        if (steps % spw == 0 && steps / spw <= max_slices) return spw;
    return 0;
}

// Profiling name of a launch of one FFN part.
const char *part_name(int part, const char *all, const char *hot, const char *cold) {
    return part == kPartHot ? hot : part == kPartCold ? cold : all;
}

int stage_rows(int bytes_per_row, int budget = kStageBytes) {
    const int nt = budget / bytes_per_row;
    return nt < 1 ? 1 : (nt > 16 ? 16 : nt);
}

// Gate/up block shape, a function of T and H only (an all-resident and a
// mixed run of one batch then add in the same order): from kGateUpWideTokens
// tokens two row tiles share a block, one staging of the token rows for twice
// the weight rows.
struct GateUpShape {
    int rt, spw, slices;
};
GateUpShape gate_up_shape(int T, int H) {
    const int steps = H / 128;
    GateUpShape g;
    g.rt = (T >= kGateUpWideTokens && pick_spw(steps, 2) != 0) ? 2 : 1;
    g.spw = pick_spw(steps, 4 / g.rt);
    g.slices = g.spw ? steps / g.spw : 0;
    return g;
}

template <int SPW>
void launch_gate_up_blk(const FfnArgs &a, const GroupView &gv, int part, int RT, uint16_t *hhi, uint16_t *hlo,
                        int umax, hipStream_t st) {
    const int slices = a.H / 128 / SPW;
    const int row_bytes = (a.H / 8 + 1) * 16;
    const int NT = stage_rows(row_bytes, RT == 2 ? kStageBytesWide : kStageBytes);
    const size_t lds = (size_t)NT * row_bytes + (size_t)2 * RT * slices * 64 * 16;
    MOE_LAUNCH(part_name(part, "ffn_gate_up_blk", "ffn_gate_up_blk_hot", "ffn_gate_up_blk_cold"),
               ffn_gate_up_blk<SPW>, dim3(a.I / (16 * RT), umax), dim3(128 * RT * slices), lds, st, a.x, a.H, a.I,
               a.k, NT, RT, gv, part, hhi, hlo);
}

template <int SPW, int RT>
void launch_down_blk(const FfnArgs &a, const GroupView &gv, int part, const uint16_t *hhi, const uint16_t *hlo,
                     float *y, int umax, hipStream_t st) {
    const int slices = a.I / 128 / SPW;
    const int row_bytes = (a.I / 8 + 1) * 16;
    // measured: more rows (fewer blocks per CU) is slower here; at most 8, so
    // that a pass's h hi and lo rows fit the 16 columns of one MFMA
    const int NT = stage_rows(2 * row_bytes) < 8 ? stage_rows(2 * row_bytes) : 8;
    const size_t lds = (size_t)2 * NT * row_bytes + (size_t)RT * slices * 64 * 16;
    MOE_LAUNCH(part_name(part, "ffn_down_blk", "ffn_down_blk_hot", "ffn_down_blk_cold"),
               (ffn_down_blk<SPW, RT>), dim3(a.H / (16 * RT), umax), dim3(64 * RT * slices), lds, st, a.H,
               a.I, NT, gv, part, hhi, hlo, y, combine_out(a));
}

void gate_up_blk(const FfnArgs &a, const GroupView &gv, int part, uint16_t *hhi, uint16_t *hlo, int umax,
                 hipStream_t st) {
    const GateUpShape g = gate_up_shape(a.T, a.H);
    switch (g.spw) {
        case 1: launch_gate_up_blk<1>(a, gv, part, g.rt, hhi, hlo, umax, st); break;
        case 2: launch_gate_up_blk<2>(a, gv, part, g.rt, hhi, hlo, umax, st); break;
        case 4: launch_gate_up_blk<4>(a, gv, part, g.rt, hhi, hlo, umax, st); break;
        case 8: launch_gate_up_blk<8>(a, gv, part, g.rt, hhi, hlo, umax, st); break;
        default: launch_gate_up_blk<16>(a, gv, part, g.rt, hhi, hlo, umax, st); break;
    }
}

template <int RT>
void down_blk_rt(int spw, const FfnArgs &a, const GroupView &gv, int part, const uint16_t *hhi,
                 const uint16_t *hlo, float *y, int umax, hipStream_t st) {
    switch (spw) {
        case 1: launch_down_blk<1, RT>(a, gv, part, hhi, hlo, y, umax, st); break;
        case 2: launch_down_blk<2, RT>(a, gv, part, hhi, hlo, y, umax, st); break;
        case 4: launch_down_blk<4, RT>(a, gv, part, hhi, hlo, y, umax, st); break;
        case 8: launch_down_blk<8, RT>(a, gv, part, hhi, hlo, y, umax, st); break;
        default: launch_down_blk<16, RT>(a, gv, part, hhi, hlo, y, umax, st); break;
    }
}

// Down kernel shape.  More rows per block share one staging of the h rows,
// which pays once experts see several tokens; with about one token per
// expert, twice as many smaller blocks keep more loads in flight.
void down_blk(const FfnArgs &a, const GroupView &gv, int part, const uint16_t *hhi, const uint16_t *hlo,
              float *y, int umax, hipStream_t st) {
    const int steps = a.I / 128;
    const bool wide = a.T >= kWideTokens && a.H % 64 == 0 && pick_spw(steps, 2) != 0;
    if (wide)
        down_blk_rt<4>(pick_spw(steps, 2), a, gv, part, hhi, hlo, y, umax, st);
    else
        down_blk_rt<2>(pick_spw(steps, 4), a, gv, part, hhi, hlo, y, umax, st);
}

// LDS bytes of ffn_down_combine, or 0 when the shape does not qualify.
size_t down_combine_lds(int T, int k, int H, int I) {
    const int P = T * k, spw = pick_spw(I / 128, 8);
    if (P > kDcMaxPairs || H % 16 != 0 || spw == 0) return 0;
    const int slices = I / 128 / spw;
    const size_t lds = (size_t)2 * P * (I / 8 + 1) * 16 + (size_t)P * slices * 64 * 16 + (size_t)(4 + 16) * P * 4;
    return lds <= kMaxLdsBytes ? lds : 0;
}

template <int SPW, int UMAX>
void launch_down_combine_u(const FfnArgs &a, const GroupView &gv, const uint16_t *hhi, const uint16_t *hlo,
                           size_t lds, hipStream_t st) {
    const int slices = a.I / 128 / SPW;
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&ffn_down_combine<SPW, UMAX>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    MOE_LAUNCH("ffn_down_combine", (ffn_down_combine<SPW, UMAX>), dim3(a.H / 16), dim3(64 * slices), lds, st,
               a.H, a.I, a.T, a.k, a.E, gv, hhi, hlo, a.ids, a.w, a.out_bf16, a.out);
}

template <int SPW>
void launch_down_combine_spw(const FfnArgs &a, const GroupView &gv, const uint16_t *hhi, const uint16_t *hlo,
                             size_t lds, hipStream_t st) {
    switch (a.T * a.k) {   // the expert slots: exactly the pairs
        case 1: launch_down_combine_u<SPW, 1>(a, gv, hhi, hlo, lds, st); break;
        case 2: launch_down_combine_u<SPW, 2>(a, gv, hhi, hlo, lds, st); break;
        case 3: launch_down_combine_u<SPW, 3>(a, gv, hhi, hlo, lds, st); break;
        case 4: launch_down_combine_u<SPW, 4>(a, gv, hhi, hlo, lds, st); break;
        case 5: launch_down_combine_u<SPW, 5>(a, gv, hhi, hlo, lds, st); break;
        case 6: launch_down_combine_u<SPW, 6>(a, gv, hhi, hlo, lds, st); break;
        case 7: launch_down_combine_u<SPW, 7>(a, gv, hhi, hlo, lds, st); break;
        default: launch_down_combine_u<SPW, 8>(a, gv, hhi, hlo, lds, st); break;
    }
}

void launch_down_combine(const FfnArgs &a, const GroupView &gv, const uint16_t *hhi, const uint16_t *hlo,
                         hipStream_t st) {
    const size_t lds = down_combine_lds(a.T, a.k, a.H, a.I);
    switch (pick_spw(a.I / 128, 8)) {
        case 1: launch_down_combine_spw<1>(a, gv, hhi, hlo, lds, st); break;
        case 2: launch_down_combine_spw<2>(a, gv, hhi, hlo, lds, st); break;
        case 4: launch_down_combine_spw<4>(a, gv, hhi, hlo, lds, st); break;
        case 8: launch_down_combine_spw<8>(a, gv, hhi, hlo, lds, st); break;
        default: launch_down_combine_spw<16>(a, gv, hhi, hlo, lds, st); break;
    }
}

void launch_combine(const FfnArgs &a, const float *y, hipStream_t st) {
    const int n4 = a.H / 4;
    const int ty = a.T < 65535 ? a.T : 65535;
    MOE_LAUNCH("ffn_combine", ffn_combine, dim3((n4 + 255) / 256, ty), dim3(256), 0, st, y, combine_out(a), a.H);
}

}  // namespace

template <int SPW, int NPL>
void launch_gate_up_sel(const FfnArgs &a, int RT, const SelectArgs &sa, const GroupOut &o, int hot_only,
                        uint16_t *hhi, uint16_t *hlo, int umax, hipStream_t st) {
    const int slices = a.H / 128 / SPW;
    const int row_bytes = (a.H / 8 + 1) * 16;
    const int NT = stage_rows(row_bytes, RT == 2 ? kStageBytesWide : kStageBytes);
    const size_t lds = (size_t)NT * row_bytes + (size_t)2 * RT * slices * 64 * 16;
    MOE_LAUNCH("ffn_gate_up_sel", (ffn_gate_up_sel<SPW, NPL>), dim3(a.I / (16 * RT), umax),
               dim3(128 * RT * slices), lds, st, a.x, a.H, a.I, a.k, NT, RT, sa, o, hot_only, hhi, hlo);
}

template <int SPW>
void gate_up_sel_npl(int npl, const FfnArgs &a, int RT, const SelectArgs &sa, const GroupOut &o, int hot_only,
                     uint16_t *hhi, uint16_t *hlo, int umax, hipStream_t st) {
    switch (npl) {
        case 1: launch_gate_up_sel<SPW, 1>(a, RT, sa, o, hot_only, hhi, hlo, umax, st); break;
        case 2: launch_gate_up_sel<SPW, 2>(a, RT, sa, o, hot_only, hhi, hlo, umax, st); break;
        case 4: launch_gate_up_sel<SPW, 4>(a, RT, sa, o, hot_only, hhi, hlo, umax, st); break;
        case 8: launch_gate_up_sel<SPW, 8>(a, RT, sa, o, hot_only, hhi, hlo, umax, st); break;
        default: launch_gate_up_sel<SPW, 16>(a, RT, sa, o, hot_only, hhi, hlo, umax, st); break;
    }
}

// The gate/up launch with the selection in every block, for every expert or
// (hot_only) the HBM-resident ones.
static void gate_up_sel(const FfnArgs &a, const SelectArgs &sa, const GroupOut &o, int hot_only, uint16_t *hhi,
                 uint16_t *hlo, int umax, hipStream_t st) {
    const int npl = topk_npl(a.E);
    const GateUpShape gs = gate_up_shape(a.T, a.H);
    switch (gs.spw) {
        case 1: gate_up_sel_npl<1>(npl, a, gs.rt, sa, o, hot_only, hhi, hlo, umax, st); break;
        case 2: gate_up_sel_npl<2>(npl, a, gs.rt, sa, o, hot_only, hhi, hlo, umax, st); break;
        case 4: gate_up_sel_npl<4>(npl, a, gs.rt, sa, o, hot_only, hhi, hlo, umax, st); break;
        case 8: gate_up_sel_npl<8>(npl, a, gs.rt, sa, o, hot_only, hhi, hlo, umax, st); break;
        default: gate_up_sel_npl<16>(npl, a, gs.rt, sa, o, hot_only, hhi, hlo, umax, st); break;
    }
}

bool ffn_select_fusable(int T, int k, int E, int H, int I) {
    if (!ffn_block_path(T, H, I)) return false;
    const GateUpShape g = gate_up_shape(T, H);
    const int P = T * k, threads = 128 * g.rt * g.slices;
    // the block selection takes one pair per thread and two residency
    // entries per thread
    return P <= kFusedSelectMaxPairs && P <= threads && E <= 2 * threads;
}

bool ffn_block_path(int T, int H, int I) {
    return T <= 32 && pick_spw(H / 128, 4) != 0 && pick_spw(I / 128, 4) != 0;
}

hipError_t launch_ffn(const FfnArgs &a, char *ws, const WsLayout &L, hipStream_t st) {
    const GroupView gv = group_view(ws, L);
    const size_t P = (size_t)a.T * a.k;
    const int umax = (int)((size_t)a.E < P ? (size_t)a.E : P);
    uint16_t *hhi = reinterpret_cast<uint16_t *>(ws + L.hbuf);
    uint16_t *hlo = hhi + P * (size_t)a.I;
    float *y = reinterpret_cast<float *>(ws + L.ybuf);

    if (ffn_gemm_path(a.T, a.H, a.I, a.k)) {
        const hipError_t e = launch_ffn_gemm(a, gv, WsLayout::max_tiles(a.E, P), hhi, hlo, y, st);
        if (e != hipSuccess) return e;
    } else if (ffn_block_path(a.T, a.H, a.I)) {
        gate_up_blk(a, gv, kPartAll, hhi, hlo, umax, st);
        if (down_combine_lds(a.T, a.k, a.H, a.I)) {
            launch_down_combine(a, gv, hhi, hlo, st);
            return hipGetLastError();
        }
        down_blk(a, gv, kPartAll, hhi, hlo, y, umax, st);
        if (down_combines(a.T)) return hipGetLastError();
    } else {
        const int sgu = a.H / 128;
        const dim3 ggu(a.I / 16, umax);
        if (sgu % 4 == 0)
            MOE_LAUNCH("ffn_gate_up_wave", ffn_gate_up_wave<4>, ggu, dim3(64), 0, st, a.x, a.H, a.I, a.k, gv, hhi,
                       hlo);
        else if (sgu % 2 == 0)
            MOE_LAUNCH("ffn_gate_up_wave", ffn_gate_up_wave<2>, ggu, dim3(64), 0, st, a.x, a.H, a.I, a.k, gv, hhi,
                       hlo);
        else
            MOE_LAUNCH("ffn_gate_up_wave", ffn_gate_up_wave<1>, ggu, dim3(64), 0, st, a.x, a.H, a.I, a.k, gv, hhi,
                       hlo);
        const int sd = a.I / 128;
        const dim3 gd(a.H / 16, umax);
        if (sd % 2 == 0)
            MOE_LAUNCH("ffn_down_wave", ffn_down_wave<2>, gd, dim3(64), 0, st, a.H, a.I, gv, hhi, hlo, y);
        else
            MOE_LAUNCH("ffn_down_wave", ffn_down_wave<1>, gd, dim3(64), 0, st, a.H, a.I, gv, hhi, hlo, y);
    }

    launch_combine(a, y, st);
    return hipGetLastError();
}

hipError_t launch_ffn_select(const FfnArgs &a, const float *z, int renorm, int32_t *ids, float *w,
                             const GroupArgs &g, char *ws, const WsLayout &L, hipStream_t st) {
    const GroupView gv = group_view(ws, L);
    const GroupOut o = GroupOut::at(ws, L);
    SelectArgs sa = select_args(z, a.T, a.k, renorm, ids, w, g);
    sa.nsync = down_counter_words(a);
    const size_t P = (size_t)a.T * a.k;
    const int umax = (int)((size_t)a.E < P ? (size_t)a.E : P);
    uint16_t *hhi = reinterpret_cast<uint16_t *>(ws + L.hbuf);
    uint16_t *hlo = hhi + P * (size_t)a.I;
    float *y = reinterpret_cast<float *>(ws + L.ybuf);
    gate_up_sel(a, sa, o, 0, hhi, hlo, umax, st);
    if (down_combine_lds(a.T, a.k, a.H, a.I)) {
        launch_down_combine(a, gv, hhi, hlo, st);
    } else {
        down_blk(a, gv, kPartAll, hhi, hlo, y, umax, st);
        if (!down_combines(a.T)) launch_combine(a, y, st);
    }
    return hipGetLastError();
}

hipError_t launch_ffn_select_hot(const FfnArgs &a, const float *z, int renorm, int32_t *ids, float *w,
                                 const GroupArgs &g, char *ws, const WsLayout &L, hipStream_t st) {
    const GroupView gv = group_view(ws, L);
    const GroupOut o = GroupOut::at(ws, L);
    SelectArgs sa = select_args(z, a.T, a.k, renorm, ids, w, g);
    sa.nsync = down_counter_words(a);
    const size_t P = (size_t)a.T * a.k;
    const int umax = (int)((size_t)a.E < P ? (size_t)a.E : P);
    uint16_t *hhi = reinterpret_cast<uint16_t *>(ws + L.hbuf);
    uint16_t *hlo = hhi + P * (size_t)a.I;
    float *y = reinterpret_cast<float *>(ws + L.ybuf);
    gate_up_sel(a, sa, o, 1, hhi, hlo, umax, st);
    if (!down_combine_lds(a.T, a.k, a.H, a.I)) down_blk(a, gv, kPartHot, hhi, hlo, y, umax, st);
    return hipGetLastError();
}

hipError_t launch_ffn_part(const FfnArgs &a, int part, int umax_part, char *ws, const WsLayout &L,
                           hipStream_t st) {
    const GroupView gv = group_view(ws, L);
    const size_t P = (size_t)a.T * a.k;
    uint16_t *hhi = reinterpret_cast<uint16_t *>(ws + L.hbuf);
    uint16_t *hlo = hhi + P * (size_t)a.I;
    float *y = reinterpret_cast<float *>(ws + L.ybuf);
    // with few pairs the down projection runs fused with the combine over
    // every expert after the cold part's gate/up (the same kernel as in the
    // all-resident sequence, so the results stay bit-identical)
    const bool fused = down_combine_lds(a.T, a.k, a.H, a.I) != 0;
    if (umax_part > 0) {
        gate_up_blk(a, gv, part, hhi, hlo, umax_part, st);
        if (!fused) down_blk(a, gv, part, hhi, hlo, y, umax_part, st);
    }
    // below kFusedCombineTokens the down blocks of the two parts combine
    // (without a cold launch, those of the hot part alone cover every
    // distinct expert; the combine launch then only writes the same values
    // again)
    if (part == kPartCold) {
        if (fused)
            launch_down_combine(a, gv, hhi, hlo, st);
        else if (!down_combines(a.T) || umax_part == 0)
            launch_combine(a, y, st);
    }
    return hipGetLastError();
}

}  // namespace moe
