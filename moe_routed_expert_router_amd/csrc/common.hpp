// Shared device helpers and the workspace / blob layout of the HIP path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;

// ------------------------------ expert blob --------------------------------
// One contiguous blob per expert (MXFP4, two e2m1 codes per byte, even element
// in the low nibble, one e8m0 scale per 32 elements along the contraction):
//   w13 codes (2I x H) | w13 scales | w2 codes (H x I) | w2 scales
// (w13 rows 0..I-1 gate, I..2I-1 up).  Each plane of R rows and K columns
// (R % 16 == 0, K % 128 == 0, nst = K / 128 steps) is stored in tiles: the
// codes of 16-row group G and step s (64 bytes per row) are one contiguous
// 1 KB chunk at (G nst + s) 1024, row r of the group at 64 r in it; the
// group's scales of that step (4 bytes per row) one 64-byte chunk at
// (G nst + s) 64.  So a wave reading 16 rows x 64 bytes of one step (the
// matrix-core operand layout) reads whole 128-byte lines: with streaming
// loads that lifts the decode FFN from ~0.62 to ~0.70 of 8 TB/s at batch 8
// and 32 against the row-major layout's half lines.
constexpr size_t kCodeStep = 1024;   // bytes between a tiled row's consecutive 128-column steps (codes)
constexpr size_t kScaleStep = 64;    // the same for its scales

// Offset of row `row`'s step-0 codes (add s * kCodeStep + byte) and scales
// (add s * kScaleStep + block) in a tiled plane of nst steps.
__host__ __device__ __forceinline__ size_t tiled_code_row(size_t row, size_t nst) {
    return ((row >> 4) * nst * 16 + (row & 15)) * 64;
}
__host__ __device__ __forceinline__ size_t tiled_scale_row(size_t row, size_t nst) {
    return ((row >> 4) * nst * 16 + (row & 15)) * 4;
}

struct BlobLayout {
    size_t w13_codes, w13_scales, w2_codes, w2_scales, bytes;
    __host__ __device__ static BlobLayout make(int H, int I) {
        BlobLayout b;
        size_t h = (size_t)H, i = (size_t)I;
        b.w13_codes = 0;
        b.w13_scales = b.w13_codes + 2 * i * (h / 2);
        b.w2_codes = b.w13_scales + 2 * i * (h / 32);
        b.w2_scales = b.w2_codes + h * (i / 2);
        b.bytes = b.w2_scales + h * (i / 32);
        return b;
    }
};

// ------------------------------- workspace ---------------------------------
// Regions of the caller's workspace for T tokens (all 256-byte aligned).
struct WsLayout {
    size_t sync;       // int32 [kSyncWords]: FFN completion counters (zeroed by the grouping)
    size_t logits;     // float [T][E]
    size_t status;     // int32 [16]: [0] invalid-pair count, [1] bad-residency count
    size_t nuniq;      // int32 [4]: [0] distinct experts U, [1] picked-cold count, [2] token tiles
    size_t uniq;       // int32 [E]: distinct picked experts, increasing
    size_t ucnt;       // int32 [E]: pairs per distinct expert
    size_t uoff;       // int32 [E+1]: start of each expert's run in plist
    size_t uptr;       // uint64 [E]: blob address of each distinct expert (0: skip)
    size_t cold;       // int32 [E]: picked cold experts, increasing
    size_t ucold;      // int32 [E]: 1 if distinct expert u reads a scratch slot, else 0
    size_t cu;         // int32 [E]: distinct-expert index of each picked cold expert
    size_t counts;     // int32 [E]: pairs per expert id
    size_t hist;       // int32 [nchunks][E+1]: per-chunk counts (+ bad ids), then chunk bases
    size_t rank;       // int32 [P]: rank of a pair among its chunk's pairs of that expert
    size_t plist;      // int32 [P]: pair ids t*k+j grouped by expert, increasing inside
    size_t tlist;      // int32 [max_tiles]: token tiles, distinct-expert index | part << 10
    size_t hbuf;       // uint16 [2][P][I]: SwiGLU output as bf16 hi and lo parts (the prefill GEMMs
                       // keep three planes of e4m3 codes and their scale slots here instead)
    size_t ybuf;       // float [P][H]: per-pair expert outputs
    size_t total;
    int nchunks;

    static constexpr int kChunk = 256;      // pairs per grouping chunk
    static constexpr int kSyncWords = 4096;  // >= H/32 for H <= 65536 (+ spare)
    static constexpr int kPrefillTokens = 160;  // tokens per tile of the grouped GEMM

    // Upper bound on the token tiles of P pairs over E experts.
    static int max_tiles(int E, size_t P) {
        const size_t u = (size_t)E < P ? (size_t)E : P;
        return (int)(u + (P + kPrefillTokens - 1) / kPrefillTokens);
    }

    static size_t up(size_t v) { return (v + 255) & ~(size_t)255; }
    static WsLayout make(int H, int I, int E, int k, int T) {
        WsLayout w;
        size_t P = (size_t)T * k;
        w.nchunks = (int)((P + kChunk - 1) / kChunk);
        size_t o = 0;
        auto take = [&](size_t bytes) { size_t r = o; o += up(bytes > 0 ? bytes : 1); return r; };
        w.sync = take((size_t)kSyncWords * 4);
        w.logits = take((size_t)T * E * 4);
        w.status = take(16 * 4);
        w.nuniq = take(4 * 4);
        w.uniq = take((size_t)E * 4);
        w.ucnt = take((size_t)E * 4);
        w.uoff = take((size_t)(E + 1) * 4);
        w.uptr = take((size_t)E * 8);
        w.cold = take((size_t)E * 4);
        w.ucold = take((size_t)E * 4);
        w.cu = take((size_t)E * 4);
        w.counts = take((size_t)E * 4);
        w.hist = take((size_t)w.nchunks * (E + 1) * 4);
        w.rank = take(P * 4);
        w.plist = take(P * 4);
        w.tlist = take((size_t)max_tiles(E, P) * 4);
        w.hbuf = take(2 * P * (size_t)I * 2);
        w.ybuf = take(P * (size_t)H * 4);
        w.total = o;
        return w;
    }
};

// Device view of the grouped pick set, resolved from a workspace base.
struct GroupView {
    int32_t *sync;          // completion counters, zero on entry to the FFN
    const int32_t *nuniq;   // [0] U, [1] picked-cold count
    const int32_t *uniq;
    const int32_t *ucnt;
    const int32_t *uoff;
    const uint64_t *uptr;
    const int32_t *plist;
    const int32_t *cold;
    const int32_t *ucold;
    const int32_t *cu;
    const int32_t *tlist;
};

// Mutable view of the grouping outputs, for the kernels that write them.
struct GroupOut {
    int32_t *sync, *status, *counts, *nuniq, *uniq, *ucnt, *uoff, *cold, *ucold, *cu, *plist, *tlist;
    uint64_t *uptr;
    static GroupOut at(char *ws, const WsLayout &L) {
        GroupOut o;
        o.sync = reinterpret_cast<int32_t *>(ws + L.sync);
        o.status = reinterpret_cast<int32_t *>(ws + L.status);
        o.counts = reinterpret_cast<int32_t *>(ws + L.counts);
        o.nuniq = reinterpret_cast<int32_t *>(ws + L.nuniq);
        o.uniq = reinterpret_cast<int32_t *>(ws + L.uniq);
        o.ucnt = reinterpret_cast<int32_t *>(ws + L.ucnt);
        o.uoff = reinterpret_cast<int32_t *>(ws + L.uoff);
        o.cold = reinterpret_cast<int32_t *>(ws + L.cold);
        o.ucold = reinterpret_cast<int32_t *>(ws + L.ucold);
        o.cu = reinterpret_cast<int32_t *>(ws + L.cu);
        o.plist = reinterpret_cast<int32_t *>(ws + L.plist);
        o.tlist = reinterpret_cast<int32_t *>(ws + L.tlist);
        o.uptr = reinterpret_cast<uint64_t *>(ws + L.uptr);
        return o;
    }
};

inline GroupView group_view(char *ws, const WsLayout &L) {
    GroupView v;
    v.sync = reinterpret_cast<int32_t *>(ws + L.sync);
    v.nuniq = reinterpret_cast<const int32_t *>(ws + L.nuniq);
    v.uniq = reinterpret_cast<const int32_t *>(ws + L.uniq);
    v.ucnt = reinterpret_cast<const int32_t *>(ws + L.ucnt);
    v.uoff = reinterpret_cast<const int32_t *>(ws + L.uoff);
    v.uptr = reinterpret_cast<const uint64_t *>(ws + L.uptr);
    v.plist = reinterpret_cast<const int32_t *>(ws + L.plist);
    v.cold = reinterpret_cast<const int32_t *>(ws + L.cold);
    v.ucold = reinterpret_cast<const int32_t *>(ws + L.ucold);
    v.cu = reinterpret_cast<const int32_t *>(ws + L.cu);
    v.tlist = reinterpret_cast<const int32_t *>(ws + L.tlist);
    return v;
}

// ------------------------------ numerics -----------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// e8m0 scale byte -> fp32 value 2^(b-127); 0 is the subnormal 2^-127, 255 NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    uint32_t bits = (b == 0u) ? 0x00400000u : ((b == 255u) ? 0x7fc00000u : (b << 23));
    return __uint_as_float(bits);
}

// Eight e2m1 codes (one dword, element 2i in the low nibble of byte i) times a
// scale, as eight bf16 values in element order (exact for normal results).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w, float scale) {
    bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
    bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
    bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
    bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
    bf16x8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// Load through the global address space (blob addresses come from an integer
// table, so the compiler would otherwise emit generic flat loads).
template <typename T>
__device__ __forceinline__ T gload(const void *p) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef const __attribute__((address_space(1))) T gT;
    return *(gT *)(p);   // an address-space cast needs the C form
#else
    return *reinterpret_cast<const T *>(p);   // host pass: never executed
#endif
}

// Streaming (non-temporal) load through the global address space, for
// expert weights, which are read once per launch.
template <typename T>
__device__ __forceinline__ T gload_nt(const void *p) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef const __attribute__((address_space(1))) T gT;
    return __builtin_nontemporal_load((gT *)(p));
#else
    return *reinterpret_cast<const T *>(p);   // host pass: never executed
#endif
}

// Cache-policy argument of the buffer-load builtins for streaming loads.
constexpr int kLoadNT = 2;

// 16 bytes through the global address space (a native vector, so no copy
// constructor takes a generic reference on the way).
__device__ __forceinline__ uint4 gload16(const void *p) {
    const u32x4 v = gload<u32x4>(p);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint4 gload16_nt(const void *p) {
    const u32x4 v = gload_nt<u32x4>(p);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Buffer resource over `bytes` bytes at `base`: reads past the end (all
// reads, for zero bytes) return 0 and touch no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// N (16 or 4) bytes per lane from rsrc + voff into LDS at wave base +
// N * lane.  Buffer (not flat) loads, so pending fills do not force the
// compiler to drain every LDS read before its use.  (Sub-dword sizes would
// still place lanes 4 bytes apart, so they are not used.)
template <int N>
__device__ __forceinline__ void lds_fill(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint8_t *lds_wave_base) {
    static_assert(N == 16 || N == 4, "fill size");
    auto *d = (void __attribute__((address_space(3))) *)lds_wave_base;
    if constexpr (N == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, voff, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 4, voff, 0, 0, 0);
}

// Wait for all of this wave's outstanding global loads (LDS fills included).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// Workgroup barrier for LDS fills issued before N (<= 63) later global loads
// of this wave: wait until at most N of its loads are outstanding (the
// counter retires in issue order, so the fills are done) and its LDS
// operations are done, then meet the other waves.  Unlike __syncthreads
// this does not wait for the N later loads.
template <int N>
__device__ __forceinline__ void fill_barrier() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));   // vmcnt(N) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Workgroup barrier over LDS only: waits for this wave's LDS operations, not
// for its outstanding global loads (no LDS fill may be pending).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt(63): no wait on loads
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16 MFMA.  A lane l: A[l % 32][8 (l / 32) + i]; B lane l:
// B[8 (l / 32) + i][l % 32]; D lane l, element i: D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32].
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float g) {
    return g / (1.0f + __expf(-g));
}

}  // namespace moe
