// Measurement aids beside the layer (they compute nothing of it).
//
// Streaming-read probe: the time one launch takes to read N bytes of HBM with
// nothing else to do, the ceiling a bandwidth-bound kernel of that size can
// approach.
//
// Each block reads one contiguous run of 256 * L 16-byte units: thread t
// issues its L loads (units t, t + 256, ...) before using any, so a wave
// instruction covers 1 KB contiguous and the whole grid's loads are in
// flight at once.  The loaded words are folded by XOR and stored to sink[0]
// only when the fold equals `key`, a value the compiler cannot know, so the
// loads cannot be dropped; the store (harmless when it happens) is rare.
#include "kernels.hpp"

namespace moe {

constexpr int kProbeThreads = 256;

template <int L>
__global__ __launch_bounds__(kProbeThreads) void probe_read(const u32x4 *__restrict__ src, size_t units,
                                                            uint32_t key, uint32_t *__restrict__ sink) {
    const size_t base = (size_t)blockIdx.x * kProbeThreads * L + threadIdx.x;
    u32x4 v[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const size_t u = base + (size_t)i * kProbeThreads;
        v[i] = u < units ? __builtin_nontemporal_load(src + u) : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    if (x == key) sink[0] = x;
}

hipError_t launch_probe_read(const void *src, size_t bytes, int loads_per_thread, uint32_t *sink,
                             hipStream_t st) {
    const size_t units = bytes / 16;
    const size_t per_block = (size_t)kProbeThreads * loads_per_thread;
    const dim3 g((unsigned)((units + per_block - 1) / per_block)), b(kProbeThreads);
    const u32x4 *s = static_cast<const u32x4 *>(src);
    switch (loads_per_thread) {
        case 1: MOE_LAUNCH("probe_read", probe_read<1>, g, b, 0, st, s, units, 0x5EEDF00Du, sink); break;
        case 2: MOE_LAUNCH("probe_read", probe_read<2>, g, b, 0, st, s, units, 0x5EEDF00Du, sink); break;
        case 4: MOE_LAUNCH("probe_read", probe_read<4>, g, b, 0, st, s, units, 0x5EEDF00Du, sink); break;
        case 8: MOE_LAUNCH("probe_read", probe_read<8>, g, b, 0, st, s, units, 0x5EEDF00Du, sink); break;
        default: MOE_LAUNCH("probe_read", probe_read<16>, g, b, 0, st, s, units, 0x5EEDF00Du, sink); break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Matrix-core rate probe: every wave of a grid that fills the GPU (two
// 4-wave blocks per CU) issues `iters` rounds of four independent MFMAs of
// one kind on register operands, so the kernel time gives the rate that kind
// sustains under a full load (clock included).  Kinds (flops per instruction):
//   0  bf16 32x32x16                        (32768)
//   1  scaled f8f6f4 32x32x64, fp8 x fp4    (131072)
//   2  scaled f8f6f4 32x32x64, fp8 x fp8    (131072)
//   3  scaled f8f6f4 32x32x64, fp6 x fp4    (131072; fp6 = e2m3)
//   4  scaled f8f6f4 32x32x64, fp4 x fp4    (131072)
// The scaled forms take an e8m0 scale per operand row and 32 K (here 127,
// i.e. 1.0).  The accumulators are folded and stored to sink[0] only when
// the fold equals `key`, so no MFMA can be dropped.
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

template <int KIND>
__global__ __launch_bounds__(256) void probe_mfma(int iters, uint32_t key, uint32_t *__restrict__ sink) {
    const uint32_t l = threadIdx.x;
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
    if constexpr (KIND == 0) {
        bf16x8 a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (__bf16)(0.001f * (float)((l + i) & 7));
            b[i] = (__bf16)(0.001f * (float)((l * 3 + i) & 7));
        }
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = mfma32x32x16(a, b, acc[j]);
    } else {
        // small codes in every format (a few low mantissa / exponent bits)
        i32x8 a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (int32_t)(0x11111111u * ((l + i) & 3));
            b[i] = (int32_t)(0x11111111u * ((l + 2 * i) & 3));
        }
        constexpr int fa = KIND == 1 ? 0 : KIND == 2 ? 0 : KIND == 3 ? 2 : 4;
        constexpr int fb = KIND == 2 ? 0 : 4;
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], fa, fb, 0, 127, 0, 127);
    }
    float f = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) f += acc[j][i];
    if (__float_as_uint(f) == key) sink[0] = key;
}

hipError_t launch_probe_mfma(int kind, int iters, int cus, uint32_t *sink, hipStream_t st) {
    const dim3 g(2 * cus), b(256);
    switch (kind) {
        case 0: MOE_LAUNCH("probe_mfma", probe_mfma<0>, g, b, 0, st, iters, 0x5EEDF00Du, sink); break;
        case 1: MOE_LAUNCH("probe_mfma", probe_mfma<1>, g, b, 0, st, iters, 0x5EEDF00Du, sink); break;
        case 2: MOE_LAUNCH("probe_mfma", probe_mfma<2>, g, b, 0, st, iters, 0x5EEDF00Du, sink); break;
        case 3: MOE_LAUNCH("probe_mfma", probe_mfma<3>, g, b, 0, st, iters, 0x5EEDF00Du, sink); break;
        default: MOE_LAUNCH("probe_mfma", probe_mfma<4>, g, b, 0, st, iters, 0x5EEDF00Du, sink); break;
    }
    return hipGetLastError();
}

}  // namespace moe
