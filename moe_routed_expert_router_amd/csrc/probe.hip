// Streaming-read probe: the time one launch takes to read N bytes of HBM with
// nothing else to do, the ceiling a bandwidth-bound kernel of that size can
// approach (a measurement aid beside the layer; it computes nothing of it).
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

}  // namespace moe
