// Cold gather: copy the picked cold experts from pinned host memory into
// their HBM scratch slots.  The gracetier write-up (section 1) keeps the 129
// cold experts of a layer in pinned host memory the GPU reads directly and has
// one small kernel per layer copy just the picked ones into their slots; its
// section 3 measures that copy at 2.60 ms of a 10.49 ms decode step.
//
// Here the kernel reads the picked-cold list the grouping left in the
// workspace (no host round trip) and streams each expert's bytes across the
// host link with 128-bit device-initiated loads: every thread keeps two loads
// in flight, a block covers 8 KB contiguous per iteration, and a wave
// instruction covers 1 KB contiguous.  Expert bytes are a multiple of 16.
//
// The grid is small on purpose: 32 blocks keep about 256 KB of host reads in
// flight, which already holds the link at its measured rate (~56 GB/s).  A
// grid eight times larger (2 MB in flight) copied no faster, and a kernel
// running beside it (the hot experts' FFN during a layer's gather) started
// 50-170 us late and ran up to five times slower; at 256 KB it starts within
// about 20 us and runs 10-40% longer than alone.
#include "device_util.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 2;
constexpr int kGatherBlocks = 32;

__global__ __launch_bounds__(kGatherThreads) void gather_cold(const uint8_t *__restrict__ host_cold,
                                                              uint8_t *__restrict__ scratch, size_t blob_bytes,
                                                              const int32_t *__restrict__ slot,
                                                              const int32_t *__restrict__ nuniq,
                                                              const int32_t *__restrict__ cold) {
    const int m = nuniq[1];
    const size_t units = blob_bytes / 16;
    const size_t per_iter = (size_t)kGatherThreads * kGatherUnroll;
    for (int i = 0; i < m; ++i) {
        const int c = -slot[cold[i]] - 1;   // grouping only lists valid cold slots
        const u32x4 *src = reinterpret_cast<const u32x4 *>(host_cold + (size_t)c * blob_bytes);
        u32x4 *dst = reinterpret_cast<u32x4 *>(scratch + (size_t)c * blob_bytes);
        for (size_t base = (size_t)blockIdx.x * per_iter; base < units; base += (size_t)gridDim.x * per_iter) {
            u32x4 v[kGatherUnroll];
#pragma unroll
            for (int j = 0; j < kGatherUnroll; ++j) {
                const size_t u = base + (size_t)j * kGatherThreads + threadIdx.x;
                if (u < units) v[j] = __builtin_nontemporal_load(src + u);
            }
#pragma unroll
            for (int j = 0; j < kGatherUnroll; ++j) {
                const size_t u = base + (size_t)j * kGatherThreads + threadIdx.x;
                if (u < units) dst[u] = v[j];
            }
        }
    }
}

// Decode variant that does not wait for a grouping launch: every block takes
// the top-k of the T tokens from the logits itself (the same wave top-k as
// the FFN kernels, so the same picks), marks the picked experts, lists the
// cold ones in increasing expert order, then copies them as gather_cold does.
// T*k <= kMaxPairsSel; every list index stays below m <= min(E, T*k).
constexpr int kMaxPairsSel = 1024;

template <int NPL>
__global__ __launch_bounds__(kGatherThreads) void gather_cold_sel(const float *__restrict__ z, int T, int E, int k,
                                                                  const int32_t *__restrict__ slot, int n_cold,
                                                                  const uint8_t *__restrict__ host_cold,
                                                                  uint8_t *__restrict__ scratch, size_t blob_bytes) {
    __shared__ uint8_t picked[kMaxExperts];
    __shared__ int32_t list[kMaxPairsSel];
    __shared__ int32_t count;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < E; e += kGatherThreads) picked[e] = 0;
    __syncthreads();
    for (int t = wave; t < T; t += kGatherThreads / 64) {
        int pe;
        float pw;
        topk_wave<NPL>(z + (size_t)t * E, E, k, 1, &pe, &pw);
        if (lane < k) picked[pe] = 1;
    }
    __syncthreads();
    if (wave == 0) {   // picked cold experts in increasing order, by ballots over 64 experts at a time
        int m = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            int c = -1;
            if (e < E && picked[e]) {
                const int sv = slot[e];
                if (sv < 0 && -sv - 1 < n_cold) c = -sv - 1;
            }
            const uint64_t b = __ballot(c >= 0);
            const int before = __popcll(b & ((1ull << lane) - 1ull));
            if (c >= 0) list[m + before] = c;
            m += __popcll(b);
        }
        if (lane == 0) count = m;
    }
    __syncthreads();
    const int m = count;
    const size_t units = blob_bytes / 16;
    const size_t per_iter = (size_t)kGatherThreads * kGatherUnroll;
    for (int i = 0; i < m; ++i) {
        const int c = list[i];
        const u32x4 *src = reinterpret_cast<const u32x4 *>(host_cold + (size_t)c * blob_bytes);
        u32x4 *dst = reinterpret_cast<u32x4 *>(scratch + (size_t)c * blob_bytes);
        for (size_t base = (size_t)blockIdx.x * per_iter; base < units; base += (size_t)gridDim.x * per_iter) {
            u32x4 v[kGatherUnroll];
#pragma unroll
            for (int j = 0; j < kGatherUnroll; ++j) {
                const size_t u = base + (size_t)j * kGatherThreads + threadIdx.x;
                if (u < units) v[j] = __builtin_nontemporal_load(src + u);
            }
#pragma unroll
            for (int j = 0; j < kGatherUnroll; ++j) {
                const size_t u = base + (size_t)j * kGatherThreads + threadIdx.x;
                if (u < units) dst[u] = v[j];
            }
        }
    }
}

hipError_t launch_gather_sel(const float *z, int T, int E, int k, const int32_t *slot, int n_cold,
                             const uint8_t *host_cold, uint8_t *scratch, size_t blob_bytes, hipStream_t st) {
    if (T * k > kMaxPairsSel || E > kMaxExperts) return hipErrorInvalidValue;
    const size_t units = blob_bytes / 16;
    const size_t per_iter = (size_t)kGatherThreads * kGatherUnroll;
    size_t blocks = (units + per_iter - 1) / per_iter;
    if (blocks > kGatherBlocks) blocks = kGatherBlocks;
    const dim3 g((unsigned)blocks), b(kGatherThreads);
    switch (topk_npl(E)) {
        case 1: MOE_LAUNCH("gather_cold", gather_cold_sel<1>, g, b, 0, st, z, T, E, k, slot, n_cold, host_cold, scratch, blob_bytes); break;
        case 2: MOE_LAUNCH("gather_cold", gather_cold_sel<2>, g, b, 0, st, z, T, E, k, slot, n_cold, host_cold, scratch, blob_bytes); break;
        case 4: MOE_LAUNCH("gather_cold", gather_cold_sel<4>, g, b, 0, st, z, T, E, k, slot, n_cold, host_cold, scratch, blob_bytes); break;
        case 8: MOE_LAUNCH("gather_cold", gather_cold_sel<8>, g, b, 0, st, z, T, E, k, slot, n_cold, host_cold, scratch, blob_bytes); break;
        default: MOE_LAUNCH("gather_cold", gather_cold_sel<16>, g, b, 0, st, z, T, E, k, slot, n_cold, host_cold, scratch, blob_bytes); break;
    }
    return hipGetLastError();
}

hipError_t launch_gather(const uint8_t *host_cold, uint8_t *scratch, size_t blob_bytes, const int32_t *slot,
                         const char *ws, const WsLayout &L, hipStream_t st) {
    const size_t units = blob_bytes / 16;
    const size_t per_iter = (size_t)kGatherThreads * kGatherUnroll;
    size_t blocks = (units + per_iter - 1) / per_iter;
    if (blocks > kGatherBlocks) blocks = kGatherBlocks;
    MOE_LAUNCH("gather_cold", gather_cold, dim3((unsigned)blocks), dim3(kGatherThreads), 0, st, host_cold, scratch,
                       blob_bytes, slot, reinterpret_cast<const int32_t *>(ws + L.nuniq),
                       reinterpret_cast<const int32_t *>(ws + L.cold));
    return hipGetLastError();
}

}  // namespace moe
