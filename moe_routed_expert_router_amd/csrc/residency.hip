// Adaptive residency: pick counting, moving experts between the HBM pool and
// the pinned host pool, the byte-audit fingerprint, and the host-side swap
// rule.  The gracetier write-up has a manager swap often-picked experts into
// the hot set between steps and quiet ones out (section 1), gated by a
// hysteresis threshold of 3.0 (section 3), and audits every moved expert
// against a boot-time fingerprint (section 4).
//
// Moves run in four stream-ordered launches, so no kernel waits on another
// block: (0) the promoted expert's bytes host -> its scratch slot (staging),
// (1) the demoted expert's bytes HBM -> the promoted one's host slot,
// (2) the staged bytes -> the demoted one's HBM slot, (3) the residency table
// update.  Copies use 128-bit vector loads and stores only; host memory is
// written through the device mapping with ordinary vector stores.
#include <algorithm>
#include <cmath>
#include <vector>

#include "kernels.hpp"

namespace moe {

// ------------------------------- pick counts --------------------------------
constexpr int kCountThreads = 256;
constexpr int kCountPerThread = 4;

__global__ __launch_bounds__(kCountThreads) void fill_i32(int32_t *__restrict__ p, int n, int32_t v) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
}

// counts[e] += number of pairs with id e: a per-block LDS histogram, then one
// atomic add per non-empty bin.
__global__ __launch_bounds__(kCountThreads) void count_picks(const int32_t *__restrict__ ids, int n_pairs, int E,
                                                            int32_t *__restrict__ counts) {
    __shared__ int32_t hist[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += kCountThreads) hist[e] = 0;
    __syncthreads();
    const int base = blockIdx.x * kCountThreads * kCountPerThread;
#pragma unroll
    for (int j = 0; j < kCountPerThread; ++j) {
        const int p = base + j * kCountThreads + threadIdx.x;
        if (p < n_pairs) {
            const int e = ids[p];
            if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kCountThreads)
        if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

// Up to kCountOneBlock pairs (every decode step): one block counts them all
// and writes (or adds) every bin itself, one launch and no global atomics.
constexpr int kCountOneBlock = 8192;
constexpr int kCountOneThreads = 1024;

__global__ __launch_bounds__(kCountOneThreads) void count_picks_one(const int32_t *__restrict__ ids, int n_pairs,
                                                                    int E, int32_t *__restrict__ counts,
                                                                    int clear) {
    __shared__ int32_t hist[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += kCountOneThreads) hist[e] = 0;
    __syncthreads();
    for (int p = threadIdx.x; p < n_pairs; p += kCountOneThreads) {
        const int e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kCountOneThreads) counts[e] = (clear ? 0 : counts[e]) + hist[e];
}

hipError_t launch_count_picks(const int32_t *ids, int n_pairs, int E, int32_t *counts, bool clear, hipStream_t st) {
    if (n_pairs <= kCountOneBlock) {
        MOE_LAUNCH("count_picks_one", count_picks_one, dim3(1), dim3(kCountOneThreads), 0, st, ids, n_pairs, E,
                   counts, clear ? 1 : 0);
        return hipGetLastError();
    }
    if (clear) MOE_LAUNCH("fill_i32", fill_i32, dim3((E + kCountThreads - 1) / kCountThreads), dim3(kCountThreads),
                          0, st, counts, E, 0);
    if (n_pairs > 0) {
        const int per = kCountThreads * kCountPerThread;
        MOE_LAUNCH("count_picks", count_picks, dim3((n_pairs + per - 1) / per), dim3(kCountThreads), 0, st, ids,
                   n_pairs, E, counts);
    }
    return hipGetLastError();
}

// ---------------------------------- moves -----------------------------------
constexpr int kMoveThreads = 256;
constexpr int kMoveUnroll = 2;

struct MoveArgs {
    const int32_t *slot;   // read by phases 0-2, written by phase 3
    int32_t *slot_w;
    uint8_t *hot_base;
    uint8_t *host_cold;
    uint8_t *scratch;
    size_t blob_bytes;
    int E, n_hot, n_cold;
};

// Pre-swap homes of pair p, or false when the table does not describe a
// (cold, hot) pair there (then every phase leaves the pair alone).
__device__ __forceinline__ bool pair_homes(const MoveArgs &a, const SwapList &l, int p, int &ci, int &hi) {
    const int c = l.cold[p], h = l.hot[p];
    if (c < 0 || c >= a.E || h < 0 || h >= a.E) return false;
    const int sc = a.slot[c], sh = a.slot[h];
    ci = -sc - 1;
    hi = sh;
    return sc < 0 && ci < a.n_cold && sh >= 0 && sh < a.n_hot;
}

__global__ __launch_bounds__(kMoveThreads) void residency_move(MoveArgs a, SwapList l, int phase) {
    const int p = blockIdx.y;
    int ci, hi;
    if (!pair_homes(a, l, p, ci, hi)) return;
    const u32x4 *src;
    u32x4 *dst;
    const size_t B = a.blob_bytes;
    if (phase == 0) {          // promoted expert: host slot -> its scratch slot
        src = reinterpret_cast<const u32x4 *>(a.host_cold + (size_t)ci * B);
        dst = reinterpret_cast<u32x4 *>(a.scratch + (size_t)ci * B);
    } else if (phase == 1) {   // demoted expert: HBM slot -> the freed host slot
        src = reinterpret_cast<const u32x4 *>(a.hot_base + (size_t)hi * B);
        dst = reinterpret_cast<u32x4 *>(a.host_cold + (size_t)ci * B);
    } else {                   // staged promoted expert -> the freed HBM slot
        src = reinterpret_cast<const u32x4 *>(a.scratch + (size_t)ci * B);
        dst = reinterpret_cast<u32x4 *>(a.hot_base + (size_t)hi * B);
    }
    const size_t units = B / 16;
    const size_t per_iter = (size_t)kMoveThreads * kMoveUnroll;
    for (size_t base = (size_t)blockIdx.x * per_iter; base < units; base += (size_t)gridDim.x * per_iter) {
        u32x4 v[kMoveUnroll];
#pragma unroll
        for (int j = 0; j < kMoveUnroll; ++j) {
            const size_t u = base + (size_t)j * kMoveThreads + threadIdx.x;
            if (u < units) v[j] = __builtin_nontemporal_load(src + u);
        }
#pragma unroll
        for (int j = 0; j < kMoveUnroll; ++j) {
            const size_t u = base + (size_t)j * kMoveThreads + threadIdx.x;
            if (u < units) dst[u] = v[j];
        }
    }
}

// One thread per pair; pairs name distinct experts, so no two threads touch
// the same entry.
__global__ void residency_move_table(MoveArgs a, SwapList l) {
    const int p = threadIdx.x;
    if (p >= l.n) return;
    int ci, hi;
    if (!pair_homes(a, l, p, ci, hi)) return;
    a.slot_w[l.cold[p]] = hi;
    a.slot_w[l.hot[p]] = -ci - 1;
}

hipError_t launch_residency_swap(int32_t *slot, uint8_t *hot_base, uint8_t *host_cold, uint8_t *scratch,
                                 size_t blob_bytes, int E, int n_hot, int n_cold, const SwapList &l,
                                 hipStream_t st) {
    if (l.n <= 0) return hipSuccess;
    MoveArgs a{slot, slot, hot_base, host_cold, scratch, blob_bytes, E, n_hot, n_cold};
    const size_t units = blob_bytes / 16;
    const size_t per_iter = (size_t)kMoveThreads * kMoveUnroll;
    const size_t max_blocks = (units + per_iter - 1) / per_iter;
    // host-link phases: ~32 blocks in all (as the gather: enough reads in
    // flight to hold the link); the HBM phase: 256 blocks per expert
    const size_t link = std::min(max_blocks, (size_t)std::max(1, 32 / l.n));
    const size_t hbm = std::min(max_blocks, (size_t)256);
    MOE_LAUNCH("residency_move", residency_move, dim3((unsigned)link, l.n), dim3(kMoveThreads), 0, st, a, l, 0);
    MOE_LAUNCH("residency_move", residency_move, dim3((unsigned)link, l.n), dim3(kMoveThreads), 0, st, a, l, 1);
    MOE_LAUNCH("residency_move", residency_move, dim3((unsigned)hbm, l.n), dim3(kMoveThreads), 0, st, a, l, 2);
    MOE_LAUNCH("residency_move_table", residency_move_table, dim3(1), dim3(kMaxSwaps), 0, st, a, l);
    return hipGetLastError();
}

// ------------------------------- fingerprint --------------------------------
// Sum mod 2^64 over the blob's little-endian 64-bit words w_i of
// mix(w_i + (i+1)*G), mix = SplitMix64's output function (Steele, Lea and
// Flood 2014, with Stafford's Mix13 constants), G = 0x9E3779B97F4A7C15.
constexpr int kFpThreads = 256;
constexpr int kFpBlocksPerExpert = 64;

__device__ __forceinline__ uint64_t splitmix_out(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__global__ __launch_bounds__(kFpThreads) void fill_u64(uint64_t *__restrict__ p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

__global__ __launch_bounds__(kFpThreads) void fingerprint(const int32_t *__restrict__ experts,
                                                          const int32_t *__restrict__ slot,
                                                          const uint8_t *__restrict__ hot_base,
                                                          const uint8_t *__restrict__ host_cold, size_t blob_bytes,
                                                          int E, int n_hot, int n_cold,
                                                          uint64_t *__restrict__ out) {
    const int p = blockIdx.y;
    const int e = experts[p];
    if (e < 0 || e >= E) return;
    const int s = slot[e];
    const uint8_t *blob;
    if (s >= 0) {
        if (s >= n_hot) return;
        blob = hot_base + (size_t)s * blob_bytes;
    } else {
        if (-s - 1 >= n_cold) return;
        blob = host_cold + (size_t)(-s - 1) * blob_bytes;
    }
    const u32x4 *src = reinterpret_cast<const u32x4 *>(blob);
    const size_t units = blob_bytes / 16;
    constexpr uint64_t G = 0x9E3779B97F4A7C15ull;
    uint64_t acc = 0;
    for (size_t u = (size_t)blockIdx.x * kFpThreads + threadIdx.x; u < units; u += (size_t)gridDim.x * kFpThreads) {
        const u32x4 v = __builtin_nontemporal_load(src + u);
        const uint64_t w0 = (uint64_t)v.x | ((uint64_t)v.y << 32);
        const uint64_t w1 = (uint64_t)v.z | ((uint64_t)v.w << 32);
        const uint64_t i0 = 2 * (uint64_t)u;   // word index of w0
        acc += splitmix_out(w0 + (i0 + 1) * G);
        acc += splitmix_out(w1 + (i0 + 2) * G);
    }
    // wave sum, then one atomic per wave
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)acc, off);
        const uint32_t hi = __shfl_xor((uint32_t)(acc >> 32), off);
        acc += (uint64_t)lo | ((uint64_t)hi << 32);
    }
    if ((threadIdx.x & 63) == 0) atomicAdd((unsigned long long *)&out[p], (unsigned long long)acc);
}

hipError_t launch_fingerprint(const int32_t *experts, int n, const int32_t *slot, const uint8_t *hot_base,
                              const uint8_t *host_cold, size_t blob_bytes, int E, int n_hot, int n_cold,
                              uint64_t *out, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    MOE_LAUNCH("fill_u64", fill_u64, dim3((n + kFpThreads - 1) / kFpThreads), dim3(kFpThreads), 0, st, out, n);
    for (int p0 = 0; p0 < n; p0 += 65535) {   // grid.y limit
        const int m = std::min(65535, n - p0);
        MOE_LAUNCH("fingerprint", fingerprint, dim3(kFpBlocksPerExpert, m), dim3(kFpThreads), 0, st, experts + p0,
                   slot, hot_base, host_cold, blob_bytes, E, n_hot, n_cold, out + p0);
    }
    return hipGetLastError();
}

// ------------------------------ the swap rule -------------------------------
// score <- decay*score + counts (the product rounded, then the sum: no fused
// multiply-add), then cold experts by decreasing score against hot experts by
// increasing score (equal scores: lower index first); the i-th cold expert
// replaces the i-th hot one while score_c > threshold * max(score_h, min_score).
#pragma clang fp contract(off)
int plan_swaps(int E, int32_t *slot, double *score, const int32_t *counts, double decay, double threshold,
               double min_score, int max_swaps, int32_t *pairs) {
    for (int e = 0; e < E; ++e) {
        const double prod = decay * score[e];
        score[e] = prod + (double)counts[e];
    }
    std::vector<int> cold, hot;
    for (int e = 0; e < E; ++e) (slot[e] < 0 ? cold : hot).push_back(e);
    std::sort(cold.begin(), cold.end(), [&](int a, int b) {
        return score[a] > score[b] || (score[a] == score[b] && a < b);
    });
    std::sort(hot.begin(), hot.end(), [&](int a, int b) {
        return score[a] < score[b] || (score[a] == score[b] && a < b);
    });
    int n = 0;
    for (size_t i = 0; i < cold.size() && i < hot.size() && n < max_swaps; ++i) {
        const int c = cold[i], h = hot[i];
        const double bar = threshold * std::max(score[h], min_score);
        if (!(score[c] > bar)) break;
        pairs[2 * n] = c;
        pairs[2 * n + 1] = h;
        std::swap(slot[c], slot[h]);
        ++n;
    }
    return n;
}

}  // namespace moe
