// Pick set / grouping: which experts the router picked, the (token, pick)
// pairs of each, and the picked cold experts.  The gracetier write-up (section
// 1) has one small kernel look at the router's picks; here that look is these
// three small kernels, and nothing goes back to the host.
//
// Pairs p = t*k + j are cut into chunks of 256.  Per chunk: a histogram over
// experts and each pair's rank among the chunk's earlier pairs of the same
// expert.  One block then turns the histograms into per-expert runs (stable:
// inside a run pairs keep increasing p), the distinct-expert list, the
// blob-address table and the picked-cold list.  A last pass scatters pair ids.
#include "device_util.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kChunk = WsLayout::kChunk;

// hist row layout: [E] per-expert counts then [1] count of out-of-range ids.
__global__ __launch_bounds__(kChunk) void group_hist(const int32_t *__restrict__ ids, int P, int E,
                                                     int32_t *__restrict__ hist,
                                                     int32_t *__restrict__ rank) {
    __shared__ int32_t cnt[kMaxExperts + 1];
    __shared__ int32_t sid[kChunk];
    const int tid = threadIdx.x;
    const int p = blockIdx.x * kChunk + tid;
    for (int i = tid; i <= E; i += kChunk) cnt[i] = 0;
    int e = -1;
    if (p < P) {
        e = ids[p];
        if (e < 0 || e >= E) e = -2;   // out of range: counted, then ignored
    }
    sid[tid] = e;
    __syncthreads();
    if (e >= 0) {
        atomicAdd(&cnt[e], 1);
        int r = 0;
        for (int q = 0; q < tid; ++q) r += (sid[q] == e);
        rank[p] = r;
    } else if (e == -2) {
        atomicAdd(&cnt[E], 1);
    }
    __syncthreads();
    int32_t *row = hist + (size_t)blockIdx.x * (E + 1);
    for (int i = tid; i <= E; i += kChunk) row[i] = cnt[i];
}

constexpr int kScanBatch = 16;   // chunk counts loaded together per thread

__global__ __launch_bounds__(1024) void group_scan(int nchunks, int E, const int32_t *__restrict__ slot,
                                                   int n_hot, int n_cold, const uint8_t *hot_base,
                                                   const uint8_t *scratch, size_t blob_bytes,
                                                   int32_t *__restrict__ hist, int32_t *__restrict__ counts,
                                                   int32_t *__restrict__ nuniq, int32_t *__restrict__ uniq,
                                                   int32_t *__restrict__ ucnt, int32_t *__restrict__ uoff,
                                                   uint64_t *__restrict__ uptr, int32_t *__restrict__ cold,
                                                   int32_t *__restrict__ ucold, int32_t *__restrict__ cu,
                                                   int32_t *__restrict__ status, int32_t *__restrict__ sync,
                                                   int32_t *__restrict__ tlist) {
    __shared__ int lds[40];
    const int e = threadIdx.x;
    for (int i = e; i < WsLayout::kSyncWords; i += 1024) sync[i] = 0;
    const int stride = E + 1;
    // the expert's pair count over all chunks, kScanBatch loads in flight at
    // a time (one dependent round trip per chunk would cost ~0.5 us each)
    int total = 0;
    if (e < E) {
        for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
            int v[kScanBatch];
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j)
                v[j] = c0 + j < nchunks ? hist[(size_t)(c0 + j) * stride + e] : 0;
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j) total += v[j];
        }
    }
    const bool is_exp = e < E;
    const int cnt = is_exp ? total : 0;
    int ntot;
    const int off = block_exscan1024(cnt, lds, &ntot);
    // residency: never point outside [0, n_hot) / [0, n_cold)
    bool ok = false, in_cold = false;
    const uint64_t addr =
        is_exp ? expert_address(slot[e], n_hot, n_cold, hot_base, scratch, blob_bytes, &ok, &in_cold) : 0;
    const bool picked = cnt > 0;
    int nu;
    const int ui = block_exscan1024(picked ? 1 : 0, lds, &nu);
    const bool is_cold = picked && ok && in_cold;
    int nc;
    const int ci = block_exscan1024(is_cold ? 1 : 0, lds, &nc);
    int nbad;
    block_exscan1024((picked && !ok) ? 1 : 0, lds, &nbad);
    // token tiles of the grouped GEMM: expert order, kPrefillTokens pairs each
    const int ntile = (cnt + WsLayout::kPrefillTokens - 1) / WsLayout::kPrefillTokens;
    int ntiles;
    const int toff = block_exscan1024(ntile, lds, &ntiles);
    for (int part = 0; part < ntile; ++part) tlist[toff + part] = ui | (part << 10);
    if (is_exp) {
        counts[e] = cnt;
        if (picked) {
            uniq[ui] = e;
            ucnt[ui] = cnt;
            uoff[ui] = off;
            uptr[ui] = addr;
            ucold[ui] = is_cold ? 1 : 0;
        }
        if (is_cold) {
            cold[ci] = e;
            cu[ci] = ui;
        }
        // each chunk's base for the expert: its global offset plus the pairs
        // of the earlier chunks
        int run = off;
        for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
            int v[kScanBatch];
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j)
                v[j] = c0 + j < nchunks ? hist[(size_t)(c0 + j) * stride + e] : 0;
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j)
                if (c0 + j < nchunks) {
                    hist[(size_t)(c0 + j) * stride + e] = run;
                    run += v[j];
                }
        }
    }
    int bad = 0;   // out-of-range pair count, over the chunks in parallel
    for (int c0 = 0; c0 < nchunks; c0 += 1024) {
        int part;
        block_exscan1024(c0 + e < nchunks ? hist[(size_t)(c0 + e) * stride + E] : 0, lds, &part);
        bad += part;
    }
    if (e == 0) {
        status[0] = bad;
        nuniq[0] = nu;
        nuniq[1] = nc;
        nuniq[2] = ntiles;
        status[1] = nbad;
        uoff[nu] = ntot;
    }
}

__global__ __launch_bounds__(kChunk) void group_place(const int32_t *__restrict__ ids, int P, int E,
                                                      const int32_t *__restrict__ hist,
                                                      const int32_t *__restrict__ rank,
                                                      int32_t *__restrict__ plist) {
    const int p = blockIdx.x * kChunk + threadIdx.x;
    if (p >= P) return;
    const int e = ids[p];
    if (e < 0 || e >= E) return;
    plist[hist[(size_t)blockIdx.x * (E + 1) + e] + rank[p]] = p;
}

hipError_t launch_group(const GroupArgs &a, char *ws, const WsLayout &L, hipStream_t st) {
    const int P = a.T * a.k;
    int32_t *hist = reinterpret_cast<int32_t *>(ws + L.hist);
    int32_t *rank = reinterpret_cast<int32_t *>(ws + L.rank);
    if (L.nchunks > 0) {
        MOE_LAUNCH("group_hist", group_hist, dim3(L.nchunks), dim3(kChunk), 0, st, a.ids, P, a.E, hist, rank);
    }
    MOE_LAUNCH("group_scan", group_scan, dim3(1), dim3(1024), 0, st, L.nchunks, a.E, a.slot, a.n_hot, a.n_cold,
                       a.hot_base, a.scratch, a.blob_bytes, hist,
                       reinterpret_cast<int32_t *>(ws + L.counts), reinterpret_cast<int32_t *>(ws + L.nuniq),
                       reinterpret_cast<int32_t *>(ws + L.uniq), reinterpret_cast<int32_t *>(ws + L.ucnt),
                       reinterpret_cast<int32_t *>(ws + L.uoff), reinterpret_cast<uint64_t *>(ws + L.uptr),
                       reinterpret_cast<int32_t *>(ws + L.cold), reinterpret_cast<int32_t *>(ws + L.ucold),
                       reinterpret_cast<int32_t *>(ws + L.cu), reinterpret_cast<int32_t *>(ws + L.status),
                       reinterpret_cast<int32_t *>(ws + L.sync), reinterpret_cast<int32_t *>(ws + L.tlist));
    if (L.nchunks > 0) {
        MOE_LAUNCH("group_place", group_place, dim3(L.nchunks), dim3(kChunk), 0, st, a.ids, P, a.E, hist, rank,
                           reinterpret_cast<int32_t *>(ws + L.plist));
    }
    return hipGetLastError();
}

__global__ __launch_bounds__(1024) void pick_set_out(const int32_t *__restrict__ counts,
                                                     const int32_t *__restrict__ nuniq,
                                                     const int32_t *__restrict__ cold, int E,
                                                     int32_t *__restrict__ counts_out,
                                                     int32_t *__restrict__ cold_out) {
    const int m = nuniq[1];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        counts_out[e] = counts[e];
        cold_out[1 + e] = (e < m) ? cold[e] : -1;
    }
    if (threadIdx.x == 0) cold_out[0] = m;
}

hipError_t launch_pick_set_out(const char *ws, const WsLayout &L, int E, int32_t *counts_out,
                               int32_t *cold_out, hipStream_t st) {
    MOE_LAUNCH("pick_set_out", pick_set_out, dim3(1), dim3(1024), 0, st,
                       reinterpret_cast<const int32_t *>(ws + L.counts),
                       reinterpret_cast<const int32_t *>(ws + L.nuniq),
                       reinterpret_cast<const int32_t *>(ws + L.cold), E, counts_out, cold_out);
    return hipGetLastError();
}

}  // namespace moe
