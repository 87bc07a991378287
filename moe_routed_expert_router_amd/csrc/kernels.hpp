// Internal launchers of the HIP path (one translation unit per kernel family).
#pragma once

#include <hip/hip_ext.h>

#include "common.hpp"

namespace moe {

// Per-kernel timing (profile.hip).  When enabled, prof_events() hands out a
// start/stop event pair that the launch itself records (hipExtLaunchKernel
// stamps them from the dispatch), so the elapsed time is the kernel's own
// execution time; otherwise it returns false and the launch is plain.
bool prof_events(const char *name, hipEvent_t *start, hipEvent_t *stop);

#define MOE_LAUNCH(name, kernel, grid, block, shmem, st, ...)                                       \
    do {                                                                                            \
        hipEvent_t _moe_e0 = nullptr, _moe_e1 = nullptr;                                            \
        if (::moe::prof_events((name), &_moe_e0, &_moe_e1))                                         \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, _moe_e0, _moe_e1, 0, __VA_ARGS__); \
        else                                                                                        \
            hipLaunchKernelGGL(kernel, grid, block, shmem, st, __VA_ARGS__);                        \
    } while (0)

// Router logits z[T][E] = x Wr^T + bias (fp32 accumulation).
hipError_t launch_route_logits(const uint16_t *x, const float *wr, const float *bias,
                               int T, int H, int E, float *z, hipStream_t st);

// Top-k selection and softmax weights from logits z[T][E].
hipError_t launch_topk(const float *z, int T, int E, int k, int renorm,
                       int32_t *ids, float *w, hipStream_t st);

// Pick set / grouping of the T*k pairs; fills the workspace regions of WsLayout.
struct GroupArgs {
    const int32_t *ids;
    int T, k, E;
    const int32_t *slot;
    int n_hot, n_cold;
    const uint8_t *hot_base;
    const uint8_t *scratch;
    size_t blob_bytes;
};
hipError_t launch_group(const GroupArgs &a, char *ws, const WsLayout &L, hipStream_t st);

// Arguments of the block-level selection (select.hpp).
struct SelectArgs;
SelectArgs select_args(const float *z, int T, int k, int renorm, int32_t *ids, float *w, const GroupArgs &a);

// Decode path (T*k <= 1024): top-k of every token and the whole pick set in
// one single-block launch.
hipError_t launch_select_group_small(const float *z, int T, int k, int renorm, int32_t *ids, float *w,
                                     const GroupArgs &a, char *ws, const WsLayout &L, hipStream_t st);

// Copies counts [E] and the picked-cold list [E+1] out of a grouped workspace.
hipError_t launch_pick_set_out(const char *ws, const WsLayout &L, int E,
                               int32_t *counts_out, int32_t *cold_out, hipStream_t st);

// Copies the picked cold experts host -> scratch.
hipError_t launch_gather(const uint8_t *host_cold, uint8_t *scratch, size_t blob_bytes,
                         const int32_t *slot, const char *ws, const WsLayout &L,
                         hipStream_t st);

// Decode gather that takes the top-k from the logits z [T][E] itself (no
// grouping launch before it): copies the picked cold experts host -> scratch.
hipError_t launch_gather_sel(const float *z, int T, int E, int k, const int32_t *slot, int n_cold,
                             const uint8_t *host_cold, uint8_t *scratch, size_t blob_bytes, hipStream_t st);

// Grouped SwiGLU FFN over the grouped pairs and the weighted combine into out.
struct FfnArgs {
    const uint16_t *x;
    const int32_t *ids;
    const float *w;
    int T, H, I, E, k;
    int out_bf16;
    void *out;
};
hipError_t launch_ffn(const FfnArgs &a, char *ws, const WsLayout &L, hipStream_t st);

// Decode FFN in two parts so that the hot experts' FFN can run while the cold
// ones are still being gathered: kPartHot covers the distinct experts whose
// blob is in HBM proper, kPartCold those read from a scratch slot (grid rows
// = picked cold experts, at most umax_part), then the combine.  The two parts
// together do exactly what launch_ffn does.  Needs ffn_block_path.
constexpr int kPartAll = 0, kPartHot = 1, kPartCold = 2;
hipError_t launch_ffn_part(const FfnArgs &a, int part, int umax_part, char *ws, const WsLayout &L,
                           hipStream_t st);

// Decode layer with no cold expert: the gate/up kernel recomputes the top-k
// and the grouping in every block (block 0 publishes ids, w and the pick set),
// then down and combine as in launch_ffn.  Needs ffn_select_fusable.
constexpr int kFusedSelectPairs = 512;
// Pairs up to which the layer uses the gate/up kernel that selects in every
// block.  The per-block selection grows with T while the launch it saves
// does not: measured per layer (4 layers rotating, graph replay), it wins at
// one token (34 against 35.5 us all resident) and loses from two tokens on
// (58 against 54 us at T = 2, 155 against 111 at T = 8, 848 against 256 at
// T = 32).
constexpr int kFusedSelectMaxPairs = 8;
hipError_t launch_ffn_select(const FfnArgs &a, const float *z, int renorm, int32_t *ids, float *w,
                             const GroupArgs &g, char *ws, const WsLayout &L, hipStream_t st);

// Decode layer with cold experts: the hot experts' gate/up (and, past the
// fused down + combine sizes, their down) with the selection recomputed in
// every block as in launch_ffn_select; block 0 publishes ids, w and the whole
// pick set, so launch_ffn_part(kPartCold) can follow once the gather is done.
// Needs ffn_select_fusable.
hipError_t launch_ffn_select_hot(const FfnArgs &a, const float *z, int renorm, int32_t *ids, float *w,
                                 const GroupArgs &g, char *ws, const WsLayout &L, hipStream_t st);

// True when launch_ffn_select applies (block path, T*k within both the
// selection's LDS and the gate/up block's threads, E within two entries per
// thread).
bool ffn_select_fusable(int T, int k, int E, int H, int I);

// True when launch_ffn uses the block kernels (decode sizes).
bool ffn_block_path(int T, int H, int I);

// True when launch_ffn uses the grouped-GEMM kernels (prefill sizes).
bool ffn_gemm_path(int T, int H, int I, int k);

// Grouped-GEMM gate/up + SwiGLU and down over the token tiles of the grouping
// (h as bf16 hi/lo planes indexed by grouped position, y by pair id).
hipError_t launch_ffn_gemm(const FfnArgs &a, const GroupView &gv, int max_tiles, uint16_t *hhi, uint16_t *hlo,
                           float *y, hipStream_t st);

// Largest T routed by the single-block select-and-group kernel.
constexpr int kSmallRouteTokens = 32;

// Adaptive residency (residency.hip).
// counts[E] (+)= pairs per expert; ids outside [0,E) ignored; clear zeroes
// counts first (in the same kernel at decode sizes, else a fill kernel).
hipError_t launch_count_picks(const int32_t *ids, int n_pairs, int E, int32_t *counts, bool clear, hipStream_t st);

// Swaps of (cold expert, hot expert) pairs, passed by value to the kernels.
constexpr int kMaxSwaps = 64;
struct SwapList {
    int32_t n;
    int32_t cold[kMaxSwaps];
    int32_t hot[kMaxSwaps];
};
hipError_t launch_residency_swap(int32_t *slot, uint8_t *hot_base, uint8_t *host_cold, uint8_t *scratch,
                                 size_t blob_bytes, int E, int n_hot, int n_cold, const SwapList &l,
                                 hipStream_t st);

// out[p] = fingerprint of expert experts[p] at its home (HBM pool or host pool).
hipError_t launch_fingerprint(const int32_t *experts, int n, const int32_t *slot, const uint8_t *hot_base,
                              const uint8_t *host_cold, size_t blob_bytes, int E, int n_hot, int n_cold,
                              uint64_t *out, hipStream_t st);

// Streaming read of `bytes` (a multiple of 16) from src by one launch with
// `loads_per_thread` (1, 2, 4, 8 or 16) 16-byte loads per thread; writes nothing.
hipError_t launch_probe_read(const void *src, size_t bytes, int loads_per_thread, uint32_t *sink,
                             hipStream_t st);
// Matrix-core rate of one MFMA kind (0 bf16, 1 fp8 x fp4, 2 fp8 x fp8, 3 fp6 x
// fp4, 4 fp4 x fp4): 2 * cus blocks of 4 waves, iters rounds of 4 MFMAs each.
hipError_t launch_probe_mfma(int kind, int iters, int cus, uint32_t *sink, hipStream_t st);

// Host side of the manager: decayed scores and the swap rule; returns the
// number of pairs written to pairs[2*i], pairs[2*i+1] and updates slot and score.
int plan_swaps(int E, int32_t *slot, double *score, const int32_t *counts, double decay, double threshold,
               double min_score, int max_swaps, int32_t *pairs);

}  // namespace moe
