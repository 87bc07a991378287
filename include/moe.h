/*
 * moe.h — C ABI of the routed-expert layer with a cold-expert gather, for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (the "gracetier" write-up, section 1 "The idea"; the GB300
 * inference write-up's paragraph on the mixture-of-experts design):
 *   1. a router scores E experts per token and keeps the top k;
 *   2. a gather copies only the picked COLD experts from pinned host memory
 *      into their fixed slot of one HBM scratch area, which every layer
 *      reuses because layers run one after another;
 *   3. one grouped SwiGLU FFN runs every picked expert, reading hot experts
 *      from HBM and cold ones from scratch, as if all were resident, and the
 *      expert outputs are added with the routing weights.
 *
 * Conventions for every entry point
 *   - Returns a moe_status; never throws, never aborts.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any error nothing is enqueued.  moe_last_error() describes the last
 *     error of the calling thread.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     No entry point synchronises the host with the device.  Device faults
 *     surface at the caller's next synchronisation.
 *   - "device" pointers must be device-accessible memory (hipMalloc'd,
 *     or pinned host memory mapped for the device); the library checks them
 *     with the HIP runtime and returns MOE_ERR_NOT_DEVICE_ACCESSIBLE when a
 *     pointer is not, or MOE_ERR_INVALID_ARG when its allocation is too small.
 *   - The caller owns all memory; the library allocates nothing on these
 *     paths.  Scratch space comes from a caller workspace `ws` of at least
 *     moe_workspace_bytes() bytes, 256-byte aligned; its contents on entry are
 *     ignored and it may be reused between calls on the same stream.
 *   - Calls that share a workspace or a scratch area must be ordered (same
 *     stream, or events).  Stream order alone makes the scratch safe to
 *     share across layers: a later layer's gather starts after the earlier
 *     layer's FFN has finished reading it.
 *
 * Layouts
 *   - Activations x: bf16 bit patterns, row-major [T][H].
 *   - Router weight: fp32 [E][H]; optional logit bias: fp32 [E].
 *   - Expert blob (one contiguous block of moe_expert_bytes() bytes per
 *     expert; MXFP4: FP4 E2M1 codes, two per byte with the even element in the
 *     low nibble, and one E8M0 scale per 32 consecutive elements along the
 *     contraction axis, following the OCP MX v1.0 formats):
 *         w13 codes  (2I x H)   rows 0..I-1 gate (w1), rows I..2I-1 up (w3)
 *         w13 scales
 *         w2  codes  (H x I)    down projection
 *         w2  scales
 *     in that order, each plane of R rows and K columns stored in tiles of
 *     16 rows x 128 columns (nst = K/128): the codes of row r, column c are
 *     byte ((r/16)*nst + c/128)*1024 + (r%16)*64 + (c%128)/2 of the plane's
 *     codes section, and the scale of row r, block b = c/32 is byte
 *     ((r/16)*nst + b/4)*64 + (r%16)*4 + b%4 of its scales section.
 *   - Residency table slot[E] (int32): slot[e] >= 0 means expert e is hot and
 *     lives at hot_base + slot[e]*B; slot[e] < 0 means cold, with cold index
 *     c = -slot[e]-1: its bytes are at host_cold + c*B and it runs from
 *     scratch + c*B (B = moe_expert_bytes()).
 *   - Routing output: topk_ids int32 [T][k] and topk_w fp32 [T][k], the k
 *     picks of each token by decreasing weight (ties: lower expert index).
 *   - Layer output: [T][H], fp32 (MOE_OUT_F32) or bf16 bits (MOE_OUT_BF16).
 *
 * Shape limits: H and I multiples of 128; 1 <= k <= min(E, 32); E <= 1024;
 * 0 <= T <= 1<<20 (T = 0 enqueues nothing and returns MOE_OK).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,           /* NULL / negative / inconsistent argument */
    MOE_ERR_UNSUPPORTED_SHAPE = 2,     /* outside the shape limits above */
    MOE_ERR_MISALIGNED = 3,            /* pointer not aligned as documented */
    MOE_ERR_NOT_DEVICE_ACCESSIBLE = 4, /* pointer the GPU cannot read or write */
    MOE_ERR_BAD_RESIDENCY = 5,         /* residency table inconsistent */
    MOE_ERR_WORKSPACE_TOO_SMALL = 6,   /* ws_bytes < moe_workspace_bytes() */
    MOE_ERR_HIP = 7                    /* a HIP runtime call or launch failed */
} moe_status;

typedef enum { MOE_OUT_F32 = 0, MOE_OUT_BF16 = 1 } moe_out_dtype;

/* Model shape: hidden size H, expert FFN width I, experts E, picks k. */
typedef struct {
    int32_t hidden;
    int32_t inter;
    int32_t n_experts;
    int32_t top_k;
} moe_shape;

/* Where one layer's experts live.  All memory is caller-owned.
 *   slot      device [E] residency table (see Layouts).
 *   hot_base  device [n_hot][B]; may be NULL when n_hot == 0.
 *   host_cold device-visible pointer to pinned host memory [n_cold][B]
 *             (moe_host_alloc()); may be NULL when n_cold == 0.
 *   scratch   device [n_cold][B]; the cold experts' HBM slots, which may be
 *             shared by every layer; may be NULL when n_cold == 0.
 *             scratch == host_cold selects direct read: the FFN reads each
 *             picked cold expert in place from pinned host memory over the
 *             host link, and nothing is copied (the pages' mapped / UVA
 *             alternative to the copy kernel: gracetier write-up, section 1,
 *             against the row-level UVA offload of the GB300 write-up's
 *             results table and the mapped W2 plane of the RTX PRO 6000
 *             write-up, "Five layers made the difference"). */
typedef struct {
    const int32_t *slot;
    const uint8_t *hot_base;
    const uint8_t *host_cold;
    uint8_t *scratch;
    int32_t n_hot;
    int32_t n_cold;
} moe_residency;

/* Human-readable name of a status code (static string). */
const char *moe_status_string(moe_status st);

/* Detail of the last error returned to the calling thread ("" if none). */
const char *moe_last_error(void);

/* MOE_OK if the shape is within the limits, else MOE_ERR_UNSUPPORTED_SHAPE
 * or MOE_ERR_INVALID_ARG (NULL). */
moe_status moe_shape_check(const moe_shape *s);

/* Bytes of one expert blob: 3*H*I*17/32 (0 if the shape is invalid). */
size_t moe_expert_bytes(const moe_shape *s);

/* Workspace bytes needed by any entry point for T tokens (0 if invalid). */
size_t moe_workspace_bytes(const moe_shape *s, int32_t n_tokens);

/* Checks a HOST copy of a residency table: the hot entries must be exactly
 * 0..n_hot-1 and the cold entries exactly 0..n_cold-1 (each once), with
 * n_hot + n_cold == E.  Returns MOE_ERR_BAD_RESIDENCY otherwise.  Run it once
 * per residency change (the fast paths trust the device copy, but still
 * never read outside [0,n_hot) / [0,n_cold): a bad entry makes that
 * expert's pairs contribute zero). */
moe_status moe_residency_check(const moe_shape *s, const int32_t *slot_host,
                               int32_t n_hot, int32_t n_cold);

/* Allocate `bytes` of pinned host memory mapped for the current device and
 * return its host address and the device-visible address the kernels use
 * (the page-locked, device-mapped host buffer that the mapped-host design in
 * the 96 GB RTX PRO 6000 write-up, "Five layers made the difference", also
 * installs into its kernel path).  flags: bit 0 = coherent (fine-grained)
 * mapping, else non-coherent.  Free with moe_host_free(). */
moe_status moe_host_alloc(size_t bytes, int32_t flags, void **host_ptr, void **device_ptr);
moe_status moe_host_free(void *host_ptr);

/* Router (the inference-engineering write-up, "Milo and James try inference
 * engineering", its opening paragraph on the mixture-of-experts design: per
 * token a small router chooses 6 of 384 experts; the gracetier write-up,
 * "DeepSeek-V4.1-Flash on One GB300 Without the Second GPU", section 1, runs
 * the copy and the experts on those picks).
 * Logits z[t,e] = sum_h x[t,h]*Wr[e,h] + bias[e] in fp32, then
 * per token the k largest logits (ties to the lower expert index), listed by
 * decreasing weight, with softmax weights renormalised over the k picks
 * (renormalize != 0) or plain softmax probabilities over all E
 * (renormalize == 0).
 *   x [T][H] bf16 (16-B aligned), w_router [E][H] fp32 (16-B aligned),
 *   bias [E] fp32 or NULL, topk_ids [T][k] int32, topk_w [T][k] fp32,
 *   logits_out [T][E] fp32 or NULL (written when given). */
moe_status moe_route(const moe_shape *s, int32_t n_tokens, const uint16_t *x,
                     const float *w_router, const float *bias, int32_t renormalize,
                     int32_t *topk_ids, float *topk_w, float *logits_out,
                     void *ws, size_t ws_bytes, void *stream);

/* Pick set (gracetier write-up, section 1: the copy kernel first looks at
 * which experts the router picked and which of them are cold).
 * For the (token, pick) pairs in topk_ids, writes
 *   counts_out [E] int32: number of pairs routed to each expert, and
 *   cold_out [E+1] int32: cold_out[0] = number m of distinct picked experts
 *   whose slot is cold, cold_out[1..m] = those experts in increasing order.
 * Pairs whose id is outside [0,E) are not counted.  slot: device [E]. */
moe_status moe_pick_set(const moe_shape *s, int32_t n_tokens, const int32_t *topk_ids,
                        const int32_t *slot, int32_t n_hot, int32_t n_cold,
                        int32_t *counts_out, int32_t *cold_out,
                        void *ws, size_t ws_bytes, void *stream);

/* Cold gather (gracetier write-up, section 1 "The idea": the cold experts
 * stay in pinned host memory that the GPU reads directly, one HBM scratch
 * area has a slot per cold expert and is shared by every layer, and one
 * small kernel per layer copies just the picked cold experts into their
 * slots; section 3 times that kernel at 2.60 ms of a 10.49 ms step).
 * Every distinct picked expert e with slot[e] < 0 is
 * copied whole, once, from host_cold + c*B to scratch + c*B (c = -slot[e]-1),
 * by a kernel that reads the pinned host memory directly; unpicked slots are
 * not touched.  No host round trip decides what is copied.  With
 * r->n_cold == 0, or in direct read (scratch == host_cold), nothing is
 * enqueued. */
moe_status moe_gather_cold(const moe_shape *s, int32_t n_tokens, const int32_t *topk_ids,
                           const moe_residency *r, void *ws, size_t ws_bytes, void *stream);

/* Grouped expert FFN and combine (gracetier write-up, section 1: after the
 * copy, every picked expert runs in one call as though all were in HBM; the
 * routed experts are MXFP4, per the two-workstation report, "A 475 GB Model
 * Across Two Workstations", Abstract and section 1; the offloaded planes
 * are w13 and w2, per the inference-engineering write-up's flag table).
 * For every pair (t, j) with
 * e = topk_ids[t][j], y = W2_e (silu(W1_e x_t) * (W3_e x_t)) with fp32
 * accumulation, and out[t] = sum_j topk_w[t][j] * y_(t,j) added in j order
 * (no float atomics: the result does not depend on where experts live).
 * Cold experts are read from their scratch slot, so moe_gather_cold must have
 * run for these ids.  Pairs with an id outside [0,E) contribute nothing.
 *   out [T][H]: fp32 or bf16 per out_dtype (16-B aligned). */
moe_status moe_expert_ffn(const moe_shape *s, int32_t n_tokens, const uint16_t *x,
                          const int32_t *topk_ids, const float *topk_w,
                          const moe_residency *r, int32_t out_dtype, void *out,
                          void *ws, size_t ws_bytes, void *stream);

/* The whole layer (gracetier write-up, section 1: route, copy the picked
 * cold experts into their slots, then one call over every picked expert;
 * layers run one after another, which is what lets them share the scratch).
 * moe_route, then the pick set, the cold gather
 * (skipped when r->n_cold == 0 or in direct read) and the grouped FFN with
 * the combine, ordered
 * on `stream`: the call returns with everything enqueued after work already
 * on `stream` and later work on `stream` sees the finished layer.  At decode
 * sizes above a few tokens (T*k > 24) with cold experts, the gather runs on a
 * library-owned side stream of the current device (default priority, created
 * on first use) forked from and joined back into `stream` by events, while
 * the hot experts' FFN runs on `stream`; the pattern is valid under stream
 * capture.  Below that everything runs on `stream`.  topk_ids / topk_w
 * receive the routing. */
moe_status moe_layer_forward(const moe_shape *s, int32_t n_tokens, const uint16_t *x,
                             const float *w_router, const float *bias, int32_t renormalize,
                             const moe_residency *r, int32_t *topk_ids, float *topk_w,
                             int32_t out_dtype, void *out,
                             void *ws, size_t ws_bytes, void *stream);

/* moe_layer_forward for callers that cannot allocate (code under graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer with the same results, but no caller workspace and no allocation
 * of any kind.  Its workspace is a static device array of
 * MOE_NOALLOC_WS_BYTES bytes inside the library, one per GPU it runs on,
 * held until the process ends; T tokens need moe_workspace_bytes(s, T)
 * bytes of it (16 MiB covers up to ~110 decode tokens at H=4096, I=2048,
 * E=384, k=6), and larger calls return MOE_ERR_WORKSPACE_TOO_SMALL with
 * nothing enqueued.  Everything runs on `stream` (no side stream), in the
 * in-order launch sequence.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (two streams, two threads) race and must be
 * ordered by the caller.  With moe_profile_enable on, the timing events are
 * still created as for every entry point. */
#define MOE_NOALLOC_WS_BYTES (16u << 20)
moe_status moe_layer_forward_noalloc(const moe_shape *s, int32_t n_tokens, const uint16_t *x,
                                     const float *w_router, const float *bias, int32_t renormalize,
                                     const moe_residency *r, int32_t *topk_ids, float *topk_w,
                                     int32_t out_dtype, void *out, void *stream);

/* ---------------------------------------------------------------------------
 * Adaptive residency and the byte audit.  The gracetier write-up: between
 * decode steps a manager swaps experts that are being picked often into the
 * hot set and moves quiet ones out (section 1, "The idea"), with a
 * hysteresis threshold whose published default is 3.0, twice the first
 * setting (section 3, "Where the time goes"); every expert is fingerprinted
 * at boot and every moved expert, plus a sample, again after swapping,
 * wherever it now lives (section 4, the table of checks).  A manager tick is:
 * moe_count_picks after each layer's routing (on the device, capturable),
 * then between steps a host copy of the counts, moe_residency_plan (host),
 * and moe_residency_swap (device).  Outputs do not depend on where experts
 * live, so a swap never changes a layer's results.
 * ------------------------------------------------------------------------- */

/* Most swaps one moe_residency_swap / moe_residency_plan call handles. */
#define MOE_MAX_SWAPS 64

/* counts[e] += number of (token, pick) pairs of topk_ids [T][k] routed to e
 * (ids outside [0,E) not counted); with clear != 0 counts is zeroed first
 * (by a kernel, so the call may be captured in a graph).  counts: device
 * int32 [E].  T = 0 with clear only zeroes. */
moe_status moe_count_picks(const moe_shape *s, int32_t n_tokens, const int32_t *topk_ids, int32_t *counts,
                           int32_t clear, void *stream);

/* Host-side swap rule of one layer (no GPU work; all pointers are host memory).
 *   score[e] <- decay * score[e] + counts_host[e]  (float64; the product is
 *   rounded, then the sum); then cold experts in decreasing score against hot
 *   experts in increasing score (equal scores: lower expert index first): the
 *   i-th cold expert replaces the i-th hot one while
 *   score_cold > threshold * max(score_hot, min_score), at most max_swaps times.
 * Writes the pairs as pairs_out[2i] = cold expert promoted, pairs_out[2i+1] =
 * hot expert demoted (room for 2*max_swaps int32), their number to
 * *n_pairs_out, and applies them to slot_host (the promoted expert takes the
 * demoted one's HBM index, the demoted one the promoted one's cold slot).
 * slot_host must pass moe_residency_check; score entries must be finite and
 * >= 0, counts >= 0, decay in [0,1], threshold > 0, min_score >= 0,
 * 0 <= max_swaps <= MOE_MAX_SWAPS.  On error nothing is modified except
 * *n_pairs_out = 0. */
moe_status moe_residency_plan(const moe_shape *s, int32_t *slot_host, int32_t n_hot, int32_t n_cold,
                              double *score, const int32_t *counts_host, double decay, double threshold,
                              double min_score, int32_t max_swaps, int32_t *pairs_out, int32_t *n_pairs_out);

/* Moves the experts of n_pairs (cold expert c, hot expert h) pairs, host array
 * pairs[2*n_pairs] as written by moe_residency_plan: c's bytes from its host
 * slot to h's HBM slot and h's bytes from HBM to c's host slot, then the
 * device table r->slot is updated as moe_residency_plan updated its host
 * copy.  The call WRITES r->slot, r->hot_base and r->host_cold (the pointers
 * are const only for the layer entry points) and uses c's scratch slot as
 * staging, so it must be ordered after any layer that still reads these
 * (same stream) and before the next layer that uses this layer's table.  A
 * pair that the device table does not show as (cold, hot) is left alone.
 * Errors: experts outside [0,E), an expert named twice, n_pairs outside
 * [0, MOE_MAX_SWAPS], a residency with no hot or no cold experts, or direct
 * read (no staging) -> nothing enqueued. */
moe_status moe_residency_swap(const moe_shape *s, const moe_residency *r, const int32_t *pairs, int32_t n_pairs,
                              void *stream);

/* Byte audit: out[p] (device uint64 [n]) = fingerprint of expert experts[p]
 * (device int32 [n]) at its home: hot_base + slot*B when hot, host_cold +
 * c*B when cold (the pinned pool, not the scratch copy).  Fingerprint: the
 * sum modulo 2^64 over the blob's little-endian 64-bit words w_i of
 * SplitMix64's output function (Steele, Lea and Flood 2014) applied to
 * w_i + (i+1) * 0x9E3779B97F4A7C15.  An id outside [0,E) or an unusable table
 * entry gives 0. */
moe_status moe_fingerprint(const moe_shape *s, const moe_residency *r, const int32_t *experts, int32_t n,
                           uint64_t *out, void *stream);

/* Per-kernel timing, a tracing aid (off by default).  While enabled, each
 * kernel the library enqueues carries a start/stop HIP event pair stamped by
 * its own dispatch, so the times are kernel execution times.
 * moe_profile_read(i, ...) waits for the recorded events, folds them
 * into per-kernel totals and returns kernel i's name (static until the next
 * reset), launch count and summed milliseconds; MOE_ERR_INVALID_ARG past the
 * last kernel.  Not meant for use under graph capture.  moe_profile_reset()
 * clears the totals. */
moe_status moe_profile_enable(int32_t on);
moe_status moe_profile_reset(void);
moe_status moe_profile_read(int32_t index, const char **name, int64_t *count, double *total_ms);

/* Streaming-read probe, a measurement aid (no part of the layer): one launch
 * reads `bytes` bytes at src (device, 16-B aligned, a positive multiple of
 * 16) with `loads_per_thread` (1, 2, 4, 8 or 16) 16-byte loads per thread, every
 * load of a thread issued before any is used, and computes nothing from
 * them.  Its kernel time (moe_profile_*, kernel "probe_read") is the time a
 * single launch of that many bytes takes when reading is all it does, the
 * ceiling for a bandwidth-bound kernel of the same size.  sink: device
 * uint32 [1], written only when the loaded words happen to fold to a fixed
 * value (it keeps the loads alive). */
moe_status moe_probe_read(const void *src, size_t bytes, int32_t loads_per_thread, uint32_t *sink, void *stream);

/* Matrix-core rate probe, a measurement aid (no part of the layer): one
 * launch of two 256-thread blocks per compute unit in which every wave
 * issues `iters` (1..2^20) rounds of four independent MFMAs of one kind on
 * register operands.  kind: 0 bf16 32x32x16 (32768 flops per instruction);
 * the gfx950 scaled 32x32x64 f8f6f4 form (131072 flops) with operands 1 fp8
 * x fp4, 2 fp8 x fp8, 3 fp6 (e2m3) x fp4, 4 fp4 x fp4.  The kernel time
 * (moe_profile_*, kernel "probe_mfma") gives the rate each kind sustains
 * with the GPU full.  sink: device uint32 [1], written only when the
 * accumulators fold to a fixed value.  MOE_ERR_INVALID_ARG for a kind or
 * iters out of range. */
moe_status moe_probe_mfma(int32_t kind, int32_t iters, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
