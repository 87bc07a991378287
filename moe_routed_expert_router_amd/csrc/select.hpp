// Top-k selection and pick-set grouping by one block, shared by the decode
// select kernel and the decode gate/up kernel that recomputes the selection in
// every block (so the selection costs no launch of its own).
#pragma once

#include "device_util.hpp"

namespace moe {

struct SelectArgs {
    const float *z;   // logits [T][E]
    int T, E, k, renorm;
    int32_t *ids;     // [T][k] (written when publishing)
    float *w;         // [T][k]
    const int32_t *slot;
    int n_hot, n_cold;
    const uint8_t *hot_base, *scratch;
    size_t blob_bytes;
    int nsync;        // completion counter words to clear when publishing
};

// LDS of select_group_block: P ints each for sid and sflag, T ints for the
// pair list of the wanted expert, and 4 ints of its summary.
struct SelectLds {
    int *sid, *sflag, *spl, *sinfo;   // sinfo: [0] pairs n, [1] first position q0, [2..3] blob address
    int *sslot;                       // [E]: the residency table, copied in while the top-k runs
};

// Top-k of every token (one wave per token), then the grouping computed from
// the pair side: pair p = t*k+j of expert e goes to position
// #{pairs of smaller experts} + #{earlier pairs of e} of the pair list, and
// the distinct index of e is the number of distinct smaller experts.  Needs
// T*k <= blockDim.x.  If `publish`, writes ids, w and the whole pick set to
// `o`.  For the distinct expert number `want`, leaves its pair count, first
// position and blob address in s.sinfo and its pairs, in order, in s.spl
// (count 0 if there is no such expert).  Every thread of the block calls it.
// Needs E <= 2 * blockDim.x.
template <int NPL>
__device__ __forceinline__ void select_group_block(const SelectArgs &a, const GroupOut &o, bool publish, int want,
                                                   const SelectLds &s) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
    const int k = a.k, bd = blockDim.x;
    if (tid == 0) s.sinfo[0] = 0;
    if (publish)   // the down blocks' per-row-tile completion counters
        for (int i = tid; i < a.nsync; i += bd) o.sync[i] = 0;
    // the residency entries are requested before the logits and land in LDS
    // after the top-k, so looking up the picked experts' entries costs no
    // round trip of its own
    const int sl0 = a.slot[tid < a.E ? tid : 0];
    const int sl1 = a.slot[tid + bd < a.E ? tid + bd : 0];
    for (int t = wave; t < a.T; t += nwaves) {
        int pe;
        float pw;
        topk_wave<NPL>(a.z + (size_t)t * a.E, a.E, k, a.renorm, &pe, &pw);
        if (lane < k) {
            s.sid[t * k + lane] = pe;
            if (publish) {
                a.ids[(size_t)t * k + lane] = pe;
                a.w[(size_t)t * k + lane] = pw;
            }
        }
    }
    if (tid < a.E) s.sslot[tid] = sl0;
    if (tid + bd < a.E) s.sslot[tid + bd] = sl1;
    __syncthreads();
    const int P = a.T * k;
    if (P <= 64) {
        // One wave groups the pairs, lane p holding pair p; the other pairs'
        // values come by lane reads and the counts by ballots, so no
        // block-wide count reduction (two barriers each) is needed.
        if (wave == 0) {
            const bool act = lane < P;
            const int e = s.sid[act ? lane : 0];
            int lt = 0, eqb = 0, cnt = 0;
            for (int q = 0; q < P; ++q) {
                const int eq = __builtin_amdgcn_readlane(e, q);
                lt += eq < e;
                cnt += eq == e;
                eqb += (eq == e) & (q < lane);
            }
            int flag = 0;
            uint64_t addr = 0;
            if (act && eqb == 0) {   // first pair of its expert: 1 first, 2 cold, 4 unusable
                bool ok, cold;
                addr = expert_address(s.sslot[e], a.n_hot, a.n_cold, a.hot_base, a.scratch, a.blob_bytes, &ok, &cold);
                flag = 1 | ((ok && cold) ? 2 : 0) | (ok ? 0 : 4);
            }
            if (act && publish) o.plist[lt + eqb] = lane;
            const int nu = __popcll(__ballot(flag & 1)), nc = __popcll(__ballot(flag & 2));
            const int nb = __popcll(__ballot(flag & 4));
            int ui = 0, ci = 0;
            for (int q = 0; q < P; ++q) {
                const int fq = __builtin_amdgcn_readlane(flag, q), less = __builtin_amdgcn_readlane(e, q) < e;
                ui += (fq & 1) & less;
                ci += ((fq >> 1) & 1) & less;
            }
            if (act && publish && (flag & 1)) {
                o.uniq[ui] = e;
                o.ucnt[ui] = cnt;
                o.uoff[ui] = lt;
                o.uptr[ui] = addr;
                o.ucold[ui] = (flag >> 1) & 1;
                if (flag & 2) {
                    o.cold[ci] = e;
                    o.cu[ci] = ui;
                }
            }
            if (act && ui == want) {
                s.spl[eqb] = lane;
                if (flag & 1) {
                    s.sinfo[0] = cnt;
                    s.sinfo[1] = lt;
                    s.sinfo[2] = (int)(uint32_t)addr;
                    s.sinfo[3] = (int)(uint32_t)(addr >> 32);
                }
            }
            if (publish && lane == 0) {
                o.nuniq[0] = nu;
                o.nuniq[1] = nc;
                o.status[0] = 0;
                o.status[1] = nb;
                o.uoff[nu] = P;
            }
        }
        __syncthreads();
        return;
    }
    int e = 0, lt = 0, eqb = 0, cnt = 0, flag = 0;
    uint64_t addr = 0;
    if (tid < P) {
        e = s.sid[tid];
        for (int q = 0; q < P; ++q) {
            const int eq = s.sid[q];
            lt += eq < e;
            cnt += eq == e;
            eqb += (eq == e) & (q < tid);
        }
        if (eqb == 0) {   // first pair of its expert: 1 first, 2 cold, 4 unusable
            bool ok, cold;
            addr = expert_address(s.sslot[e], a.n_hot, a.n_cold, a.hot_base, a.scratch, a.blob_bytes, &ok, &cold);
            flag = 1 | ((ok && cold) ? 2 : 0) | (ok ? 0 : 4);
        }
        s.sflag[tid] = flag;
        if (publish) o.plist[lt + eqb] = tid;
    }
    const int nu = __syncthreads_count(flag & 1);
    const int nc = __syncthreads_count(flag & 2);
    const int nb = __syncthreads_count(flag & 4);
    if (tid < P) {
        int ui = 0, ci = 0;
        for (int q = 0; q < P; ++q) {
            const int fq = s.sflag[q], less = s.sid[q] < e;
            ui += (fq & 1) & less;
            ci += ((fq >> 1) & 1) & less;
        }
        if (publish && (flag & 1)) {
            o.uniq[ui] = e;
            o.ucnt[ui] = cnt;
            o.uoff[ui] = lt;
            o.uptr[ui] = addr;
            o.ucold[ui] = (flag >> 1) & 1;
            if (flag & 2) {
                o.cold[ci] = e;
                o.cu[ci] = ui;
            }
        }
        if (ui == want) {
            s.spl[eqb] = tid;
            if (flag & 1) {
                s.sinfo[0] = cnt;
                s.sinfo[1] = lt;
                s.sinfo[2] = (int)(uint32_t)addr;
                s.sinfo[3] = (int)(uint32_t)(addr >> 32);
            }
        }
    }
    if (publish && tid == 0) {
        o.nuniq[0] = nu;
        o.nuniq[1] = nc;
        o.status[0] = 0;
        o.status[1] = nb;
        o.uoff[nu] = P;
    }
    __syncthreads();
}

}  // namespace moe
