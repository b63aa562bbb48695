// The token-to-expert worklist built by a single wave (small pair counts),
// shared by the decode preparation kernel and the fused f32 decode kernel.
// pxq_llama.cpp release notes, "Device-side MoE row map": histogram, scan
// and fill on the device, bit-identical to a host build.
#pragma once

#include "common.h"
#include "launch.h"

namespace qmoe {

// Inclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    // Hillis-Steele inside each row of 16 lanes (row shifts read 0 past the
    // row start), then the row totals carried forward with row broadcasts:
    // lane 15 into rows 1 and 3, lane 31 into rows 2 and 3.  DPP only, no LDS.
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
    return x;
}

// The same worklist built by one wave, for small pair counts: no block
// barriers, only the in-order LDS traffic of a single wave (its fences are
// wave-scope: they order the compiler, the hardware already keeps one
// wave's LDS operations in order).
__device__ inline void wl_wave(const int32_t *__restrict__ ids, const float *__restrict__ topk_w, int n,
                        int k, int E, const Worklist &wl, const DecodePlan &plan,
                        int *cnt /* [E+1] */, int *run /* [E+1] */) {
    const int lane = lane_id();
    for (int e = lane; e <= E; e += QMOE_WAVE) cnt[e] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int p = lane; p < n; p += QMOE_WAVE) {
        int e = ids[p];
        if (e < 0 || e >= E) e = E;
        atomicAdd(&cnt[e], 1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // Plan records of expert e (c pairs from sorted position off): passes of
    // tb pairs from record slot `slot` on.
    auto records = [&](int32_t *rec, int tb, int slot, int e, int off, int c) {
        for (int j = 0; j * tb < c; j++)
            *(u32x4 *)(rec + 4 * (slot + j)) =
                u32x4{(uint32_t)e, (uint32_t)(off + j * tb),
                      (uint32_t)min(off + (j + 1) * tb, off + c), 0u};
    };
    const bool planned = plan.rec_gu != nullptr;
    int carry = 0, acarry = 0, gcarry = 0, dcarry = 0;
    for (int base = 0; base < E; base += QMOE_WAVE) {
        const int e = base + lane;
        const int c = e < E ? cnt[e] : 0;
        const int inc = wave_inclusive_scan(c);
        const int off = carry + inc - c;
        const int a = c > 0 ? 1 : 0;
        const int ainc = wave_inclusive_scan(a);
        const int ng = planned ? (c + plan.tb_gu - 1) / plan.tb_gu : 0;
        const int nd = planned ? (c + plan.tb_dn - 1) / plan.tb_dn : 0;
        const int ginc = wave_inclusive_scan(ng), dinc = wave_inclusive_scan(nd);
        if (e < E) {
            wl.counts[e] = c;
            wl.offsets[e] = off;
            run[e] = off;
            if (a && wl.active) wl.active[acarry + ainc - 1] = e;
            if (a && planned) {
                records(plan.rec_gu, plan.tb_gu, gcarry + ginc - ng, e, off, c);
                records(plan.rec_dn, plan.tb_dn, dcarry + dinc - nd, e, off, c);
            }
        }
        carry += __builtin_amdgcn_readlane(inc, QMOE_WAVE - 1);
        acarry += __builtin_amdgcn_readlane(ainc, QMOE_WAVE - 1);
        gcarry += __builtin_amdgcn_readlane(ginc, QMOE_WAVE - 1);
        dcarry += __builtin_amdgcn_readlane(dinc, QMOE_WAVE - 1);
    }
    if (lane == 0) {
        wl.offsets[E] = carry;
        wl.n_invalid[0] = cnt[E];
        run[E] = carry;
        if (wl.n_active) wl.n_active[0] = acarry;
    }
    if (planned) {
        for (int a = gcarry + lane; a < plan.max_rec; a += QMOE_WAVE) plan.rec_gu[4 * a] = -1;
        for (int a = dcarry + lane; a < plan.max_rec; a += QMOE_WAVE) plan.rec_dn[4 * a] = -1;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    int nbits = 1;
    while ((1 << nbits) <= E) nbits++;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < n; base += QMOE_WAVE) {
        const int p = base + lane;
        const bool act = p < n;
        int e = E;
        if (act) {
            e = ids[p];
            if (e < 0 || e >= E) e = E;
        }
        uint64_t m = __ballot(act);
        for (int bit = 0; bit < nbits; bit++) {
            const bool set = (e >> bit) & 1;
            const uint64_t bb = __ballot(set);
            m &= set ? bb : ~bb;
        }
        const int rank = __popcll(m & below);
        const int cnt_e = __popcll(m);
        if (act) {
            const int pos = run[e] + rank;
            wl.pairs[pos] = e < E ? p : -1;
            wl.inv[p] = e < E ? pos : -1;
            if (e < E && plan.tok) {
                plan.tok[pos] = p / k;
                plan.wsort[pos] = topk_w[p];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (act && rank == 0) run[e] += cnt_e;
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace qmoe
