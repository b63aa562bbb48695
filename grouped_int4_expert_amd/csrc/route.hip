// Router: top-k of each token's E logits and the softmax over the picked k,
// the step that produces the routing ids and weights the layer consumes.
//
// What is computed follows the colibri pull request "cuda+engine: full fmt=4
// (grouped int4 gs=64) support", the quoted issue's list of CPU work: top-K
// with one "taken" flag per expert, K passes over the E logits.  Readings:
// a pass picks the untaken expert with the largest logit, the lowest id
// among equal logits, NaN ranking as -infinity; slot order is pick order;
// weight of slot s = exp(l_s - l_0) / sum_j exp(l_j - l_0) over the picked.
//
// MI355X mapping: one wave per token.  Lane l holds the logits of experts
// l, l + 64, ... (EPL per lane, read with coalesced 4-byte loads) and a bit
// mask of which of them are taken.  A pass is a per-lane scan in ascending
// id followed by a wave argmax over (key, -id) with DPP row shifts and row
// broadcasts (VALU only, no LDS round trips), so the pick equals the
// sequential scan's; lane 63 holds the winner and a readlane broadcasts it.
// The softmax runs on lane 0 in f32 over the k picked logits.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace qmoe {

// (key, id) order: larger key first, then lower id.
__device__ __forceinline__ bool route_better(float ka, int ia, float kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

// One step of the argmax: combine with the (key, id) of the lane the DPP
// control selects; lanes without a source (or masked off) see the identity
// (-inf, INT_MAX).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_step(float &bk, int &bi) {
    const float ok = __int_as_float(__builtin_amdgcn_update_dpp(
        (int)0xff800000, __float_as_int(bk), CTRL, ROW_MASK, 0xf, false));
    const int oi = __builtin_amdgcn_update_dpp(0x7fffffff, bi, CTRL, ROW_MASK, 0xf, false);
    if (route_better(ok, oi, bk, bi)) {
        bk = ok;
        bi = oi;
    }
}

// Wave argmax of (key, id): row shifts 1, 2, 4, 8 fold each row of 16 into
// its last lane, row_bcast:15 and row_bcast:31 fold the rows into lane 63.
// Returns the winning id in every lane.
__device__ __forceinline__ int route_wave_argmax(float bk, int bi) {
    argmax_step<0x111, 0xf>(bk, bi);
    argmax_step<0x112, 0xf>(bk, bi);
    argmax_step<0x114, 0xf>(bk, bi);
    argmax_step<0x118, 0xf>(bk, bi);
    argmax_step<0x142, 0xa>(bk, bi);
    argmax_step<0x143, 0xc>(bk, bi);
    return __builtin_amdgcn_readlane(bi, 63);
}

template <int EPL>
__global__ void __launch_bounds__(256) route_kernel(const float *__restrict__ logits, int tokens,
                                                    int E, int k, int32_t *__restrict__ ids,
                                                    float *__restrict__ w) {
    const int t = blockIdx.x * 4 + wave_id();
    if (t >= tokens) return;
    const int lane = lane_id();
    const float *row = logits + (int64_t)t * E;
    float key[EPL];
    uint32_t absent = 0;   // bit i: expert lane + 64 i is taken or does not exist
#pragma unroll
    for (int i = 0; i < EPL; i++) {
        const int e = lane + 64 * i;
        if (e < E) {
            const float v = row[e];
            key[i] = isnan(v) ? -INFINITY : v;
        } else {
            key[i] = -INFINITY;
            absent |= 1u << i;
        }
    }
    float picked[MAX_ROUTE_TOPK];
    int pick_id[MAX_ROUTE_TOPK];
    for (int s = 0; s < k; s++) {
        float bk = -INFINITY;
        int bi = 0x7fffffff;   // no candidate in this lane
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            const int e = lane + 64 * i;
            if (!(absent >> i & 1u) && route_better(key[i], e, bk, bi)) {
                bk = key[i];
                bi = e;
            }
        }
        bi = route_wave_argmax(bk, bi);
        // every lane now holds the winner
        if ((bi & 63) == lane) absent |= 1u << (bi >> 6);
        pick_id[s] = bi;
    }
    if (lane == 0) {
        // logit values of the picks (NaN kept as NaN for the weights)
        for (int s = 0; s < k; s++) picked[s] = row[pick_id[s]];
        const float top = picked[0];
        float sum = 0.f;
        for (int s = 0; s < k; s++) {
            picked[s] = expf(picked[s] - top);
            sum += picked[s];
        }
        for (int s = 0; s < k; s++) {
            ids[(int64_t)t * k + s] = pick_id[s];
            w[(int64_t)t * k + s] = picked[s] / sum;
        }
    }
}

bool route_supported(int experts, int k) {
    return experts >= 1 && experts <= 64 * 16 && k >= 1 && k <= experts && k <= MAX_ROUTE_TOPK;
}

hipError_t launch_route(const float *logits, int tokens, int experts, int k, int32_t *ids,
                        float *w, hipStream_t st) {
    const dim3 grid((tokens + 3) / 4);
    const int epl = (experts + 63) / 64;
#define R(N)                                                                                \
    if (epl <= N) {                                                                         \
        hipLaunchKernelGGL((route_kernel<N>), grid, dim3(256), 0, st, logits, tokens, experts, \
                           k, ids, w);                                                      \
        return hipGetLastError();                                                           \
    }
    R(1) R(2) R(4) R(8) R(16)
#undef R
    return hipErrorInvalidValue;
}

}  // namespace qmoe
