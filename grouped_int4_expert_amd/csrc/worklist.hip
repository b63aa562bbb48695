// Token-to-expert worklist built on the device, with no host round trip.
//
// pxq_llama.cpp release notes, section "Device-side MoE row map": the table
// mapping tokens to experts for one batched MoE layer is built entirely on
// the device (histogram, scan, fill), replacing a host build whose
// device-to-host sync sat on the critical path; the device and host builds
// agree bit for bit.  Here the table is a stable counting sort of the pairs
// p = t*k + j by expert id, so the result is unique:
//   counts[e], offsets[e] (exclusive scan), pairs[pos] (ascending expert,
//   ascending p inside an expert, -1 in the tail), inv[p] (position or -1),
//   n_invalid (ids outside [0, E), dropped).
// The same pass also lists the experts that have work (ascending) and cuts
// each expert's rows into tiles of tile_m rows for the grouped GEMMs: at
// most ceil(n / tile_m) + E tiles, so grids are launched at that bound and
// surplus blocks exit.  For the bf16 prefill, experts with at most
// skinny_max pairs are listed as 16-pair passes instead (skinny.hip).
#include "common.h"
#include "launch.h"
#include "split16.h"
#include "wl_wave.h"

namespace qmoe {

constexpr int WL_THREADS = 1024;
constexpr int WL_MAX_E = 1024;
constexpr int WL_CHUNK = 2048;          // pairs per block in the multi-block build (4096: 5 us slower at 65536 pairs)

// Exclusive scan of v over the block (blockDim.x == 1024); returns the
// exclusive prefix of this thread and writes the block total to *total.
__device__ int block_exclusive_scan(int v, int *sh_wave, int *total) {
    const int lane = lane_id(), w = wave_id();
    int x = v;
#pragma unroll
    for (int o = 1; o < QMOE_WAVE; o <<= 1) {
        const int y = __shfl_up(x, o, QMOE_WAVE);
        if (lane >= o) x += y;
    }
    if (lane == QMOE_WAVE - 1) sh_wave[w] = x;
    __syncthreads();
    if (w == 0) {
        const int nw = blockDim.x / QMOE_WAVE;
        int s = lane < nw ? sh_wave[lane] : 0;
#pragma unroll
        for (int o = 1; o < QMOE_WAVE; o <<= 1) {
            const int y = __shfl_up(s, o, QMOE_WAVE);
            if (lane >= o) s += y;
        }
        if (lane < nw) sh_wave[lane] = s;   // inclusive wave totals
    }
    __syncthreads();
    const int before = (w > 0 ? sh_wave[w - 1] : 0) + x - v;
    *total = sh_wave[blockDim.x / QMOE_WAVE - 1];
    __syncthreads();
    return before;
}

struct WlShared {
    int tot[WL_MAX_E + 1];   // pairs per expert (slot E: dropped ids)
    int run[WL_MAX_E + 1];   // next free position of this block per expert
    int wave[WL_THREADS / QMOE_WAVE];
};

// Per-block histogram of the pair range [lo, hi).
__global__ void __launch_bounds__(256) wl_hist_kernel(const int32_t *__restrict__ ids, int n,
                                                      int E, int32_t *__restrict__ hist) {
    __shared__ int h[WL_MAX_E + 1];
    for (int e = threadIdx.x; e <= E; e += blockDim.x) h[e] = 0;
    __syncthreads();
    const int lo = blockIdx.x * WL_CHUNK, hi = min(n, lo + WL_CHUNK);
    for (int p = lo + threadIdx.x; p < hi; p += blockDim.x) {
        int e = ids[p];
        if (e < 0 || e >= E) e = E;
        atomicAdd(&h[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += blockDim.x)
        hist[(int64_t)blockIdx.x * (E + 1) + e] = h[e];
}

// Build (or, with nb > 1, finish) the worklist for the pairs of block b.
// nb == 1: the block counts its own pairs; otherwise hist holds the per-block
// histograms from wl_hist_kernel.
__device__ void wl_block(const int32_t *__restrict__ ids, int n, int E, const Worklist &wl,
                         const int32_t *__restrict__ hist, int nb, int b, WlShared &sh) {
    const int tid = threadIdx.x;
    const int lo = nb == 1 ? 0 : b * WL_CHUNK;
    const int hi = nb == 1 ? n : min(n, lo + WL_CHUNK);

    // 1. totals per expert and this block's starting rank inside each expert
    if (nb == 1) {
        for (int e = tid; e <= E; e += blockDim.x) { sh.tot[e] = 0; sh.run[e] = 0; }
        __syncthreads();
        for (int p = tid; p < n; p += blockDim.x) {
            int e = ids[p];
            if (e < 0 || e >= E) e = E;
            atomicAdd(&sh.tot[e], 1);
        }
    } else {
        for (int e = tid; e <= E; e += blockDim.x) {
            // eight independent loads in flight at a time (a plain loop
            // waits for each block's count before loading the next)
            int tot = 0, pre = 0;
            for (int j0 = 0; j0 < nb; j0 += 8) {
                int c[8];
#pragma unroll
                for (int u = 0; u < 8; u++)
                    c[u] = j0 + u < nb ? hist[(int64_t)(j0 + u) * (E + 1) + e] : 0;
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    tot += c[u];
                    pre += (j0 + u < b) ? c[u] : 0;
                }
            }
            sh.tot[e] = tot;
            sh.run[e] = pre;
        }
    }
    __syncthreads();

    // 2. exclusive scan over experts -> offsets; dropped ids go after them
    const int my = tid < E ? sh.tot[tid] : 0;
    int n_valid;
    const int off = block_exclusive_scan(my, sh.wave, &n_valid);
    if (tid < E) sh.run[tid] += off;
    if (tid == 0) sh.run[E] += n_valid;
    if (b == 0) {
        if (tid < E) {
            wl.counts[tid] = my;
            wl.offsets[tid] = off;
        }
        if (tid == 0) {
            wl.offsets[E] = n_valid;
            wl.n_invalid[0] = sh.tot[E];
        }
    }
    __syncthreads();

    // 3. block 0: list of experts with work and the tile list
    if (b == 0 && wl.active) {
        int na;
        const int pos = block_exclusive_scan(my > 0 ? 1 : 0, sh.wave, &na);
        if (tid < E && my > 0) wl.active[pos] = tid;
        if (tid == 0) wl.n_active[0] = na;
    }
    if (b == 0 && wl.tiles) {
        // experts with 1..skinny_max pairs take SK_TP-row passes instead
        const bool pass = wl.spass && my <= wl.skinny_max;
        const int nt = pass ? 0 : (my + wl.tile_m - 1) / wl.tile_m;
        int ntot;
        const int t0 = block_exclusive_scan(nt, sh.wave, &ntot);
        for (int i = 0; i < nt; i++) {
            wl.tiles[2 * (t0 + i)] = tid;
            wl.tiles[2 * (t0 + i) + 1] = i * wl.tile_m;
        }
        if (tid == 0) wl.n_tiles[0] = ntot;
        if (wl.spass) {
            const int np = pass ? (my + SK_TP - 1) / SK_TP : 0;
            int ptot;
            const int p0 = block_exclusive_scan(np, sh.wave, &ptot);
            for (int i = 0; i < np; i++) {
                wl.spass[2 * (p0 + i)] = tid;
                wl.spass[2 * (p0 + i) + 1] = i * SK_TP;
            }
            if (tid == 0) wl.n_spass[0] = ptot;
        }
    }

    // 4. stable fill: pairs of this block in order, one wave at a time
    int nbits = 1;
    while ((1 << nbits) <= E) nbits++;
    const int lane = lane_id(), w = wave_id(), nw = blockDim.x / QMOE_WAVE;
    for (int base = lo; base < hi; base += blockDim.x) {
        const int p = base + tid;
        const bool act = p < hi;
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
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        const int rank = __popcll(m & below);
        const int cnt = __popcll(m);
        for (int turn = 0; turn < nw; turn++) {
            if (w == turn && act) {
                const int pos = sh.run[e] + rank;
                if (e < E) {
                    wl.pairs[pos] = p;
                    wl.inv[p] = pos;
                } else {
                    wl.pairs[pos] = -1;
                    wl.inv[p] = -1;
                }
                if (rank == 0) sh.run[e] += cnt;
            }
            __syncthreads();
        }
    }
}

__global__ void __launch_bounds__(WL_THREADS) wl_fill_kernel(const int32_t *__restrict__ ids,
                                                             int n, int E, Worklist wl,
                                                             const int32_t *__restrict__ hist,
                                                             int nb) {
    __shared__ WlShared sh;
    wl_block(ids, n, E, wl, hist, nb, blockIdx.x, sh);
}

int64_t wl_scratch_ints(int64_t n, int E) {
    const int64_t nb = (n + WL_CHUNK - 1) / WL_CHUNK;
    return nb > 1 ? nb * (E + 1) : 0;
}

hipError_t launch_worklist(const int32_t *ids, int n, int k, int E, const Worklist &wl,
                           int32_t *scratch, hipStream_t st) {
    (void)k;
    const int nb = n > WL_CHUNK ? (n + WL_CHUNK - 1) / WL_CHUNK : 1;
    if (nb > 1)
        hipLaunchKernelGGL(wl_hist_kernel, dim3(nb), dim3(256), 0, st, ids, n, E, scratch);
    hipLaunchKernelGGL(wl_fill_kernel, dim3(nb), dim3(WL_THREADS), 0, st, ids, n, E, wl,
                       (const int32_t *)scratch, nb);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Activation digits (see common.h).  One 32-lane half-wave per chunk.
// ---------------------------------------------------------------------------
__device__ void xdigits_chunks(const float *__restrict__ x, int rows, int cols, int src_cols,
                               XDigits xd, int64_t first_half, int64_t stride_halves) {
    const int cpr = cols / XD_CHUNK;
    const int64_t nchunks = (int64_t)rows * cpr;
    const int half = (threadIdx.x >> 5);
    const int sub = threadIdx.x & 31;
    for (int64_t c = first_half + half; c < nchunks; c += stride_halves) {
        const int64_t r = c / cpr, ch = c - r * cpr;
        const int e = (int)ch * XD_CHUNK + sub;
        const float v = e < src_cols ? x[r * src_cols + e] : 0.0f;
        uint32_t *dst = xd.dig + c * XD_DWORDS;
        const float f = quantise_chunk32<true>(v, [&](int plane, int dw, uint32_t val) {
            dst[plane * 4 + dw] = val;
        });
        if (sub == 0) xd.fac[c] = f;
    }
}

__global__ void __launch_bounds__(256) xdigits_kernel(const float *__restrict__ x, int rows,
                                                      int cols, int src_cols, XDigits xd) {
    const int64_t halves_per_block = blockDim.x / 32;
    xdigits_chunks(x, rows, cols, src_cols, xd, (int64_t)blockIdx.x * halves_per_block,
                   (int64_t)gridDim.x * halves_per_block);
}

hipError_t launch_xdigits(const float *x, int rows, int cols, int src_cols, XDigits xd,
                          hipStream_t st) {
    const int64_t nchunks = (int64_t)rows * (cols / XD_CHUNK);
    int64_t g = (nchunks + 7) / 8;
    if (g > 4096) g = 4096;
    hipLaunchKernelGGL(xdigits_kernel, dim3((int)g), dim3(256), 0, st, x, rows, cols, src_cols,
                       xd);
    return hipGetLastError();
}

// Block 0 builds the worklist; the other blocks turn x into digits (when
// xd.dig is set: the digit variant of the decode path) and clear out (the down
// projection accumulates into it).
__global__ void __launch_bounds__(WL_THREADS) decode_prep_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ topk_w, int n, int k, int E,
    Worklist wl, DecodePlan plan, const float *__restrict__ x, int tokens, int hidden, XDigits xd,
    XSplit xs, float *__restrict__ out) {
    if (blockIdx.x == 0) {
        __shared__ int cnt[WL_MAX_E + 1], run[WL_MAX_E + 1];
        if (wave_id() == 0) wl_wave(ids, topk_w, n, k, E, wl, plan, cnt, run);
        return;
    }
    const int64_t hpb = blockDim.x / 32;
    const int64_t first = (int64_t)(blockIdx.x - 1) * hpb;
    const int64_t stride = (int64_t)(gridDim.x - 1) * hpb;
    if (xd.dig) xdigits_chunks(x, tokens, hidden, hidden, xd, first, stride);
    if (xs.v) {
        // one block per row: 16 inputs per thread cover rows up to 16384
        __shared__ uint32_t red;
        sp_split_rows<2>(x, tokens, hidden, xs.v, xs.f, blockIdx.x - 1, gridDim.x - 1, &red);
    }
    const int64_t total = (int64_t)tokens * hidden;
    for (int64_t i = (int64_t)(blockIdx.x - 1) * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)(gridDim.x - 1) * blockDim.x)
        out[i] = 0.0f;
}

hipError_t launch_decode_prep(const int32_t *ids, const float *topk_w, int n, int k, int E,
                              const Worklist &wl, const DecodePlan &plan, const float *x,
                              int tokens, int hidden, XDigits xd, XSplit xs, float *out,
                              hipStream_t st) {
    const int64_t nchunks = (int64_t)tokens * (hidden / XD_CHUNK);
    int64_t g = (nchunks + 31) / 32;     // 32 half-waves per 1024-thread block
    if (g < 1) g = 1;
    if (g > 1024) g = 1024;
    hipLaunchKernelGGL(decode_prep_kernel, dim3((int)g + 1), dim3(WL_THREADS), 0, st, ids,
                       topk_w, n, k, E, wl, plan, x, tokens, hidden, xd, xs, out);
    return hipGetLastError();
}

}  // namespace qmoe
