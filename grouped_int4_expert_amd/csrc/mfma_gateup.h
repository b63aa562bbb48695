// Prefill gate+up kernel (see mfma.hip for the design).  Its two
// instances (group 32, and group 64 * 2^j or per row) are compiled in
// separate sources, mfma.hip and mfma_gateup_g32.hip.
#pragma once

#include "mfma_loop.h"

namespace qmoe {

// ---------------------------------------------------------------------------
// gate+up: block = (128 features of F for gate and up, one tile of <=256
// rows).  Wave w: features n0 + 32w .. +32 of gate (frag 0) and up (frag 1).
// Output h = silu(g) * u as f16 at sorted position pos0 + m, octet-permuted
// in the feature index (the down projection's k).
// ---------------------------------------------------------------------------
template <int BMK, bool G32>
__global__ void __launch_bounds__(MF_THREADS, occ_of<BMK>()) mfma_gateup_kernel(
    QMat G, QMat Up, const uint16_t *__restrict__ x16, const float *__restrict__ xinv,
    uint16_t *__restrict__ h16, MfmaRoute r) {
    constexpr int MF = mf_of<BMK>();
    __shared__ __attribute__((aligned(1024))) uint16_t s0[BMK * 64], s1[BMK * 64],
        s2[BMK * 64], s3[BMK * 64];
    __shared__ __attribute__((aligned(16))) float sInv[BMK];

    const int H = G.cols, F = G.rows, ng = H / 64;
    int tile, cb;
    if (!work_item<BMK>(r, (F + 127) / 128, tile, cb)) return;
    TileInfo ti;
    if (!tile_info<BMK>(r, tile, ti)) return;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int n = cb * 128 + 32 * w + (lane & 31);
    const bool wave_on = cb * 128 + 32 * w < F;
    auto token = [&](int m) -> int64_t {
        return r.wl.pairs ? r.wl.pairs[ti.pos0 + m] / r.k : ti.pos0 + m;
    };

    LoopSrc<MF> src;
    src.a = make_rsrc(x16, (int64_t)r.x_rows * H * 2);
    src.gshift = group_shift(G);
    tile_offsets(src, ti.rows, H, token);
    for (int m = tid; m < BMK; m += MF_THREADS) sInv[m] = m < ti.rows ? xinv[token(m)] : 0.f;
    const int hh = lane >> 5;
    const int nn = wave_on ? n : 0;       // idle waves read row 0 (valid) and store nothing
    const QMat *mats[NF] = {&G, &Up};
#pragma unroll
    for (int j = 0; j < NF; j++) {
        const QMat &M = *mats[j];
        src.q[j] = make_rsrc(M.q + (int64_t)ti.e * M.q_stride, (int64_t)F * (H / 2));
        const int spr = scales_per_row(M);
        src.s[j] = make_rsrc(M.s + (int64_t)ti.e * M.s_stride, (int64_t)F * spr * 4);
        src.qoff[j] = (uint32_t)(nn * (H / 2) + 16 * hh);
        src.soff[j] = (uint32_t)(nn * spr * 4 + (G32 ? 4 * hh : 0));
    }

    Frags<MF> fr;
    run_mainloop<MF, G32>(fr, src, ng, ti.rows, s0, s1, s2, s3);

    if (!wave_on) return;
    // h rows of the tile through a descriptor that ends at row ti.rows:
    // stores of rows past the tile fall outside it and are dropped, so the
    // loop has no branches; the row offset rides in the vector offset.
    const int npos = (n & ~7) + octet_pos(n & 7);
    const __amdgpu_buffer_rsrc_t hr =
        make_rsrc(h16 + (int64_t)ti.pos0 * F, (int64_t)ti.rows * F * 2);
    const uint32_t hoff = (uint32_t)((4 * hh * F + npos) * 2);
#pragma unroll
    for (int i = 0; i < MF; i++) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const f32x4 sc4 = *(const f32x4 *)&sInv[32 * i + 8 * q + 4 * hh];
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
                const int v = 4 * q + rr;   // row 32 i + 8 q + 4 hh + rr
                const float h = silu_fast(fr.acc[i][0][v] * sc4[rr]) * (fr.acc[i][1][v] * sc4[rr]);
                __builtin_amdgcn_raw_buffer_store_b16(
                    __builtin_bit_cast(uint16_t, (_Float16)h), hr,
                    hoff + (uint32_t)((32 * i + 8 * q + rr) * F * 2), 0, 0);
            }
        }
    }
}

template <bool G32>
hipError_t launch_gateup(const QMat &gate, const QMat &up, const uint16_t *x16, const float *xinv,
                         uint16_t *h16, const MfmaRoute &r, hipStream_t st) {
    constexpr int BMK = GATEUP_BM;
    const int64_t items = r.wl.pairs ? (int64_t)r.max_tiles * (BM / BMK) : (r.ntok + BMK - 1) / BMK;
    const dim3 grid(xcd_grid(items * ((gate.rows + 127) / 128)));
    hipLaunchKernelGGL((mfma_gateup_kernel<BMK, G32>), grid, dim3(MF_THREADS), 0, st, gate, up,
                       x16, xinv, h16, r);
    return hipGetLastError();
}

// Group-32 instance (mfma_gateup_g32.hip).
hipError_t launch_gateup_g32(const QMat &gate, const QMat &up, const uint16_t *x16,
                             const float *xinv, uint16_t *h16, const MfmaRoute &r, hipStream_t st);

}  // namespace qmoe
