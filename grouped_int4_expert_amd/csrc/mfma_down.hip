// Prefill down projection on the matrix cores (see mfma.hip for the design).
#include "mfma_loop.h"

namespace qmoe {

// ---------------------------------------------------------------------------
// down: block = (256 features of H, one tile of <=256 rows); wave w:
// features n0 + 64w + 32j + (lane%32), j = 0, 1.
// Routed: Y[pos] = w * (D h); direct: out[pos] = D h.
// ---------------------------------------------------------------------------
template <int BMK, bool G32>
__global__ void __launch_bounds__(MF_THREADS, occ_of<BMK>()) mfma_down_kernel(
    QMat D, const uint16_t *__restrict__ h16, float *__restrict__ out, YBuf yb, MfmaRoute r) {
    constexpr int MF = mf_of<BMK>();
    __shared__ __attribute__((aligned(1024))) uint16_t s0[BMK * 64], s1[BMK * 64],
        s2[BMK * 64], s3[BMK * 64];
    __shared__ __attribute__((aligned(16))) float sW[BMK];

    const int H = D.rows, F = D.cols, ng = F / 64;
    int tile, cb;
    if (!work_item<BMK>(r, (H + 255) / 256, tile, cb)) return;
    TileInfo ti;
    if (!tile_info<BMK>(r, tile, ti)) return;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int hh = lane >> 5;
    const bool routed = r.wl.pairs != nullptr;
    // routing weight of each row, fetched before the main loop (the barriers
    // inside it publish sW)
    for (int m = tid; m < BMK; m += MF_THREADS)
        sW[m] = m >= ti.rows ? 0.f : routed ? r.topk_w[r.wl.pairs[ti.pos0 + m]] : 1.0f;

    LoopSrc<MF> src;
    src.a = make_rsrc(h16, (int64_t)r.h_rows * F * 2);
    src.gshift = group_shift(D);
    tile_offsets(src, ti.rows, F, [&](int m) -> int64_t { return ti.pos0 + m; });
    int ncol[NF];
#pragma unroll
    for (int j = 0; j < NF; j++) {
        ncol[j] = cb * 256 + 64 * w + 32 * j + (lane & 31);
        const int nn = ncol[j] < H ? ncol[j] : 0;
        src.q[j] = make_rsrc(D.q + (int64_t)ti.e * D.q_stride, (int64_t)H * (F / 2));
        const int spr = scales_per_row(D);
        src.s[j] = make_rsrc(D.s + (int64_t)ti.e * D.s_stride, (int64_t)H * spr * 4);
        src.qoff[j] = (uint32_t)(nn * (F / 2) + 16 * hh);
        src.soff[j] = (uint32_t)(nn * spr * 4 + (G32 ? 4 * hh : 0));
    }

    Frags<MF> fr;
    run_mainloop<MF, G32>(fr, src, ng, ti.rows, s0, s1, s2, s3);

    if (!routed) {   // direct mode (one expert): out = D h in f32
#pragma unroll
        for (int i = 0; i < MF; i++) {
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int m = acc_row(i, v, lane);
                if (m < ti.rows) {
#pragma unroll
                    for (int j = 0; j < NF; j++)
                        if (ncol[j] < H) out[(int64_t)(ti.pos0 + m) * H + ncol[j]] = fr.acc[i][j][v];
                }
            }
        }
        return;
    }
    // Routed: Y = w (D h) as f16 with a power-of-two exponent per block of 4
    // rows (the lane's accumulators 4g..4g+3) x 16 columns (one DPP row of
    // lanes): the block maximum is scaled into [2^14, 2^15), so every value
    // keeps f16's 11-bit significand and none overflows.  Lane r (< 4) of each
    // 16-lane row stores the exponent of row r of the block.
    // Stores go through descriptors that end at row ti.rows (rows past the
    // tile are dropped); columns past H and the exponent stores of lanes
    // 4..15 of each DPP row take an offset past any descriptor.
    const int hs = H / 16;
    const __amdgpu_buffer_rsrc_t yv = make_rsrc(yb.v + (int64_t)ti.pos0 * H, (int64_t)ti.rows * H * 2);
    const __amdgpu_buffer_rsrc_t ye = make_rsrc(yb.e + (int64_t)ti.pos0 * hs, (int64_t)ti.rows * hs);
    const int er = lane & 15;   // row of the block whose exponent this lane stores
    uint32_t voff[NF], eoff[NF];
#pragma unroll
    for (int j = 0; j < NF; j++) {
        const bool on = ncol[j] < H;
        voff[j] = on ? (uint32_t)((4 * hh * H + ncol[j]) * 2) : OOB_OFFSET;
        eoff[j] = on && er < 4 ? (uint32_t)((4 * hh + er) * hs + ((ncol[j] - er) >> 4)) : OOB_OFFSET;
    }
#pragma unroll
    for (int i = 0; i < MF; i++) {
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int rb = 32 * i + 8 * g;   // rows rb + 4 hh .. + 3
            const f32x4 w4 = *(const f32x4 *)&sW[rb + 4 * hh];
#pragma unroll
            for (int j = 0; j < NF; j++) {
                float val[4], mx = 0.f;
#pragma unroll
                for (int rr = 0; rr < 4; rr++) {
                    val[rr] = w4[rr] * fr.acc[i][j][4 * g + rr];
                    mx = fmaxf(mx, fabsf(val[rr]));
                }
                // mx >= 0 and never NaN (fmaxf drops NaN), so its bits order
                // like its value; mx in [2^(ex-1), 2^ex) with ex = exponent
                // field - 126.  ex is kept in [-111, 127]: 2^(15-ex) and the
                // combine's 2^(ex-15) stay normal f32 numbers and ex fits int8
                // (blocks below 2^-111 keep fewer bits; |Y| >= 2^127 saturates).
                const uint32_t mb = max16_u32_dpp(__float_as_uint(mx));
                int ex = 0;
                if (mb != 0 && mb < 0x7f800000u) ex = min(max((int)(mb >> 23) - 126, -111), 127);
                const float sc = __uint_as_float((uint32_t)(142 - ex) << 23);   // 2^(15 - ex)
#pragma unroll
                for (int rr = 0; rr < 4; rr++)
                    __builtin_amdgcn_raw_buffer_store_b16(
                        __builtin_bit_cast(uint16_t, (_Float16)(val[rr] * sc)), yv,
                        voff[j] + (uint32_t)((rb + rr) * H * 2), 0, 0);
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(int8_t)ex, ye,
                                                     eoff[j] + (uint32_t)(rb * hs), 0, 0);
            }
        }
    }
}

// out[t] = sum_j Y[inv[t*k + j]], slots in order; 4 floats per thread.
hipError_t launch_mfma_down(const QMat &down, const uint16_t *h16, float *out, YBuf y,
                            const MfmaRoute &r, hipStream_t st) {
    constexpr int BMK = DOWN_BM;
    const int64_t items = r.wl.pairs ? (int64_t)r.max_tiles * (BM / BMK) : (r.ntok + BMK - 1) / BMK;
    const dim3 grid(xcd_grid(items * ((down.rows + 255) / 256)));
    if (down.group == 32)
        hipLaunchKernelGGL((mfma_down_kernel<BMK, true>), grid, dim3(MF_THREADS), 0, st, down, h16,
                           out, y, r);
    else
        hipLaunchKernelGGL((mfma_down_kernel<BMK, false>), grid, dim3(MF_THREADS), 0, st, down,
                           h16, out, y, r);
    return hipGetLastError();
}

}  // namespace qmoe
