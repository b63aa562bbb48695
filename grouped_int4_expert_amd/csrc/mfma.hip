// Prefill path (bf16 activations): grouped per-expert GEMMs on the gfx950
// matrix cores.
//
// The pages describe the operation (colibri pull request "cuda+engine: full
// fmt=4 (grouped int4 gs=64) support": per-group scale scales[o*ng + i/gs],
// the fused gate+up pair, the down projection; the tensor-core W4A16
// kernels it names are per-row only and self-guarded, so they are prior art,
// not a design).  The design here is MI355X's own:
//
//  * Tiles come from the device worklist: (expert, first sorted row), at
//    most 256 rows each; activation rows are gathered through the sorted
//    pair list.
//  * A one-pass prep turns each bf16 activation row into f16 scaled by a
//    power of two 2^k_t (so the row maximum sits in [2^14, 2^15); bf16 -> f16
//    is then exact for all but subnormal-range values), with k permuted
//    inside every 8-element octet to the order the nibble unpack produces
//    (0,4,1,5,2,6,3,7) -- a dot product does not depend on term order.  The
//    gate/up epilogue multiplies by 2^-k_t.
//  * Weights never pass through LDS: each lane loads the 16 packed bytes its
//    MFMA operand needs straight from HBM/L2 and unpacks them in registers to
//    f16 q*s (nibble into the mantissa of 1024.0, packed add of -1032 gives
//    the exact code, packed multiply by the f16 group scale), so the f32
//    group scale costs no per-group accumulator work; rounding q*s to f16
//    adds ~2^-12 relative error per weight (bf16 would be 2^-9).
//  * v_mfma_f32_32x32x16_f16.  gate+up: block = 4 waves x (256 rows x 32
//    features of gate and of up), so each unpacked weight fragment feeds 8
//    row fragments (accumulators in AGPRs, one block per CU).  down
//    (mfma_down.hip): block = 4 waves x (128 rows x 64 features), two blocks
//    per CU.  A tile needing at most 1/2 or 1/4 of the block's rows runs a
//    loop with that many row fragments.
//  * The activation tile (rows x 64 f16 per group) reaches LDS by buffer
//    loads that write LDS directly, into a 4-stage ring with octets
//    XOR-swizzled by row; weights and scales run 4 groups ahead in
//    registers; the main loop (mfma_loop.h) interleaves the next k-step's
//    LDS reads and unpack with the current k-step's MFMAs.
#include "mfma_loop.h"

namespace qmoe {

// ---------------------------------------------------------------------------
// Activation prep: x bf16 [T][H] -> x16 f16 (scaled by 2^k_t, octet-permuted)
// and xinv[t] = 2^-k_t.  One block per row.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) xprep_kernel(const uint16_t *__restrict__ x, int H,
                                                    uint16_t *__restrict__ x16,
                                                    float *__restrict__ xinv) {
    __shared__ float red[4];
    const int64_t t = blockIdx.x;
    const uint16_t *row = x + t * H;
    float m = 0.f;
    for (int i = threadIdx.x * 8; i < H; i += 256 * 8) {
        const u32x4 v = *(const u32x4 *)(row + i);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            m = fmaxf(m, fabsf(__uint_as_float(w[j] << 16)));
            m = fmaxf(m, fabsf(__uint_as_float(w[j] & 0xffff0000u)));
        }
    }
    m = group_max<64>(m);
    if (lane_id() == 0) red[wave_id()] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int k = 0;
    if (m > 0.f && m <= 3.0e38f) {
        int e;
        frexpf(m, &e);
        k = min(15 - e, 126);
    }
    if (threadIdx.x == 0) xinv[t] = ldexpf(1.0f, -k);
    for (int i = threadIdx.x * 8; i < H; i += 256 * 8) {
        const u32x4 v = *(const u32x4 *)(row + i);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        _Float16 o[8];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            o[octet_pos(2 * j)] = (_Float16)ldexpf(__uint_as_float(w[j] << 16), k);
            o[octet_pos(2 * j + 1)] = (_Float16)ldexpf(__uint_as_float(w[j] & 0xffff0000u), k);
        }
        u32x4 out;
        out.x = __builtin_bit_cast(uint32_t, f16x2{o[0], o[1]});
        out.y = __builtin_bit_cast(uint32_t, f16x2{o[2], o[3]});
        out.z = __builtin_bit_cast(uint32_t, f16x2{o[4], o[5]});
        out.w = __builtin_bit_cast(uint32_t, f16x2{o[6], o[7]});
        *(u32x4 *)(x16 + t * H + i) = out;
    }
}

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

// out[t][n..n+3] = sum over j in pick order of Y[inv[t k + j]][n..n+3]; the
// four columns share one exponent (n % 4 == 0 stays inside a 16-column block).
__global__ void __launch_bounds__(256) combine_kernel(YBuf y, const int32_t *__restrict__ inv,
                                                      int k, int hidden, float *__restrict__ out) {
    const int t = blockIdx.y;
    const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (n >= hidden) return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; j++) {
        const int pos = inv[(int64_t)t * k + j];
        if (pos >= 0) {
            const f16x4 v = *(const f16x4 *)(y.v + (int64_t)pos * hidden + n);
            const float sc = ldexpf(1.0f, (int)y.e[(int64_t)pos * (hidden / 16) + n / 16] - 15);
            acc += f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]} * sc;
        }
    }
    *(f32x4 *)(out + (int64_t)t * hidden + n) = acc;
}

hipError_t launch_xprep(const uint16_t *x, int tokens, int hidden, uint16_t *x16, float *xinv,
                        hipStream_t st) {
    hipLaunchKernelGGL(xprep_kernel, dim3(tokens), dim3(256), 0, st, x, hidden, x16, xinv);
    return hipGetLastError();
}

hipError_t launch_mfma_gateup(const QMat &gate, const QMat &up, const uint16_t *x16,
                              const float *xinv, uint16_t *h16, const MfmaRoute &r,
                              hipStream_t st) {
    constexpr int BMK = GATEUP_BM;
    const int64_t items = r.wl.pairs ? (int64_t)r.max_tiles * (BM / BMK) : (r.ntok + BMK - 1) / BMK;
    const dim3 grid(xcd_grid(items * ((gate.rows + 127) / 128)));
    if (gate.group == 32)
        hipLaunchKernelGGL((mfma_gateup_kernel<BMK, true>), grid, dim3(MF_THREADS), 0, st, gate,
                           up, x16, xinv, h16, r);
    else
        hipLaunchKernelGGL((mfma_gateup_kernel<BMK, false>), grid, dim3(MF_THREADS), 0, st, gate,
                           up, x16, xinv, h16, r);
    return hipGetLastError();
}

hipError_t launch_combine(YBuf y, const int32_t *inv, int tokens, int k, int hidden, float *out,
                          hipStream_t st) {
    const dim3 grid((hidden / 4 + 255) / 256, tokens);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, y, inv, k, hidden, out);
    return hipGetLastError();
}

}  // namespace qmoe
