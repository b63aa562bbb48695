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
//    per CU.  A tile of `rows` rows runs a loop over ceil(rows / 32) row
//    fragments.
//  * The activation tile (rows x 64 f16 per group) reaches LDS by buffer
//    loads that write LDS directly, into a 4-stage ring with octets
//    XOR-swizzled by row; weights and scales run 4 groups ahead in
//    registers; the main loop (mfma_loop.h) interleaves the next k-step's
//    LDS reads and unpack with the current k-step's MFMAs.
#include "mfma_gateup.h"

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

// out[t][n..n+7] = sum over j in pick order of Y[inv[t k + j]][n..n+7]; the
// eight columns share one exponent (n % 8 == 0 stays inside a 16-column
// block), one 16-byte load per row.  Token t = blockIdx.z * gridDim.y +
// blockIdx.y (a grid dimension other than x holds at most 65535 blocks).
__global__ void __launch_bounds__(256) combine_kernel(YBuf y, const int32_t *__restrict__ inv,
                                                      int tokens, int k, int hidden,
                                                      float *__restrict__ out) {
    const int t = blockIdx.z * gridDim.y + blockIdx.y;
    const int n = (blockIdx.x * 256 + threadIdx.x) * 8;
    if (t >= tokens || n >= hidden) return;
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; j++) {
        const int pos = inv[(int64_t)t * k + j];
        if (pos >= 0) {
            const f16x8 v = *(const f16x8 *)(y.v + (int64_t)pos * hidden + n);
            const float sc = ldexpf(1.0f, (int)y.e[(int64_t)pos * (hidden / 16) + n / 16] - 15);
            lo += f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]} * sc;
            hi += f32x4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]} * sc;
        }
    }
    float *o = out + (int64_t)t * hidden + n;
    *(f32x4 *)o = lo;
    *(f32x4 *)(o + 4) = hi;
}

hipError_t launch_xprep(const uint16_t *x, int tokens, int hidden, uint16_t *x16, float *xinv,
                        hipStream_t st) {
    hipLaunchKernelGGL(xprep_kernel, dim3(tokens), dim3(256), 0, st, x, hidden, x16, xinv);
    return hipGetLastError();
}

hipError_t launch_mfma_gateup(const QMat &gate, const QMat &up, const uint16_t *x16,
                              const float *xinv, uint16_t *h16, const MfmaRoute &r,
                              hipStream_t st) {
    if (gate.group == 32) return launch_gateup_g32(gate, up, x16, xinv, h16, r, st);
    return launch_gateup<false>(gate, up, x16, xinv, h16, r, st);
}

hipError_t launch_combine(YBuf y, const int32_t *inv, int tokens, int k, int hidden, float *out,
                          hipStream_t st) {
    const int gy = tokens < 65535 ? tokens : 65535;
    const dim3 grid((hidden / 8 + 255) / 256, gy, (tokens + gy - 1) / gy);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, y, inv, tokens, k, hidden, out);
    return hipGetLastError();
}

}  // namespace qmoe
