// Exact three-part f16 form of f32 activations, the operand of the
// matrix-core decode kernels (gemv_mfma.hip).
//
// A row of f32 activations is scaled by one power of two 2^E per row so that
// its largest magnitude lies in [2^14, 2^15), and each scaled element xs is
// written as p0 + p1 + p2 with p0 = f16(xs), p1 = f16(xs - p0),
// p2 = f16(xs - p0 - p1) (round to nearest).  Each residual is exact in f32;
// xs has 24 significant bits and every part takes 11, so the three parts sum
// to xs exactly whenever the last residual's bits are f16-representable,
// which holds for |xs| >= 1/2 (elements within 2^15 of the row maximum).
// Smaller elements lose at most 2^-25 in scaled units, 2^-39 of the row
// maximum.  Products of the parts with exact f16 weight codes are exact, and
// the matrix cores accumulate them in f32.
//
// Operand layout.  A load step covers 128 consecutive inputs.  The weight
// side (B operand of v_mfma_f32_16x16x32_f16: lane l holds row l % 16 and
// inputs 8 (l / 16) .. + 8 of an MFMA step) reads 16 packed bytes per lane
// at byte 16 g of the step's 64 bytes (g = l / 16), so lane group g holds
// inputs 32 g .. 32 g + 31 and dword j of the load holds 32 g + 8 j .. + 7.
// A swap of the upper 32 lanes of dwords 0, 1 with the lower 32 lanes of
// dwords 2, 3 (v_permlane32_swap) leaves MFMA steps 0 and 1 with inputs of
// the first 64-input half only and steps 2 and 3 with the second, so a scale
// group of 64 never straddles an MFMA step.  Inside a dword, nibble pair
// (j, j + 4) unpacks into f16 elements (2 j, 2 j + 1).  Input c of a load
// step is therefore MFMA step i, lane group g, element e with
//   i = 2 c[6] + c[3],  g = c[5] + 2 c[4],  e = 2 (c & 3) + c[2]
// and, inversely, c = 64 (i >> 1) + 8 (i & 1) + 32 (g & 1) + 16 (g >> 1)
//                    + (e >> 1) + 4 (e & 1).
// The activation side (A operand: lane l holds row m = l % 16 and the same
// inputs as the weight lane l) uses the same map, so the elements pair up.
#pragma once

#include "common.h"

namespace qmoe {

// Inputs per load step and f16 parts per activation.
constexpr int SP_STEP = 128;
constexpr int SP_PARTS = 3;

// First input of the 8-input run that MFMA step i, lane group g holds.
__host__ __device__ constexpr int sp_run(int i, int g) {
    return 64 * (i >> 1) + 8 * (i & 1) + 32 * (g & 1) + 16 * (g >> 1);
}
// Input (inside the run) of element e.
__host__ __device__ constexpr int sp_elem(int e) { return (e >> 1) + 4 * (e & 1); }

// Row scale: 2^E with max|x| * 2^E in [2^14, 2^15) (E clamped to
// [-126, 126]: an all-zero row takes 2^126); *inv = 2^-E.
__device__ __forceinline__ float sp_scale(float amax, float *inv) {
    const int be = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
    int e = 141 - be;
    e = e < -126 ? -126 : (e > 126 ? 126 : e);
    *inv = __uint_as_float((uint32_t)(127 - e) << 23);
    return __uint_as_float((uint32_t)(127 + e) << 23);
}

// The three parts of one scaled element.  An infinity or NaN stays in the
// first part (the residual inf - inf would turn an infinity into NaN).
__device__ __forceinline__ void sp_split1(float xs, _Float16 &a, _Float16 &b, _Float16 &c) {
    a = (_Float16)xs;
    const float r1 = __builtin_isfinite(xs) ? xs - (float)a : 0.f;
    b = (_Float16)r1;
    c = (_Float16)(r1 - (float)b);
}

// The three parts of 8 scaled elements of one run, in element order.
__device__ __forceinline__ void sp_split8(const float (&run)[8], float scale, f16x8 (&part)[3]) {
#pragma unroll
    for (int e = 0; e < 8; e++) {
        _Float16 a, b, c;
        sp_split1(run[sp_elem(e)] * scale, a, b, c);
        part[0][e] = a;
        part[1][e] = b;
        part[2][e] = c;
    }
}

// Split of activation rows (x f32 [rows][cols], cols % 128 == 0, rows 16-byte
// aligned) into v = [rows][cols / 128][4 steps][4 lane groups][3 parts]
// operands of 8 f16 and f[row] = 2^-E.  One block per row (blocks
// first_block, first_block + block_stride, ...; block-uniform arguments);
// each thread takes 8-input runs: it loads them once, the block finds the
// row maximum, and the thread splits and stores its runs.  `red` is LDS of
// one word; every thread of the block calls this.
template <int RUNS>
__device__ inline void sp_split_rows(const float *__restrict__ x, int64_t rows, int cols,
                                     uint16_t *__restrict__ v, float *__restrict__ f,
                                     int64_t first_block, int64_t block_stride, uint32_t *red) {
    const int NL = cols / SP_STEP;
    const int nrun = NL * 16;
    for (int64_t r = first_block; r < rows; r += block_stride) {
        const float *xr = x + r * cols;
        float run[RUNS][8];
        // |x| as unsigned bits orders like |x| (NaN above inf)
        uint32_t m = 0u;
#pragma unroll
        for (int j = 0; j < RUNS; j++) {
            const int q = threadIdx.x + j * blockDim.x;
            if (q < nrun) {
                const int L = q >> 4, i = (q >> 2) & 3, g = q & 3;
                const float *src = xr + L * SP_STEP + sp_run(i, g);
                const f32x4 lo = *(const f32x4 *)src, hi = *(const f32x4 *)(src + 4);
                run[j][0] = lo.x; run[j][1] = lo.y; run[j][2] = lo.z; run[j][3] = lo.w;
                run[j][4] = hi.x; run[j][5] = hi.y; run[j][6] = hi.z; run[j][7] = hi.w;
#pragma unroll
                for (int e = 0; e < 8; e++) m = max(m, __float_as_uint(fabsf(run[j][e])));
            }
        }
        if (threadIdx.x == 0) *red = 0u;
        __syncthreads();
#pragma unroll
        for (int o = QMOE_WAVE / 2; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
        if (lane_id() == 0 && m) atomicMax(red, m);
        __syncthreads();
        float inv;
        const float sc = sp_scale(__uint_as_float(*red), &inv);
        if (threadIdx.x == 0) f[r] = inv;
        f16x8 *dst = reinterpret_cast<f16x8 *>(v) + r * NL * 48;
#pragma unroll
        for (int j = 0; j < RUNS; j++) {
            const int q = threadIdx.x + j * blockDim.x;
            if (q < nrun) {
                f16x8 part[3];
                sp_split8(run[j], sc, part);
                // run q = (L, i, g) is operand ((L * 4 + i) * 4 + g) * 3 + part
                f16x8 *d = dst + q * 3;
                d[0] = part[0];
                d[1] = part[1];
                d[2] = part[2];
            }
        }
        __syncthreads();   // *red is reused by the next row
    }
}

// 8 packed codes (one dword) -> 8 exact f16 codes q - 8 in element order:
// nibbles j and j + 4 land in the mantissas of two f16 1024.0 (one and-or)
// and a packed add of -1032 leaves the code.
__device__ __forceinline__ f16x8 sp_codes8(uint32_t d) {
    uint32_t mask = 0x000F000Fu, expo = 0x64006400u;
    asm("" : "+v"(mask));
    asm("" : "+v"(expo));
    const f16x2 off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    f16x8 r;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t t = ((d >> (4 * j)) & mask) | expo;
        const f16x2 v = __builtin_bit_cast(f16x2, t) + off;
        r[2 * j] = v[0];
        r[2 * j + 1] = v[1];
    }
    return r;
}

}  // namespace qmoe
