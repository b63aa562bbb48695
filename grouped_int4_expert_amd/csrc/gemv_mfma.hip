// Decode GEMVs of the routed layer on the matrix cores, in f32 arithmetic.
//
// What is computed is the same as the f32 GEMVs of gemv_f32.hip (per-group
// f32 scale applied once per 64-input group, f32 accumulation; colibri pull
// request "cuda+engine: full fmt=4 (grouped int4 gs=64) support", Summary and
// comment "blocked by GPU driver instability"), for passes of up to four
// tokens of one expert.  The f32 activations are carried as three exact f16
// parts each (split16.h), the codes as exact f16 q - 8, and
// v_mfma_f32_16x16x32_f16 forms the products exactly and adds them in f32.
// Where the VALU kernels spend one f32 FMA per code and token on top of the
// unpack, here the code-times-token work moves to the matrix cores and the
// vector ALUs only unpack, so a pass of several tokens costs about what one
// token does.
//
// MFMA roles.  A operand (16 rows m): m = 4 t + p, token t of the pass
// (0..3), part p (0..2; p = 3 is zero).  B operand (16 columns): 16 weight
// rows.  D: lane l holds the four parts of token l / 16 for weight row
// l % 16, so a lane needs one scale per group and sums its own parts at the
// end.  Per 128-input load step a lane reads 16 packed bytes of its row
// (lane group l / 16 at byte 16 (l / 16)), two dwords swap lane halves
// (split16.h), and four MFMAs follow: steps 0 and 1 accumulate the first
// 64-input group, steps 2 and 3 the second; each group's partial sums are
// multiplied by the row's f32 scale and added to the f32 totals.
//
// Weight stream.  Each wave reads a row block's four load steps back to back
// (256 contiguous bytes of each of 16 rows): a probe of this stream on
// MI355X read 5.8 TB/s, against 4.2 TB/s when every row advanced only 64
// bytes per step.
//
// gate+up reads the activation parts from the preparation kernel's split of
// x (L2-resident) and writes h as the down projection's parts (a power of
// two per 64 rows of h, whose inverse goes into down's group scales); down
// reads them the same way.  Records, sorted positions and the routed atomic
// adds into out are those of the record mode of the VALU kernels.
#include "mfd_loop.h"

namespace qmoe {

// ---------------------------------------------------------------------------
// gate+up: block = one pass x 8 row blocks (128 rows) of gate and of up;
// h = silu(g) * u for rows row0 .. row0 + 127 of the pass's tokens, written
// as f32 h[p0 + t][f] or (hs.v set) as the down projection's operands: the
// three f16 parts of h scaled per 64 rows (two groups per block), hs.f the
// group's 2^-E.
// ---------------------------------------------------------------------------
template <int RB>
__global__ void __launch_bounds__(MFD_GU_WAVES * QMOE_WAVE) mfd_gateup_kernel(
    F32Mat G, F32Mat U, XSplit xs, int64_t xs_bytes, float *__restrict__ h, XSplit hs,
    const int32_t *__restrict__ rec, const int32_t *__restrict__ tokp, int max_rec) {
    // [S][RB][64] partials; then h of the block [4][8 RB] and the group maxima [4][RB / 4]
    extern __shared__ float part_lds[];
    constexpr int ROWS = 16 * RB / 2;   // rows of gate (and of up) per block
    const int slot = blockIdx.z * gridDim.y + blockIdx.y;
    if (slot >= max_rec) return;
    const MfdPass ps = mfd_pass(rec, slot);
    if (ps.e < 0 || ps.nt <= 0) return;
    const int F = G.rows, NL = G.cols / SP_STEP, S = G.cols / MFD_KW;
    const int row0 = blockIdx.x * ROWS;
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int lane = lane_id(), n = lane & 15;
    const MfdMat mg = mfd_mat(G, ps.e, row0, w), mu = mfd_mat(U, ps.e, row0, w);
    f16x8 a[MFD_LPW][4];
    // activation operands (after the first weights are on their way): A row
    // m = n is token n / 4, part n % 4 (part 3 and missing tokens read past
    // the descriptor: zero)
    auto ready = [&] {
        const __amdgpu_buffer_rsrc_t ar = make_rsrc(xs.v, xs_bytes);
        uint32_t aoff = OOB_OFFSET;
        const int ta = n >> 2, pa = n & 3;
        if (ta < ps.nt && pa < SP_PARTS) {
            const int tok = tokp[ps.p0 + ta];
            aoff = (uint32_t)(((int64_t)tok * NL * 48 + (lane >> 4) * 3 + pa) * 16);
        }
#pragma unroll
        for (int L = 0; L < MFD_LPW; L++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                a[L][i] = __builtin_bit_cast(
                    f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                               ar, aoff, (uint32_t)((MFD_LPW * w + L) * 768 + i * 192), 0));
        // these are the newest loads: wait for them once here, not in every
        // step of the row-block loop
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    };
    const float nogf[2 * MFD_LPW] = {};
    float *sl = part_lds + S * RB * QMOE_WAVE + w * MFD_STAGES * 2 * QMOE_WAVE;
    mfd_mainloop<RB, RB / 2, false>(
        a, mg, mu, w, nogf, sl,
        [&](int b, f32x4 t) {
            // parts of the lane's token (register 3 is the zero part), smallest first
            part_lds[(w * RB + b) * QMOE_WAVE + lane] = (t[2] + t[1]) + t[0];
        }, ready);
    const int tid = threadIdx.x, nth = blockDim.x;
    __syncthreads();
    // rows row0 + 16 b + n of token t: gate partials in row block b, up in RB/2 + b
    float hreg[RB / 2];
#pragma unroll
    for (int j = 0; j < RB / 2; j++) {
        const int i = tid + j * nth;
        hreg[j] = 0.f;
        if (i >= (RB / 2) * QMOE_WAVE) continue;
        const int b = i / QMOE_WAVE, l = i % QMOE_WAVE;
        const int t = l >> 4, f = row0 + 16 * b + (l & 15);
        if (t >= ps.nt || f >= F) continue;
        float gv = 0.f, uv = 0.f;
        for (int k = 0; k < S; k++) {
            gv += part_lds[(k * RB + b) * QMOE_WAVE + l];
            uv += part_lds[(k * RB + RB / 2 + b) * QMOE_WAVE + l];
        }
        const float inv = xs.f[tokp[ps.p0 + t]];
        hreg[j] = silu(gv * inv) * (uv * inv);
        if (!hs.v) h[(int64_t)(ps.p0 + t) * F + f] = hreg[j];
    }
    if (!hs.v) return;
    float *hv = part_lds;                                        // [4][ROWS]
    uint32_t *gmax = reinterpret_cast<uint32_t *>(part_lds + MFD_TB * ROWS);   // [4][ROWS / 64]
    __syncthreads();   // every partial has been read
    if (tid < MFD_TB * ROWS / 64) gmax[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < RB / 2; j++) {
        const int i = tid + j * nth;
        if (i >= (RB / 2) * QMOE_WAVE) continue;
        const int b = i / QMOE_WAVE, l = i % QMOE_WAVE;
        const int t = l >> 4, r = 16 * b + (l & 15);
        if (t >= ps.nt || row0 + r >= F) continue;
        hv[t * ROWS + r] = hreg[j];
        // |h| as unsigned bits orders like |h| (NaN above inf)
        atomicMax(&gmax[t * (ROWS / 64) + (r >> 6)], __float_as_uint(fabsf(hreg[j])));
    }
    __syncthreads();
    // input r of the block (down's load step (row0 + r) / 128, input r % 128
    // of it) sits in MFMA step i, lane group g, element e of the operand layout
    const int NLd = F / SP_STEP;
    for (int i = tid; i < ps.nt * ROWS; i += nth) {
        const int t = i / ROWS, r = i % ROWS, f = row0 + r;
        if (f >= F) continue;
        float inv;
        const float sc = sp_scale(__uint_as_float(gmax[t * (ROWS / 64) + (r >> 6)]), &inv);
        _Float16 p[3];
        sp_split1(hv[t * ROWS + r] * sc, p[0], p[1], p[2]);
        const int c = f % SP_STEP;
        const int si = 2 * ((c >> 6) & 1) + ((c >> 3) & 1), g = ((c >> 5) & 1) + 2 * ((c >> 4) & 1);
        const int e = 2 * (c & 3) + ((c >> 2) & 1);
        const int64_t pos = ps.p0 + t;
        _Float16 *dst = reinterpret_cast<_Float16 *>(hs.v) +
                        ((((pos * NLd + f / SP_STEP) * 4 + si) * 4 + g) * 3) * 8 + e;
        dst[0] = p[0];
        dst[8] = p[1];
        dst[16] = p[2];
        if ((f & 63) == 0) hs.f[pos * (F / 64) + f / 64] = inv;
    }
}

// ---------------------------------------------------------------------------
// down: block = one pass x 16 row blocks (256 output rows), operands from the
// gate+up kernel's split of h (per 64 inputs a power of two, taken into the
// group scales).  out[tok] += w * y (f32 atomics).
// ---------------------------------------------------------------------------
template <int RB>
__global__ void __launch_bounds__(MFD_DN_WAVES * QMOE_WAVE) mfd_down_kernel(
    F32Mat D, XSplit hs, int64_t hs_bytes, float *__restrict__ out,
    const int32_t *__restrict__ rec, const int32_t *__restrict__ tokp,
    const float *__restrict__ wsort, int max_rec) {
    extern __shared__ float part_lds[];   // [S][R][64]
    const int slot = blockIdx.z * gridDim.y + blockIdx.y;
    if (slot >= max_rec) return;
    const MfdPass ps = mfd_pass(rec, slot);
    if (ps.e < 0 || ps.nt <= 0) return;
    const int O = D.rows, K = D.cols, NL = K / SP_STEP, S = K / MFD_KW;
    const int row0 = blockIdx.x * (16 * RB);
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(hs.v, hs_bytes);
    uint32_t aoff = OOB_OFFSET;
    const int ta = n >> 2, pa = n & 3;
    if (ta < ps.nt && pa < SP_PARTS)
        aoff = (uint32_t)(((int64_t)(ps.p0 + ta) * NL * 48 + g * 3 + pa) * 16);
    f16x8 a[MFD_LPW][4];
#pragma unroll
    for (int L = 0; L < MFD_LPW; L++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            a[L][i] = __builtin_bit_cast(
                f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                           ar, aoff, (uint32_t)((MFD_LPW * w + L) * 768 + i * 192), 0));
    // group factors of the lane's token (D rows: token l / 16) for the
    // slice's 8 groups
    float gf[2 * MFD_LPW];
    {
        const int gt = g < ps.nt ? g : 0;
        const f32x4 *fp =
            reinterpret_cast<const f32x4 *>(hs.f + (int64_t)(ps.p0 + gt) * (K / 64) + 8 * w);
        const f32x4 f0 = fp[0], f1 = fp[1];
        gf[0] = f0.x; gf[1] = f0.y; gf[2] = f0.z; gf[3] = f0.w;
        gf[4] = f1.x; gf[5] = f1.y; gf[6] = f1.z; gf[7] = f1.w;
    }
    const MfdMat md = mfd_mat(D, ps.e, row0, w);
    float *sl = part_lds + S * RB * QMOE_WAVE + w * MFD_STAGES * 2 * QMOE_WAVE;
    mfd_mainloop<RB, RB, true>(
        a, md, md, w, gf, sl,
        [&](int b, f32x4 t) {
            // parts of the lane's token (register 3 is the zero part), smallest first
            part_lds[(w * RB + b) * QMOE_WAVE + lane] = (t[2] + t[1]) + t[0];
        }, [] {});
    __syncthreads();
    const int tid = threadIdx.x, nth = blockDim.x;
    for (int i = tid; i < RB * QMOE_WAVE; i += nth) {
        const int b = i / QMOE_WAVE, l = i % QMOE_WAVE;
        const int t = l >> 4, o = row0 + 16 * b + (l & 15);
        if (t >= ps.nt || o >= O) continue;
        float y = 0.f;
        for (int k = 0; k < S; k++) y += part_lds[(k * RB + b) * QMOE_WAVE + l];
        const int pos = ps.p0 + t;
        unsafeAtomicAdd(out + (int64_t)tokp[pos] * O + o, wsort[pos] * y);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static bool mfd_group_ok(const QMat &m) { return m.group >= 64; }

bool mfd_gateup_supported(const QMat &gate, const QMat &up) {
    return gate.cols % MFD_KW == 0 && gate.cols <= MFD_KW * MFD_GU_WAVES &&
           mfd_group_ok(gate) && mfd_group_ok(up);
}

bool mfd_down_supported(const QMat &down) {
    return down.cols % MFD_KW == 0 && down.cols <= MFD_DOWN_MAX_COLS && mfd_group_ok(down);
}

static dim3 mfd_grid(unsigned x, int64_t slots) {
    const int64_t gy = slots < 65535 ? (slots > 0 ? slots : 1) : 65535;
    return dim3(x, (unsigned)gy, (unsigned)((slots + gy - 1) / gy));
}

// 16-row blocks per block (32 measured no faster for gate+up and slower for
// down, whose 16-token launch then has too few blocks to fill the GPU).
static int mfd_rb(int) { return 16; }

// LDS of a block: the partials [S][RB][64] and each wave's scale stages
// [MFD_STAGES][2][64], floats.
static size_t mfd_lds(int cols, int rb) {
    const int S = cols / MFD_KW;
    return (size_t)S * (rb + MFD_STAGES * 2) * QMOE_WAVE * sizeof(float);
}

hipError_t launch_mfd_gateup(const QMat &gate, const QMat &up, XSplit xs, int tokens, float *h,
                             XSplit hs, const int32_t *rec, const int32_t *tok, int max_rec,
                             hipStream_t st) {
    if (!mfd_gateup_supported(gate, up)) return hipErrorInvalidValue;
    if (hs.v && gate.rows % MFD_KW) return hipErrorInvalidValue;
    const int64_t xs_bytes = xsplit_bytes(tokens, gate.cols);
    if (xs_bytes >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int rb = mfd_rb(gate.cols);
    const int rows_per_block = 16 * rb / 2;
    const dim3 grid = mfd_grid((gate.rows + rows_per_block - 1) / rows_per_block, max_rec);
    const dim3 block((gate.cols / MFD_KW) * QMOE_WAVE);
    const size_t lds = mfd_lds(gate.cols, rb);
    const F32Mat G = f32_mat(gate), U = f32_mat(up);
#define X(RB_)                                                                                  \
    if (rb == RB_) {                                                                            \
        hipLaunchKernelGGL((mfd_gateup_kernel<RB_>), grid, block, lds, st, G, U, xs, xs_bytes,   \
                           h, hs, rec, tok, max_rec);                                           \
        return hipGetLastError();                                                               \
    }
    X(16)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_mfd_down(const QMat &down, XSplit hs, int pairs, float *out, const int32_t *rec,
                           const int32_t *tok, const float *wsort, int max_rec,
                           hipStream_t st) {
    if (!mfd_down_supported(down)) return hipErrorInvalidValue;
    const int64_t hs_bytes = xsplit_bytes(pairs, down.cols);
    if (hs_bytes >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int rb = mfd_rb(down.cols);
    const int rows_per_block = 16 * rb;
    const dim3 grid = mfd_grid((down.rows + rows_per_block - 1) / rows_per_block, max_rec);
    const dim3 block((down.cols / MFD_KW) * QMOE_WAVE);
    const size_t lds = mfd_lds(down.cols, rb);
    const F32Mat D = f32_mat(down);
#define X(RB_)                                                                                  \
    if (rb == RB_) {                                                                            \
        hipLaunchKernelGGL((mfd_down_kernel<RB_>), grid, block, lds, st, D, hs, hs_bytes, out,   \
                           rec, tok, wsort, max_rec);                                           \
        return hipGetLastError();                                                               \
    }
    X(16)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace qmoe
