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
#include "common.h"
#include "launch.h"
#include "split16.h"

namespace qmoe {

// A block = one pass x RB 16-row blocks x the whole input width: wave w
// takes inputs 512 w .. 512 w + 511 (four load steps), so its activation
// operands (64 registers) are read once; it streams its R row blocks, each
// as four back-to-back loads of 64 bytes per row (256 contiguous bytes), and
// leaves one partial sum per row and token in LDS; the block adds the
// slices' partials at the end.  gate+up: row blocks 0..RB/2-1 of gate and the
// same rows of up.
constexpr int MFD_KW = 512;        // inputs per wave
constexpr int MFD_LPW = MFD_KW / SP_STEP;
constexpr int MFD_GU_WAVES = 12;   // gate+up inputs up to 6144
constexpr int MFD_DN_WAVES = MFD_DOWN_MAX_COLS / MFD_KW;
constexpr int MFD_STAGES = 2;      // row blocks in flight per wave

struct MfdPass {
    int e, p0, nt;
};

// Record `slot` of the plan (expert, first and end sorted position).
__device__ __forceinline__ MfdPass mfd_pass(const int32_t *rec, int slot) {
    MfdPass p;
    p.e = __builtin_amdgcn_readfirstlane(rec[4 * slot]);
    p.p0 = __builtin_amdgcn_readfirstlane(rec[4 * slot + 1]);
    const int end = __builtin_amdgcn_readfirstlane(rec[4 * slot + 2]);
    p.nt = min(end - p.p0, MFD_TB);
    return p;
}

// One expert's matrix as the main loop reads it: descriptors over its codes
// and scales, lane offsets of row lane % 16 at this wave's first input, the
// byte stride of 16 rows.
struct MfdMat {
    __amdgpu_buffer_rsrc_t q, s;
    uint32_t qlane, slane;     // per lane
    uint32_t qwave, swave;     // this wave's slice (uniform)
    uint32_t q16, s16;         // 16 rows
    int gshift;
};

__device__ __forceinline__ MfdMat mfd_mat(const F32Mat &M, int e, int row0, int w) {
    MfdMat m;
    const int lane = lane_id();
    m.q = make_rsrc(M.q + (int64_t)e * M.q_stride, M.qbytes);
    m.s = make_rsrc(M.s + (int64_t)e * M.s_stride, M.sbytes);
    m.qlane = (uint32_t)(lane & 15) * M.rb + 16u * (uint32_t)(lane >> 4);
    m.slane = (uint32_t)(lane & 15) * M.sb;
    m.qwave = (uint32_t)row0 * M.rb + (uint32_t)(MFD_KW / 2) * (uint32_t)w;
    m.swave = (uint32_t)row0 * M.sb;
    m.q16 = 16u * M.rb;
    m.s16 = 16u * M.sb;
    m.gshift = M.gshift;
    return m;
}

// Main loop of one wave: a[L][i] = activation operands of its four load
// steps; row blocks b = 0..R-1 of matrix M0 (b < R0) or M1 (b >= R0, row
// block b - R0); `part(b, y)` receives the lane's part sum of row block b.
// Input k0 of the wave: MFD_KW * w.  GF: gf holds per-lane factors of the
// slice's 8 groups (the activation parts' power of two per 64 inputs), taken
// into the group scales.  `ready()` runs once the first row blocks' loads
// are issued, before `a` is read (it may fill `a`).
template <int R, int R0, bool GF, typename Part, typename Ready>
__device__ __forceinline__ void mfd_mainloop(const f16x8 (&a)[MFD_LPW][4], const MfdMat &M0,
                                             const MfdMat &M1, int w,
                                             const float (&gf)[2 * MFD_LPW], float *sl,
                                             Part part, Ready ready) {
    u32x4 wq[MFD_STAGES][MFD_LPW];
    const int lane = lane_id(), g = lane >> 4, n = lane & 15;
    // scales: lane (g, n) fetches the scales of row n for the slice's groups
    // h = g and h = 4 + g straight into LDS (sl[st][h / 4][16 (h % 4) + n]),
    // so in-flight scales hold no registers
    uint32_t sv0[2], sv1[2];
#pragma unroll
    for (int m = 0; m < 2; m++) {
        const MfdMat &M = m ? M1 : M0;
        sv0[m] = M.slane + ((uint32_t)(MFD_KW * w + 64 * g) >> M.gshift) * 4u;
        sv1[m] = M.slane + ((uint32_t)(MFD_KW * w + 64 * (4 + g)) >> M.gshift) * 4u;
    }
    // (a row block past R reads past the descriptors: no memory access)
    auto issue = [&](int b, int st) {
        __builtin_amdgcn_sched_barrier(0);
        const int m = b < R0 ? 0 : 1;
        const MfdMat &M = m ? M1 : M0;
        const int bb = b < R0 ? b : b - R0;
        const uint32_t qo = b < R ? M.qwave + (uint32_t)bb * M.q16 : OOB_OFFSET;
#pragma unroll
        for (int L = 0; L < MFD_LPW; L++)
            wq[st][L] = __builtin_amdgcn_raw_buffer_load_b128(M.q, M.qlane, qo + 64u * L, 0);
        const uint32_t so = b < R ? M.swave + (uint32_t)bb * M.s16 : OOB_OFFSET;
        float *dst = sl + st * 2 * QMOE_WAVE;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(M.s, QMOE_LDS(dst), 4, m ? sv0[1] : sv0[0], so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(M.s, QMOE_LDS(dst + QMOE_WAVE), 4,
                                                 m ? sv1[1] : sv1[0], so, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // loads per stage, in issue order: MFD_LPW weight loads, 2 scale loads
    constexpr int LPS = MFD_LPW + 2;
    auto compute = [&](int b, int st) {
        // the scales of stage st arrive in LDS, which the compiler does not
        // track: wait until only the later stages' loads are in flight
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPS * (MFD_STAGES - 1)));
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 tot = zero;
        const float *ss = sl + st * 2 * QMOE_WAVE + n;
#pragma unroll
        for (int L = 0; L < MFD_LPW; L++) {
            const u32x4 q = wq[st][L];
            // lanes 32..63 of dwords 0, 1 <-> lanes 0..31 of dwords 2, 3
            const auto s02 = __builtin_amdgcn_permlane32_swap(q[0], q[2], false, false);
            const auto s13 = __builtin_amdgcn_permlane32_swap(q[1], q[3], false, false);
            const f16x8 b0 = sp_codes8(s02[0]), b1 = sp_codes8(s13[0]);
            const f16x8 b2 = sp_codes8(s02[1]), b3 = sp_codes8(s13[1]);
            f32x4 pa = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[L][0], b0, zero, 0, 0, 0);
            pa = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[L][1], b1, pa, 0, 0, 0);
            f32x4 pb = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[L][2], b2, zero, 0, 0, 0);
            pb = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[L][3], b3, pb, 0, 0, 0);
            const int h0 = 2 * L, h1 = 2 * L + 1;
            const float s0 = ss[(h0 / 4) * QMOE_WAVE + 16 * (h0 % 4)];
            const float s1 = ss[(h1 / 4) * QMOE_WAVE + 16 * (h1 % 4)];
            const float sa = GF ? s0 * gf[h0] : s0;
            const float sb = GF ? s1 * gf[h1] : s1;
#pragma unroll
            for (int v = 0; v < 4; v++) tot[v] = fmaf(sa, pa[v], fmaf(sb, pb[v], tot[v]));
        }
        // parts of the lane's token (register 3 is the zero part), smallest first
        part(b, (tot[2] + tot[1]) + tot[0]);
    };
    static_assert(R % MFD_STAGES == 0, "row blocks per block");
#pragma unroll
    for (int st = 0; st < MFD_STAGES; st++) issue(st, st);
    ready();
    for (int b = 0; b < R; b += MFD_STAGES) {
        b = __builtin_amdgcn_readfirstlane(b);
#pragma unroll
        for (int st = 0; st < MFD_STAGES; st++) {
            compute(b + st, st);
            issue(b + st + MFD_STAGES, st);
        }
    }
}

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
        [&](int b, float y) { part_lds[(w * RB + b) * QMOE_WAVE + lane] = y; }, ready);
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
        [&](int b, float y) { part_lds[(w * RB + b) * QMOE_WAVE + lane] = y; }, [] {});
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
