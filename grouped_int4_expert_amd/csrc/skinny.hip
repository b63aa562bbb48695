// Prefill (bf16 activations) of lightly routed experts: weight-streaming
// passes on the matrix cores instead of row tiles.
//
// The pages' operation is the same as in mfma.hip (per-group scale
// scales[o*ng + i/gs], the fused gate+up pair with SiLU gating, the down
// projection; colibri pull request "cuda+engine: full fmt=4 (grouped int4
// gs=64) support", Summary).  What changes is the shape: under skewed
// routing (the 256-expert Zipf layer) most experts receive a few dozen rows
// or fewer, and a row tile of such an expert keeps the matrix cores mostly
// idle while its weights, read once per tile, set the time.  Those experts
// are memory-bound GEMVs with a handful of right-hand sides, so they are
// cut into passes of up to 16 rows that stream the expert's weights once per
// pass at HBM rate:
//
//  * A operand of v_mfma_f32_16x16x32_f16: row m = row m of the pass (one
//    token, or one pair for down), read straight from the f16 activations
//    the tile path also uses (x16, scaled by 2^k_t per token and
//    octet-permuted; h16 octet-permuted in the feature index), because the
//    octet order is the order the weight unpack of the matrix-core passes
//    produces (split16.h).  B: 16 weight rows as exact f16 codes.  The f32
//    group scale multiplies each 64-input group's f32 partial sums, as in
//    the f32 decode passes (mfd_loop.h); no f16 rounding of q * s.
//  * D: lane l holds rows 4 (l / 16) .. + 3 of the pass for weight row
//    l % 16.  A block covers the whole input width (wave w: inputs
//    512 w .. + 511) and RB row blocks; the waves' partial sums meet in LDS
//    and are added in wave order (deterministic).
//  * gate+up writes h16 rows of the pass exactly where the tile kernel
//    would (sorted pair position, f16, octet-permuted); down writes Y in the
//    combine's format (f16 with a power-of-two exponent per row and 16
//    columns).  Tile and pass kernels therefore share the workspace, and the
//    combine does not know which produced a row.
//  * The worklist lists the passes: experts with 1..skinny_max rows are cut
//    into 16-row passes instead of tiles.  Blocks walk the pass list with a
//    grid-stride loop (gridDim.y is capped), so a call whose experts all
//    take tiles costs a few thousand blocks that exit at once.
#include <atomic>

#include "mfd_loop.h"
#include "mfma_loop.h"

namespace qmoe {

static_assert(SK_TP == 16, "a pass fills the 16 A rows of one MFMA");

struct SkPass {
    int e, pos0, nt;
};

__device__ __forceinline__ SkPass sk_pass(const SkRoute &r, int p) {
    SkPass s;
    s.e = __builtin_amdgcn_readfirstlane(r.wl.spass[2 * p]);
    const int row0 = __builtin_amdgcn_readfirstlane(r.wl.spass[2 * p + 1]);
    const int c = __builtin_amdgcn_readfirstlane(r.wl.counts[s.e]);
    s.pos0 = __builtin_amdgcn_readfirstlane(r.wl.offsets[s.e]) + row0;
    s.nt = min(SK_TP, c - row0);
    return s;
}

// A operands of wave w: row m = lane % 16 of the pass (byte offset `aoff` of
// its f16 row, OOB_OFFSET for a missing row: zeros), inputs
// 512 w + 128 L + sp_run(i, lane / 16) .. + 7 (one octet).
__device__ __forceinline__ void sk_load_a(f16x8 (&a)[MFD_LPW][4], __amdgpu_buffer_rsrc_t ar,
                                          uint32_t aoff, int w) {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int L = 0; L < MFD_LPW; L++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            a[L][i] = __builtin_bit_cast(
                f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                           ar, aoff, (uint32_t)((MFD_KW * w + SP_STEP * L + sp_run(i, g)) * 2), 0));
}

// ---------------------------------------------------------------------------
// gate+up: block = one pass x RB row blocks (RB/2 x 16 features of gate and
// the same features of up).  h16[pos][f] = silu(g) * u for the pass's rows.
// ---------------------------------------------------------------------------
template <int RB>
__global__ void __launch_bounds__(MFD_GU_WAVES * QMOE_WAVE) sk_gateup_kernel(
    F32Mat G, F32Mat U, const uint16_t *__restrict__ x16, int64_t x16_bytes,
    const float *__restrict__ xinv, uint16_t *__restrict__ h16, SkRoute r) {
    // [S][RB][4][64] partials, then each wave's scale stages
    extern __shared__ float part_lds[];
    constexpr int ROWS = 16 * RB / 2;
    const int H = G.cols, F = G.rows, S = H / MFD_KW;
    const int row0 = blockIdx.x * ROWS;
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int lane = lane_id(), tid = threadIdx.x, nth = blockDim.x;
    const int np = __builtin_amdgcn_readfirstlane(r.wl.n_spass[0]);
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(x16, x16_bytes);
    float *sl = part_lds + S * RB * 4 * QMOE_WAVE + w * MFD_STAGES * 2 * QMOE_WAVE;
    const float nogf[2 * MFD_LPW] = {};
    for (int p = blockIdx.y; p < np; p += gridDim.y) {
        const SkPass ps = sk_pass(r, p);
        const MfdMat mg = mfd_mat(G, ps.e, row0, w), mu = mfd_mat(U, ps.e, row0, w);
        f16x8 a[MFD_LPW][4];
        auto ready = [&] {
            const int m = lane & 15;
            uint32_t aoff = OOB_OFFSET;
            if (m < ps.nt) aoff = (uint32_t)((int64_t)(r.wl.pairs[ps.pos0 + m] / r.k) * H * 2);
            sk_load_a(a, ar, aoff, w);
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        };
        mfd_mainloop<RB, RB / 2, false>(
            a, mg, mu, w, nogf, sl,
            [&](int b, f32x4 t) {
#pragma unroll
                for (int v = 0; v < 4; v++)
                    part_lds[((w * RB + b) * 4 + v) * QMOE_WAVE + lane] = t[v];
            },
            ready);
        __syncthreads();
        // feature f = row0 + 16 b + l % 16 of pass row t = 4 (l / 16) + v
        for (int i = tid; i < (RB / 2) * 4 * QMOE_WAVE; i += nth) {
            const int b = i / (4 * QMOE_WAVE), v = (i / QMOE_WAVE) & 3, l = i % QMOE_WAVE;
            const int t = 4 * (l >> 4) + v, f = row0 + 16 * b + (l & 15);
            if (t >= ps.nt || f >= F) continue;
            float gv = 0.f, uv = 0.f;
            for (int s = 0; s < S; s++) {
                gv += part_lds[((s * RB + b) * 4 + v) * QMOE_WAVE + l];
                uv += part_lds[((s * RB + RB / 2 + b) * 4 + v) * QMOE_WAVE + l];
            }
            const int pos = ps.pos0 + t;
            const float inv = xinv[r.wl.pairs[pos] / r.k];
            const float h = silu(gv * inv) * (uv * inv);
            h16[(int64_t)pos * F + (f & ~7) + octet_pos(f & 7)] =
                __builtin_bit_cast(uint16_t, (_Float16)h);
        }
        __syncthreads();   // the next pass reuses the partials
    }
}

// ---------------------------------------------------------------------------
// down: block = one pass x RB row blocks (16 RB output features).
// Y[pos][o] = w * (D h) as f16 with the exponent of the row's 16-column
// block (the block maximum scaled into [2^14, 2^15), as the tile kernel
// does per 4 rows).
// ---------------------------------------------------------------------------
template <int RB>
__global__ void __launch_bounds__(MFD_DN_WAVES * QMOE_WAVE) sk_down_kernel(
    F32Mat D, const uint16_t *__restrict__ h16, int64_t h16_bytes, YBuf yb, SkRoute r) {
    extern __shared__ float part_lds[];
    const int O = D.rows, K = D.cols, S = K / MFD_KW, hs = O / 16;
    const int row0 = blockIdx.x * (16 * RB);
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int lane = lane_id(), tid = threadIdx.x, nth = blockDim.x;
    const int np = __builtin_amdgcn_readfirstlane(r.wl.n_spass[0]);
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(h16, h16_bytes);
    float *sl = part_lds + S * RB * 4 * QMOE_WAVE + w * MFD_STAGES * 2 * QMOE_WAVE;
    const float nogf[2 * MFD_LPW] = {};
    for (int p = blockIdx.y; p < np; p += gridDim.y) {
        const SkPass ps = sk_pass(r, p);
        const MfdMat md = mfd_mat(D, ps.e, row0, w);
        f16x8 a[MFD_LPW][4];
        auto ready = [&] {
            const int m = lane & 15;
            const uint32_t aoff = m < ps.nt ? (uint32_t)((int64_t)(ps.pos0 + m) * K * 2) : OOB_OFFSET;
            sk_load_a(a, ar, aoff, w);
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        };
        mfd_mainloop<RB, RB, false>(
            a, md, md, w, nogf, sl,
            [&](int b, f32x4 t) {
#pragma unroll
                for (int v = 0; v < 4; v++)
                    part_lds[((w * RB + b) * 4 + v) * QMOE_WAVE + lane] = t[v];
            },
            ready);
        __syncthreads();
        // output o = row0 + 16 b + l % 16 of pass row t = 4 (l / 16) + v; the
        // 16 lanes of a DPP row share t and cover one 16-column block.  A
        // wave's iterations are all in range or all out (nth and the bound are
        // multiples of 64), so the DPP maximum always runs on whole rows.
        for (int i = tid; i < RB * 4 * QMOE_WAVE; i += nth) {
            const int b = i / (4 * QMOE_WAVE), v = (i / QMOE_WAVE) & 3, l = i % QMOE_WAVE;
            const int t = 4 * (l >> 4) + v, o = row0 + 16 * b + (l & 15);
            float y = 0.f;
            for (int s = 0; s < S; s++) y += part_lds[((s * RB + b) * 4 + v) * QMOE_WAVE + l];
            const int pos = ps.pos0 + t;
            const bool on = t < ps.nt && o < O;
            const float val = on ? r.topk_w[r.wl.pairs[pos]] * y : 0.f;
            // |val| >= 0 and never NaN (fmaxf drops NaN), so its bits order
            // like its value; ex as in the tile kernel
            const uint32_t mb = max16_u32_dpp(__float_as_uint(fmaxf(fabsf(val), 0.f)));
            int ex = 0;
            if (mb != 0 && mb < 0x7f800000u) ex = min(max((int)(mb >> 23) - 126, -111), 127);
            const float sc = __uint_as_float((uint32_t)(142 - ex) << 23);   // 2^(15 - ex)
            if (!on) continue;
            yb.v[(int64_t)pos * O + o] = __builtin_bit_cast(uint16_t, (_Float16)(val * sc));
            if ((l & 15) == 0) yb.e[(int64_t)pos * hs + o / 16] = (int8_t)ex;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int SK_GU_RB = 8;    // 4 x 16 features of gate and of up per block
constexpr int SK_DN_RB = 16;   // 256 output features per block
constexpr int SK_GRID_Y = 64;  // passes in the grid at once (blocks loop over the rest)

static size_t sk_lds(int cols, int rb) {
    const int S = cols / MFD_KW;
    return (size_t)S * (rb * 4 + MFD_STAGES * 2) * QMOE_WAVE * sizeof(float);
}

// LDS of one gfx950 workgroup
constexpr size_t SK_LDS_MAX = 160 * 1024;

// hidden and inter multiples of 512 (one wave per 512 inputs), groups of 64
// or more, and blocks whose partials fit the LDS: gate+up up to hidden 6144
// (108 KB), down up to inter 4608 (153 KB)
bool sk_supported(const QMat &gate, const QMat &up, const QMat &down) {
    const int H = gate.cols, F = gate.rows;
    return gate.group >= 64 && up.group >= 64 && down.group >= 64 && H % MFD_KW == 0 &&
           H <= MFD_KW * MFD_GU_WAVES && F % MFD_KW == 0 && F <= MFD_DOWN_MAX_COLS &&
           sk_lds(H, SK_GU_RB) <= SK_LDS_MAX && sk_lds(F, SK_DN_RB) <= SK_LDS_MAX;
}

// gfx950 gives a block up to 160 KB of LDS; above 64 KB the launch needs the
// kernel's dynamic limit raised (once per kernel and device, to the largest
// size used there).
constexpr int SK_MAX_DEVICES = 64;
template <typename K>
static hipError_t sk_allow_lds(K kernel, size_t lds, std::atomic<size_t> (&raised)[SK_MAX_DEVICES]) {
    if (lds <= 65536) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::atomic<size_t> *r = dev >= 0 && dev < SK_MAX_DEVICES ? &raised[dev] : nullptr;
    if (r && lds <= r->load()) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess && r) r->store(lds);
    return e;
}
static std::atomic<size_t> sk_gu_lds[SK_MAX_DEVICES], sk_dn_lds[SK_MAX_DEVICES];

hipError_t launch_sk_gateup(const QMat &gate, const QMat &up, const uint16_t *x16, int tokens,
                            const float *xinv, uint16_t *h16, const SkRoute &r, hipStream_t st) {
    const int H = gate.cols, F = gate.rows;
    const int rows_per_block = 16 * SK_GU_RB / 2;
    const dim3 grid((F + rows_per_block - 1) / rows_per_block,
                    r.max_passes < SK_GRID_Y ? (r.max_passes > 0 ? r.max_passes : 1) : SK_GRID_Y);
    const dim3 block((H / MFD_KW) * QMOE_WAVE);
    const size_t lds = sk_lds(H, SK_GU_RB);
    hipError_t e = sk_allow_lds(sk_gateup_kernel<SK_GU_RB>, lds, sk_gu_lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((sk_gateup_kernel<SK_GU_RB>), grid, block, lds, st, f32_mat(gate),
                       f32_mat(up), x16, (int64_t)tokens * H * 2, xinv, h16, r);
    return hipGetLastError();
}

hipError_t launch_sk_down(const QMat &down, const uint16_t *h16, int64_t pairs, YBuf y,
                          const SkRoute &r, hipStream_t st) {
    const int O = down.rows, K = down.cols;
    const int rows_per_block = 16 * SK_DN_RB;
    const dim3 grid((O + rows_per_block - 1) / rows_per_block,
                    r.max_passes < SK_GRID_Y ? (r.max_passes > 0 ? r.max_passes : 1) : SK_GRID_Y);
    const dim3 block((K / MFD_KW) * QMOE_WAVE);
    const size_t lds = sk_lds(K, SK_DN_RB);
    hipError_t e = sk_allow_lds(sk_down_kernel<SK_DN_RB>, lds, sk_dn_lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((sk_down_kernel<SK_DN_RB>), grid, block, lds, st, f32_mat(down), h16,
                       pairs * K * 2, y, r);
    return hipGetLastError();
}

}  // namespace qmoe
