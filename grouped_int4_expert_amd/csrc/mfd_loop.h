// Main loop of the matrix-core passes over int4-g64 weights: one wave takes
// 512 inputs of a pass's activation operands (A of v_mfma_f32_16x16x32_f16,
// held in registers) and streams 16-row blocks of one or two matrices past
// them (B: exact f16 codes), multiplying each 64-input group's f32 partial
// sums by the row's f32 group scale.  Used by the f32 decode passes
// (gemv_mfma.hip: A rows are the three f16 parts of four tokens) and by the
// bf16 prefill passes of lightly routed experts (skinny.hip: A rows are
// sixteen tokens).  Operand layout: split16.h.
#pragma once

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
        part(b, tot);
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

}  // namespace qmoe
