// Decode GEMVs in f32 arithmetic (f32 activations): grouped int4 weights are
// streamed once per expert with 128-bit buffer loads, every code is unpacked
// in registers to an exact f32, multiplied with the f32 activation in an f32
// FMA chain, scaled by its f32 group scale and reduced across lanes with DPP.
//
// What is computed follows the colibri pull request "cuda+engine: full fmt=4
// (grouped int4 gs=64) support": the per-group scale scales[o*ng + i/gs]
// applied once per group (comment "blocked by GPU driver instability": the
// grouped kernel accumulates a group and then applies its scale), and the
// fused gate+up pair that loads the activation once for both matrices
// (Summary, "matmul_i4_grouped_pair").  The routed layer's tokens are grouped
// by expert on the device, with no host round trip (pxq_llama.cpp release
// notes, "Device-side MoE row map").
//
// MI355X mapping.  A lane owns one 32-input chunk of a row (16 packed bytes,
// one 128-bit load per row) and keeps that chunk of each token's activation
// in 32 registers, so activations are read once per block and weights stream
// past them.  L lanes (16, 32 or 64: one, two or four DPP rows) cover L
// chunks of a row; a row of C chunks is split into S slices of L chunks, one
// wave per slice, and a wave instruction covers 64/L rows.  A 32-input chunk
// lies inside one scale group for every supported group size (32, 64 * 2^j,
// one per row), so each lane needs one scale per row, at index
// (32 * chunk) >> log2(group).
//
// Unpack: w' = w ^ 0x88888888 turns the offset nibbles into two's
// complement; (w' & 0xF0F0F0F0) then holds 16 q of the odd elements as signed
// bytes and ((w' << 4) & 0xF0F0F0F0) 16 q of the even ones, and each byte
// converts exactly in one sign-extending instruction (11 VALU instructions
// per 8 codes), then one f32 FMA per code and token; the power of two 16 is
// taken out together with the group scale.  The lane sums of 16 row steps
// are reduced together by a lane-transposed butterfly (one DPP level per
// lane bit) instead of one full DPP reduction per row.
//
// Every size a buffer descriptor or a scalar offset is built from comes from
// the host (F32Mat), so descriptors and row offsets stay in scalar registers.
#include "common.h"
#include "launch.h"
#include "wl_wave.h"

namespace qmoe {

// Rows per gate+up block and row steps per down wave, chosen per launch from
// the waves the launch would have at 32 rows / 16 steps: small launches (the
// single expert, the one-token layer) are latency-bound and take more,
// shorter waves; passes of several tokens take longer down waves (fewer block
// set-ups for the same weights).
constexpr int F32_GU_ROWS = 32, F32_GU_ROWS_MID = 16, F32_GU_ROWS_SHORT = 8;
constexpr int F32_DN_STEPS_LONG = 32, F32_DN_STEPS = 16, F32_DN_STEPS_SHORT = 4;
constexpr int F32_MAX_WAVES = 8;

// The pass of a block, in LDS: expert, token count and per token the row of
// the pass's input (x: token; h: pair or sorted position), its token (the row
// of out) and its routing weight.
struct PassLds {
    int e, nt;
    int hrow[4], tok[4];
    float w[4];
};

// Plan of slot a, computed by one wave into LDS (lane 0 writes).
// inline: slot = pair a; it starts a pass when a's rank among its expert's
//   pairs (ascending) is a multiple of TB, and the pass takes the next TB - 1
//   pairs of that expert.  sid = the ids staged in LDS (n <= F32_INLINE_MAX).
// record: plan record a over sorted positions (preparation kernel).
// direct: expert 0, tokens a*TB ...
template <int TB>
__device__ void plan_wave(const F32Route &r, int a, const int *sid, PassLds *pl) {
    const int lane = lane_id();
    int e = -1, nt = 0;
    int hrow[TB], tok[TB];
    float w[TB];
#pragma unroll
    for (int j = 0; j < TB; j++) {
        hrow[j] = 0;
        tok[j] = 0;
        w[j] = 0.f;
    }
    if (r.ids) {
        if (a < r.n) {
            const int e0 = sid[a];
            if (e0 >= 0 && e0 < r.E) {
                e = e0;
                nt = 1;
                hrow[0] = a;
                int rank = 0;
                if (TB > 1) {
                    const int nc = (r.n + QMOE_WAVE - 1) / QMOE_WAVE;
                    const int ca = a / QMOE_WAVE, la = a % QMOE_WAVE;
                    for (int c = 0; c < nc; c++) {
                        const int q = c * QMOE_WAVE + lane;
                        const int v = q < r.n ? sid[q] : -1;
                        uint64_t m = __ballot(v == e);
                        if (c < ca) {
                            rank += __popcll(m);
                            continue;
                        }
                        if (c == ca) {
                            rank += __popcll(m & ((1ull << la) - 1ull));
                            m = la == 63 ? 0ull : (m & ~((2ull << la) - 1ull));
                        }
#pragma unroll
                        for (int j = 1; j < TB; j++)
                            if (nt == j && m) {
                                hrow[j] = c * QMOE_WAVE + __builtin_ctzll(m);
                                m &= m - 1ull;
                                nt++;
                            }
                        if (nt == TB) break;
                    }
                    // a pair whose rank is not a multiple of TB belongs to an
                    // earlier pass; the ranks of the pairs before a suffice
                    // because the partners only come after a
                    if (rank % TB) nt = 0;
                }
#pragma unroll
                for (int j = 0; j < TB; j++)
                    if (j < nt) {
                        tok[j] = hrow[j] / r.k;
                        w[j] = r.topk_w[hrow[j]];
                    }
            }
        }
    } else if (r.rec) {
        if (a < r.max_rec) {
            const u32x4 rc = *(const u32x4 *)(r.rec + 4 * a);
            if ((int)rc.x >= 0) {
                e = (int)rc.x;
                nt = (int)rc.z - (int)rc.y;
#pragma unroll
                for (int j = 0; j < TB; j++)
                    if (j < nt) {
                        hrow[j] = (int)rc.y + j;
                        tok[j] = r.tok[hrow[j]];
                        w[j] = r.wsort[hrow[j]];
                    }
            }
        }
    } else {
        const int t0 = a * TB;
        if (t0 < r.ntok) {
            e = 0;
            nt = min(TB, r.ntok - t0);
#pragma unroll
            for (int j = 0; j < TB; j++) {
                hrow[j] = t0 + (j < nt ? j : 0);
                tok[j] = hrow[j];
                w[j] = 1.f;
            }
        }
    }
    if (lane == 0) {
        pl->e = e;
        pl->nt = e < 0 ? 0 : nt;
#pragma unroll
        for (int j = 0; j < TB; j++) {
            pl->hrow[j] = hrow[j];
            pl->tok[j] = tok[j];
            pl->w[j] = w[j];
        }
    }
}

// Stage the plan of this block into LDS and return its token count (0:
// nothing to do; uniform over the block).  Inline mode with several tokens per
// pass stages the ids and lets one wave search the partners; otherwise every
// wave plans for itself from global memory (all write the same values), which
// keeps the block's barriers off the path to its first weight loads.
template <int TB>
__device__ __forceinline__ int stage_plan(const F32Route &r, int a, int *sid, PassLds *pl) {
    if (r.ids && TB > 1) {
        for (int i = threadIdx.x; i < r.n; i += blockDim.x) sid[i] = r.ids[i];
        __syncthreads();
        if (wave_id() == 0) plan_wave<TB>(r, a, sid, pl);
        __syncthreads();
    } else {
        plan_wave<TB>(r, a, r.ids, pl);
    }
    return __builtin_amdgcn_readfirstlane(pl->nt);
}

// Buffer descriptors of one expert's matrix and this lane's byte offsets
// (its chunk's 16 packed bytes and its scale) inside a row.
struct SliceSrc {
    __amdgpu_buffer_rsrc_t q, s;
    uint32_t qlane, slane;
};

__device__ __forceinline__ SliceSrc slice_src(const F32Mat &M, int e, int chunk) {
    SliceSrc r;
    r.q = make_rsrc(M.q + (int64_t)e * M.q_stride, M.qbytes);
    r.s = make_rsrc(M.s + (int64_t)e * M.s_stride, M.sbytes);
    const bool ok = chunk < M.chunks;
    r.qlane = ok ? (uint32_t)chunk * 16u : OOB_OFFSET;
    r.slane = ok ? (((uint32_t)chunk * 32u) >> M.gshift) * 4u : OOB_OFFSET;
    return r;
}

// This lane's 32 activations of `row` (a row of `cols` f32 starting at
// base + row * ld); zero for a chunk past the row.  `vec` = 16-byte loads.
__device__ __forceinline__ void load_chunk(float (&x)[32], const float *base, int64_t row,
                                           int64_t ld, int col0, int cols, bool vec) {
    if (col0 >= cols) {
#pragma unroll
        for (int i = 0; i < 32; i++) x[i] = 0.f;
        return;
    }
    const float *p = base + row * ld + col0;
    if (vec && col0 + 32 <= cols) {
#pragma unroll
        for (int v = 0; v < 8; v++) {
            const f32x4 t = *(const f32x4 *)(p + 4 * v);
            x[4 * v + 0] = t.x;
            x[4 * v + 1] = t.y;
            x[4 * v + 2] = t.z;
            x[4 * v + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; i++) x[i] = col0 + i < cols ? p[i] : 0.f;
    }
}

// acc[t] = sum over the chunk of (16 q_i) x[t][i]: the 32 codes of one 16-byte
// load against NT tokens' activations.
template <int TB, int NT>
__device__ __forceinline__ void chunk_fma(const u32x4 &w, const float (&x)[TB][32],
                                          float (&acc)[TB]) {
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = 0.f;
#pragma unroll
    for (int d = 0; d < 4; d++) {
        const uint32_t v = w[d];
        const uint32_t hi = (v & 0xF0F0F0F0u) ^ 0x80808080u;
        const uint32_t lo = ((v << 4) & 0xF0F0F0F0u) ^ 0x80808080u;
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const float fe = (float)(int8_t)(lo >> (8 * b));
            const float fo = (float)(int8_t)(hi >> (8 * b));
#pragma unroll
            for (int t = 0; t < NT; t++) {
                acc[t] = fmaf(fe, x[t][8 * d + 2 * b], acc[t]);
                acc[t] = fmaf(fo, x[t][8 * d + 2 * b + 1], acc[t]);
            }
        }
    }
}

// Lane-transposed sum of 2^D row steps (a butterfly over lane bits 0..D-1).
// Step values arrive one at a time; level b combines two partial sums that
// each cover 2^b steps: every lane adds its value to the partner's (lane bit b
// flipped: quad_perm for bits 0 and 1, a rotation by 4 or 8 inside the DPP row
// for bits 2 and 3, which keeps the lower bits) and keeps the half of the
// steps whose bit b equals its own lane bit b.  After all D levels lane l
// holds a partial sum for step l mod 2^D; the lanes of an L-lane row that hold
// the same step (they differ only in bits D and up) cover disjoint lane sets
// whose union is the whole row, so their partial sums add up to the row sum.
// Every level costs one output per 2^(b+1) steps, three VALU instructions
// each (two DPP adds and a bit select).
template <int D>
struct Butterfly {
    float v[D + 1];   // v[b]: the pending partial sum that covers 2^b steps
};
template <int CTRL>
__device__ __forceinline__ float dpp_sum(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// Level B of the butterfly for a value of batch step `step`; false when the
// value waits for its partner block (the push ends there).
template <int B, int D>
__device__ __forceinline__ bool butterfly_level(Butterfly<D> &bf, float &v, int step) {
    if constexpr (B < D) {
        if (((step >> B) & 1) == 0) {
            bf.v[B] = v;
            return false;
        }
        constexpr int ctrl = B == 0 ? 0xB1 : B == 1 ? 0x4E : B == 2 ? 0x124 : 0x128;
        const float lo = dpp_sum<ctrl>(bf.v[B]), hi = dpp_sum<ctrl>(v);
        // lane bit B ? hi : lo, as a bit select (truth table 0xD8 = c ? b : a)
        const uint32_t m = 0u - (uint32_t)((lane_id() >> B) & 1);
        v = __uint_as_float(__builtin_amdgcn_bitop3_b32(__float_as_uint(lo), __float_as_uint(hi), m, 0xD8));
    }
    return true;
}
// Push the value of batch step `step` (compile-time after unrolling); returns
// the lane's finished sum after the batch's last step.
template <int D>
__device__ __forceinline__ float butterfly_push(Butterfly<D> &bf, float v, int step) {
    if (!butterfly_level<0, D>(bf, v, step)) return 0.f;
    if (!butterfly_level<1, D>(bf, v, step)) return 0.f;
    if (!butterfly_level<2, D>(bf, v, step)) return 0.f;
    if (!butterfly_level<3, D>(bf, v, step)) return 0.f;
    return v;
}

// Butterfly depth of a stream of NST steps, and the parts (lane groups whose
// partial sums are added in the epilogue) per row: L >> depth.
static inline int f32_depth_rt(int nst) { return nst >= 16 ? 4 : nst >= 8 ? 3 : nst >= 4 ? 2 : 1; }
template <int NST>
constexpr int f32_depth() { return NST >= 16 ? 4 : NST >= 8 ? 3 : NST >= 4 ? 2 : 1; }
template <int L, int NST>
constexpr int f32_parts() { return L >> f32_depth<NST>(); }

// Load steps in flight per wave, per tokens per pass.
template <int TB>
constexpr int f32_prefetch() { return TB == 1 ? 12 : TB == 2 ? 8 : 4; }

// Stream NST row steps of one slice: step j reads row row0 + j*(64/L) + the
// lane's sub-row (the last row of the matrix past its end).  Loads run PD
// steps ahead.  Each step's chunk sums, times the lane's group scale, go
// through a butterfly of depth D (2^D steps); lane l then writes, for step
// 2^D * batch + (l mod 2^D), its partial row sum to
// red[t * ld_t + part * ld_p + step * (64/L) + sub-row], part = (l mod L) >> D.
template <int L, int TB, int NT, int NST, int PD>
__device__ __forceinline__ void stream_slice(const SliceSrc &src, uint32_t rb, uint32_t sb,
                                             int row0, int rows, const float (&x)[TB][32],
                                             float *red, int ld_t, int ld_p) {
    constexpr int RPI = QMOE_WAVE / L;
    constexpr int D = f32_depth<NST>();
    constexpr int BD = 1 << D;
    static_assert(NST % BD == 0, "steps must be a multiple of the butterfly batch");
    const int lane = lane_id();
    const int sr = lane / L;
    u32x4 wq[PD];
    float ws[PD];
    auto load = [&](int j) {
        if (RPI == 1) {
            // one row per wave instruction: the row offset is scalar
            const int row = min(row0 + j, rows - 1);
            wq[j % PD] = __builtin_amdgcn_raw_buffer_load_b128(src.q, src.qlane, (uint32_t)row * rb, 0);
            ws[j % PD] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(src.s, src.slane, (uint32_t)row * sb, 0));
        } else {
            const int row = min(row0 + j * RPI + sr, rows - 1);
            wq[j % PD] = __builtin_amdgcn_raw_buffer_load_b128(src.q, src.qlane + (uint32_t)row * rb, 0u, 0);
            ws[j % PD] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(src.s, src.slane + (uint32_t)row * sb, 0u, 0));
        }
    };
#pragma unroll
    for (int j = 0; j < PD && j < NST; j++) load(j);
    Butterfly<D> bf[NT];
    float *dst = red + ((lane % L) >> D) * ld_p + (lane & (BD - 1)) * RPI + sr;
#pragma unroll
    for (int j = 0; j < NST; j++) {
        float acc[TB];
        chunk_fma<TB, NT>(wq[j % PD], x, acc);
        const float sc = ws[j % PD] * 0.0625f;
        if (j + PD < NST) load(j + PD);
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const float v = butterfly_push<D>(bf[t], acc[t] * sc, j % BD);
            if (j % BD == BD - 1) dst[t * ld_t + (j / BD) * BD * RPI] = v;
        }
    }
}

// The NT-token instance of a slice stream, chosen by the pass's token count.
template <int L, int TB, int NST, int PD>
__device__ __forceinline__ void stream_slice_nt(int nt, const SliceSrc &src, uint32_t rb,
                                                uint32_t sb, int row0, int rows,
                                                const float (&x)[TB][32], float *red, int ld_t,
                                                int ld_p) {
    if (TB >= 4 && nt == 4)
        stream_slice<L, TB, (TB >= 4 ? 4 : 1), NST, PD>(src, rb, sb, row0, rows, x, red, ld_t, ld_p);
    else if (TB >= 3 && nt == 3)
        stream_slice<L, TB, (TB >= 3 ? 3 : 1), NST, PD>(src, rb, sb, row0, rows, x, red, ld_t, ld_p);
    else if (TB >= 2 && nt == 2)
        stream_slice<L, TB, (TB >= 2 ? 2 : 1), NST, PD>(src, rb, sb, row0, rows, x, red, ld_t, ld_p);
    else
        stream_slice<L, TB, 1, NST, PD>(src, rb, sb, row0, rows, x, red, ld_t, ld_p);
}

// Blocks per SIMD the register allocation targets, per tokens per pass (no
// instance spills at these targets).
template <int TB>
constexpr int f32_waves_per_eu() { return TB == 1 ? 4 : 2; }

// Slot index of this block (grid y and z together).
__device__ __forceinline__ int f32_slot() { return blockIdx.z * gridDim.y + blockIdx.y; }

// Leading row of an inline gate+up launch: the worklist view of the call
// (block 0, one wave) and out <- 0 for the down projection's atomic adds.
__device__ void f32_lead_row(const F32Route &r, int *lds) {
    const int64_t total = (int64_t)r.out_tokens * r.out_cols;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride)
        r.out[i] = 0.f;
    if (blockIdx.x == 0 && wave_id() == 0) {
        DecodePlan none{};
        wl_wave(r.ids, r.topk_w, r.n, r.k, r.E, r.wl, none, lds, lds + (r.E + 1));
    }
}

// LDS of a block: the cross-slice sums (nred floats), the pass, the staged ids.
struct F32Lds {
    float *red;
    PassLds *pl;
    int *sid;
};
__device__ __forceinline__ F32Lds f32_lds(float *base, int nred) {
    F32Lds l;
    l.red = base;
    l.pl = reinterpret_cast<PassLds *>(base + nred);
    l.sid = reinterpret_cast<int *>(base + nred) + sizeof(PassLds) / sizeof(int);
    return l;
}

// ---------------------------------------------------------------------------
// gate+up: block = (ROWS rows of F, one pass).  Waves 0..S-1 stream the gate
// slices, waves S..2S-1 the same rows of up; the epilogue writes
// h = silu(g) * u in f32 for the pass's tokens, row hrow of h.  Cross-slice
// sums: red[(((m * S + s) * TB + t) * P + part) * ROWS + row], P parts per row.
// ---------------------------------------------------------------------------
template <int L, int TB, int ROWS>
__global__ void __launch_bounds__(F32_MAX_WAVES * QMOE_WAVE)
    __attribute__((amdgpu_waves_per_eu(f32_waves_per_eu<TB>())))
    f32_gateup_kernel(F32Mat G, F32Mat Up, const float *__restrict__ x, float *__restrict__ h,
                      F32Route r, int S) {
    extern __shared__ float lds_gu[];
    constexpr int RPI = QMOE_WAVE / L;
    constexpr int NST = ROWS / RPI;
    constexpr int P = f32_parts<L, NST>();
    int a = f32_slot();
    if (r.lead_row) {
        if (a == 0) {
            f32_lead_row(r, (int *)lds_gu);
            return;
        }
        a -= 1;
    }
    const int nred = 2 * S * TB * P * ROWS;
    const F32Lds l = f32_lds(lds_gu, nred);
    const int nt = stage_plan<TB>(r, a, l.sid, l.pl);
    if (nt == 0) return;
    const int e = __builtin_amdgcn_readfirstlane(l.pl->e);
    const int H = G.cols, F = G.rows;
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int m = w / S, s = w % S;
    const int chunk = s * L + lane_id() % L;
    const F32Mat &M = m ? Up : G;
    const SliceSrc src = slice_src(M, e, chunk);
    float xr[TB][32];
#pragma unroll
    for (int t = 0; t < TB; t++)
        if (t < nt) load_chunk(xr[t], x, l.pl->tok[t], H, chunk * 32, H, true);
    const int row0 = blockIdx.x * ROWS;
    float *red = l.red + (m * S + s) * TB * P * ROWS;
    stream_slice_nt<L, TB, NST, f32_prefetch<TB>()>(nt, src, M.rb, M.sb, row0, F, xr, red,
                                                    P * ROWS, ROWS);
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid < nt * ROWS) {
        const int t = tid / ROWS, rr = tid % ROWS;
        const int f = row0 + rr;
        if (f < F) {
            float g = 0.f, u = 0.f;
            for (int k = 0; k < S * P; k++) {
                const int sk = k / P, pk = k % P;
                g += l.red[((sk * TB + t) * P + pk) * ROWS + rr];
                u += l.red[(((S + sk) * TB + t) * P + pk) * ROWS + rr];
            }
            h[(int64_t)l.pl->hrow[t] * F + f] = silu(g) * u;
        }
    }
}

// ---------------------------------------------------------------------------
// down (and the plain matvec): block = (R * STEPS * 64/L output rows, one pass);
// wave w streams slice w % S of row group w / S.  Routed: out[tok] += w * y
// with f32 atomics (out was cleared ahead of the launch); direct: out = y.
// Cross-slice sums: red[((s * TB + t) * P + part) * NR + row].
// ---------------------------------------------------------------------------
template <int L, int TB, int STEPS>
__global__ void __launch_bounds__(F32_MAX_WAVES * QMOE_WAVE)
    __attribute__((amdgpu_waves_per_eu(f32_waves_per_eu<TB>())))
    f32_down_kernel(F32Mat D, const float *__restrict__ hin, int64_t h_ld, int h_cols,
                    float *__restrict__ out, F32Route r, int S, int R, bool routed, bool vec) {
    extern __shared__ float lds_dn[];
    constexpr int RPI = QMOE_WAVE / L;
    constexpr int RW = STEPS * RPI;     // rows per row group
    constexpr int P = f32_parts<L, STEPS>();
    const int NR = R * RW;
    const F32Lds l = f32_lds(lds_dn, S * TB * P * NR);
    const int nt = stage_plan<TB>(r, f32_slot(), l.sid, l.pl);
    if (nt == 0) return;
    const int e = __builtin_amdgcn_readfirstlane(l.pl->e);
    const int O = D.rows;
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int s = w % S, rg = w / S;
    const int chunk = s * L + lane_id() % L;
    const SliceSrc src = slice_src(D, e, chunk);
    float xr[TB][32];
#pragma unroll
    for (int t = 0; t < TB; t++)
        if (t < nt) load_chunk(xr[t], hin, l.pl->hrow[t], h_ld, chunk * 32, h_cols, vec);
    const int row0 = blockIdx.x * NR;
    float *red = l.red + s * TB * P * NR + rg * RW;
    stream_slice_nt<L, TB, STEPS, f32_prefetch<TB>()>(nt, src, D.rb, D.sb, row0 + rg * RW,
                                                             O, xr, red, P * NR, NR);
    __syncthreads();
    for (int i = threadIdx.x; i < nt * NR; i += blockDim.x) {
        const int t = i / NR, rr = i % NR;
        const int o = row0 + rr;
        if (o >= O) continue;
        float y = 0.f;
        for (int k = 0; k < S * P; k++) y += l.red[(((k / P) * TB + t) * P + k % P) * NR + rr];
        float *dst = out + (int64_t)l.pl->tok[t] * O + o;
        if (routed) unsafeAtomicAdd(dst, l.pl->w[t] * y);
        else *dst = y;
    }
}

// Lane layout for rows of `cols` inputs: L lanes per slice, S slices, at most
// smax slices; fewest idle lanes, then widest L.  {0, 0} if none fits.
struct F32Shape {
    int L, S;
};
static F32Shape f32_shape(int cols, int smax) {
    const int C = cols / 32;
    F32Shape best{0, 0};
    int best_waste = 1 << 30;
    const int Ls[3] = {64, 32, 16};
    for (int i = 0; i < 3; i++) {
        const int L = Ls[i];
        const int S = (C + L - 1) / L;
        if (S > smax) continue;
        const int waste = S * L - C;
        if (waste < best_waste) {
            best_waste = waste;
            best = F32Shape{L, S};
        }
    }
    return best;
}

bool f32_gateup_supported(int hidden) {
    return hidden % 64 == 0 && f32_shape(hidden, F32_MAX_WAVES / 2).L != 0;
}
bool f32_down_supported(int cols) {
    return cols % 64 == 0 && f32_shape(cols, F32_MAX_WAVES).L != 0;
}

// The uniform sizes of a matrix the kernels use (no division on the device).
F32Mat f32_mat(const QMat &m) {
    F32Mat f;
    f.q = m.q;
    f.s = m.s;
    f.q_stride = m.q_stride;
    f.s_stride = m.s_stride;
    f.rows = m.rows;
    f.cols = m.cols;
    f.chunks = m.cols / 32;
    f.rb = (uint32_t)(m.cols / 2);
    f.sb = (uint32_t)scales_per_row(m) * 4u;
    f.qbytes = (int64_t)m.rows * f.rb;
    f.sbytes = (int64_t)m.rows * f.sb;
    if (m.group >= m.cols) {
        f.gshift = 31;                 // one scale per row: index 0
    } else {
        int j = 0;
        while ((1 << j) < m.group) j++;
        f.gshift = j;                  // group 32 or 64 * 2^i: a power of two
    }
    return f;
}

// Tokens per weight pass (a pass shares one read and one unpack of the weights
// among its tokens; more tokens per pass cost registers and occupancy).  Four
// from two pairs per expert on average for gate+up (skewed layers put tens of
// tokens on a few experts: 64-token Zipf layer 1.64 -> 1.57 ms per call), from
// four for down (its four-token instance runs at lower occupancy).
int f32_tokens_per_pass(int pairs, int experts, bool gateup) {
    if (pairs >= (gateup ? 2 : 4) * (int64_t)experts) return 4;
    if (pairs > 1 && 2 * (int64_t)pairs >= experts) return 2;
    return 1;
}

static dim3 f32_grid(unsigned x, int64_t slots) {
    const int64_t gy = slots < 65535 ? (slots > 0 ? slots : 1) : 65535;
    return dim3(x, (unsigned)gy, (unsigned)((slots + gy - 1) / gy));
}

// Grid slots of a launch: inline = one per pair (+ the leading row), record =
// max_rec, direct = ceil(ntok / tb).
static int64_t f32_slots(const F32Route &r, int tb) {
    if (r.ids) return (int64_t)r.n + (r.lead_row ? 1 : 0);
    if (r.rec) return r.max_rec;
    return (r.ntok + tb - 1) / tb;
}

// Dynamic LDS of a launch: the cross-slice sums, the pass and (inline) the
// staged ids; a leading row needs the one-wave worklist's two counters of
// E + 1 ints.
static size_t f32_lds_bytes(const F32Route &r, size_t nred) {
    size_t b = nred * sizeof(float) + sizeof(PassLds) + (r.ids ? (size_t)r.n * sizeof(int) : 0);
    if (r.ids && r.lead_row) {
        const size_t wl = (size_t)2 * (r.E + 1) * sizeof(int);
        b = b > wl ? b : wl;
    }
    return b;
}

// Measured per call (one-token passes): the single expert 16.8 us at 32 rows,
// 11.5 at 8; the one-token layer 29-31 us at 32 or 8 rows, 28 at 16; the
// four-token layer is best at 32 rows.  Down at 32 steps for multi-token
// passes: the 64-token Zipf layer's down 430 -> 389 us.
constexpr int64_t F32_SHORT_BELOW = 512, F32_MID_BELOW = 2048;
static int64_t f32_est_passes(const F32Route &r, int tb) {
    if (r.ids) return r.n;
    if (r.rec) return r.max_rec;
    return (r.ntok + tb - 1) / tb;
}

hipError_t launch_f32_gateup(const QMat &gate, const QMat &up, const float *x, float *h,
                             const F32Route &r, int tb, hipStream_t st) {
    const F32Shape sh = f32_shape(gate.cols, F32_MAX_WAVES / 2);
    if (!sh.L || (r.ids && r.n > F32_INLINE_MAX)) return hipErrorInvalidValue;
    const int64_t waves_long = (int64_t)2 * sh.S * ((gate.rows + F32_GU_ROWS - 1) / F32_GU_ROWS) *
                               f32_est_passes(r, tb);
    const int rows = tb > 1 ? F32_GU_ROWS
                     : waves_long < F32_SHORT_BELOW ? F32_GU_ROWS_SHORT
                     : waves_long < F32_MID_BELOW   ? F32_GU_ROWS_MID
                                                    : F32_GU_ROWS;
    const dim3 grid = f32_grid((gate.rows + rows - 1) / rows, f32_slots(r, tb));
    const dim3 block(2 * sh.S * QMOE_WAVE);
    const int P = sh.L >> f32_depth_rt(rows * sh.L / QMOE_WAVE);
    const size_t lds = f32_lds_bytes(r, (size_t)2 * sh.S * tb * P * rows);
    const F32Mat G = f32_mat(gate), U = f32_mat(up);
#define X(L_, T_, R_)                                                                          \
    if (sh.L == L_ && tb == T_ && rows == R_) {                                                \
        hipLaunchKernelGGL((f32_gateup_kernel<L_, T_, R_>), grid, block, lds, st, G, U, x, h,   \
                           r, sh.S);                                                           \
        return hipGetLastError();                                                              \
    }
    X(64, 1, F32_GU_ROWS) X(64, 2, F32_GU_ROWS) X(64, 4, F32_GU_ROWS)
    X(32, 1, F32_GU_ROWS) X(32, 2, F32_GU_ROWS) X(32, 4, F32_GU_ROWS)
    X(16, 1, F32_GU_ROWS) X(16, 2, F32_GU_ROWS) X(16, 4, F32_GU_ROWS)
    X(64, 1, F32_GU_ROWS_SHORT) X(32, 1, F32_GU_ROWS_SHORT) X(16, 1, F32_GU_ROWS_SHORT)
    X(64, 1, F32_GU_ROWS_MID) X(32, 1, F32_GU_ROWS_MID) X(16, 1, F32_GU_ROWS_MID)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_f32_down(const QMat &down, const float *hin, int64_t h_ld, int h_cols,
                           float *out, const F32Route &r, int tb, bool routed, hipStream_t st) {
    const F32Shape sh = f32_shape(down.cols, F32_MAX_WAVES);
    if (!sh.L || (r.ids && r.n > F32_INLINE_MAX) || r.lead_row) return hipErrorInvalidValue;
    int R = 4 / sh.S;
    if (R < 1) R = 1;
    const int rpi = QMOE_WAVE / sh.L;
    const int nr_long = R * F32_DN_STEPS * rpi;
    const int64_t waves_long = (int64_t)sh.S * R * ((down.rows + nr_long - 1) / nr_long) *
                               f32_est_passes(r, tb);
    const int steps = tb > 1 ? F32_DN_STEPS_LONG
                      : waves_long < F32_MID_BELOW ? F32_DN_STEPS_SHORT
                                                   : F32_DN_STEPS;
    const int NR = R * steps * rpi;
    const dim3 grid = f32_grid((down.rows + NR - 1) / NR, f32_slots(r, tb));
    const dim3 block(sh.S * R * QMOE_WAVE);
    const int P = sh.L >> f32_depth_rt(steps);
    const size_t lds = f32_lds_bytes(r, (size_t)sh.S * tb * P * NR);
    const bool vec = h_cols % 4 == 0 && h_ld % 4 == 0 &&
                     (reinterpret_cast<uintptr_t>(hin) & 15u) == 0;
    const F32Mat D = f32_mat(down);
#define X(L_, T_, S_)                                                                          \
    if (sh.L == L_ && tb == T_ && steps == S_) {                                               \
        hipLaunchKernelGGL((f32_down_kernel<L_, T_, S_>), grid, block, lds, st, D, hin, h_ld,   \
                           h_cols, out, r, sh.S, R, routed, vec);                              \
        return hipGetLastError();                                                              \
    }
    X(64, 1, F32_DN_STEPS) X(64, 2, F32_DN_STEPS_LONG) X(64, 4, F32_DN_STEPS_LONG)
    X(32, 1, F32_DN_STEPS) X(32, 2, F32_DN_STEPS_LONG) X(32, 4, F32_DN_STEPS_LONG)
    X(16, 1, F32_DN_STEPS) X(16, 2, F32_DN_STEPS_LONG) X(16, 4, F32_DN_STEPS_LONG)
    X(64, 1, F32_DN_STEPS_SHORT) X(32, 1, F32_DN_STEPS_SHORT) X(16, 1, F32_DN_STEPS_SHORT)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace qmoe
