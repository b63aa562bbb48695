// Decode GEMVs (f32 activations): grouped int4 weights streamed once per
// expert with 128-bit loads, integer dot products in registers, f32 group
// scale, f32 accumulation and a cross-lane reduction.
//
// What is computed follows the colibri pull request "cuda+engine: full fmt=4
// (grouped int4 gs=64) support": per-group scale scales[o*ng + i/gs]
// applied once per group inside the row loop (comments "blocked by GPU
// driver instability" and the maintainer's data request, which asks for a
// shift instead of a divide and the scale hoisted per group), and the fused
// gate+up pair that loads the activation once for both matrices (Summary,
// "matmul_i4_grouped_pair").
//
// MI355X mapping.  A row of I inputs is I/64 groups of 32 bytes; LPR lanes
// share a row and each lane owns GPL whole groups, so every lane issues
// 2*GPL 16-byte loads per row and needs exactly GPL scales.  The activation
// is carried as five int4 digit planes per 32-element chunk (common.h), so a
// weight dword (8 codes, XOR 0x88888888 turns offset nibbles into two's
// complement) meets an activation dword in one v_dot8_i32_i4: 5 dot
// instructions per 8 weights, integer-exact, instead of 16+ f32 ops.  The
// chunk sum is rebuilt in int32 and scaled once per chunk and group.
// Each block owns a slice of rows of one expert and one weight pass over
// them (a plan record from the device worklist): the pass's tokens (one or
// two) share the weight stream, and an expert with more tokens gets one
// block per pass.
#include "common.h"
#include "launch.h"

namespace qmoe {

constexpr int GV_THREADS = 256;

// Blocks per CU the register allocation targets (more waves in flight hide
// more HBM latency); chosen per shape so that no instance spills.
template <int GPL, int LPR, int TB, bool DOWN, bool G32>
constexpr int gv_occ() {
    if (GPL != 1 || TB != 1) return 2;
    if (DOWN) return LPR <= 32 ? (G32 ? 3 : 4) : 2;
    return G32 ? 2 : 3;
}

template <int GPL>
struct XReg {
    uint32_t d[GPL][2 * XD_DWORDS];   // two chunks per group
    float f[GPL][2];
};

// Load the digits of `pos` for the lane's groups.
template <int GPL, int LPR>
__device__ __forceinline__ void load_digits(XReg<GPL> &xr, const XDigits &xd, int64_t pos,
                                            int ncpr, int ng, int lr) {
#pragma unroll
    for (int gi = 0; gi < GPL; gi++) {
        const int g = lr + gi * LPR;
        if (g < ng) {
            const u32x4 *src = (const u32x4 *)(xd.dig + (pos * ncpr + 2 * g) * XD_DWORDS);
#pragma unroll
            for (int v = 0; v < 2 * XD_DWORDS / 4; v++) {
                const u32x4 t = src[v];
                xr.d[gi][4 * v + 0] = t.x;
                xr.d[gi][4 * v + 1] = t.y;
                xr.d[gi][4 * v + 2] = t.z;
                xr.d[gi][4 * v + 3] = t.w;
            }
            const u32x2 ff = *(const u32x2 *)(xd.fac + pos * ncpr + 2 * g);
            xr.f[gi][0] = __uint_as_float(ff.x);
            xr.f[gi][1] = __uint_as_float(ff.y);
        } else {
#pragma unroll
            for (int v = 0; v < 2 * XD_DWORDS; v++) xr.d[gi][v] = 0;
            xr.f[gi][0] = 0.f;
            xr.f[gi][1] = 0.f;
        }
    }
}

template <int GPL, int U>
struct WReg {
    uint32_t w[U][GPL][8];
    float s[U][GPL][2];   // group 32: one scale per 32-input chunk; else [1] unused
};

// One expert's matrix as buffer descriptors (base and byte size in scalar
// registers) plus this lane's byte offsets inside a row: its 64-input
// groups' 32 packed bytes and their scales (group 32: the two scales of the
// two chunks; group 64m: scale (64 g) / group).  A lane without a group gets
// offsets past the end of the buffer, which read as zero.
template <int GPL>
struct RowSrc {
    __amdgpu_buffer_rsrc_t q, s;
    uint32_t qlane[GPL], slane[GPL];
    uint32_t rb, sb;     // packed bytes and scale bytes per row
};


template <int GPL, int LPR, bool G32>
__device__ __forceinline__ RowSrc<GPL> row_src(const QMat &M, int e, int lr) {
    RowSrc<GPL> r;
    const int ng = M.cols / 64;
    r.rb = (uint32_t)(M.cols / 2);
    r.sb = (uint32_t)scales_per_row(M) * 4;
    r.q = make_rsrc(M.q + (int64_t)e * M.q_stride, (int64_t)M.rows * r.rb);
    r.s = make_rsrc(M.s + (int64_t)e * M.s_stride, (int64_t)M.rows * r.sb);
#pragma unroll
    for (int gi = 0; gi < GPL; gi++) {
        const int g = lr + gi * LPR;
        const uint32_t si = G32 ? 2u * g : (uint32_t)(g * 64 / M.group);
        r.qlane[gi] = g < ng ? (uint32_t)g * 32 : OOB_OFFSET;
        r.slane[gi] = g < ng ? si * 4 : OOB_OFFSET;
    }
    return r;
}

// Load U rows (valid row indices) for the lane's groups.  When a lane group
// is a whole wave the row is wave-uniform and its byte offset goes into the
// scalar offset operand; otherwise it is added to the lane offset (an
// out-of-range lane offset stays out of range: rows are < 2^31 bytes).
template <int GPL, int LPR, int U, bool G32>
__device__ __forceinline__ void load_rows(WReg<GPL, U> &wr, const RowSrc<GPL> &src,
                                          const int *row) {
#pragma unroll
    for (int u = 0; u < U; u++) {
        const uint32_t qrow = (uint32_t)row[u] * src.rb;
        const uint32_t srow = (uint32_t)row[u] * src.sb;
#pragma unroll
        for (int gi = 0; gi < GPL; gi++) {
            u32x4 a, b;
            u32x2 sc;
            const uint32_t qv = LPR == 64 ? src.qlane[gi] : src.qlane[gi] + qrow;
            const uint32_t qs = LPR == 64 ? qrow : 0u;
            const uint32_t sv = LPR == 64 ? src.slane[gi] : src.slane[gi] + srow;
            const uint32_t ss = LPR == 64 ? srow : 0u;
            a = __builtin_amdgcn_raw_buffer_load_b128(src.q, qv, qs, 0);
            b = __builtin_amdgcn_raw_buffer_load_b128(src.q, qv + 16, qs, 0);
            if (G32) {
                sc = __builtin_amdgcn_raw_buffer_load_b64(src.s, sv, ss, 0);
            } else {
                sc.x = __builtin_amdgcn_raw_buffer_load_b32(src.s, sv, ss, 0);
                sc.y = sc.x;
            }
            wr.w[u][gi][0] = a.x ^ 0x88888888u;
            wr.w[u][gi][1] = a.y ^ 0x88888888u;
            wr.w[u][gi][2] = a.z ^ 0x88888888u;
            wr.w[u][gi][3] = a.w ^ 0x88888888u;
            wr.w[u][gi][4] = b.x ^ 0x88888888u;
            wr.w[u][gi][5] = b.y ^ 0x88888888u;
            wr.w[u][gi][6] = b.z ^ 0x88888888u;
            wr.w[u][gi][7] = b.w ^ 0x88888888u;
            wr.s[u][gi][0] = __uint_as_float(sc.x);
            wr.s[u][gi][1] = __uint_as_float(sc.y);
        }
    }
}

// PAIRED: the activation's two chunks of each group share one factor
// (x digits; h digits have one factor per chunk).
template <int GPL, int U, bool G32, bool PAIRED>
__device__ __forceinline__ float row_dot(const WReg<GPL, U> &wr, int u, const XReg<GPL> &xr) {
    float acc = 0.f;
#pragma unroll
    for (int gi = 0; gi < GPL; gi++) {
        if (PAIRED && !G32) {
            acc = fmaf(wr.s[u][gi][0], group_dot(&wr.w[u][gi][0], &xr.d[gi][0], xr.f[gi][0]), acc);
            continue;
        }
        const float g0 = chunk_dot(&wr.w[u][gi][0], &xr.d[gi][0], xr.f[gi][0]);
        const float g1 = chunk_dot(&wr.w[u][gi][4], &xr.d[gi][XD_DWORDS], xr.f[gi][1]);
        if (G32) acc = fmaf(wr.s[u][gi][1], g1, fmaf(wr.s[u][gi][0], g0, acc));
        else acc = fmaf(wr.s[u][gi][0], g0 + g1, acc);
    }
    return acc;
}

// Lane group of this thread (LPR lanes each).  With whole-wave groups it is
// the wave index, made visibly uniform so that row offsets derived from it
// stay in scalar registers (a buffer load's scalar offset computed from a
// value the compiler takes as per-lane is wrapped in a loop over its distinct
// values).
template <int LPR>
__device__ __forceinline__ int lane_group() {
    if (LPR == 64) return __builtin_amdgcn_readfirstlane(wave_id());
    return threadIdx.x / LPR;
}

// Plan record of this block: grid y and z together (a grid dimension other
// than x holds at most 65535 blocks; there can be one record per pair).
__device__ __forceinline__ int record_index() { return blockIdx.z * gridDim.y + blockIdx.y; }

inline dim3 gemv_grid(unsigned row_blocks, const GemvRoute &r) {
    const int64_t nrec = r.rec ? r.max_rec : 1;
    const int64_t gy = nrec < 65535 ? nrec : 65535;
    return dim3(row_blocks, (unsigned)gy, (unsigned)((nrec + gy - 1) / gy));
}

// Expert and sorted-position range of this block (one plan record).
__device__ __forceinline__ bool block_expert(const GemvRoute &r, int a, int &e, int &p0,
                                             int &p1) {
    if (r.rec == nullptr) {
        if (a != 0) return false;
        e = 0;
        p0 = 0;
        p1 = r.ntok;
        return true;
    }
    if (a >= r.max_rec) return false;
    const u32x4 rc = *(const u32x4 *)(r.rec + 4 * a);
    e = (int)rc.x;
    if (e < 0) return false;
    p0 = (int)rc.y;
    p1 = (int)rc.z;
    return true;
}

__device__ __forceinline__ int64_t token_of(const GemvRoute &r, int pos) {
    return r.rec == nullptr ? pos : r.tok[pos];
}

// Rows per batch: about 128 bytes of weights in flight per lane per batch.
template <int GPL, int NSTEP>
constexpr int batch_rows() {
    return (4 / GPL) < NSTEP ? (4 / GPL < 1 ? 1 : 4 / GPL) : NSTEP;
}

// Stream NSTEP rows per lane group (LPR lanes) of matrix `src` in batches of
// U rows, the next batch's loads issued before the current batch is
// computed.  row_at(step) gives the (valid) row index; emit(step, j, value)
// runs on the last lane of the group.
template <int GPL, int LPR, int TB, int U, int NSTEP, bool G32, bool PAIRED, class RowAt,
          class Prologue, class Emit>
__device__ __forceinline__ void stream_rows(const XReg<GPL> *xr, int nt, int lr,
                                            const RowSrc<GPL> &src, RowAt row_at,
                                            Prologue prologue, Emit emit) {
    constexpr int NB = NSTEP / U;
    static_assert(NB * U == NSTEP, "NSTEP must be a multiple of U");
    WReg<GPL, U> w[2];
    auto load_batch = [&](int b, WReg<GPL, U> &dst) {
        int rows[U];
#pragma unroll
        for (int u = 0; u < U; u++) rows[u] = row_at(b * U + u);
        load_rows<GPL, LPR, U, G32>(dst, src, rows);
    };
    // The first weight batch depends only on the expert; issue it before the
    // prologue's dependent chain (pair -> token -> activation digits).
    load_batch(0, w[0]);
    prologue();
#pragma unroll
    for (int b = 0; b < NB; b++) {
        if (b + 1 < NB) load_batch(b + 1, w[(b + 1) & 1]);
#pragma unroll
        for (int j = 0; j < TB; j++) {
            if (j < nt) {
#pragma unroll
                for (int u = 0; u < U; u++) {
                    float v = row_dot<GPL, U, G32, PAIRED>(w[b & 1], u, xr[j]);
                    v = reduce_dpp<LPR>(v);
                    if (lr == LPR - 1) emit(b * U + u, j, v);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// gate+up: block = (32 rows of F, one pass of one expert); 32 gate rows and the
// same 32 up rows (64 row tasks).  Writes h = silu(g)*u for the 32 rows as
// one digit chunk per sorted position.
// ---------------------------------------------------------------------------
template <int GPL, int LPR, int TB, bool G32>
__global__ void __launch_bounds__(GV_THREADS, (gv_occ<GPL, LPR, TB, false, G32>())) gemv_gateup_kernel(QMat G, QMat Up, XDigits xd,
                                                                 XDigits hd, GemvRoute r) {
    constexpr int RS = GV_THREADS / LPR;       // lane groups per block
    constexpr int NR = 64;                     // row tasks per block
    constexpr int NSTEP = NR / RS;             // rows per lane group
    constexpr int U = batch_rows<GPL, NSTEP>();
    __shared__ float res[TB][NR];

    int e, p0, p1;
    if (!block_expert(r, record_index(), e, p0, p1)) return;
    const int H = G.cols, F = G.rows;
    const int ng = H / 64, ncx = H / XD_CHUNK, nch = F / XD_CHUNK;
    const int lr = threadIdx.x % LPR, slot = lane_group<LPR>();
    const int row0 = blockIdx.x * 32;
    // Row tasks 0..63 are the 32 gate rows then the same 32 up rows; every
    // wave owns 16 consecutive tasks (NSTEP rows for each of its 64/LPR lane
    // groups), so waves 0-1 read gate and waves 2-3 up.
    static_assert(NSTEP * (64 / LPR) == 16, "16 row tasks per wave");
    const bool up_wave = __builtin_amdgcn_readfirstlane(wave_id()) >= 2;
    const RowSrc<GPL> src = row_src<GPL, LPR, G32>(up_wave ? Up : G, e, lr);
    auto row_at = [&](int step) { return row0 + ((slot * NSTEP + step) & 31); };

    for (int t0 = p0; t0 < p1; t0 += TB) {
        const int nt = min(TB, p1 - t0);
        XReg<GPL> xr[TB];
        stream_rows<GPL, LPR, TB, U, NSTEP, G32, true>(
            xr, nt, lr, src, row_at,
            [&]() {
#pragma unroll
                for (int j = 0; j < TB; j++)
                    if (j < nt) load_digits<GPL, LPR>(xr[j], xd, token_of(r, t0 + j), ncx, ng, lr);
            },
            [&](int step, int j, float v) { res[j][slot * NSTEP + step] = v; });
        __syncthreads();
        // epilogue: wave j quantises token j's 32 values of h
        const int w = wave_id(), lane = lane_id();
        if (w < nt && lane < 32) {
            const float h = silu(res[w][lane]) * res[w][32 + lane];
            const int64_t c = (int64_t)(t0 + w) * nch + blockIdx.x;
            uint32_t *dst = hd.dig + c * XD_DWORDS;
            const float f = quantise_chunk32(h, [&](int plane, int dw, uint32_t val) {
                dst[plane * 4 + dw] = val;
            });
            if (lane == 0) hd.fac[c] = f;
        }
        __syncthreads();
    }
}

// Output rows per down block: 64 for one group per lane, fewer for wider
// rows (32 at two groups, 16 at three), whose fully unrolled 64-row stream
// would not fit the register file; at least one row per lane group.
__host__ __device__ constexpr int down_rows_per_block(int gpl, int lpr) {
    const int base = gpl >= 3 ? 16 : gpl == 2 ? 32 : 64;
    return GV_THREADS / lpr > base ? GV_THREADS / lpr : base;
}

// ---------------------------------------------------------------------------
// down (and plain matvec): block = (down_rows_per_block output rows, one
// pass of one expert).
// Routed mode adds w * y into out[token] with f32 atomics (out was cleared by
// the preparation kernel); direct mode stores y to out[pos].
// ---------------------------------------------------------------------------
template <int GPL, int LPR, int TB, bool G32>
__global__ void __launch_bounds__(GV_THREADS, (gv_occ<GPL, LPR, TB, true, G32>())) gemv_down_kernel(QMat D, XDigits hd,
                                                               float *__restrict__ out,
                                                               GemvRoute r) {
    constexpr int RS = GV_THREADS / LPR;
    constexpr int NR = down_rows_per_block(GPL, LPR);
    constexpr int NSTEP = NR / RS;
    constexpr int U = batch_rows<GPL, NSTEP>();

    int e, p0, p1;
    if (!block_expert(r, record_index(), e, p0, p1)) return;
    const int O = D.rows, I = D.cols;
    const int ng = I / 64, ncx = I / XD_CHUNK;
    const int lr = threadIdx.x % LPR, slot = lane_group<LPR>();
    const int row0 = blockIdx.x * NR + slot * NSTEP;
    const bool routed = r.rec != nullptr;
    const RowSrc<GPL> src = row_src<GPL, LPR, G32>(D, e, lr);
    // rows past O re-read row O-1 and are never emitted
    auto row_at = [&](int step) { return min(row0 + step, O - 1); };

    for (int t0 = p0; t0 < p1; t0 += TB) {
        const int nt = min(TB, p1 - t0);
        XReg<GPL> xr[TB];
        float wj[TB];
        int64_t tj[TB];
        auto prologue = [&]() {
#pragma unroll
            for (int j = 0; j < TB; j++) {
                wj[j] = 0.f;
                tj[j] = 0;
                if (j < nt) {
                    load_digits<GPL, LPR>(xr[j], hd, t0 + j, ncx, ng, lr);
                    if (routed) {
                        tj[j] = r.tok[t0 + j];
                        wj[j] = r.wsort[t0 + j];
                    } else {
                        tj[j] = t0 + j;
                        wj[j] = 1.f;
                    }
                }
            }
        };
        stream_rows<GPL, LPR, TB, U, NSTEP, G32, false>(xr, nt, lr, src, row_at, prologue,
                                            [&](int step, int j, float v) {
                                                const int o = row0 + step;
                                                if (o < O) {
                                                    float *dst = out + tj[j] * O + o;
                                                    if (routed) unsafeAtomicAdd(dst, wj[j] * v);
                                                    else *dst = v;
                                                }
                                            });
    }
}

// Lane layout for a row of ng groups: LPR lanes x GPL groups per lane.
struct GemvShape {
    int gpl, lpr;
};

// Fewer groups per lane is preferred: one group per lane keeps two tokens'
// digits in registers (a second token costs no second weight pass), so it
// wins whenever at least 70% of the lanes have a group.
static GemvShape choose_shape(int ng) {
    const int lprs[4] = {64, 32, 16, 8};
    for (int gpl = 1; gpl <= 3; gpl++) {
        GemvShape best{0, 0};
        double best_eff = 0;
        for (int li = 0; li < 4; li++) {
            const int lpr = lprs[li];
            if (gpl * lpr < ng || (gpl - 1) * lpr >= ng) continue;
            const double eff = (double)ng / (gpl * lpr);
            if (eff > best_eff + 1e-9) {
                best_eff = eff;
                best = GemvShape{gpl, lpr};
            }
        }
        if (best.gpl && best_eff >= 0.7) return best;
    }
    GemvShape best{0, 0};
    double best_eff = 0;
    for (int gpl = 1; gpl <= 3; gpl++)
        for (int li = 0; li < 4; li++) {
            const int lpr = lprs[li];
            if (gpl * lpr < ng || (gpl - 1) * lpr >= ng) continue;
            const double eff = (double)ng / (gpl * lpr);
            if (eff > best_eff + 1e-9) {
                best_eff = eff;
                best = GemvShape{gpl, lpr};
            }
        }
    return best;
}

bool gemv_supported(int cols) {
    if (cols % 64) return false;
    return choose_shape(cols / 64).gpl != 0;
}

// (groups per lane, lanes per row, tokens per pass).  Two tokens per pass
// only with one group per lane (register budget).
#define QMOE_GEMV_SHAPES(X)                                                                     \
    X(1, 64, 1) X(1, 32, 1) X(1, 16, 1) X(1, 8, 1) X(1, 64, 2) X(1, 32, 2) X(1, 16, 2) X(1, 8, 2) \
        X(2, 64, 1) X(2, 32, 1) X(2, 16, 1) X(2, 8, 1) X(3, 64, 1) X(3, 32, 1) X(3, 16, 1)      \
            X(3, 8, 1)

// Tokens per weight pass (measured on MI355X): gate+up keeps two tokens'
// digits in registers once there are at least half as many pairs as experts
// (128 experts: 16 tokens x top-8 186.8 vs 189.4 us per call with one; at 4
// tokens most experts have a single token, and the one-token instance, with
// its higher occupancy, is faster: 69.4 vs 70.8 us); the down projection runs
// faster with one token per pass at every batch size (fewer registers, more
// waves in flight; its extra passes hit in L2).
static int tokens_per_pass(const GemvShape &s, int pairs, int experts, bool gateup) {
    if (s.gpl != 1 || !gateup) return 1;
    return pairs > 1 && 2 * (int64_t)pairs >= experts ? 2 : 1;
}

int gemv_tokens_per_pass(const QMat &m, int pairs, int experts, bool gateup) {
    return tokens_per_pass(choose_shape(m.cols / 64), pairs, experts, gateup);
}

hipError_t launch_gemv_gateup(const QMat &gate, const QMat &up, XDigits xd, XDigits hd,
                              const GemvRoute &r, hipStream_t st) {
    const GemvShape s = choose_shape(gate.cols / 64);
    const int tb = tokens_per_pass(s, r.pairs, r.experts, true);
    const dim3 grid = gemv_grid(gate.rows / 32, r);
    const bool g32 = gate.group == 32;
#define X(G_, L_, T_)                                                                          \
    if (s.gpl == G_ && s.lpr == L_ && tb == T_) {                                              \
        if (g32)                                                                               \
            hipLaunchKernelGGL((gemv_gateup_kernel<G_, L_, T_, true>), grid, dim3(GV_THREADS), \
                               0, st, gate, up, xd, hd, r);                                    \
        else                                                                                   \
            hipLaunchKernelGGL((gemv_gateup_kernel<G_, L_, T_, false>), grid, dim3(GV_THREADS), \
                               0, st, gate, up, xd, hd, r);                                    \
        return hipGetLastError();                                                              \
    }
    QMOE_GEMV_SHAPES(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_gemv_down(const QMat &down, XDigits hd, float *out, const GemvRoute &r,
                            hipStream_t st) {
    const GemvShape s = choose_shape(down.cols / 64);
    const int tb = tokens_per_pass(s, r.pairs, r.experts, false);
    const int nr = down_rows_per_block(s.gpl, s.lpr);
    const dim3 grid = gemv_grid((down.rows + nr - 1) / nr, r);
    const bool g32 = down.group == 32;
#define X(G_, L_, T_)                                                                        \
    if (s.gpl == G_ && s.lpr == L_ && tb == T_) {                                            \
        if (g32)                                                                             \
            hipLaunchKernelGGL((gemv_down_kernel<G_, L_, T_, true>), grid, dim3(GV_THREADS), \
                               0, st, down, hd, out, r);                                     \
        else                                                                                 \
            hipLaunchKernelGGL((gemv_down_kernel<G_, L_, T_, false>), grid, dim3(GV_THREADS), \
                               0, st, down, hd, out, r);                                     \
        return hipGetLastError();                                                            \
    }
    QMOE_GEMV_SHAPES(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_gemv_matvec(const QMat &w, XDigits xd, int batch, float *y, hipStream_t st) {
    GemvRoute r{};
    r.ntok = batch;
    r.pairs = batch;
    r.experts = 1;
    return launch_gemv_down(w, xd, y, r, st);
}

}  // namespace qmoe
