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
//  * v_mfma_f32_32x32x16_f16; block = 4 waves x (256 rows x 32 features of
//    gate and of up) or 4 waves x (256 rows x 64 features) for down, so each
//    unpacked weight fragment feeds 8 row fragments (accumulators live in
//    AGPRs); row fragments past the tile's rows are skipped; the
//    activation tile (128 x 64 f16 per group) is double-buffered in LDS with
//    octets XOR-swizzled by row; global loads of group g+1 are issued
//    before the MFMAs of group g, and two blocks per CU overlap waits.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace qmoe {

constexpr int MF_THREADS = 256;
constexpr int BM = MFMA_BM;   // token rows per worklist tile
// A block takes BMK rows: a whole tile or a part of it (BM / BMK parts).
template <int BMK>
constexpr int mf_of() { return BMK / 32; }   // 32-row MFMA fragments per block
template <int BMK>
constexpr int occ_of() { return BMK > 128 ? 1 : 2; }   // blocks per CU
// gate+up takes whole 256-row tiles (each unpacked weight fragment feeds 8
// row fragments; one block per CU); down, with a third of the k-depth and
// four times the output bytes per row, takes half tiles at two blocks per
// CU so one block's prologue and stores overlap the other's MFMAs.
constexpr int GATEUP_BM = 256;
constexpr int DOWN_BM = 128;

// LDS offset (in 16-bit elements) of octet `o` of row `m` in a BMK x 64 tile.
__device__ __forceinline__ int sw_off(int m, int o) { return m * 64 + ((o ^ (m & 7)) << 3); }

// s_waitcnt immediate (gfx9 layout) that waits until at most n vector memory
// loads of this wave are outstanding and leaves the other counters alone.
__host__ __device__ constexpr int waitcnt_vm(int n) {
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// Position of element e (0..7) of an octet after the unpack permutation.
__device__ __forceinline__ int octet_pos(int e) { return e < 4 ? 2 * e : 2 * (e - 4) + 1; }

// 8 packed codes (one dword) -> 8 f16 values q*s in unpack order.  Pair i
// (nibbles i and 4+i) lands in the mantissas of two f16 1024.0 with one
// and-or (mask and exponent bits held in registers, so the compiler can use
// the 3-operand form), then a packed add of -1032 gives the exact code and a
// packed multiply applies the group scale.
__device__ __forceinline__ f16x8 dequant8(uint32_t d, f16x2 s2) {
    uint32_t mask = 0x000F000Fu, expo = 0x64006400u;
    asm("" : "+v"(mask));
    asm("" : "+v"(expo));
    const f16x2 off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t t = ((d >> (4 * i)) & mask) | expo;
        const f16x2 v = (__builtin_bit_cast(f16x2, t) + off) * s2;
        r[2 * i] = v[0];
        r[2 * i + 1] = v[1];
    }
    return r;
}

struct TileInfo {
    int e, row0, rows, pos0;
};

// Rows of block item `item`: part item % (BM / BMK) of worklist tile
// item / (BM / BMK); direct mode has plain BMK-row items.
template <int BMK>
__device__ __forceinline__ bool tile_info(const MfmaRoute &r, int item, TileInfo &ti) {
    if (r.wl.pairs == nullptr) {
        const int row0 = item * BMK;
        if (row0 >= r.ntok) return false;
        ti.e = 0;
        ti.row0 = row0;
        ti.pos0 = row0;
        ti.rows = min(BMK, r.ntok - row0);
        return true;
    }
    constexpr int SPLIT = BM / BMK;
    const int tile = item / SPLIT, part = item - tile * SPLIT;
    if (tile >= r.wl.n_tiles[0]) return false;
    ti.e = r.wl.tiles[2 * tile];
    ti.row0 = r.wl.tiles[2 * tile + 1] + part * BMK;
    const int c = r.wl.counts[ti.e];
    if (ti.row0 >= c) return false;
    ti.pos0 = r.wl.offsets[ti.e] + ti.row0;
    ti.rows = min(BMK, c - ti.row0);
    return true;
}

// Work item (tile, column block) of this block.  The GPU hands linear block
// ids to its 8 XCDs round-robin, and each XCD has its own L2; so each XCD is
// given one contiguous run of the real items (their count comes from the
// device worklist), column blocks of a tile adjacent: a tile's activation
// rows and an expert's weight slices are then fetched into one L2 instead of
// up to eight.  gridDim.x is a multiple of 8 and >= the largest item count.
template <int BMK>
__device__ __forceinline__ bool work_item(const MfmaRoute &r, int ncb, int &tile, int &cb) {
    const int ntiles = r.wl.pairs ? r.wl.n_tiles[0] * (BM / BMK) : (r.ntok + BMK - 1) / BMK;
    const int W = ntiles * ncb;
    const int per_xcd = (W + 7) / 8;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int w = xcd * per_xcd + local;
    if (local >= per_xcd || w >= W) return false;
    tile = w / ncb;
    cb = w - tile * ncb;
    return true;
}

static unsigned xcd_grid(int64_t items) { return (unsigned)(((items + 7) / 8) * 8); }

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
// Shared main loop.  The block owns a BM-row tile of f16 activation rows and
// each wave NF = 2 column fragments of 32 weight rows.  acc[i][j]: row
// fragment i (32 rows), column fragment j.  MFC (8 or 4) row fragments are
// computed; a tile of at most 128 rows takes the MFC = 4 instance.
//
// All global reads are buffer loads: the 128-bit descriptor (base, byte
// size) sits in scalar registers, each lane keeps a 32-bit byte offset, and
// the per-group advance is the scalar offset operand, so the loop spends no
// vector instructions on addresses; reads past the descriptor's size return 0.
//
// Pipeline.  A 64-k group g (one scale group) is 4 k-steps of 16:
//  * activation tile: buffer loads straight into LDS (16 B per lane) into a
//    ring of 4 LDS stages.  One such load of a wave writes 1 KB of LDS in
//    lane order; load i of wave w fills rows 32i + 8w + lane/8 (row fragment
//    i), and lane l fetches the octet that the XOR swizzle places at slot l%8
//    of its row.
//  * packed weights + scales: registers, 4 slots.
//  * operands of k-step s+1 (LDS reads of the activation fragments, unpack
//    of the weight fragments) are produced while the MFMAs of step s run;
//    with one wave per SIMD nothing else hides their latency, so the
//    instruction scheduler is told to interleave them (1 MFMA, 1 LDS read,
//    a few VALU ops, repeated).
//  * group g+1 is synchronised just before the last k-step of group g:
//    counted vmcnt wait (each thread issues exactly MFC + 2*NF loads per
//    group in a fixed order, so letting the two newest groups' loads stay in
//    flight guarantees group g+1 has landed), then one s_barrier.  Every
//    wave has by then finished its LDS reads of stage g, so the loads of
//    group g+4 into that stage are issued right after the barrier, and the
//    last k-step's MFMAs overlap group g+1's first operand reads.
// ---------------------------------------------------------------------------
constexpr int NF = 2;

template <int MF>
struct Frags {
    f32x16 acc[MF][NF];
};

// Buffer descriptor over [base, base + bytes); bytes < 2^32 is checked by
// the host.  Word 3 selects 32-bit data format, as raw loads require.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             (int)(uint32_t)bytes, 0x00020000);
}

// Sources of one block: activation tile (one descriptor, MF lane offsets at
// group 0) and the wave's two weight column fragments.
template <int MF>
struct LoopSrc {
    __amdgpu_buffer_rsrc_t a;
    uint32_t aoff[MF];
    __amdgpu_buffer_rsrc_t q[NF], s[NF];
    uint32_t qoff[NF], soff[NF];
};

#define QMOE_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Scheduling hint for one k-step: n_mfma MFMAs, each followed by one LDS
// read (while any remain) and `valu` VALU instructions.
template <int N_MFMA, int N_DS, int VALU>
__device__ __forceinline__ void interleave_hint() {
#pragma unroll
    for (int t = 0; t < N_MFMA; t++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (t < N_DS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, VALU, 0);
    }
}

template <int MF, int MFC>
__device__ __forceinline__ void mfma_mainloop(Frags<MF> &fr, const LoopSrc<MF> &src, int ng,
                                              uint16_t *__restrict__ s0,
                                              uint16_t *__restrict__ s1,
                                              uint16_t *__restrict__ s2,
                                              uint16_t *__restrict__ s3) {
    static_assert(MFC <= MF, "row fragments");
    constexpr int LPG = MFC + 2 * NF;   // loads per thread per group, in issue order
    constexpr int VALU_PER_MFMA = (40 + MFC * NF - 1) / (MFC * NF);
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int hh = lane >> 5, nl = lane & 31;
#pragma unroll
    for (int i = 0; i < MFC; i++)
#pragma unroll
        for (int j = 0; j < NF; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) fr.acc[i][j][v] = 0.f;

    u32x4 rb[4][NF];
    float rs[4][NF];
    f16x8 av[2][MFC], bq[2][NF];
    f16x2 sc[NF];
    // Loads of group g (clamped to the last real group; the padding groups
    // past ng get a zero scale) into register slot `slot` and LDS stage buf.
    auto issue_loads = [&](int g, int slot, uint16_t *buf) {
        const int gc = g < ng ? g : ng - 1;
#pragma unroll
        for (int i = 0; i < MFC; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(src.a, QMOE_LDS(buf + (i * 4 + w) * 512), 16,
                                                     src.aoff[i], gc * 128, 0, 0);
#pragma unroll
        for (int j = 0; j < NF; j++) {
            rb[slot][j] = __builtin_amdgcn_raw_buffer_load_b128(src.q[j], src.qoff[j], gc * 32, 0);
            rs[slot][j] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(src.s[j], src.soff[j], gc * 4, 0));
        }
    };
    // Operands of k-step kk of group g (ring slot/stage `slot`, buf) into
    // operand buffer p.
    auto operands = [&](int p, int g, int slot, const uint16_t *buf, int kk) {
        if (kk == 0) {
#pragma unroll
            for (int j = 0; j < NF; j++) {
                const _Float16 sh = g < ng ? (_Float16)rs[slot][j] : (_Float16)0.0f;
                sc[j] = f16x2{sh, sh};
            }
        }
#pragma unroll
        for (int i = 0; i < MFC; i++)
            av[p][i] = *(const f16x8 *)&buf[sw_off(32 * i + nl, 4 * hh + kk)];
#pragma unroll
        for (int j = 0; j < NF; j++) bq[p][j] = dequant8(rb[slot][j][kk], sc[j]);
    };
    auto mfmas = [&](int p) {
#pragma unroll
        for (int i = 0; i < MFC; i++)
#pragma unroll
            for (int j = 0; j < NF; j++)
                fr.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[p][i], bq[p][j],
                                                                     fr.acc[i][j], 0, 0, 0);
    };
    // Group g (ring slot/stage `slot`, stages cur and next): k-steps 0..2
    // prefetch the next step's operands; before step 3, group g+1 is
    // synchronised (this wave's LDS reads of cur are done, every thread's
    // loads of group g+1 have landed, barrier), group g+4's loads go into
    // cur, and step 3 prefetches group g+1's first operands.  Nothing here
    // is conditional, so no register holding an in-flight load is ever
    // copied (a copy would wait for the load).
    auto group = [&](int g, int slot, uint16_t *cur, uint16_t *next) {
#pragma unroll
        for (int kk = 0; kk < 3; kk++) {
            operands((kk + 1) & 1, g, slot, cur, kk + 1);
            mfmas(kk & 1);
            interleave_hint<MFC * NF, MFC, VALU_PER_MFMA>();
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPG));
        __builtin_amdgcn_s_barrier();
        issue_loads(g + 4, slot, cur);
        operands(0, g + 1, (slot + 1) & 3, next, 0);
        mfmas(1);
        interleave_hint<MFC * NF, MFC, VALU_PER_MFMA>();
    };

    // Prologue: groups 0..2 in flight, group 0 synchronised, group 3 issued,
    // operands of group 0 step 0 read.  The loop runs ng rounded up to a
    // multiple of 4 groups; loads past the end re-read the last group and
    // the padding groups multiply by a zero scale.
    issue_loads(0, 0, s0);
    issue_loads(1, 1, s1);
    issue_loads(2, 2, s2);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPG));
    __builtin_amdgcn_s_barrier();
    issue_loads(3, 3, s3);
    operands(0, 0, 0, s0, 0);
    for (int g = 0; g < ng; g += 4) {
        group(g, 0, s0, s1);
        group(g + 1, 1, s1, s2);
        group(g + 2, 2, s2, s3);
        group(g + 3, 3, s3, s0);
    }
    // no load may still be writing LDS when the block ends
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
}

// Row (within the tile) held by accumulator v of lane `lane` in m-frag i.
__device__ __forceinline__ int acc_row(int i, int v, int lane) {
    return 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// Runs the main loop over the row fragments a tile of `rows` rows needs
// (rounded up to MF, MF/2 or MF/4 fragments).
template <int MF>
__device__ __forceinline__ void run_mainloop(Frags<MF> &fr, const LoopSrc<MF> &src, int ng, int rows,
                                             uint16_t *__restrict__ s0,
                                             uint16_t *__restrict__ s1,
                                             uint16_t *__restrict__ s2,
                                             uint16_t *__restrict__ s3) {
    if (rows > 16 * MF) mfma_mainloop<MF, MF>(fr, src, ng, s0, s1, s2, s3);
    else if (rows > 8 * MF) mfma_mainloop<MF, MF / 2>(fr, src, ng, s0, s1, s2, s3);
    else mfma_mainloop<MF, MF / 4>(fr, src, ng, s0, s1, s2, s3);
}

// Activation tile sources: load i of wave w fills rows 32i + 8w + lane/8,
// whose swizzle slot lane%8 holds octet (lane%8) ^ (row%8).  Rows past the
// tile read a valid row (row 0) and are never stored.
template <int MF, typename RowOf>
__device__ __forceinline__ void tile_offsets(LoopSrc<MF> &src, int rows, int row_elems,
                                             RowOf row_of) {
    const int lane = lane_id(), w = wave_id();
    const int oct = (lane & 7) ^ ((lane >> 3) & 7);
#pragma unroll
    for (int i = 0; i < MF; i++) {
        int m = 32 * i + 8 * w + (lane >> 3);
        if (m >= rows) m = 0;
        src.aoff[i] = (uint32_t)(row_of(m) * row_elems * 2 + oct * 16);
    }
}

// ---------------------------------------------------------------------------
// gate+up: block = (128 features of F for gate and up, one tile of <=256
// rows).  Wave w: features n0 + 32w .. +32 of gate (frag 0) and up (frag 1).
// Output h = silu(g) * u as f16 at sorted position pos0 + m, octet-permuted
// in the feature index (the down projection's k).
// ---------------------------------------------------------------------------
template <int BMK>
__global__ void __launch_bounds__(MF_THREADS, occ_of<BMK>()) mfma_gateup_kernel(
    QMat G, QMat Up, const uint16_t *__restrict__ x16, const float *__restrict__ xinv,
    uint16_t *__restrict__ h16, MfmaRoute r) {
    constexpr int MF = mf_of<BMK>();
    __shared__ __attribute__((aligned(1024))) uint16_t s0[BMK * 64], s1[BMK * 64],
        s2[BMK * 64], s3[BMK * 64];
    __shared__ float sInv[BMK];

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
    tile_offsets(src, ti.rows, H, token);
    for (int m = tid; m < BMK; m += MF_THREADS) sInv[m] = m < ti.rows ? xinv[token(m)] : 0.f;
    const int hh = lane >> 5;
    const int nn = wave_on ? n : 0;       // idle waves read row 0 (valid) and store nothing
    const QMat *mats[NF] = {&G, &Up};
#pragma unroll
    for (int j = 0; j < NF; j++) {
        const QMat &M = *mats[j];
        src.q[j] = make_rsrc(M.q + (int64_t)ti.e * M.q_stride, (int64_t)F * (H / 2));
        src.s[j] = make_rsrc(M.s + (int64_t)ti.e * M.s_stride, (int64_t)F * ng * 4);
        src.qoff[j] = (uint32_t)(nn * (H / 2) + 16 * hh);
        src.soff[j] = (uint32_t)(nn * ng * 4);
    }

    Frags<MF> fr;
    run_mainloop<MF>(fr, src, ng, ti.rows, s0, s1, s2, s3);

    if (!wave_on) return;
    const int npos = (n & ~7) + octet_pos(n & 7);
#pragma unroll
    for (int i = 0; i < MF; i++) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = acc_row(i, v, lane);
            if (m < ti.rows) {
                const float sc = sInv[m];
                const float h = silu(fr.acc[i][0][v] * sc) * (fr.acc[i][1][v] * sc);
                h16[(int64_t)(ti.pos0 + m) * F + npos] =
                    __builtin_bit_cast(uint16_t, (_Float16)h);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// down: block = (256 features of H, one tile of <=256 rows); wave w:
// features n0 + 64w + 32j + (lane%32), j = 0, 1.
// Routed: Y[pos] = w * (D h); direct: out[pos] = D h.
// ---------------------------------------------------------------------------
template <int BMK>
__global__ void __launch_bounds__(MF_THREADS, occ_of<BMK>()) mfma_down_kernel(
    QMat D, const uint16_t *__restrict__ h16, float *__restrict__ y, MfmaRoute r) {
    constexpr int MF = mf_of<BMK>();
    __shared__ __attribute__((aligned(1024))) uint16_t s0[BMK * 64], s1[BMK * 64],
        s2[BMK * 64], s3[BMK * 64];
    __shared__ float sW[BMK];

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
    tile_offsets(src, ti.rows, F, [&](int m) -> int64_t { return ti.pos0 + m; });
    int ncol[NF];
#pragma unroll
    for (int j = 0; j < NF; j++) {
        ncol[j] = cb * 256 + 64 * w + 32 * j + (lane & 31);
        const int nn = ncol[j] < H ? ncol[j] : 0;
        src.q[j] = make_rsrc(D.q + (int64_t)ti.e * D.q_stride, (int64_t)H * (F / 2));
        src.s[j] = make_rsrc(D.s + (int64_t)ti.e * D.s_stride, (int64_t)H * ng * 4);
        src.qoff[j] = (uint32_t)(nn * (F / 2) + 16 * hh);
        src.soff[j] = (uint32_t)(nn * ng * 4);
    }

    Frags<MF> fr;
    run_mainloop<MF>(fr, src, ng, ti.rows, s0, s1, s2, s3);

#pragma unroll
    for (int i = 0; i < MF; i++) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = acc_row(i, v, lane);
            if (m < ti.rows) {
                const int pos = ti.pos0 + m;
                const float wgt = sW[m];
#pragma unroll
                for (int j = 0; j < NF; j++)
                    if (ncol[j] < H) y[(int64_t)pos * H + ncol[j]] = wgt * fr.acc[i][j][v];
            }
        }
    }
}

// out[t] = sum_j Y[inv[t*k + j]], slots in order; 4 floats per thread.
__global__ void __launch_bounds__(256) combine_kernel(const float *__restrict__ y,
                                                      const int32_t *__restrict__ inv, int k,
                                                      int hidden, float *__restrict__ out) {
    const int t = blockIdx.y;
    const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (n >= hidden) return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; j++) {
        const int pos = inv[(int64_t)t * k + j];
        if (pos >= 0) acc += *(const f32x4 *)(y + (int64_t)pos * hidden + n);
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
    hipLaunchKernelGGL(mfma_gateup_kernel<BMK>, grid, dim3(MF_THREADS), 0, st, gate, up, x16,
                       xinv, h16, r);
    return hipGetLastError();
}

hipError_t launch_mfma_down(const QMat &down, const uint16_t *h16, float *y, const MfmaRoute &r,
                            hipStream_t st) {
    constexpr int BMK = DOWN_BM;
    const int64_t items = r.wl.pairs ? (int64_t)r.max_tiles * (BM / BMK) : (r.ntok + BMK - 1) / BMK;
    const dim3 grid(xcd_grid(items * ((down.rows + 255) / 256)));
    hipLaunchKernelGGL(mfma_down_kernel<BMK>, grid, dim3(MF_THREADS), 0, st, down, h16, y, r);
    return hipGetLastError();
}

hipError_t launch_combine(const float *y, const int32_t *inv, int tokens, int k, int hidden,
                          float *out, hipStream_t st) {
    const dim3 grid((hidden / 4 + 255) / 256, tokens);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, y, inv, k, hidden, out);
    return hipGetLastError();
}

}  // namespace qmoe
