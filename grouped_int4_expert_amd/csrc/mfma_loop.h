// Shared pieces of the prefill MFMA kernels (gate+up in mfma.hip, down in
// mfma_down.hip): tile bookkeeping, the activation-tile swizzle, the int4 ->
// f16 operand unpack and the software-pipelined main loop.  The design notes
// are at the top of mfma.hip.
#pragma once

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

// Swizzle slot of octet `o` (16 bytes) in row `m` of a BMK x 64 f16 tile
// (128-byte rows), and its LDS offset in 16-bit elements.  gfx950's LDS has
// 64 four-byte banks and serves a 128-bit read 16 lanes at a time; an
// operand read has those lanes on 16 consecutive rows at one octet.  XOR with
// m % 8 spreads 8 rows over the 8 slots of a row, and XOR with bit 3 of m
// separates rows m and m + 8, which sit on the same banks (row stride 128
// bytes, bank line 256): the 16 reads then hit 16 distinct bank quads
// (SQ_LDS_BANK_CONFLICT reads 0; with m % 8 alone, every read was 2-way).
__device__ __forceinline__ int sw_slot(int m, int o) { return o ^ (m & 7) ^ ((m >> 3) & 1); }
__device__ __forceinline__ int sw_off(int m, int o) { return m * 64 + (sw_slot(m, o) << 3); }

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

inline unsigned xcd_grid(int64_t items) { return (unsigned)(((items + 7) / 8) * 8); }

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

// Sources of one block: activation tile (one descriptor, MF lane offsets at
// group 0) and the wave's two weight column fragments.
template <int MF>
struct LoopSrc {
    __amdgpu_buffer_rsrc_t a;
    uint32_t aoff[MF];
    __amdgpu_buffer_rsrc_t q[NF], s[NF];
    // soff: byte offset of the lane's scale in the row at group 0.  A lane
    // holds the codes of inputs 32 hh .. 32 hh + 31 of each 64-input group,
    // so with group 32 its scale is number 2 g + hh (soff includes hh) and
    // with group 64 * 2^j it is g >> j (gshift = j; a group as wide as the
    // row has gshift 31: scale 0).
    uint32_t qoff[NF], soff[NF];
    int gshift;
};

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

// G32: group 32 (scale stride 8 bytes per 64-input group).
template <int MF, int MFC, bool G32>
__device__ __forceinline__ void mfma_mainloop(Frags<MF> &fr, const LoopSrc<MF> &src, int ng,
                                              uint16_t *__restrict__ s0,
                                              uint16_t *__restrict__ s1,
                                              uint16_t *__restrict__ s2,
                                              uint16_t *__restrict__ s3) {
    static_assert(MFC <= MF, "row fragments");
    constexpr int LPG = MFC + 2 * NF;   // loads per thread per group, in issue order
    // VALU slots the scheduler may place after each MFMA: a k-step has about
    // 31 VALU instructions (two 8-code unpacks and the scale conversion); a
    // budget of 32 per k-step measured 1-2 % faster than 40 or 64.
    constexpr int VALU_PER_MFMA = (32 + MFC * NF - 1) / (MFC * NF);
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
            const int sbyte = G32 ? gc * 8 : (gc >> src.gshift) * 4;
            rs[slot][j] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(src.s[j], src.soff[j], sbyte, 0));
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

// Runs the main loop over the row fragments a tile of `rows` rows needs:
// ceil(rows / 32) of them, so a tile's padding is under one fragment.
template <int MF, bool G32, int C = MF>
__device__ __forceinline__ void run_mainloop(Frags<MF> &fr, const LoopSrc<MF> &src, int ng, int rows,
                                             uint16_t *__restrict__ s0,
                                             uint16_t *__restrict__ s1,
                                             uint16_t *__restrict__ s2,
                                             uint16_t *__restrict__ s3) {
    if constexpr (C == 1) {
        mfma_mainloop<MF, 1, G32>(fr, src, ng, s0, s1, s2, s3);
    } else {
        if (rows > 32 * (C - 1)) mfma_mainloop<MF, C, G32>(fr, src, ng, s0, s1, s2, s3);
        else run_mainloop<MF, G32, C - 1>(fr, src, ng, rows, s0, s1, s2, s3);
    }
}

// Activation tile sources: load i of wave w fills rows m = 32i + 8w + lane/8,
// and lane l fetches the octet that swizzle slot l % 8 of row m holds (the
// swizzle is an involution on the slot: sw_slot(m, l % 8)).  Rows past the
// tile read a valid row (row 0) and are never stored.
template <int MF, typename RowOf>
__device__ __forceinline__ void tile_offsets(LoopSrc<MF> &src, int rows, int row_elems,
                                             RowOf row_of) {
    const int lane = lane_id(), w = wave_id();
#pragma unroll
    for (int i = 0; i < MF; i++) {
        int m = 32 * i + 8 * w + (lane >> 3);
        const int oct = sw_slot(m, lane & 7);
        if (m >= rows) m = 0;
        src.aoff[i] = (uint32_t)(row_of(m) * row_elems * 2 + oct * 16);
    }
}

}  // namespace qmoe
