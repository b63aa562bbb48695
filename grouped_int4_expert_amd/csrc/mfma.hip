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
//    most 128 rows each; activation rows are gathered through the sorted
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
//  * v_mfma_f32_32x32x16_f16; block = 4 waves x (128 rows x 32 features of
//    gate and of up) or 4 waves x (128 rows x 64 features) for down; the
//    activation tile (128 x 64 f16 per group) is double-buffered in LDS with
//    octets XOR-swizzled by row; global loads of group g+1 are issued
//    before the MFMAs of group g, and two blocks per CU overlap waits.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace qmoe {

constexpr int MF_THREADS = 256;
constexpr int BM = MFMA_BM;   // 128 token rows per tile

// LDS offset (in 16-bit elements) of octet `o` of row `m` in a 128 x 64 tile.
__device__ __forceinline__ int sw_off(int m, int o) { return m * 64 + ((o ^ (m & 7)) << 3); }

// s_waitcnt immediate (gfx9 layout) that waits until at most n vector memory
// loads of this wave are outstanding and leaves the other counters alone.
__host__ __device__ constexpr int waitcnt_vm(int n) {
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// Position of element e (0..7) of an octet after the unpack permutation.
__device__ __forceinline__ int octet_pos(int e) { return e < 4 ? 2 * e : 2 * (e - 4) + 1; }

// 8 packed codes (one dword) -> 8 f16 values q*s in unpack order.
__device__ __forceinline__ f16x8 dequant8(uint32_t d, f16x2 s2) {
    const f16x2 off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t t = ((d >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
        const f16x2 v = (__builtin_bit_cast(f16x2, t) + off) * s2;
        r[2 * i] = v[0];
        r[2 * i + 1] = v[1];
    }
    return r;
}

struct TileInfo {
    int e, row0, rows, pos0;
};

__device__ __forceinline__ bool tile_info(const MfmaRoute &r, int tile, TileInfo &ti) {
    if (r.wl.pairs == nullptr) {
        const int row0 = tile * BM;
        if (row0 >= r.ntok) return false;
        ti.e = 0;
        ti.row0 = row0;
        ti.pos0 = row0;
        ti.rows = min(BM, r.ntok - row0);
        return true;
    }
    if (tile >= r.wl.n_tiles[0]) return false;
    ti.e = r.wl.tiles[2 * tile];
    ti.row0 = r.wl.tiles[2 * tile + 1];
    const int c = r.wl.counts[ti.e];
    ti.pos0 = r.wl.offsets[ti.e] + ti.row0;
    ti.rows = min(BM, c - ti.row0);
    return true;
}

// Work item (tile, column block) of this block.  The GPU hands linear block
// ids to its 8 XCDs round-robin, and each XCD has its own L2; so each XCD is
// given one contiguous run of the real items (their count comes from the
// device worklist), column blocks of a tile adjacent: a tile's activation
// rows and an expert's weight slices are then fetched into one L2 instead of
// up to eight.  gridDim.x is a multiple of 8 and >= the largest item count.
__device__ __forceinline__ bool work_item(const MfmaRoute &r, int ncb, int &tile, int &cb) {
    const int ntiles = r.wl.pairs ? r.wl.n_tiles[0] : (r.ntok + BM - 1) / BM;
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
// Shared main loop.  The block owns a 128-row tile of f16 activation rows and
// each wave NF 32-column weight fragments.  acc[i][j]: m-frag i (32 rows),
// n-frag j.
//
// Pipeline, per 64-k group g (one scale group):
//  * activation tile: direct global->LDS loads (global_load_lds_dwordx4) into
//    a ring of NS = 4 LDS stages, issued 3 groups ahead.  A wave's DMA writes
//    1 KB of LDS in lane order, so lane l of chunk c fetches the octet that the
//    XOR swizzle places at slot l%8 of row 8c + l/8.
//  * packed weights + scales: registers, 4 slots, issued 3 groups ahead.
//  * one s_barrier per group, preceded by a counted vmcnt wait: each thread
//    issues exactly LPG loads per group in a fixed order, so allowing the two
//    newest groups' loads to stay in flight guarantees this group's tile and
//    weights have landed (near the end, where fewer groups follow, the wait
//    is vmcnt(0)).  Stage g%4 is rewritten only by the DMA issued after the
//    barrier of group g+1, when every wave has finished reading it.
// ---------------------------------------------------------------------------
template <int NF>
struct Frags {
    f32x16 acc[4][NF];
};

#define QMOE_LDS(p) ((__attribute__((address_space(3))) void *)(p))

template <int NF>
__device__ __forceinline__ void mfma_mainloop(Frags<NF> &fr, const uint16_t *const *arow,
                                              const uint8_t *const *brow,
                                              const float *const *srow, int ng,
                                              uint16_t *__restrict__ s0,
                                              uint16_t *__restrict__ s1,
                                              uint16_t *__restrict__ s2,
                                              uint16_t *__restrict__ s3) {
    const int lane = lane_id(), w = wave_id();
    const int hh = lane >> 5, nl = lane & 31;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < NF; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) fr.acc[i][j][v] = 0.f;

    u32x4 rb[4][NF];
    float rs[4][NF];
    // Issue the tile DMA of group g into stage buffer `buf` (4 loads).
    auto dma_a = [&](int g, uint16_t *buf) {
#pragma unroll
        for (int i = 0; i < 4; i++)
            __builtin_amdgcn_global_load_lds((const void *)(arow[i] + g * 64),
                                             QMOE_LDS(buf + (w * 4 + i) * 512), 16, 0, 0);
    };
    // Issue the weight loads of group g into register slot `slot` (2*NF loads).
    auto fetch_b = [&](int g, int slot) {
#pragma unroll
        for (int j = 0; j < NF; j++) {
            rb[slot][j] = *(const u32x4 *)(brow[j] + (int64_t)g * 32);
            rs[slot][j] = srow[j][g];
        }
    };
    constexpr int LPG = 4 + 2 * NF;   // loads per thread per group
    auto compute = [&](int slot, const uint16_t *buf) {
        f16x2 s2[NF];
#pragma unroll
        for (int j = 0; j < NF; j++) {
            const _Float16 sh = (_Float16)rs[slot][j];
            s2[j] = f16x2{sh, sh};
        }
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            f16x8 av[4];
#pragma unroll
            for (int i = 0; i < 4; i++)
                av[i] = *(const f16x8 *)&buf[sw_off(32 * i + nl, 4 * hh + kk)];
            f16x8 bq[NF];
#pragma unroll
            for (int j = 0; j < NF; j++) bq[j] = dequant8(rb[slot][j][kk], s2[j]);
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < NF; j++)
                    fr.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bq[j],
                                                                          fr.acc[i][j], 0, 0, 0);
        }
    };
    // Top of group g: wait for its tile and weights, then barrier.
    auto sync_group = [&](int g) {
        if (g + 2 < ng) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPG));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __builtin_amdgcn_s_barrier();
    };
    auto iter = [&](int g, int slot, uint16_t *cur, uint16_t *ahead) {
        sync_group(g);
        if (g + 3 < ng) {
            dma_a(g + 3, ahead);
            fetch_b(g + 3, (slot + 3) & 3);
        }
        compute(slot, cur);
    };

    // prologue: groups 0, 1, 2 in flight (tile and weights of each group)
    dma_a(0, s0);
    fetch_b(0, 0);
    if (ng > 1) {
        dma_a(1, s1);
        fetch_b(1, 1);
    }
    if (ng > 2) {
        dma_a(2, s2);
        fetch_b(2, 2);
    }
    for (int g = 0; g < ng; g += 4) {
        iter(g, 0, s0, s3);
        if (g + 1 < ng) iter(g + 1, 1, s1, s0);
        if (g + 2 < ng) iter(g + 2, 2, s2, s1);
        if (g + 3 < ng) iter(g + 3, 3, s3, s2);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
}

// Row (within the tile) held by accumulator v of lane `lane` in m-frag i.
__device__ __forceinline__ int acc_row(int i, int v, int lane) {
    return 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// ---------------------------------------------------------------------------
// gate+up: block = (128 features of F for gate and up, one tile of <=128
// rows).  Wave w: features n0 + 32w .. +32 of gate (frag 0) and up (frag 1).
// Output h = silu(g) * u as f16 at sorted position pos0 + m, octet-permuted
// in the feature index (the down projection's k).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(MF_THREADS, 2) mfma_gateup_kernel(
    QMat G, QMat Up, const uint16_t *__restrict__ x16, const float *__restrict__ xinv,
    uint16_t *__restrict__ h16, MfmaRoute r) {
    __shared__ __attribute__((aligned(1024))) uint16_t s0[BM * 64], s1[BM * 64], s2[BM * 64],
        s3[BM * 64];
    __shared__ float sInv[BM];

    const int H = G.cols, F = G.rows, ng = H / 64;
    int tile, cb;
    if (!work_item(r, (F + 127) / 128, tile, cb)) return;
    TileInfo ti;
    if (!tile_info(r, tile, ti)) return;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int n = cb * 128 + 32 * w + (lane & 31);
    const bool wave_on = cb * 128 + 32 * w < F;
    auto token = [&](int m) -> int64_t {
        return r.wl.pairs ? r.wl.pairs[ti.pos0 + m] / r.k : ti.pos0 + m;
    };

    // Tile DMA sources: chunk 4w+i holds rows 8(4w+i) + lane/8, swizzle slot lane%8.
    const uint16_t *arow[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        int m = 8 * (4 * w + i) + (lane >> 3);
        const int oct = (lane & 7) ^ ((lane >> 3) & 7);
        if (m >= ti.rows) m = 0;          // padding rows: any valid row, never stored
        arow[i] = x16 + token(m) * H + oct * 8;
    }
    if (tid < BM) sInv[tid] = tid < ti.rows ? xinv[token(tid)] : 0.f;
    const uint8_t *brow[2];
    const float *srow[2];
    const int hh = lane >> 5;
    const int nn = wave_on ? n : 0;       // idle waves read row 0 (valid) and store nothing
    brow[0] = G.q + (int64_t)ti.e * G.q_stride + (int64_t)nn * (H / 2) + 16 * hh;
    brow[1] = Up.q + (int64_t)ti.e * Up.q_stride + (int64_t)nn * (H / 2) + 16 * hh;
    srow[0] = G.s + (int64_t)ti.e * G.s_stride + (int64_t)nn * ng;
    srow[1] = Up.s + (int64_t)ti.e * Up.s_stride + (int64_t)nn * ng;

    Frags<2> fr;
    mfma_mainloop<2>(fr, arow, brow, srow, ng, s0, s1, s2, s3);

    if (!wave_on) return;
    const int npos = (n & ~7) + octet_pos(n & 7);
#pragma unroll
    for (int i = 0; i < 4; i++) {
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
// down: block = (256 features of H, one tile of <=128 rows); wave w:
// features n0 + 64w + 32j + (lane%32), j = 0, 1.
// Routed: Y[pos] = w * (D h); direct: out[pos] = D h.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(MF_THREADS, 2) mfma_down_kernel(QMat D,
                                                                  const uint16_t *__restrict__ h16,
                                                                  float *__restrict__ y,
                                                                  MfmaRoute r) {
    __shared__ __attribute__((aligned(1024))) uint16_t s0[BM * 64], s1[BM * 64], s2[BM * 64],
        s3[BM * 64];

    const int H = D.rows, F = D.cols, ng = F / 64;
    int tile, cb;
    if (!work_item(r, (H + 255) / 256, tile, cb)) return;
    TileInfo ti;
    if (!tile_info(r, tile, ti)) return;
    const int lane = lane_id(), w = wave_id();
    const int hh = lane >> 5;

    const uint16_t *arow[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        int m = 8 * (4 * w + i) + (lane >> 3);
        const int oct = (lane & 7) ^ ((lane >> 3) & 7);
        if (m >= ti.rows) m = 0;
        arow[i] = h16 + (int64_t)(ti.pos0 + m) * F + oct * 8;
    }
    const uint8_t *brow[2];
    const float *srow[2];
    int ncol[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        ncol[j] = cb * 256 + 64 * w + 32 * j + (lane & 31);
        const int nn = ncol[j] < H ? ncol[j] : 0;
        brow[j] = D.q + (int64_t)ti.e * D.q_stride + (int64_t)nn * (F / 2) + 16 * hh;
        srow[j] = D.s + (int64_t)ti.e * D.s_stride + (int64_t)nn * ng;
    }

    Frags<2> fr;
    mfma_mainloop<2>(fr, arow, brow, srow, ng, s0, s1, s2, s3);

    const bool routed = r.wl.pairs != nullptr;
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = acc_row(i, v, lane);
            if (m < ti.rows) {
                const int pos = ti.pos0 + m;
                const float wgt = routed ? r.topk_w[r.wl.pairs[pos]] : 1.0f;
#pragma unroll
                for (int j = 0; j < 2; j++)
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
    const int ntiles = r.wl.pairs ? r.max_tiles : (r.ntok + BM - 1) / BM;
    const dim3 grid(xcd_grid((int64_t)ntiles * ((gate.rows + 127) / 128)));
    hipLaunchKernelGGL(mfma_gateup_kernel, grid, dim3(MF_THREADS), 0, st, gate, up, x16, xinv,
                       h16, r);
    return hipGetLastError();
}

hipError_t launch_mfma_down(const QMat &down, const uint16_t *h16, float *y, const MfmaRoute &r,
                            hipStream_t st) {
    const int ntiles = r.wl.pairs ? r.max_tiles : (r.ntok + BM - 1) / BM;
    const dim3 grid(xcd_grid((int64_t)ntiles * ((down.rows + 255) / 256)));
    hipLaunchKernelGGL(mfma_down_kernel, grid, dim3(MF_THREADS), 0, st, down, h16, y, r);
    return hipGetLastError();
}

hipError_t launch_combine(const float *y, const int32_t *inv, int tokens, int k, int hidden,
                          float *out, hipStream_t st) {
    const dim3 grid((hidden / 4 + 255) / 256, tokens);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, y, inv, k, hidden, out);
    return hipGetLastError();
}

}  // namespace qmoe
