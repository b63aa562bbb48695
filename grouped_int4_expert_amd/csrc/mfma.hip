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
// Shared main loop.  The block owns a 128-row tile of f16 activation rows
// (arow[i]: row pointers of the 4 pieces this thread stages) and each wave
// NF 32-column weight fragments (brow/srow per fragment).  acc[i][j]: m-frag i
// (32 rows), n-frag j.
// ---------------------------------------------------------------------------
template <int NF>
struct Frags {
    f32x16 acc[4][NF];
};

template <int NF>
__device__ __forceinline__ void mfma_mainloop(Frags<NF> &fr, const uint16_t *const *arow,
                                              const uint8_t *const *brow,
                                              const float *const *srow, int ng,
                                              uint16_t *sA /* [2][128*64] */) {
    const int tid = threadIdx.x, lane = lane_id();
    const int a_oct = tid & 7;
    const int hh = lane >> 5, nl = lane & 31;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < NF; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) fr.acc[i][j][v] = 0.f;

    // Registers in flight: the A pieces of the next group, and the packed
    // weights + scales of the current (slot S) and next (slot 1-S) group.
    u32x4 ra[4];
    u32x4 rb[2][NF];
    float rs[2][NF];
    auto fetch_a = [&](int g) {
#pragma unroll
        for (int i = 0; i < 4; i++)
            ra[i] = arow[i] ? *(const u32x4 *)(arow[i] + g * 64) : u32x4{0, 0, 0, 0};
    };
    auto fetch_b = [&](int g, int slot) {
#pragma unroll
        for (int j = 0; j < NF; j++) {
            if (brow[j]) {
                rb[slot][j] = *(const u32x4 *)(brow[j] + (int64_t)g * 32);
                rs[slot][j] = srow[j][g];
            } else {
                rb[slot][j] = u32x4{0, 0, 0, 0};
                rs[slot][j] = 0.f;
            }
        }
    };
    auto stage_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int m = (tid >> 3) + 32 * i;
            *(u32x4 *)&sA[buf * BM * 64 + sw_off(m, a_oct)] = ra[i];
        }
    };
    // One group: operands A in sA[S], weights in rb[S].
    auto iter = [&](int g, auto slot_c) {
        constexpr int S = decltype(slot_c)::value;
        const bool more = g + 1 < ng;
        if (more) {
            fetch_a(g + 1);
            fetch_b(g + 1, 1 - S);
        }
        f16x2 s2[NF];
#pragma unroll
        for (int j = 0; j < NF; j++) {
            const _Float16 sh = (_Float16)rs[S][j];
            s2[j] = f16x2{sh, sh};
        }
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            f16x8 av[4];
#pragma unroll
            for (int i = 0; i < 4; i++)
                av[i] = *(const f16x8 *)&sA[S * BM * 64 + sw_off(32 * i + nl, 4 * hh + kk)];
            f16x8 bq[NF];
#pragma unroll
            for (int j = 0; j < NF; j++) bq[j] = dequant8(rb[S][j][kk], s2[j]);
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < NF; j++)
                    fr.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bq[j],
                                                                          fr.acc[i][j], 0, 0, 0);
        }
        if (more) stage_a(1 - S);
        __syncthreads();
    };

    fetch_a(0);
    fetch_b(0, 0);
    stage_a(0);
    __syncthreads();
    for (int g = 0; g < ng; g += 2) {
        iter(g, std::integral_constant<int, 0>{});
        if (g + 1 < ng) iter(g + 1, std::integral_constant<int, 1>{});
    }
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
    __shared__ __attribute__((aligned(16))) uint16_t sA[2 * BM * 64];
    __shared__ float sInv[BM];

    TileInfo ti;
    if (!tile_info(r, blockIdx.y, ti)) return;
    const int H = G.cols, F = G.rows, ng = H / 64;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int n = blockIdx.x * 128 + 32 * w + (lane & 31);
    const bool wave_on = blockIdx.x * 128 + 32 * w < F;

    const uint16_t *arow[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int m = (tid >> 3) + 32 * i;
        arow[i] = nullptr;
        if (m < ti.rows) {
            const int64_t t = r.wl.pairs ? r.wl.pairs[ti.pos0 + m] / r.k : ti.pos0 + m;
            arow[i] = x16 + t * H + (tid & 7) * 8;
        }
    }
    if (tid < BM) {
        float v = 0.f;
        if (tid < ti.rows) {
            const int64_t t = r.wl.pairs ? r.wl.pairs[ti.pos0 + tid] / r.k : ti.pos0 + tid;
            v = xinv[t];
        }
        sInv[tid] = v;
    }
    const uint8_t *brow[2];
    const float *srow[2];
    const int hh = lane >> 5;
    brow[0] = wave_on ? G.q + (int64_t)ti.e * G.q_stride + (int64_t)n * (H / 2) + 16 * hh
                      : nullptr;
    brow[1] = wave_on ? Up.q + (int64_t)ti.e * Up.q_stride + (int64_t)n * (H / 2) + 16 * hh
                      : nullptr;
    srow[0] = G.s + (int64_t)ti.e * G.s_stride + (int64_t)(wave_on ? n : 0) * ng;
    srow[1] = Up.s + (int64_t)ti.e * Up.s_stride + (int64_t)(wave_on ? n : 0) * ng;

    Frags<2> fr;
    mfma_mainloop<2>(fr, arow, brow, srow, ng, sA);

    if (!wave_on) return;
    const int npos = (n & ~7) + octet_pos(n & 7);
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = acc_row(i, v, lane);
            if (m < ti.rows) {
                const float s = sInv[m];
                const float h = silu(fr.acc[i][0][v] * s) * (fr.acc[i][1][v] * s);
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
    __shared__ __attribute__((aligned(16))) uint16_t sA[2 * BM * 64];

    TileInfo ti;
    if (!tile_info(r, blockIdx.y, ti)) return;
    const int H = D.rows, F = D.cols, ng = F / 64;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int hh = lane >> 5;

    const uint16_t *arow[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int m = (tid >> 3) + 32 * i;
        arow[i] = m < ti.rows ? h16 + (int64_t)(ti.pos0 + m) * F + (tid & 7) * 8 : nullptr;
    }
    const uint8_t *brow[2];
    const float *srow[2];
    int ncol[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        ncol[j] = blockIdx.x * 256 + 64 * w + 32 * j + (lane & 31);
        const bool on = ncol[j] < H;
        brow[j] = on ? D.q + (int64_t)ti.e * D.q_stride + (int64_t)ncol[j] * (F / 2) + 16 * hh
                     : nullptr;
        srow[j] = D.s + (int64_t)ti.e * D.s_stride + (int64_t)(on ? ncol[j] : 0) * ng;
    }

    Frags<2> fr;
    mfma_mainloop<2>(fr, arow, brow, srow, ng, sA);

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
    const dim3 grid((gate.rows + 127) / 128, ntiles);
    hipLaunchKernelGGL(mfma_gateup_kernel, grid, dim3(MF_THREADS), 0, st, gate, up, x16, xinv,
                       h16, r);
    return hipGetLastError();
}

hipError_t launch_mfma_down(const QMat &down, const uint16_t *h16, float *y, const MfmaRoute &r,
                            hipStream_t st) {
    const int ntiles = r.wl.pairs ? r.max_tiles : (r.ntok + BM - 1) / BM;
    const dim3 grid((down.rows + 255) / 256, ntiles);
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
