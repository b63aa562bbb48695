// Prefill path (bf16 activations): grouped per-expert GEMMs on the gfx950
// matrix cores, int4 tiles dequantised into LDS.
//
// The pages describe the operation (colibri pull request "cuda+engine: full
// fmt=4 (grouped int4 gs=64) support": per-group scale scales[o*ng + i/gs],
// fused gate+up pair, down projection; the tensor-core W4A16 kernels it
// names are per-row only and self-guarded, so they are prior art, not a
// design).  The design here is MI355X's own:
//
//  * Tiles come from the device worklist: (expert, first sorted row) with at
//    most 128 rows each; rows of x are gathered through the sorted pair list.
//  * Int4 codes are unpacked in registers to bf16 values 128 + u = 136 + q
//    (one AND-OR per two values: the nibble goes into the mantissa of 128.0)
//    and written to LDS.  Each MFMA group of 64 k starts its accumulator at
//    -136 * sum(x over the group) instead of zero, so the matrix core itself
//    removes the offset, and the f32 group scale is applied once per 64 k to
//    that group's partial sums (q is exact in bf16; rounding q*s to bf16
//    would cost ~3e-3 relative error).
//  * The down projection uses f16 (h is produced as f16): codes become exact
//    f16 q with one packed f16 add (1024 + u - 1032), no offset term.
//  * k is permuted inside every 8-element octet, identically for both
//    operands, to the order the nibble unpack produces (0,4,1,5,2,6,3,7);
//    a dot product does not depend on the order of its terms.
//  * v_mfma_f32_32x32x16_{bf16,f16}; block tile 128 rows x 128 columns, four
//    waves of 64x64, K step 64 (one scale group), LDS octets XOR-swizzled by
//    row to spread banks.
#include "common.h"
#include "launch.h"

namespace qmoe {

constexpr int MF_THREADS = 256;
constexpr int BM = MFMA_BM;   // 128 token rows per tile
constexpr int BK = 64;        // one scale group per K step

// LDS addressing: row of 64 16-bit values = 8 octets of 16 B, octet
// position XOR-swizzled with the row.
__device__ __forceinline__ int sw_off(int row, int octet) {
    return row * 64 + ((octet ^ (row & 7)) << 3);   // in 16-bit elements
}

// bf16 (or f16) octet [x0..x7] -> [x0,x4,x1,x5,x2,x6,x3,x7]
__device__ __forceinline__ u32x4 permute_octet(u32x4 a) {
    u32x4 o;
    o.x = perm_b32(a.z, a.x, 0x05040100u);
    o.y = perm_b32(a.z, a.x, 0x07060302u);
    o.z = perm_b32(a.w, a.y, 0x05040100u);
    o.w = perm_b32(a.w, a.y, 0x07060302u);
    return o;
}

// 8 nibbles -> 8 bf16 values 128 + u in the permuted octet order.
__device__ __forceinline__ u32x4 unpack_bf16_biased(uint32_t x) {
    u32x4 o;
    o.x = (x & 0x000F000Fu) | 0x43004300u;
    o.y = ((x >> 4) & 0x000F000Fu) | 0x43004300u;
    o.z = ((x >> 8) & 0x000F000Fu) | 0x43004300u;
    o.w = ((x >> 12) & 0x000F000Fu) | 0x43004300u;
    return o;
}

// 8 nibbles -> 8 exact f16 codes u - 8 in the permuted octet order.
__device__ __forceinline__ u32x4 unpack_f16_exact(uint32_t x) {
    const f16x2 off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    u32x4 o;
    uint32_t t[4];
    t[0] = (x & 0x000F000Fu) | 0x64006400u;
    t[1] = ((x >> 4) & 0x000F000Fu) | 0x64006400u;
    t[2] = ((x >> 8) & 0x000F000Fu) | 0x64006400u;
    t[3] = ((x >> 12) & 0x000F000Fu) | 0x64006400u;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        f16x2 h = __builtin_bit_cast(f16x2, t[i]);
        h = h + off;
        t[i] = __builtin_bit_cast(uint32_t, h);
    }
    o.x = t[0];
    o.y = t[1];
    o.z = t[2];
    o.w = t[3];
    return o;
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

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
// gate+up: block = (64 features of F for gate and up, one tile of <=128 rows)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(MF_THREADS) mfma_gateup_kernel(QMat G, QMat Up,
                                                                 const uint16_t *__restrict__ x,
                                                                 uint16_t *__restrict__ h16,
                                                                 MfmaRoute r) {
    constexpr int BN = 64;
    __shared__ __attribute__((aligned(16))) uint16_t sA[BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];
    __shared__ __attribute__((aligned(16))) float sBias[BM];
    __shared__ float sScale[2][BN];

    TileInfo ti;
    if (!tile_info(r, blockIdx.y, ti)) return;
    const int H = G.cols, F = G.rows, ng = H / 64;
    const int n0 = blockIdx.x * BN;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();

    // A pieces: 4 per thread, rows tid/8 + 32*i, octet tid%8
    const int a_oct = tid & 7;
    const uint16_t *arow[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int m = (tid >> 3) + 32 * i;
        if (m < ti.rows) {
            int64_t t;
            if (r.wl.pairs == nullptr) t = ti.pos0 + m;
            else t = r.wl.pairs[ti.pos0 + m] / r.k;
            arow[i] = x + t * H + a_oct * 8;
        } else {
            arow[i] = nullptr;
        }
    }
    // B piece: 1 per thread: matrix, row, half-group
    const int b_mat = tid >> 7, b_row = (tid & 127) >> 1, b_half = tid & 1;
    const QMat &BMt = b_mat == 0 ? G : Up;
    const uint8_t *brow = BMt.q + (int64_t)ti.e * BMt.q_stride + (int64_t)(n0 + b_row) * (H / 2) +
                          b_half * 16;
    const float *srow = (tid < 128) ? ((tid < 64 ? G.s + (int64_t)ti.e * G.s_stride
                                                 : Up.s + (int64_t)ti.e * Up.s_stride) +
                                       (int64_t)(n0 + (tid & 63)) * ng)
                                    : nullptr;

    // wave tile: rows wm*64 + [0,64), features wn*32 + [0,32) of both matrices
    const int wm = w >> 1, wn = w & 1;
    f32x16 acc[2][2];   // [m-subtile][matrix]
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    u32x4 ra[4];
    u32x4 rb;
    float rs = 0.f;
    auto fetch = [&](int g) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (arow[i]) ra[i] = *(const u32x4 *)(arow[i] + g * 64);
            else ra[i] = u32x4{0, 0, 0, 0};
        }
        rb = *(const u32x4 *)(brow + (int64_t)g * 32);
        if (srow) rs = srow[g];
    };
    auto stage = [&]() {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int m = (tid >> 3) + 32 * i;
            const u32x4 a = ra[i];
            float s = bf16_lo(a.x) + bf16_hi(a.x) + bf16_lo(a.y) + bf16_hi(a.y) + bf16_lo(a.z) +
                      bf16_hi(a.z) + bf16_lo(a.w) + bf16_hi(a.w);
            s = group_sum<8>(s);
            if (a_oct == 0) sBias[m] = -136.0f * s;
            *(u32x4 *)&sA[sw_off(m, a_oct)] = permute_octet(a);
        }
        const uint32_t wv[4] = {rb.x, rb.y, rb.z, rb.w};
#pragma unroll
        for (int d = 0; d < 4; d++)
            *(u32x4 *)&sB[b_mat][sw_off(b_row, b_half * 4 + d)] = unpack_bf16_biased(wv[d]);
        if (tid < 128) sScale[tid >> 6][tid & 63] = rs;
    };

    fetch(0);
    stage();
    __syncthreads();
    for (int g = 0; g < ng; g++) {
        if (g + 1 < ng) fetch(g + 1);
        // bias rows of this lane: m = base + 8*jj + 4*(lane/32) + i
        f32x16 gacc[2][2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int mb = wm * 64 + i * 32 + 4 * (lane >> 5);
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
                const f32x4 b4 = *(const f32x4 *)&sBias[mb + 8 * jj];
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    gacc[i][0][4 * jj + q] = b4[q];
                    gacc[i][1][4 * jj + q] = b4[q];
                }
            }
        }
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            const int oct = 2 * kk + (lane >> 5);
            bf16x8 av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int m = wm * 64 + i * 32 + (lane & 31);
                av[i] = *(const bf16x8 *)&sA[sw_off(m, oct)];
            }
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int n = wn * 32 + (lane & 31);
                bv[j] = *(const bf16x8 *)&sB[j][sw_off(n, oct)];
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    gacc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], gacc[i][j],
                                                                         0, 0, 0);
        }
        const float sg = sScale[0][wn * 32 + (lane & 31)];
        const float su = sScale[1][wn * 32 + (lane & 31)];
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                acc[i][0][v] = fmaf(sg, gacc[i][0][v], acc[i][0][v]);
                acc[i][1][v] = fmaf(su, gacc[i][1][v], acc[i][1][v]);
            }
        __syncthreads();
        if (g + 1 < ng) {
            stage();
            __syncthreads();
        }
    }

    // epilogue: h = silu(g) * u -> f16 at sorted position pos0 + m
    const int n = n0 + wn * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 2; i++) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (m < ti.rows) {
                const float h = silu(acc[i][0][v]) * acc[i][1][v];
                const _Float16 hh = (_Float16)h;
                h16[(int64_t)(ti.pos0 + m) * F + n] = __builtin_bit_cast(uint16_t, hh);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// down: block = (128 features of H, one tile of <=128 rows); f16 MFMA.
// Routed: Y[pos] = w * (D h); direct: out[pos] = D h.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(MF_THREADS) mfma_down_kernel(QMat D,
                                                               const uint16_t *__restrict__ h16,
                                                               float *__restrict__ y,
                                                               MfmaRoute r) {
    constexpr int BN = 128;
    __shared__ __attribute__((aligned(16))) uint16_t sA[BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[BN * BK];
    __shared__ float sScale[BN];

    TileInfo ti;
    if (!tile_info(r, blockIdx.y, ti)) return;
    const int H = D.rows, F = D.cols, ng = F / 64;
    const int n0 = blockIdx.x * BN;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();

    const int a_oct = tid & 7;
    const uint16_t *arow[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int m = (tid >> 3) + 32 * i;
        arow[i] = m < ti.rows ? h16 + (int64_t)(ti.pos0 + m) * F + a_oct * 8 : nullptr;
    }
    const int b_row = tid >> 1, b_half = tid & 1;
    const uint8_t *brow = D.q + (int64_t)ti.e * D.q_stride + (int64_t)(n0 + b_row) * (F / 2) +
                          b_half * 16;
    const float *srow = tid < BN ? D.s + (int64_t)ti.e * D.s_stride + (int64_t)(n0 + tid) * ng
                                 : nullptr;

    const int wm = w >> 1, wn = w & 1;   // wave tile rows wm*64.., features wn*64..
    f32x16 acc[2][2];                    // [m-subtile][n-subtile]
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.f;

    u32x4 ra[4];
    u32x4 rb;
    float rs = 0.f;
    auto fetch = [&](int g) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (arow[i]) ra[i] = *(const u32x4 *)(arow[i] + g * 64);
            else ra[i] = u32x4{0, 0, 0, 0};
        }
        rb = *(const u32x4 *)(brow + (int64_t)g * 32);
        if (srow) rs = srow[g];
    };
    auto stage = [&]() {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int m = (tid >> 3) + 32 * i;
            *(u32x4 *)&sA[sw_off(m, a_oct)] = permute_octet(ra[i]);
        }
        const uint32_t wv[4] = {rb.x, rb.y, rb.z, rb.w};
#pragma unroll
        for (int d = 0; d < 4; d++)
            *(u32x4 *)&sB[sw_off(b_row, b_half * 4 + d)] = unpack_f16_exact(wv[d]);
        if (tid < BN) sScale[tid] = rs;
    };

    fetch(0);
    stage();
    __syncthreads();
    for (int g = 0; g < ng; g++) {
        if (g + 1 < ng) fetch(g + 1);
        f32x16 gacc[2][2];
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int v = 0; v < 16; v++) gacc[i][j][v] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            const int oct = 2 * kk + (lane >> 5);
            f16x8 av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int m = wm * 64 + i * 32 + (lane & 31);
                av[i] = *(const f16x8 *)&sA[sw_off(m, oct)];
            }
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int n = wn * 64 + j * 32 + (lane & 31);
                bv[j] = *(const f16x8 *)&sB[sw_off(n, oct)];
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    gacc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], gacc[i][j],
                                                                        0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const float s = sScale[wn * 64 + j * 32 + (lane & 31)];
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int v = 0; v < 16; v++) acc[i][j][v] = fmaf(s, gacc[i][j][v], acc[i][j][v]);
        }
        __syncthreads();
        if (g + 1 < ng) {
            stage();
            __syncthreads();
        }
    }

    const bool routed = r.wl.pairs != nullptr;
#pragma unroll
    for (int i = 0; i < 2; i++) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (m < ti.rows) {
                const int pos = ti.pos0 + m;
                const float wgt = routed ? r.topk_w[r.wl.pairs[pos]] : 1.0f;
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const int n = n0 + wn * 64 + j * 32 + (lane & 31);
                    y[(int64_t)pos * H + n] = wgt * acc[i][j][v];
                }
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

hipError_t launch_mfma_gateup(const QMat &gate, const QMat &up, const uint16_t *x_bf16,
                              uint16_t *h16, const MfmaRoute &r, hipStream_t st) {
    const int ntiles = r.wl.pairs ? r.max_tiles : (r.ntok + BM - 1) / BM;
    const dim3 grid(gate.rows / 64, ntiles);
    hipLaunchKernelGGL(mfma_gateup_kernel, grid, dim3(MF_THREADS), 0, st, gate, up, x_bf16, h16,
                       r);
    return hipGetLastError();
}

hipError_t launch_mfma_down(const QMat &down, const uint16_t *h16, float *y, const MfmaRoute &r,
                            hipStream_t st) {
    const int ntiles = r.wl.pairs ? r.max_tiles : (r.ntok + BM - 1) / BM;
    const dim3 grid(down.rows / 128, ntiles);
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
