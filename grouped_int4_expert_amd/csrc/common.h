// Device-side helpers shared by the qmoe HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define QMOE_WAVE 64

namespace qmoe {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef _Float16 __attribute__((ext_vector_type(2))) f16x2;
typedef _Float16 __attribute__((ext_vector_type(4))) f16x4;

// Lanes per wave and the lane index.
__device__ __forceinline__ int lane_id() { return threadIdx.x & (QMOE_WAVE - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / QMOE_WAVE; }

// Butterfly sum over groups of `width` consecutive lanes (width a power of
// two, <= 64); every lane of a group ends with the group's sum.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, QMOE_WAVE);
    return v;
}

template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, QMOE_WAVE));
    return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
    for (int o = QMOE_WAVE / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, QMOE_WAVE);
    return v;
}

template <int WIDTH>
__device__ __forceinline__ uint32_t group_or(uint32_t v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v |= (uint32_t)__shfl_xor((int)v, o, QMOE_WAVE);
    return v;
}

// DPP lane permutations inside a row of 16 lanes (every source lane lies in
// the same row, so all of them are valid whenever the row is active).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
constexpr int DPP_QUAD_SWAP1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int DPP_QUAD_SWAP2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;

// OR over each group of 8 lanes, in every lane of the group: quad pairs,
// quads, then the two quads of a half row (half mirror maps one onto the
// other).
__device__ __forceinline__ uint32_t or8_dpp(uint32_t v) {
    v |= dpp_u32<DPP_QUAD_SWAP1>(v);
    v |= dpp_u32<DPP_QUAD_SWAP2>(v);
    v |= dpp_u32<DPP_ROW_HALF_MIRROR>(v);
    return v;
}

// Max over each row of 16 lanes, in every lane of the row (DPP only).
__device__ __forceinline__ float max16_dpp(float v) {
    v = fmaxf(v, __uint_as_float(dpp_u32<DPP_QUAD_SWAP1>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<DPP_QUAD_SWAP2>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<DPP_ROW_HALF_MIRROR>(__float_as_uint(v))));
    return fmaxf(v, __uint_as_float(dpp_u32<DPP_ROW_MIRROR>(__float_as_uint(v))));
}

// Unsigned max over each row of 16 lanes, in every lane (DPP only).  For
// non-negative floats that are not NaN the bit patterns order like the values.
__device__ __forceinline__ uint32_t max16_u32_dpp(uint32_t v) {
    v = max(v, dpp_u32<DPP_QUAD_SWAP1>(v));
    v = max(v, dpp_u32<DPP_QUAD_SWAP2>(v));
    v = max(v, dpp_u32<DPP_ROW_HALF_MIRROR>(v));
    return max(v, dpp_u32<DPP_ROW_MIRROR>(v));
}

// Max over each group of 32 lanes, in every lane: within 16 lanes by DPP
// (quad pairs, quads, half rows, rows), then one exchange between the two
// rows.
__device__ __forceinline__ float max32_dpp(float v) {
    v = max16_dpp(v);
    return fmaxf(v, __shfl_xor(v, 16, QMOE_WAVE));
}

// Signed int4 x int4 dot of 8 nibbles, accumulated into c (v_dot8_i32_i4).
__device__ __forceinline__ int sdot8(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
}

// Byte permute: result byte i = byte sel_i of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// The same with the hardware exp2 and reciprocal (about 1 ulp each), for
// results that are rounded to f16 next: z * 1/(1 + 2^(-z log2 e)).  Large
// negative z gives 2^t = inf, 1/inf = 0 and a zero of z's sign, as above.
__device__ __forceinline__ float silu_fast(float z) {
    const float e = __builtin_amdgcn_exp2f(z * -1.4426950408889634f);
    return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---------------------------------------------------------------------------
// Activation digits ("x digits").  A 32-element chunk of an f32 activation
// row is carried as a block fixed-point integer v_i = rint(x_i * 2^(18-E))
// (2^(E-1) <= max|x| < 2^E), written in five balanced base-16 digits
// d_k in [-8, 7] (v = sum_k d_k 16^k) so that a packed int4 weight nibble
// and a digit nibble multiply exactly in v_dot8_i32_i4.  Layout of one row
// of I elements: I/32 chunks x 5 planes x 4 dwords (plane k, dword d holds
// the digits of chunk elements 8d..8d+7, element 8d+i in nibble i), plus one
// f32 factor 2^(E-18) per chunk in a separate array.  |v| <= 2^18 fits the
// five-digit range [-559240, 489335].  Activation rows (x) take E from the
// maximum over both chunks of each 64-element group, so the two factors of a
// group are equal and the fused gate+up kernel combines a group's digit sums
// once; h (produced 32 features per block) keeps one E per chunk.
// ---------------------------------------------------------------------------
constexpr int XD_PLANES = 5;
constexpr int XD_CHUNK = 32;                       // elements per factor
constexpr int XD_DWORDS = XD_PLANES * 4;           // dwords per chunk
constexpr int XD_FRAC_BITS = 18;

// Quantise one chunk held one element per lane by 32 consecutive lanes
// (lanes with `valid` false hold zero).  Lane (8d + i) of the chunk gets its
// five digit nibbles; returns the factor.  Writes plane dwords through
// `store(plane, dword, value)` from lanes with (lane % 8) == 0.  PAIR: the
// two halves of the wave hold the two chunks of one 64-element group and
// share one exponent (every lane of the wave must take part).
template <bool PAIR = false, typename Store>
__device__ __forceinline__ float quantise_chunk32(float x, Store store) {
    float m = max32_dpp(fabsf(x));
    if (PAIR) m = fmaxf(m, __shfl_xor(m, 32, QMOE_WAVE));
    // fmaxf drops NaN, so NaN is found on its own: a ballot over the chunk's
    // lanes (both halves of the wave for PAIR)
    const uint64_t nan_lanes = __ballot(x != x);
    const bool any_nan =
        PAIR ? nan_lanes != 0ull : ((nan_lanes >> (lane_id() & 32)) & 0xffffffffull) != 0ull;
    float factor;
    int v = 0;
    if (any_nan || !(m <= 3.0e38f)) {         // NaN or inf in the chunk: no digits
        factor = __int_as_float(0x7fc00000);
    } else if (m == 0.0f) {
        factor = 0.0f;
    } else {
        int e;
        frexpf(m, &e);                        // m = f * 2^e, f in [0.5, 1)
        v = (int)rintf(ldexpf(x, XD_FRAC_BITS - e));
        factor = ldexpf(1.0f, e - XD_FRAC_BITS);
    }
    const int sub = lane_id() & 7;            // element inside the dword
    const int dw = (lane_id() & 31) >> 3;     // dword inside the plane
#pragma unroll
    for (int k = 0; k < XD_PLANES; k++) {
        const int d = ((v + 8) & 15) - 8;
        v = (v - d) >> 4;
        uint32_t nib = (uint32_t)(d & 15) << (4 * sub);
        nib = or8_dpp(nib);
        if (sub == 0) store(k, dw, nib);
    }
    return factor;
}

// Dot of one 64-element group whose two chunks share the factor `fac`:
// weights w[0..7] against the digit planes at x[0..39], both chunks of a
// plane summed in one chain.  The planes are folded in Horner order inside
// the dot chain (v = 16 v + plane sum), so the chain needs one zero to start
// and no separate recombination; every partial value is bounded by the full
// sum, |sum| <= 64 * 8 * 2^18.
__device__ __forceinline__ float group_dot(const uint32_t *w, const uint32_t *x, float fac) {
    int v = 0;
#pragma unroll
    for (int k = XD_PLANES - 1; k >= 0; k--) {
        v *= 16;
#pragma unroll
        for (int d = 0; d < 4; d++) v = sdot8(w[d], x[4 * k + d], v);
#pragma unroll
        for (int d = 0; d < 4; d++) v = sdot8(w[4 + d], x[XD_DWORDS + 4 * k + d], v);
    }
    return (float)v * fac;
}

// Dot of one 32-element chunk: weights w[0..3] (two's-complement nibbles)
// against the five digit planes at x[0..19], in the same Horner order.
__device__ __forceinline__ float chunk_dot(const uint32_t *w, const uint32_t *x, float fac) {
    int v = 0;
#pragma unroll
    for (int k = XD_PLANES - 1; k >= 0; k--) {
        v *= 16;
#pragma unroll
        for (int d = 0; d < 4; d++) v = sdot8(w[d], x[4 * k + d], v);
    }
    return (float)v * fac;
}

// Sum over groups of LPR consecutive lanes (LPR = 8, 16, 32 or 64) with DPP
// row shifts and row broadcasts (VALU only); the sum is valid in the last
// lane of each group.
__device__ __forceinline__ float dpp_add(float v, int t) { return v + __int_as_float(t); }
template <int LPR>
__device__ __forceinline__ float reduce_dpp(float v) {
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));
    if (LPR >= 16)
        v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));
    if (LPR >= 32)   // row_bcast:15 into rows 1 and 3
        v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
    if (LPR >= 64)   // row_bcast:31 into rows 2 and 3
        v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
    return v;
}

// ---------------------------------------------------------------------------
// Buffer loads.  A descriptor (base, byte size) lives in scalar registers and
// each lane supplies a 32-bit byte offset; bytes past the size read as zero.
// Where a lane is switched off with OOB_OFFSET, the descriptor covers less
// than 2^31 bytes and the other offsets of the access stay below 2^31, so
// the sum stays out of range.
// ---------------------------------------------------------------------------
constexpr uint32_t OOB_OFFSET = 0x80000000u;

// Word 3 selects the 32-bit data format that raw loads require.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             (int)(uint32_t)bytes, 0x00020000);
}

// An LDS pointer as the address-space-3 pointer that loads writing LDS take.
#define QMOE_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// s_waitcnt immediate (gfx9 layout) that waits until at most n (< 64) vector
// memory operations of this wave are outstanding and leaves the other
// counters alone.
__host__ __device__ constexpr int waitcnt_vm(int n) {
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

}  // namespace qmoe
