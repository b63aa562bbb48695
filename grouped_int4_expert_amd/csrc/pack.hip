// Packing of int8 codes into the grouped int4 container and back.
//
// Format (colibri pull request "cuda+engine: full fmt=4 (grouped int4 gs=64)
// support", Summary: int4 rows are (I+1)/2 bytes, same nibble layout as the
// per-row format; comment "implementation complete but system-instability":
// the container keeps each code as a nibble 0..15 offset by 8): byte j of a row holds
// element 2j in its low nibble and 2j+1 in its high nibble, each as q + 8.
#include "common.h"
#include "launch.h"

namespace qmoe {

// One thread per output byte; grid-stride over rows*row_bytes bytes.
__global__ void pack_kernel(const int8_t *__restrict__ q, int64_t rows, int64_t cols,
                            uint8_t *__restrict__ packed, int32_t *__restrict__ n_bad) {
    const int64_t rb = (cols + 1) / 2;
    const int64_t total = rows * rb;
    int bad = 0;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t o = idx / rb, j = idx - o * rb;
        const int64_t i0 = 2 * j;
        const int v0 = q[o * cols + i0];
        bad += (v0 < -8 || v0 > 7);
        uint32_t b = (uint32_t)(v0 + 8) & 15u;
        uint32_t hi = 8u;                       // pad nibble: value 0
        if (i0 + 1 < cols) {
            const int v1 = q[o * cols + i0 + 1];
            bad += (v1 < -8 || v1 > 7);
            hi = (uint32_t)(v1 + 8) & 15u;
        }
        packed[idx] = (uint8_t)(b | (hi << 4));
    }
    if (n_bad) {
        bad = wave_sum_i32(bad);
        if (lane_id() == 0 && bad) atomicAdd(n_bad, bad);
    }
}

__global__ void unpack_kernel(const uint8_t *__restrict__ packed, int64_t rows, int64_t cols,
                              int8_t *__restrict__ q) {
    const int64_t rb = (cols + 1) / 2;
    const int64_t total = rows * rb;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t o = idx / rb, j = idx - o * rb;
        const uint32_t b = packed[idx];
        q[o * cols + 2 * j] = (int8_t)((int)(b & 15u) - 8);
        if (2 * j + 1 < cols) q[o * cols + 2 * j + 1] = (int8_t)((int)(b >> 4) - 8);
    }
}

// Two's-complement nibble container (what the pages' GPU upload holds) to
// the offset container: a nibble n becomes n XOR 8 (signed value + 8), so a
// byte XOR 0x88.  16 bytes per thread where both buffers are 16-byte aligned,
// single bytes otherwise; in place is allowed.
__global__ void import_twos_kernel(const uint8_t *twos, int64_t n, uint8_t *packed, int vec) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t done = 0;
    if (vec) {
        const int64_t n16 = n / 16;
        for (int64_t j = i; j < n16; j += stride) {
            const u32x4 v = ((const u32x4 *)twos)[j];
            ((u32x4 *)packed)[j] = v ^ 0x88888888u;
        }
        done = n16 * 16;
    }
    for (int64_t j = done + i; j < n; j += stride) packed[j] = (uint8_t)(twos[j] ^ 0x88u);
}

// Re-lay a matrix of `cols` inputs (rows of ceil(cols/2) packed bytes, ng
// scales) as one of cols_out >= cols inputs (cols_out/2 bytes per row, ng_out
// >= ng scales): the added nibbles are 8 (code 0) and the added scales 0, so
// every added column contributes nothing.  Byte-wise: a row of the input may
// start at any byte.
__global__ void pad_cols_kernel(const uint8_t *__restrict__ q, const float *__restrict__ s,
                                int64_t rows, int64_t cols, int64_t ng, uint8_t *__restrict__ qo,
                                int64_t cols_out, float *__restrict__ so, int64_t ng_out) {
    const int64_t rb = (cols + 1) / 2, rbo = cols_out / 2;
    const int64_t nq = rows * rbo, n = nq + rows * ng_out;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (i < nq) {
            const int64_t r = i / rbo, b = i - r * rbo;
            qo[i] = b < rb ? q[r * rb + b] : (uint8_t)0x88;
        } else {
            const int64_t j = i - nq, r = j / ng_out, c = j - r * ng_out;
            so[j] = c < ng ? s[r * ng + c] : 0.0f;
        }
    }
}

__global__ void zero_i32_kernel(int32_t *p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

static int grid_for(int64_t n, int block) {
    int64_t g = (n + block - 1) / block;
    if (g > 65536) g = 65536;
    if (g < 1) g = 1;
    return (int)g;
}

hipError_t launch_pack(const int8_t *q, int64_t rows, int64_t cols, uint8_t *packed,
                       int32_t *n_bad, hipStream_t st) {
    if (n_bad) hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(64), 0, st, n_bad, (int64_t)1);
    const int64_t total = rows * ((cols + 1) / 2);
    hipLaunchKernelGGL(pack_kernel, dim3(grid_for(total, 256)), dim3(256), 0, st, q, rows,
                       cols, packed, n_bad);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, int64_t rows, int64_t cols, int8_t *q,
                         hipStream_t st) {
    const int64_t total = rows * ((cols + 1) / 2);
    hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(total, 256)), dim3(256), 0, st, packed,
                       rows, cols, q);
    return hipGetLastError();
}


hipError_t launch_import_twos(const uint8_t *twos, int64_t rows, int64_t cols, uint8_t *packed,
                              hipStream_t st) {
    const int64_t n = rows * ((cols + 1) / 2);
    const int vec = ((reinterpret_cast<uintptr_t>(twos) | reinterpret_cast<uintptr_t>(packed)) &
                     15u) == 0;
    hipLaunchKernelGGL(import_twos_kernel, dim3(grid_for(vec ? n / 16 + 1 : n, 256)), dim3(256),
                       0, st, twos, n, packed, vec);
    return hipGetLastError();
}

hipError_t launch_pad_cols(const uint8_t *q, const float *s, int64_t rows, int64_t cols, int64_t ng,
                           uint8_t *qo, int64_t cols_out, float *so, int64_t ng_out,
                           hipStream_t st) {
    const int64_t n = rows * (cols_out / 2 + ng_out);
    hipLaunchKernelGGL(pad_cols_kernel, dim3(grid_for(n, 256)), dim3(256), 0, st, q, s, rows, cols,
                       ng, qo, cols_out, so, ng_out);
    return hipGetLastError();
}
}  // namespace qmoe
