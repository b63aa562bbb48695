// Read-stream probe: how fast this GPU streams a buffer from HBM with the
// load shapes the decode kernels use.  A measurement aid beside the path
// (it computes nothing the layer needs): the decode kernels are judged
// against 8 TB/s, and this gives the rate a plain read of the same shape
// reaches on the same part.
//
//  * QMOE_PROBE_LINEAR: every wave instruction reads 1 KB of consecutive
//    bytes (16 B per lane) and a wave keeps 16 such loads in flight.
//  * QMOE_PROBE_ROWS: the buffer as rows of 2 KB (a 4096-input int4 row);
//    a wave reads row blocks of 16 rows x 256 consecutive bytes of each row
//    as four back-to-back loads (lane l: row l % 16, bytes 16 (l / 16) +
//    64 L), two row blocks in flight, as the matrix-core decode passes do;
//    the eight waves of a block take the eight 256-byte slices of a row.
//
// Each lane adds the dwords it read (mod 2^32) and each block writes one sum,
// so the loads cannot be dropped and the sum checks that every byte was read
// once.
#include "common.h"
#include "launch.h"

namespace qmoe {

constexpr int PR_THREADS = 256;
constexpr int PR_LINEAR_DEPTH = 16;   // 1 KB loads in flight per wave

__device__ __forceinline__ uint32_t add4(u32x4 v) { return v.x + v.y + v.z + v.w; }

__global__ void __launch_bounds__(PR_THREADS) probe_linear_kernel(const uint8_t *__restrict__ buf,
                                                                  int64_t bytes,
                                                                  uint32_t *__restrict__ sink) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(buf, bytes);
    const int lane = lane_id();
    const int64_t wave = (int64_t)blockIdx.x * (PR_THREADS / QMOE_WAVE) + wave_id();
    const int64_t waves = (int64_t)gridDim.x * (PR_THREADS / QMOE_WAVE);
    constexpr int64_t CHUNK = (int64_t)PR_LINEAR_DEPTH * QMOE_WAVE * 16;   // 16 KB per wave step
    uint32_t acc = 0;
    for (int64_t c = wave * CHUNK; c < bytes; c += waves * CHUNK) {
        // the chunk's offset rides in the scalar offset (below 2^31 for the
        // sizes the host allows); loads past the end return zero
        const uint32_t base = (uint32_t)__builtin_amdgcn_readfirstlane((int)c);
        u32x4 v[PR_LINEAR_DEPTH];
#pragma unroll
        for (int i = 0; i < PR_LINEAR_DEPTH; i++)
            v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(lane * 16 + i * 1024), base,
                                                         0);
#pragma unroll
        for (int i = 0; i < PR_LINEAR_DEPTH; i++) acc += add4(v[i]);
    }
    __shared__ uint32_t red[PR_THREADS / QMOE_WAVE];
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, QMOE_WAVE);
    if (lane == 0) red[wave_id()] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int i = 0; i < PR_THREADS / QMOE_WAVE; i++) s += red[i];
        sink[blockIdx.x] = s;
    }
}

// rows of 2 KB; block = 8 waves (one per 256-byte slice) x `rb` row blocks
__global__ void __launch_bounds__(512) probe_rows_kernel(const uint8_t *__restrict__ buf,
                                                         int64_t bytes, int rb,
                                                         uint32_t *__restrict__ sink) {
    constexpr uint32_t ROW = 2048;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(buf, bytes);
    const int lane = lane_id(), w = wave_id();
    const uint32_t lane_off = (uint32_t)(lane & 15) * ROW + 16u * (uint32_t)(lane >> 4) + 256u * w;
    const int64_t rows = bytes / ROW;
    const int64_t blocks_of_rows = (rows + 16 * rb - 1) / (16 * rb);
    uint32_t acc = 0;
    for (int64_t b = blockIdx.x; b < blocks_of_rows; b += gridDim.x) {
        const uint32_t row0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(b * 16 * rb));
        u32x4 st[2][4];
        auto issue = [&](int j, int s) {
            // row blocks past this block's share or past the buffer read zeros
            const uint32_t o = j < rb ? (row0 + 16u * j) * ROW : OOB_OFFSET;
#pragma unroll
            for (int L = 0; L < 4; L++)
                st[s][L] = __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, o + 64u * L, 0);
        };
        issue(0, 0);
        issue(1, 1);
        for (int j = 0; j < rb; j += 2) {
#pragma unroll
            for (int s = 0; s < 2; s++) {
#pragma unroll
                for (int L = 0; L < 4; L++) acc += add4(st[s][L]);
                issue(j + s + 2, s);
            }
        }
    }
    __shared__ uint32_t red[8];
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, QMOE_WAVE);
    if (lane == 0) red[w] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int i = 0; i < 8; i++) s += red[i];
        sink[blockIdx.x] = s;
    }
}

// Both shapes launch QMOE_PROBE_SINK blocks, so every sink entry is written.
int probe_grid(int) { return 2048; }

hipError_t launch_probe(const void *buf, int64_t bytes, int pattern, uint32_t *sink,
                        hipStream_t st) {
    const uint8_t *b = static_cast<const uint8_t *>(buf);
    if (pattern == 0)
        hipLaunchKernelGGL(probe_linear_kernel, dim3(probe_grid(0)), dim3(PR_THREADS), 0, st, b,
                           bytes, sink);
    else
        hipLaunchKernelGGL(probe_rows_kernel, dim3(probe_grid(1)), dim3(512), 0, st, b, bytes, 16,
                           sink);
    return hipGetLastError();
}

}  // namespace qmoe
