// Internal launchers of the qmoe kernels (host side).  Shapes are validated
// by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

// Packed int4 matrix stack on the device (see include/qmoe.h).
struct QMat {
    const uint8_t *q;
    const float *s;
    int64_t q_stride;   // bytes between experts
    int64_t s_stride;   // floats between experts
    int rows, cols;     // O, I (cols % 64 == 0)
    int group;          // inputs per scale: 32, or a multiple of 64
};

// Scales per row.
__host__ __device__ inline int scales_per_row(const QMat &m) {
    return (m.cols + m.group - 1) / m.group;
}

// For group 64 * 2^j: j, so that 64-input group g has scale g >> j; for a
// group at least as wide as the row: 31 (every g has scale 0).
__host__ __device__ inline int group_shift(const QMat &m) {
    if (m.group >= m.cols) return 31;
    int j = 0;
    while ((64 << j) < m.group) j++;
    return j;
}

// Worklist outputs inside a workspace.
struct Worklist {
    int32_t *counts;    // [E]
    int32_t *offsets;   // [E+1]
    int32_t *pairs;     // [n]
    int32_t *inv;       // [n]
    int32_t *n_invalid; // [1]
    int32_t *active;    // [E]  experts with a pair, ascending (nullable)
    int32_t *n_active;  // [1]                                 (nullable)
    int32_t *tiles;     // [2*max_tiles] (expert, first row)   (nullable)
    int32_t *n_tiles;   // [1]                                 (nullable)
    int tile_m;         // rows per tile
    // Prefill passes (with tiles only): experts with 1..skinny_max pairs are
    // cut into SK_TP-row passes (expert, first row) instead of tiles.
    int32_t *spass;     // [2*max_passes]                      (nullable)
    int32_t *n_spass;   // [1]                                 (nullable)
    int skinny_max;
};

// Decode activation digits of `rows` rows of width `cols` (see common.h).
struct XDigits {
    uint32_t *dig;      // [rows][cols/32][20]
    float *fac;         // [rows][cols/32]
};

hipError_t launch_pack(const int8_t *q, int64_t rows, int64_t cols, uint8_t *packed,
                       int32_t *n_bad, hipStream_t st);
hipError_t launch_import_twos(const uint8_t *twos, int64_t rows, int64_t cols, uint8_t *packed,
                              hipStream_t st);
hipError_t launch_unpack(const uint8_t *packed, int64_t rows, int64_t cols, int8_t *q,
                         hipStream_t st);
// Re-lay a matrix of `cols` inputs as one of cols_out inputs (code 0 and
// scale 0 in the added columns and groups).
hipError_t launch_pad_cols(const uint8_t *q, const float *s, int64_t rows, int64_t cols, int64_t ng,
                           uint8_t *qo, int64_t cols_out, float *so, int64_t ng_out,
                           hipStream_t st);

// Worklist for n = tokens*k pairs.  block_counts: scratch of
// wl_scratch_ints(n, E) int32 (unused when n is small).
int64_t wl_scratch_ints(int64_t n, int E);
hipError_t launch_worklist(const int32_t *ids, int n, int k, int E, const Worklist &wl,
                           int32_t *scratch, hipStream_t st);

// Per-call plan of the decode GEMVs, written by the preparation kernel so a
// GEMV block starts with one load.  One record per weight pass: an active
// expert with c pairs gets ceil(c / tb) records of at most tb consecutive
// sorted positions, (expert, first and end sorted position, 0), experts in
// ascending order; records past the last are (-1, 0, 0, 0) up to max_rec.
// The gate+up and down kernels take different tokens per pass, so each has
// its own list.  tok/wsort = token and routing weight of each sorted
// position.
struct DecodePlan {
    int32_t *rec_gu;    // [4 * max_rec], passes of tb_gu pairs
    int32_t *rec_dn;    // [4 * max_rec], passes of tb_dn pairs
    int32_t *tok;       // [n]
    float *wsort;       // [n]
    int max_rec;        // >= the number of records of either list (n suffices)
    int tb_gu, tb_dn;
};

// Exact three-part f16 form of f32 activation rows (split16.h): v holds
// [rows][cols / 128][4][4][3] operands of 8 f16, f[row] = 2^-E of the row.
struct XSplit {
    uint16_t *v;
    float *f;
};

// Decode preparation in one launch: the worklist and plan (block 0), x ->
// digits (xd.dig set) or x -> f16 parts (xs.v set) for all tokens, and
// out <- 0.
hipError_t launch_decode_prep(const int32_t *ids, const float *topk_w, int n, int k, int E,
                              const Worklist &wl, const DecodePlan &plan, const float *x,
                              int tokens, int hidden, XDigits xd, XSplit xs, float *out,
                              hipStream_t st);

// x -> digits only (matvec and the single-expert FFN): rows of `cols`
// digits (a multiple of 32) from x rows of src_cols <= cols elements, the
// elements past src_cols taken as 0.
hipError_t launch_xdigits(const float *x, int rows, int cols, int src_cols, XDigits xd,
                          hipStream_t st);

// Decode GEMVs.  Tokens of expert `active[a]` are the sorted positions
// offsets[e]..offsets[e+1]; in "direct" mode (wl.pairs == nullptr) there is
// one expert (0) with positions 0..ntok-1 = tokens 0..ntok-1, weight 1.
struct GemvRoute {
    const int32_t *rec;    // plan records of this kernel (nullptr: direct mode)
    const int32_t *tok;    // token of each sorted position
    const float *wsort;    // routing weight of each sorted position
    int max_rec;           // grid bound on records
    int ntok;              // direct mode: tokens
    int pairs, experts;    // pairs and experts of the call (a launch-shape hint)
};

// h digits for the down projection: silu(gate x) * (up x) per sorted pair.
hipError_t launch_gemv_gateup(const QMat &gate, const QMat &up, XDigits xd, XDigits hd,
                              const GemvRoute &r, hipStream_t st);
// out[t] += w * down(h) (routed: atomic adds; direct: plain stores).
hipError_t launch_gemv_down(const QMat &down, XDigits hd, float *out, const GemvRoute &r,
                            hipStream_t st);
// y = W x for `batch` rows of digits.
// Tokens per weight pass the decode kernels use for matrix `m` in a call of
// `pairs` (token, expert) pairs over `experts` experts (the plan's pass
// length must match).
int gemv_tokens_per_pass(const QMat &m, int pairs, int experts, bool gateup);
hipError_t launch_gemv_matvec(const QMat &w, XDigits xd, int batch, float *y,
                              hipStream_t st);

// Decode GEMVs in f32 arithmetic.  Each launch block handles one weight pass
// (one expert, up to tb tokens) found from its grid slot in one of three
// modes: inline (ids set: slot = pair, the pass grouping derived in every
// block from the ids, for at most F32_INLINE_MAX pairs), record (rec set:
// plan records over sorted positions from the preparation kernel) or direct
// (neither: expert 0, slot a = tokens a*tb ..).  The rows of h are pairs
// (inline), sorted positions (record) or tokens (direct).
constexpr int F32_INLINE_MAX = 64;
struct F32Route {
    const int32_t *ids;     // inline: topk ids [n]
    const float *topk_w;    // inline: routing weights [n]
    int n, k, E;
    const int32_t *rec;     // record: plan records (see DecodePlan)
    const int32_t *tok;     // record: token of each sorted position
    const float *wsort;     // record: weight of each sorted position
    int max_rec;
    int ntok;               // direct: tokens
    int lead_row;           // inline gate+up: grid row 0 writes the worklist view and clears out
    Worklist wl;            // lead row: worklist view arrays
    float *out;             // lead row: output to clear
    int out_tokens, out_cols;
};
// A matrix stack as the f32 kernels see it: every size a buffer descriptor
// or a row offset is built from is computed on the host.
struct F32Mat {
    const uint8_t *q;
    const float *s;
    int64_t q_stride, s_stride;   // bytes / floats between experts
    int64_t qbytes, sbytes;       // one expert's codes and scales, in bytes
    int rows, cols, chunks;       // chunks = cols / 32
    uint32_t rb, sb;              // bytes per row of codes and of scales
    int gshift;                   // scale index of input i: i >> gshift (31: one per row)
};
F32Mat f32_mat(const QMat &m);
bool f32_gateup_supported(int hidden);
bool f32_down_supported(int cols);
int f32_tokens_per_pass(int pairs, int experts, bool gateup);
// h[hrow][F] = silu(G x) * (U x) in f32 (x f32 [tokens][H]).
hipError_t launch_f32_gateup(const QMat &gate, const QMat &up, const float *x, float *h,
                             const F32Route &r, int tb, hipStream_t st);
// y = D h over rows of h (h_ld floats apart, h_cols valid inputs, zero past
// them); routed: out[tok] += w * y (atomics), else out[tok] = y.
hipError_t launch_f32_down(const QMat &down, const float *hin, int64_t h_ld, int h_cols,
                           float *out, const F32Route &r, int tb, bool routed, hipStream_t st);

// Decode GEMVs on the matrix cores (f32 activations, record mode; the
// arithmetic of the f32 GEMVs above).  xs: the exact f16 parts of x from the
// preparation kernel; passes of at most MFD_TB tokens (the plan's tb for
// these kernels).  gate+up writes h as f32 rows (h, sorted positions) or,
// for the matrix-core down projection, as that kernel's operands (hs: the
// f16 parts of each 64 rows of h scaled by a power of two, hs.f[pos][F / 64]
// its inverse).  The down projection needs a gate+up that wrote hs.
constexpr int MFD_TB = 4;
constexpr int MFD_DOWN_MAX_COLS = 6144;
bool mfd_gateup_supported(const QMat &gate, const QMat &up);
bool mfd_down_supported(const QMat &down);
// Bytes of the split of `rows` activation rows of `cols` inputs.
inline int64_t xsplit_bytes(int64_t rows, int64_t cols) { return rows * cols * 6; }
hipError_t launch_mfd_gateup(const QMat &gate, const QMat &up, XSplit xs, int tokens, float *h,
                             XSplit hs, const int32_t *rec, const int32_t *tok, int max_rec,
                             hipStream_t st);
hipError_t launch_mfd_down(const QMat &down, XSplit hs, int pairs, float *out, const int32_t *rec,
                           const int32_t *tok, const float *wsort, int max_rec, hipStream_t st);

// Prefill (bf16 activations, MFMA).
constexpr int MFMA_BM = 256;
struct MfmaRoute {
    Worklist wl;
    const float *topk_w;
    int k;
    int max_tiles;     // grid bound on tiles
    int ntok;          // direct mode
    int64_t x_rows;    // rows of x16 (tokens); x_rows * hidden * 2 < 2^32
    int64_t h_rows;    // rows of h16 (pair positions); h_rows * inter * 2 < 2^32
};
// x bf16 [tokens][hidden] -> x16 f16 scaled by 2^k_t (octet-permuted), xinv = 2^-k_t.
hipError_t launch_xprep(const uint16_t *x, int tokens, int hidden, uint16_t *x16, float *xinv,
                        hipStream_t st);
// h16[pos][F] = silu(G x) * (U x) as f16, pos = sorted pair position.
hipError_t launch_mfma_gateup(const QMat &gate, const QMat &up, const uint16_t *x16,
                              const float *xinv, uint16_t *h16, const MfmaRoute &r,
                              hipStream_t st);
// Y of the routed prefill down projection: Y[pos][n] = v[pos][n] * 2^(e - 15)
// with v f16 and e an int8 exponent shared by each 4-row x 16-column block
// (stored once per row: e[pos][n / 16]); |v| < 2^15 by construction.
struct YBuf {
    uint16_t *v;   // [pairs][hidden] f16
    int8_t *e;     // [pairs][hidden / 16]
};
// Routed: Y[pos] = w * (D h) into y; direct mode: out[t] = D h in f32.
hipError_t launch_mfma_down(const QMat &down, const uint16_t *h16, float *out, YBuf y,
                            const MfmaRoute &r, hipStream_t st);
// out[t] = sum_j Y[inv[t*k + j]] in pick order (dropped pairs skipped).
hipError_t launch_combine(YBuf y, const int32_t *inv, int tokens, int k, int hidden, float *out,
                          hipStream_t st);

// Prefill passes of lightly routed experts (skinny.hip): SK_TP rows each,
// weights streamed once per pass on the matrix cores; the same h16 and Y as
// the tile kernels.
constexpr int SK_TP = 16;
// Experts with at most this many pairs take passes by default.
constexpr int PREFILL_PASS_ROWS_DEFAULT = 16;
struct SkRoute {
    Worklist wl;           // counts, offsets, pairs, spass, n_spass
    const float *topk_w;
    int k;
    int max_passes;        // bound on n_spass
};
bool sk_supported(const QMat &gate, const QMat &up, const QMat &down);
hipError_t launch_sk_gateup(const QMat &gate, const QMat &up, const uint16_t *x16, int tokens,
                            const float *xinv, uint16_t *h16, const SkRoute &r, hipStream_t st);
hipError_t launch_sk_down(const QMat &down, const uint16_t *h16, int64_t pairs, YBuf y,
                          const SkRoute &r, hipStream_t st);


// Read-stream probe (probe.hip): pattern 0 linear, 1 rows; grid blocks =
// probe_grid(pattern), one uint32 sum each in sink.
int probe_grid(int pattern);
hipError_t launch_probe(const void *buf, int64_t bytes, int pattern, uint32_t *sink,
                        hipStream_t st);

// Router: ids [tokens][k] (pick order) and softmax weights over the picked
// logits, one wave per token.
constexpr int MAX_ROUTE_TOPK = 16;
bool route_supported(int experts, int k);
hipError_t launch_route(const float *logits, int tokens, int experts, int k, int32_t *ids,
                        float *w, hipStream_t st);

}  // namespace qmoe
