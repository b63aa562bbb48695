// C ABI of libqmoe.so: host-side validation, workspace layout and launch
// sequencing.  Every check runs before the first HIP call, so a rejected
// call launches nothing (fail closed).
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "../../include/qmoe.h"
#include "launch.h"

using namespace qmoe;

namespace qmoe {
bool gemv_supported(int cols);
}

namespace {
// f32 activations: QMOE_F32 (f32 arithmetic) or QMOE_F32_DIGITS (the
// block fixed-point digit variant); both read x as f32 [tokens][H].
inline bool is_f32(int dtype) { return dtype == QMOE_F32 || dtype == QMOE_F32_DIGITS; }
inline int x_elem_bytes(int dtype) { return is_f32(dtype) ? 4 : 2; }
// Widths the decode kernels of a dtype take (hidden into gate+up, inter into down).
inline bool decode_widths_ok(int dtype, int H, int F) {
    if (dtype == QMOE_F32) return f32_gateup_supported(H) && f32_down_supported(F);
    return gemv_supported(H) && gemv_supported(F);
}
}  // namespace

namespace {

constexpr int MAX_EXPERTS = 1024;
constexpr int MAX_TOPK = 64;

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

inline bool overlap(const void *a, int64_t na, const void *b, int64_t nb) {
    if (!a || !b || na <= 0 || nb <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

inline int status_of(hipError_t e) { return e == hipSuccess ? QMOE_OK : QMOE_ERR_HIP; }

// The prefill kernels address activations, h and each expert's weights
// through buffer descriptors with 32-bit byte sizes and offsets; the
// epilogues store a tile's rows (at most 256) through one descriptor, with
// 2^31 added to the offset of a lane that must not store, so a tile's h and Y
// rows must span less than 2^31 bytes.
inline bool mfma_fits(int64_t H, int64_t F, int64_t x_rows, int64_t h_rows) {
    const int64_t lim = (int64_t)1 << 32;
    return x_rows * H * 2 < lim && h_rows * F * 2 < lim && H * F / 2 < lim && H * F / 8 < lim &&
           256 * 2 * (H > F ? H : F) < lim / 2;
}

int64_t packed_bytes(int64_t rows, int64_t cols) { return rows * ((cols + 1) / 2); }
int64_t scale_count(int64_t rows, int64_t cols, int64_t g) { return rows * ((cols + g - 1) / g); }

// The decode kernels read one matrix (one expert) through buffer descriptors
// whose lanes past a row's end use an offset of 2^31: codes and scales of a
// matrix must stay below 2 GB.
inline bool gemv_fits(int64_t rows, int64_t cols, int64_t g) {
    const int64_t lim = (int64_t)1 << 31;
    return packed_bytes(rows, cols) < lim && 4 * scale_count(rows, cols, g) < lim;
}

// Group sizes the GPU kernels take for a row of `cols` inputs: 32, 64 times a
// power of two (64, 128, 256, ...), or at least the row (one scale per row).
bool group_supported(int group, int cols) {
    if (group == 32 || group >= cols) return group > 0;
    if (group % 64 != 0) return false;
    const int m = group / 64;
    return (m & (m - 1)) == 0;
}

// Validate one matrix descriptor for the GPU kernels: expected shape, a
// supported group, cols % 64 == 0, aligned pointers and expert strides.
int check_qmat(const qmoe_qmat *m, int rows, int cols, int experts) {
    if (!m) return QMOE_ERR_NULL;
    if (m->struct_size != sizeof(qmoe_qmat)) return QMOE_ERR_ABI;
    if (m->rows != rows || m->cols != cols || rows <= 0 || cols <= 0) return QMOE_ERR_SHAPE;
    if (m->group <= 0) return QMOE_ERR_SHAPE;
    if (!group_supported(m->group, cols) || cols % 64 != 0) return QMOE_ERR_UNSUPPORTED;
    if (!gemv_fits(rows, cols, m->group)) return QMOE_ERR_UNSUPPORTED;
    if (!m->q || !m->s) return QMOE_ERR_NULL;
    if (!aligned16(m->q) || !aligned16(m->s)) return QMOE_ERR_ALIGN;
    if (experts > 1) {
        if (m->q_expert_stride < packed_bytes(rows, cols) ||
            m->s_expert_stride < scale_count(rows, cols, m->group))
            return QMOE_ERR_SHAPE;
        if (m->q_expert_stride % 16 != 0 || m->s_expert_stride % 4 != 0) return QMOE_ERR_ALIGN;
    }
    return QMOE_OK;
}

QMat to_qmat(const qmoe_qmat *m) {
    QMat q;
    q.q = m->q;
    q.s = m->s;
    q.q_stride = m->q_expert_stride;
    q.s_stride = m->s_expert_stride;
    q.rows = m->rows;
    q.cols = m->cols;
    q.group = m->group;
    return q;
}

// Workspace carving with 256-byte alignment.
struct Carver {
    char *base;
    int64_t off = 0;
    explicit Carver(void *b) : base(static_cast<char *>(b)) {}
    template <typename T>
    T *take(int64_t count) {
        T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
        off = align256(off + count * (int64_t)sizeof(T));
        return p;
    }
};

struct LayerWs {
    Worklist wl;
    int32_t *hist;
    XDigits xd, hd;
    DecodePlan plan;
    float *hf;           // f32 path: h [pairs][F]
    XSplit xs;           // f32 path, matrix-core record mode: f16 parts of x
    XSplit hs;           // ... and of h (the down projection's operands)
    uint16_t *x16, *h16;
    float *xinv;
    YBuf y;
    int64_t bytes;
    int max_active, max_tiles;
    int max_passes;      // bf16 prefill passes (0: every expert takes tiles)
    qmoe_layer_ws_view view;
};

// Experts with at most this many pairs run the bf16 prefill as 16-row passes
// (skinny.hip) rather than row tiles; QMOE_PREFILL_PASS_ROWS overrides it
// (0 turns the passes off), read once per process.
static int prefill_pass_rows() {
    static const int v = [] {
        const char *s = getenv("QMOE_PREFILL_PASS_ROWS");
        int r = PREFILL_PASS_ROWS_DEFAULT;
        if (s && *s) r = atoi(s);
        return r < 0 ? 0 : (r > MFMA_BM ? MFMA_BM : r);
    }();
    return v;
}

LayerWs carve_layer(void *ws, int E, int H, int F, int T, int k, int dtype) {
    LayerWs L{};
    Carver c(ws);
    const int64_t n = (int64_t)T * k;
    L.max_active = (int)(n < E ? n : E);
    L.max_tiles = (int)((n + MFMA_BM - 1) / MFMA_BM + L.max_active);
    L.wl.counts = c.take<int32_t>(E);
    L.wl.offsets = c.take<int32_t>(E + 1);
    L.wl.pairs = c.take<int32_t>(n);
    L.wl.inv = c.take<int32_t>(n);
    L.wl.n_invalid = c.take<int32_t>(1);
    L.wl.active = c.take<int32_t>(E);
    L.wl.n_active = c.take<int32_t>(1);
    L.wl.tiles = c.take<int32_t>(2 * (int64_t)L.max_tiles);
    L.wl.n_tiles = c.take<int32_t>(1);
    L.wl.tile_m = MFMA_BM;
    L.hist = c.take<int32_t>(wl_scratch_ints(n, E));
    if (dtype == QMOE_F32) {
        if (n > F32_INLINE_MAX) {
            L.plan.rec_gu = c.take<int32_t>(4 * n);
            L.plan.rec_dn = c.take<int32_t>(4 * n);
            L.plan.tok = c.take<int32_t>(n);
            L.plan.wsort = c.take<float>(n);
            L.plan.max_rec = (int)n;
        }
        bool hs_ok = false;
        if (n > F32_INLINE_MAX && H % 512 == 0 && xsplit_bytes(T, H) < ((int64_t)1 << 31)) {
            L.xs.v = c.take<uint16_t>(xsplit_bytes(T, H) / 2);
            L.xs.f = c.take<float>(T);
            hs_ok = F % 512 == 0 && F <= MFD_DOWN_MAX_COLS && xsplit_bytes(n, F) < ((int64_t)1 << 31);
        }
        if (hs_ok) {
            // h is either f32 rows (VALU down) or the matrix-core down
            // projection's f16 parts, never both in one call: one region
            const int64_t hb = xsplit_bytes(n, F) > n * F * 4 ? xsplit_bytes(n, F) : n * F * 4;
            uint16_t *hr = c.take<uint16_t>(hb / 2);
            L.hf = reinterpret_cast<float *>(hr);
            L.hs.v = hr;
            L.hs.f = c.take<float>(n * (F / 64));
        } else {
            L.hf = c.take<float>(n * F);
        }
    } else if (dtype == QMOE_F32_DIGITS) {
        L.plan.rec_gu = c.take<int32_t>(4 * n);
        L.plan.rec_dn = c.take<int32_t>(4 * n);
        L.plan.tok = c.take<int32_t>(n);
        L.plan.wsort = c.take<float>(n);
        L.plan.max_rec = (int)n;
        L.xd.dig = c.take<uint32_t>((int64_t)T * (H / 32) * 20);
        L.xd.fac = c.take<float>((int64_t)T * (H / 32));
        L.hd.dig = c.take<uint32_t>(n * (F / 32) * 20);
        L.hd.fac = c.take<float>(n * (F / 32));
    } else {
        L.x16 = c.take<uint16_t>((int64_t)T * H);
        L.xinv = c.take<float>(T);
        L.h16 = c.take<uint16_t>(n * F);
        L.y.v = c.take<uint16_t>(n * H);
        L.y.e = c.take<int8_t>(n * (H / 16));
        const int pm = prefill_pass_rows();
        if (pm > 0) {
            const int64_t per_expert = (pm + SK_TP - 1) / SK_TP;
            const int64_t bound = (n + SK_TP - 1) / SK_TP + L.max_active;
            L.max_passes = (int)std::min(bound, per_expert * L.max_active);
            L.wl.spass = c.take<int32_t>(2 * (int64_t)L.max_passes);
            L.wl.n_spass = c.take<int32_t>(1);
            L.wl.skinny_max = pm;
        }
    }
    L.bytes = c.off;
    // offsets of the worklist arrays (same order as above)
    int64_t o = 0;
    L.view.struct_size = sizeof(qmoe_layer_ws_view);
    L.view.counts = o;
    o = align256(o + 4 * (int64_t)E);
    L.view.offsets = o;
    o = align256(o + 4 * (int64_t)(E + 1));
    L.view.pairs = o;
    o = align256(o + 4 * n);
    L.view.inv = o;
    o = align256(o + 4 * n);
    L.view.n_invalid = o;
    return L;
}

int check_layer_desc(const qmoe_layer_desc *d) {
    if (!d) return QMOE_ERR_NULL;
    if (d->struct_size != sizeof(qmoe_layer_desc)) return QMOE_ERR_ABI;
    if (d->experts < 1 || d->experts > MAX_EXPERTS || d->hidden <= 0 || d->inter <= 0)
        return QMOE_ERR_SHAPE;
    if (d->group <= 0) return QMOE_ERR_SHAPE;
    if (d->hidden % 64 || d->inter % 64) return QMOE_ERR_UNSUPPORTED;
    if (d->gate.group != d->group || d->up.group != d->group || d->down.group != d->group)
        return QMOE_ERR_SHAPE;
    int s;
    if ((s = check_qmat(&d->gate, d->inter, d->hidden, d->experts))) return s;
    if ((s = check_qmat(&d->up, d->inter, d->hidden, d->experts))) return s;
    if ((s = check_qmat(&d->down, d->hidden, d->inter, d->experts))) return s;
    return QMOE_OK;
}

}  // namespace

extern "C" {

int qmoe_abi_version(void) { return QMOE_ABI_VERSION; }

const char *qmoe_status_str(int status) {
    switch (status) {
        case QMOE_OK: return "ok";
        case QMOE_ERR_NULL: return "null pointer";
        case QMOE_ERR_SHAPE: return "bad shape or size";
        case QMOE_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
        case QMOE_ERR_UNSUPPORTED: return "unsupported by the GPU kernels (group 32, 64 * 2^j or a whole row; layer and FFN widths % 64 == 0; a matrix under 2 GB)";
        case QMOE_ERR_WORKSPACE: return "workspace missing or too small";
        case QMOE_ERR_ALIAS: return "output overlaps an input or the workspace";
        case QMOE_ERR_ABI: return "struct_size mismatch (library and caller built from different headers)";
        case QMOE_ERR_HIP: return "HIP launch failed";
        case QMOE_ERR_SCRATCH:
            return "needs more workspace than the allocation-free entry point's fixed scratch "
                   "(QMOE_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

size_t qmoe_packed_bytes(int64_t rows, int64_t cols) {
    if (rows < 0 || cols < 0) return 0;
    return (size_t)packed_bytes(rows, cols);
}

size_t qmoe_scale_count(int64_t rows, int64_t cols, int64_t group) {
    if (rows < 0 || cols < 0 || group <= 0) return 0;
    return (size_t)scale_count(rows, cols, group);
}

int qmoe_pack(const int8_t *q, int64_t rows, int64_t cols, uint8_t *packed, int32_t *n_bad,
              void *stream) {
    if (rows < 0 || cols < 0) return QMOE_ERR_SHAPE;
    if (rows == 0 || cols == 0) return QMOE_OK;
    if (!q || !packed) return QMOE_ERR_NULL;
    if (n_bad && !aligned4(n_bad)) return QMOE_ERR_ALIGN;
    if (overlap(q, rows * cols, packed, packed_bytes(rows, cols))) return QMOE_ERR_ALIAS;
    if (n_bad && (overlap(n_bad, 4, q, rows * cols) ||
                  overlap(n_bad, 4, packed, packed_bytes(rows, cols))))
        return QMOE_ERR_ALIAS;
    return status_of(launch_pack(q, rows, cols, packed, n_bad, as_stream(stream)));
}

int qmoe_unpack(const uint8_t *packed, int64_t rows, int64_t cols, int8_t *q, void *stream) {
    if (rows < 0 || cols < 0) return QMOE_ERR_SHAPE;
    if (rows == 0 || cols == 0) return QMOE_OK;
    if (!q || !packed) return QMOE_ERR_NULL;
    if (overlap(q, rows * cols, packed, packed_bytes(rows, cols))) return QMOE_ERR_ALIAS;
    return status_of(launch_unpack(packed, rows, cols, q, as_stream(stream)));
}

// A matvec over a width that is not a multiple of 64 (a partial last group)
// runs on a copy of W re-laid to the next multiple of 64 in the workspace:
// the added columns hold code 0 and the added groups scale 0, and x is read
// as zero past its width.  Group 32 and 64 * 2^j keep their scale index;
// one scale per row (group >= cols) becomes group = padded width.
struct MatvecPlan {
    int64_t cols;       // padded width
    int64_t group;      // group of the padded matrix
    int64_t ng_in, ng;  // scales per row before and after
    bool relaid;
};

static MatvecPlan matvec_plan(const qmoe_qmat *W) {
    MatvecPlan p;
    p.cols = (W->cols + 63) / 64 * 64;
    p.relaid = p.cols != W->cols;
    p.group = W->group >= W->cols ? p.cols : W->group;
    p.ng_in = (W->cols + W->group - 1) / W->group;
    p.ng = (p.cols + p.group - 1) / p.group;
    return p;
}

size_t qmoe_matvec_workspace_bytes(const qmoe_qmat *W, int32_t batch) {
    if (!W || batch < 0 || W->cols <= 0 || W->rows <= 0 || W->group <= 0) return 0;
    const MatvecPlan p = matvec_plan(W);
    Carver c(nullptr);
    if (p.relaid) {
        c.take<uint8_t>((int64_t)W->rows * (p.cols / 2));
        c.take<float>((int64_t)W->rows * p.ng);
    }
    return (size_t)c.off;
}

int qmoe_matvec(const qmoe_qmat *W, const float *x, int32_t batch, float *y, void *ws,
                size_t ws_bytes, void *stream) {
    if (!W) return QMOE_ERR_NULL;
    if (W->struct_size != sizeof(qmoe_qmat)) return QMOE_ERR_ABI;
    if (batch < 0 || W->rows <= 0 || W->cols <= 0 || W->group <= 0) return QMOE_ERR_SHAPE;
    if (!group_supported(W->group, W->cols)) return QMOE_ERR_UNSUPPORTED;
    const MatvecPlan p = matvec_plan(W);
    if (!f32_down_supported((int)p.cols) || !gemv_fits(W->rows, p.cols, p.group))
        return QMOE_ERR_UNSUPPORTED;
    if (!W->q || !W->s) return QMOE_ERR_NULL;
    if (!aligned16(W->q) || !aligned16(W->s)) return QMOE_ERR_ALIGN;
    if (batch == 0) return QMOE_OK;
    if (!x || !y) return QMOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(y)) return QMOE_ERR_ALIGN;
    const size_t need = qmoe_matvec_workspace_bytes(W, batch);
    if (need > 0 && (!ws || ws_bytes < need)) return QMOE_ERR_WORKSPACE;
    if (need > 0 && !aligned16(ws)) return QMOE_ERR_ALIGN;
    const int64_t xb = (int64_t)batch * W->cols * 4, yb = (int64_t)batch * W->rows * 4;
    if (overlap(y, yb, x, xb) || overlap(y, yb, ws, need) || overlap(x, xb, ws, need) ||
        overlap(y, yb, W->q, packed_bytes(W->rows, W->cols)) ||
        overlap(y, yb, W->s, 4 * scale_count(W->rows, W->cols, W->group)) ||
        overlap(ws, need, W->q, packed_bytes(W->rows, W->cols)) ||
        overlap(ws, need, W->s, 4 * scale_count(W->rows, W->cols, W->group)))
        return QMOE_ERR_ALIAS;
    Carver c(ws);
    const hipStream_t st = as_stream(stream);
    QMat M = to_qmat(W);
    hipError_t e = hipSuccess;
    if (p.relaid) {
        uint8_t *q2 = c.take<uint8_t>((int64_t)W->rows * (p.cols / 2));
        float *s2 = c.take<float>((int64_t)W->rows * p.ng);
        e = launch_pad_cols(W->q, W->s, W->rows, W->cols, p.ng_in, q2, p.cols, s2, p.ng, st);
        M.q = q2;
        M.s = s2;
        M.cols = (int)p.cols;
        M.group = (int)p.group;
    }
    F32Route r{};
    r.ntok = batch;
    const int tb = batch >= 4 ? 4 : batch >= 2 ? 2 : 1;
    if (e == hipSuccess) e = launch_f32_down(M, x, W->cols, W->cols, y, r, tb, false, st);
    return status_of(e);
}

size_t qmoe_expert_ffn_workspace_bytes(const qmoe_qmat *gate, const qmoe_qmat *up,
                                       const qmoe_qmat *down, int32_t x_dtype, int32_t batch) {
    (void)up;
    (void)down;
    if (!gate || batch < 0) return 0;
    const int64_t H = gate->cols, F = gate->rows;
    Carver c(nullptr);
    if (x_dtype == QMOE_F32) {
        c.take<float>(batch * F);
    } else if (x_dtype == QMOE_F32_DIGITS) {
        c.take<uint32_t>(batch * (H / 32) * 20);
        c.take<float>(batch * (H / 32));
        c.take<uint32_t>(batch * (F / 32) * 20);
        c.take<float>(batch * (F / 32));
    } else {
        c.take<uint16_t>(batch * H);
        c.take<float>(batch);
        c.take<uint16_t>(batch * F);
    }
    return (size_t)c.off;
}

int qmoe_expert_ffn(const qmoe_qmat *gate, const qmoe_qmat *up, const qmoe_qmat *down,
                    int32_t x_dtype, const void *x, int32_t batch, float *out, void *ws,
                    size_t ws_bytes, void *stream) {
    if (!gate || !up || !down) return QMOE_ERR_NULL;
    if (gate->struct_size != sizeof(qmoe_qmat) || up->struct_size != sizeof(qmoe_qmat) ||
        down->struct_size != sizeof(qmoe_qmat))
        return QMOE_ERR_ABI;
    const int H = gate->cols, F = gate->rows;
    if (H <= 0 || F <= 0 || batch < 0) return QMOE_ERR_SHAPE;
    int s;
    if ((s = check_qmat(gate, F, H, 1))) return s;
    if ((s = check_qmat(up, F, H, 1))) return s;
    if ((s = check_qmat(down, H, F, 1))) return s;
    if (gate->group != up->group) return QMOE_ERR_SHAPE;   // one fused gate+up pass
    if (!is_f32(x_dtype) && x_dtype != QMOE_BF16) return QMOE_ERR_UNSUPPORTED;
    if (is_f32(x_dtype) && !decode_widths_ok(x_dtype, H, F)) return QMOE_ERR_UNSUPPORTED;
    if (x_dtype == QMOE_BF16 && H % 64 != 0) return QMOE_ERR_UNSUPPORTED;
    if (batch == 0) return QMOE_OK;
    if (!x || !out) return QMOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(out)) return QMOE_ERR_ALIGN;
    const size_t need = qmoe_expert_ffn_workspace_bytes(gate, up, down, x_dtype, batch);
    if (!ws || ws_bytes < need) return QMOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return QMOE_ERR_ALIGN;
    const int64_t xb = (int64_t)batch * H * x_elem_bytes(x_dtype);
    const int64_t ob = (int64_t)batch * H * 4;
    if (overlap(out, ob, x, xb) || overlap(out, ob, ws, need) || overlap(x, xb, ws, need))
        return QMOE_ERR_ALIAS;
    const hipStream_t st = as_stream(stream);
    Carver c(ws);
    hipError_t e;
    if (x_dtype == QMOE_F32) {
        float *hf = c.take<float>((int64_t)batch * F);
        F32Route r{};
        r.ntok = batch;
        const int tb = batch >= 4 ? 4 : batch >= 2 ? 2 : 1;
        e = launch_f32_gateup(to_qmat(gate), to_qmat(up), static_cast<const float *>(x), hf, r,
                              tb, st);
        if (e == hipSuccess) e = launch_f32_down(to_qmat(down), hf, F, F, out, r, tb, false, st);
    } else if (x_dtype == QMOE_F32_DIGITS) {
        XDigits xd, hd;
        xd.dig = c.take<uint32_t>((int64_t)batch * (H / 32) * 20);
        xd.fac = c.take<float>((int64_t)batch * (H / 32));
        hd.dig = c.take<uint32_t>((int64_t)batch * (F / 32) * 20);
        hd.fac = c.take<float>((int64_t)batch * (F / 32));
        GemvRoute r{};
        r.ntok = batch;
        r.pairs = batch;
        r.experts = 1;
        e = launch_xdigits(static_cast<const float *>(x), batch, H, H, xd, st);
        if (e == hipSuccess) e = launch_gemv_gateup(to_qmat(gate), to_qmat(up), xd, hd, r, st);
        if (e == hipSuccess) e = launch_gemv_down(to_qmat(down), hd, out, r, st);
    } else {
        uint16_t *x16 = c.take<uint16_t>((int64_t)batch * H);
        float *xinv = c.take<float>(batch);
        uint16_t *h16 = c.take<uint16_t>((int64_t)batch * F);
        MfmaRoute r{};
        r.wl.pairs = nullptr;
        r.ntok = batch;
        r.k = 1;
        r.x_rows = batch;
        r.h_rows = batch;
        if (!mfma_fits(H, F, batch, batch)) return QMOE_ERR_SHAPE;
        e = launch_xprep(static_cast<const uint16_t *>(x), batch, H, x16, xinv, st);
        if (e == hipSuccess)
            e = launch_mfma_gateup(to_qmat(gate), to_qmat(up), x16, xinv, h16, r, st);
        if (e == hipSuccess) e = launch_mfma_down(to_qmat(down), h16, out, YBuf{}, r, st);
    }
    return status_of(e);
}

int qmoe_import_twos(const uint8_t *twos, int64_t rows, int64_t cols, uint8_t *packed,
                     void *stream) {
    if (rows < 0 || cols < 0) return QMOE_ERR_SHAPE;
    const int64_t n = packed_bytes(rows, cols);
    if (n == 0) return QMOE_OK;
    if (!twos || !packed) return QMOE_ERR_NULL;
    if (twos != packed && overlap(twos, n, packed, n)) return QMOE_ERR_ALIAS;
    return status_of(launch_import_twos(twos, rows, cols, packed, as_stream(stream)));
}

int qmoe_stream_probe(const void *buf, int64_t bytes, int32_t pattern, uint32_t *sink,
                      void *stream) {
    if (!buf || !sink) return QMOE_ERR_NULL;
    if (pattern != QMOE_PROBE_LINEAR && pattern != QMOE_PROBE_ROWS) return QMOE_ERR_UNSUPPORTED;
    if (bytes <= 0 || bytes > ((int64_t)1 << 30)) return QMOE_ERR_SHAPE;
    if (pattern == QMOE_PROBE_ROWS && bytes % 2048 != 0) return QMOE_ERR_SHAPE;
    if (!aligned16(buf) || !aligned4(sink)) return QMOE_ERR_ALIGN;
    if (probe_grid(pattern) > QMOE_PROBE_SINK) return QMOE_ERR_SHAPE;
    if (overlap(sink, 4 * (int64_t)QMOE_PROBE_SINK, buf, bytes)) return QMOE_ERR_ALIAS;
    return status_of(launch_probe(buf, bytes, pattern, sink, as_stream(stream)));
}

int32_t qmoe_detect_group(int64_t rows, int64_t cols, int64_t scale_bytes) {
    static const int64_t cand[8] = {16, 32, 48, 64, 96, 128, 192, 256};
    if (rows <= 0 || cols <= 0 || scale_bytes <= 0) return 0;
    for (int64_t gs : cand)
        if (scale_count(rows, cols, gs) * 4 == scale_bytes) return (int32_t)gs;
    return 0;
}

int qmoe_route(const float *logits, int32_t tokens, int32_t experts, int32_t k,
               int32_t *topk_ids, float *topk_w, void *stream) {
    if (tokens < 0 || experts < 1 || k < 1 || k > experts) return QMOE_ERR_SHAPE;
    if ((int64_t)tokens * experts > (int64_t)1 << 31) return QMOE_ERR_SHAPE;
    if (!route_supported(experts, k)) return QMOE_ERR_UNSUPPORTED;
    if (tokens == 0) return QMOE_OK;
    if (!logits || !topk_ids || !topk_w) return QMOE_ERR_NULL;
    if (!aligned4(logits) || !aligned4(topk_ids) || !aligned4(topk_w)) return QMOE_ERR_ALIGN;
    const int64_t nl = 4 * (int64_t)tokens * experts, no = 4 * (int64_t)tokens * k;
    if (overlap(topk_ids, no, logits, nl) || overlap(topk_w, no, logits, nl) ||
        overlap(topk_ids, no, topk_w, no))
        return QMOE_ERR_ALIAS;
    return status_of(launch_route(logits, tokens, experts, k, topk_ids, topk_w,
                                  as_stream(stream)));
}

size_t qmoe_worklist_workspace_bytes(int32_t tokens, int32_t k, int32_t experts) {
    if (tokens < 0 || k < 1 || experts < 1) return 0;
    return (size_t)(4 * wl_scratch_ints((int64_t)tokens * k, experts));
}

int qmoe_worklist(const int32_t *topk_ids, int32_t tokens, int32_t k, int32_t experts,
                  int32_t *counts, int32_t *offsets, int32_t *pairs, int32_t *inv,
                  int32_t *n_invalid, void *ws, size_t ws_bytes, void *stream) {
    if (tokens < 0 || k < 1 || k > MAX_TOPK || experts < 1 || experts > MAX_EXPERTS)
        return QMOE_ERR_SHAPE;
    if ((int64_t)tokens * k > (int64_t)1 << 30) return QMOE_ERR_SHAPE;
    if (!counts || !offsets || !n_invalid) return QMOE_ERR_NULL;
    const int64_t n = (int64_t)tokens * k;
    if (n > 0 && (!topk_ids || !pairs || !inv)) return QMOE_ERR_NULL;
    const void *ptrs[6] = {topk_ids, counts, offsets, pairs, inv, n_invalid};
    for (const void *p : ptrs)
        if (p && !aligned4(p)) return QMOE_ERR_ALIGN;
    const size_t need = qmoe_worklist_workspace_bytes(tokens, k, experts);
    if (need > 0 && (!ws || ws_bytes < need)) return QMOE_ERR_WORKSPACE;
    const void *outs[5] = {counts, offsets, pairs, inv, n_invalid};
    const int64_t outn[5] = {4 * (int64_t)experts, 4 * (int64_t)(experts + 1), 4 * n, 4 * n, 4};
    for (int i = 0; i < 5; i++) {
        if (overlap(outs[i], outn[i], topk_ids, 4 * n)) return QMOE_ERR_ALIAS;
        if (need > 0 && overlap(outs[i], outn[i], ws, need)) return QMOE_ERR_ALIAS;
        for (int j = i + 1; j < 5; j++)
            if (overlap(outs[i], outn[i], outs[j], outn[j])) return QMOE_ERR_ALIAS;
    }
    Worklist wl{};
    wl.counts = counts;
    wl.offsets = offsets;
    wl.pairs = pairs;
    wl.inv = inv;
    wl.n_invalid = n_invalid;
    wl.tile_m = MFMA_BM;
    return status_of(launch_worklist(topk_ids, (int)n, k, experts, wl,
                                     static_cast<int32_t *>(ws), as_stream(stream)));
}

int32_t qmoe_prefill_pass_rows(void) { return prefill_pass_rows(); }

size_t qmoe_layer_workspace_bytes(const qmoe_layer_desc *desc, int32_t tokens, int32_t k,
                                  int32_t x_dtype) {
    if (!desc || tokens < 0 || k < 1 || desc->experts < 1) return 0;
    if (!is_f32(x_dtype) && x_dtype != QMOE_BF16) return 0;
    return (size_t)carve_layer(nullptr, desc->experts, desc->hidden, desc->inter, tokens, k,
                               x_dtype)
        .bytes;
}

int qmoe_layer_ws_layout(const qmoe_layer_desc *desc, int32_t tokens, int32_t k,
                         int32_t x_dtype, qmoe_layer_ws_view *view) {
    if (!desc || !view) return QMOE_ERR_NULL;
    if (view->struct_size != sizeof(qmoe_layer_ws_view)) return QMOE_ERR_ABI;
    if (tokens < 0 || k < 1 || desc->experts < 1) return QMOE_ERR_SHAPE;
    const LayerWs L =
        carve_layer(nullptr, desc->experts, desc->hidden, desc->inter, tokens, k, x_dtype);
    *view = L.view;
    return QMOE_OK;
}

int qmoe_layer(const qmoe_layer_desc *desc, int32_t x_dtype, const void *x, int32_t tokens,
               const int32_t *topk_ids, const float *topk_w, int32_t k, float *out, void *ws,
               size_t ws_bytes, void *stream) {
    return qmoe_layer_ex(desc, x_dtype, x, tokens, topk_ids, topk_w, k, out, ws, ws_bytes,
                         stream, nullptr, 0);
}

// Everything qmoe_layer_ex checks before launching (the routing arrays are
// only addressed, never read).
static int layer_validate(const qmoe_layer_desc *desc, int32_t x_dtype, const void *x,
                          int32_t tokens, const int32_t *topk_ids, const float *topk_w, int32_t k,
                          float *out, void *ws, size_t ws_bytes, void *const *phase_events,
                          int32_t n_events) {
    int s = check_layer_desc(desc);
    if (s) return s;
    if (!is_f32(x_dtype) && x_dtype != QMOE_BF16) return QMOE_ERR_UNSUPPORTED;
    if (tokens < 0 || k < 1 || k > MAX_TOPK) return QMOE_ERR_SHAPE;
    if ((int64_t)tokens * k > (int64_t)1 << 30) return QMOE_ERR_SHAPE;
    const int E = desc->experts, H = desc->hidden, F = desc->inter;
    if (is_f32(x_dtype) && !decode_widths_ok(x_dtype, H, F)) return QMOE_ERR_UNSUPPORTED;
    if (x_dtype == QMOE_BF16 && H % 64 != 0) return QMOE_ERR_UNSUPPORTED;
    {
        const int64_t n0 = (int64_t)tokens * k;
        const int64_t tiles = (n0 + MFMA_BM - 1) / MFMA_BM + (n0 < E ? n0 : E);
        if (tiles > 65535) return QMOE_ERR_SHAPE;   // grid.y bound of the tiled kernels
        if (x_dtype == QMOE_BF16 && !mfma_fits(H, F, tokens, n0)) return QMOE_ERR_SHAPE;
    }
    if (phase_events) {
        if (n_events < (is_f32(x_dtype) ? 4 : 5)) return QMOE_ERR_SHAPE;
        for (int i = 0; i < (is_f32(x_dtype) ? 4 : 5); i++)
            if (!phase_events[i]) return QMOE_ERR_NULL;
    }
    if (tokens == 0) return QMOE_OK;
    if (!x || !topk_ids || !topk_w || !out) return QMOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(out)) return QMOE_ERR_ALIGN;
    if (!aligned4(topk_ids) || !aligned4(topk_w)) return QMOE_ERR_ALIGN;
    const LayerWs need = carve_layer(nullptr, E, H, F, tokens, k, x_dtype);
    if (!ws || (int64_t)ws_bytes < need.bytes) return QMOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return QMOE_ERR_ALIGN;
    const int64_t n = (int64_t)tokens * k;
    const int64_t xb = (int64_t)tokens * H * x_elem_bytes(x_dtype);
    const int64_t ob = (int64_t)tokens * H * 4;
    if (overlap(out, ob, x, xb) || overlap(out, ob, topk_ids, 4 * n) ||
        overlap(out, ob, topk_w, 4 * n) || overlap(out, ob, ws, need.bytes) ||
        overlap(ws, need.bytes, x, xb) || overlap(ws, need.bytes, topk_ids, 4 * n) ||
        overlap(ws, need.bytes, topk_w, 4 * n))
        return QMOE_ERR_ALIAS;
    return QMOE_OK;
}

int qmoe_layer_ex(const qmoe_layer_desc *desc, int32_t x_dtype, const void *x, int32_t tokens,
                  const int32_t *topk_ids, const float *topk_w, int32_t k, float *out,
                  void *ws, size_t ws_bytes, void *stream, void *const *phase_events,
                  int32_t n_events) {
    const int s = layer_validate(desc, x_dtype, x, tokens, topk_ids, topk_w, k, out, ws, ws_bytes,
                                 phase_events, n_events);
    if (s || tokens == 0) return s;
    const int E = desc->experts, H = desc->hidden, F = desc->inter;
    const int64_t n = (int64_t)tokens * k;
    const LayerWs L = carve_layer(ws, E, H, F, tokens, k, x_dtype);
    const hipStream_t st = as_stream(stream);
    const QMat G = to_qmat(&desc->gate), U = to_qmat(&desc->up), D = to_qmat(&desc->down);
    int phase = 0;
    auto mark = [&]() -> hipError_t {
        if (!phase_events) return hipSuccess;
        return hipEventRecord(static_cast<hipEvent_t>(phase_events[phase++]), st);
    };
    hipError_t e = mark();
    if (e != hipSuccess) return QMOE_ERR_HIP;
    if (x_dtype == QMOE_F32) {
        // record mode runs the passes on the matrix cores where the shapes allow
        const bool mf_gu = n > F32_INLINE_MAX && L.xs.v && mfd_gateup_supported(G, U);
        const bool mf_dn = mf_gu && L.hs.v && mfd_down_supported(D);
        const int tb_gu = mf_gu ? MFD_TB : f32_tokens_per_pass((int)n, E, true);
        const int tb_dn = mf_dn ? MFD_TB : f32_tokens_per_pass((int)n, E, false);
        F32Route r{};
        r.k = k;
        r.E = E;
        r.n = (int)n;
        if (n <= F32_INLINE_MAX) {
            // the gate+up launch groups the pairs itself; its leading grid
            // row writes the worklist view and clears out
            r.ids = topk_ids;
            r.topk_w = topk_w;
            r.lead_row = 1;
            r.wl = L.wl;
            r.out = out;
            r.out_tokens = tokens;
            r.out_cols = H;
            if (e == hipSuccess) e = mark();
        } else {
            Worklist wl = L.wl;
            wl.tiles = nullptr;
            wl.n_tiles = nullptr;
            DecodePlan plan = L.plan;
            plan.tb_gu = tb_gu;
            plan.tb_dn = tb_dn;
            e = launch_decode_prep(topk_ids, topk_w, (int)n, k, E, wl, plan,
                                   static_cast<const float *>(x), tokens, H, XDigits{},
                                   mf_gu ? L.xs : XSplit{}, out, st);
            if (e == hipSuccess) e = mark();
            r.rec = plan.rec_gu;
            r.tok = plan.tok;
            r.wsort = plan.wsort;
            r.max_rec = plan.max_rec;
        }
        if (e == hipSuccess) {
            if (mf_gu)
                e = launch_mfd_gateup(G, U, L.xs, tokens, L.hf, mf_dn ? L.hs : XSplit{},
                                      L.plan.rec_gu, L.plan.tok, L.plan.max_rec, st);
            else
                e = launch_f32_gateup(G, U, static_cast<const float *>(x), L.hf, r, tb_gu, st);
        }
        if (e == hipSuccess) e = mark();
        r.lead_row = 0;
        if (r.rec) r.rec = L.plan.rec_dn;
        if (e == hipSuccess) {
            if (mf_dn)
                e = launch_mfd_down(D, L.hs, (int)n, out, L.plan.rec_dn, L.plan.tok,
                                    L.plan.wsort, L.plan.max_rec, st);
            else
                e = launch_f32_down(D, L.hf, F, F, out, r, tb_dn, true, st);
        }
        if (e == hipSuccess) e = mark();
    } else if (x_dtype == QMOE_F32_DIGITS) {
        Worklist wl = L.wl;
        wl.tiles = nullptr;
        wl.n_tiles = nullptr;
        DecodePlan plan = L.plan;
        plan.tb_gu = gemv_tokens_per_pass(G, (int)n, E, true);
        plan.tb_dn = gemv_tokens_per_pass(D, (int)n, E, false);
        e = launch_decode_prep(topk_ids, topk_w, (int)n, k, E, wl, plan,
                               static_cast<const float *>(x), tokens, H, L.xd, XSplit{}, out,
                               st);
        if (e == hipSuccess) e = mark();
        GemvRoute r{};
        r.rec = plan.rec_gu;
        r.tok = plan.tok;
        r.wsort = plan.wsort;
        r.max_rec = plan.max_rec;
        r.pairs = (int)n;
        r.experts = E;
        if (e == hipSuccess) e = launch_gemv_gateup(G, U, L.xd, L.hd, r, st);
        if (e == hipSuccess) e = mark();
        r.rec = plan.rec_dn;
        if (e == hipSuccess) e = launch_gemv_down(D, L.hd, out, r, st);
        if (e == hipSuccess) e = mark();
    } else {
        // experts with few pairs take passes where the shapes allow
        const bool passes = L.max_passes > 0 && sk_supported(G, U, D);
        Worklist wl = L.wl;
        if (!passes) {
            wl.spass = nullptr;
            wl.n_spass = nullptr;
        }
        e = launch_worklist(topk_ids, (int)n, k, E, wl, L.hist, st);
        if (e == hipSuccess)
            e = launch_xprep(static_cast<const uint16_t *>(x), tokens, H, L.x16, L.xinv, st);
        if (e == hipSuccess) e = mark();
        MfmaRoute r{};
        r.wl = L.wl;
        r.topk_w = topk_w;
        r.k = k;
        r.max_tiles = L.max_tiles;
        r.x_rows = tokens;
        r.h_rows = n;
        SkRoute sr{};
        sr.wl = L.wl;
        sr.topk_w = topk_w;
        sr.k = k;
        sr.max_passes = L.max_passes;
        if (e == hipSuccess) e = launch_mfma_gateup(G, U, L.x16, L.xinv, L.h16, r, st);
        if (e == hipSuccess && passes)
            e = launch_sk_gateup(G, U, L.x16, tokens, L.xinv, L.h16, sr, st);
        if (e == hipSuccess) e = mark();
        if (e == hipSuccess) e = launch_mfma_down(D, L.h16, nullptr, L.y, r, st);
        if (e == hipSuccess && passes) e = launch_sk_down(D, L.h16, n, L.y, sr, st);
        if (e == hipSuccess) e = mark();
        if (e == hipSuccess) e = launch_combine(L.y, L.wl.inv, tokens, k, H, out, st);
        if (e == hipSuccess) e = mark();
    }
    return status_of(e);
}

size_t qmoe_layer_logits_workspace_bytes(const qmoe_layer_desc *desc, int32_t tokens,
                                         int32_t k, int32_t x_dtype) {
    const size_t layer = qmoe_layer_workspace_bytes(desc, tokens, k, x_dtype);
    if (layer == 0 && tokens > 0) return 0;
    return layer + 2 * (size_t)align256(4 * (int64_t)tokens * k);
}

int qmoe_layer_logits(const qmoe_layer_desc *desc, int32_t x_dtype, const void *x,
                      int32_t tokens, const float *logits, int32_t k, float *out, void *ws,
                      size_t ws_bytes, void *stream) {
    int s = check_layer_desc(desc);
    if (s) return s;
    if (tokens < 0 || k < 1) return QMOE_ERR_SHAPE;
    if (!route_supported(desc->experts, k)) return QMOE_ERR_UNSUPPORTED;
    if (tokens == 0) return QMOE_OK;
    if (!logits || !ws) return QMOE_ERR_NULL;
    if (!aligned4(logits)) return QMOE_ERR_ALIGN;
    const size_t need = qmoe_layer_logits_workspace_bytes(desc, tokens, k, x_dtype);
    if (need == 0) return QMOE_ERR_UNSUPPORTED;
    if (ws_bytes < need) return QMOE_ERR_WORKSPACE;
    const int64_t nl = 4 * (int64_t)tokens * desc->experts;
    if (overlap(logits, nl, ws, (int64_t)need) || overlap(logits, nl, out, 4 * (int64_t)tokens *
                                                                          desc->hidden))
        return QMOE_ERR_ALIAS;
    // routing arrays at the end of the workspace; the layer's own workspace
    // (and its worklist view) starts at offset 0
    const size_t layer = qmoe_layer_workspace_bytes(desc, tokens, k, x_dtype);
    uint8_t *base = static_cast<uint8_t *>(ws);
    int32_t *ids = reinterpret_cast<int32_t *>(base + layer);
    float *w = reinterpret_cast<float *>(base + layer + align256(4 * (int64_t)tokens * k));
    if ((s = layer_validate(desc, x_dtype, x, tokens, ids, w, k, out, ws, layer, nullptr, 0)))
        return s;
    const hipError_t e = launch_route(logits, tokens, desc->experts, k, ids, w, as_stream(stream));
    if (e != hipSuccess) return QMOE_ERR_HIP;
    return qmoe_layer(desc, x_dtype, x, tokens, ids, w, k, out, ws, layer, stream);
}

}  // extern "C"
