/*
 * qmoe -- grouped int4 (gs = 64) MoE expert matmul for AMD Instinct MI355X
 * (gfx950).  C ABI of libqmoe.so.
 *
 * The operation is the one the colibri pull request "cuda+engine: full fmt=4
 * (grouped int4 gs=64) support + diagnostic harness" adds to its engine:
 * expert weights quantised to signed int4, packed two per byte, with one f32
 * scale for every 64 consecutive input elements of a row (Summary and
 * Problem), evaluated as the fused gate+up pair (x read once for both
 * matrices) followed by the down projection (Summary, "matmul_i4_grouped_pair"
 * and "expert_gate_up"), over a top-k token-to-expert table that is built on
 * the device (pxq_llama.cpp release notes, "Device-side MoE row map").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates, frees or synchronises.  Work is enqueued on
 *    `stream` (a hipStream_t passed as void*; NULL = the null stream) and the
 *    return value comes from host-side checks made before anything is
 *    enqueued.  A non-zero status means nothing was launched: like the
 *    format guard of the same pull request (comment "implementation complete
 *    but system-instability"), an unsupported input is declined up front
 *    instead of being run with a guessed layout.
 *  - The library is stateless and thread-safe.  Concurrent calls on one
 *    stream serialise; calls on different streams that share a workspace
 *    race.
 *  - Sizes are 64-bit where they count bytes.  Shapes are int32.
 *  - Packed int4 layout ("qmat"): row-major [rows][ceil(cols/2)] bytes;
 *    element 2j of a row sits in the LOW nibble of byte j and element 2j+1
 *    in the high nibble; a nibble u stores the code q = u - 8 (offset
 *    binary, as the container on the pages stores it; XOR 0x88 per byte
 *    gives two's complement).  Scales are row-major f32 [rows][ceil(cols/g)]
 *    with scale(o, i) = s[o * ng + i / g] (comment "blocked by GPU driver
 *    instability": scales[o*ng + i/gs]).
 *  - Group sizes: 32, 64 * 2^j, or any group >= cols (one scale per row, the
 *    per-row int4 format); others return QMOE_ERR_UNSUPPORTED.  The layer
 *    and expert-FFN entry points take widths (hidden, inter) that are
 *    multiples of 64, as every MoE shape on the pages is; qmoe_matvec takes
 *    any width, a partial last group included.  Every pointer must be
 *    16-byte aligned (QMOE_ERR_ALIGN otherwise), like the vector-load guard
 *    of the pxq_llama.cpp notes (release rc3 fixes) that declines rather
 *    than faults.
 *  - Size limits (QMOE_ERR_SHAPE or QMOE_ERR_UNSUPPORTED beyond them): the
 *    kernels address memory through buffer descriptors with 32-bit byte
 *    offsets, so one expert matrix's codes and scales stay below 2 GB; on
 *    the bf16 path the activations [tokens][hidden] and h [pairs][inter] as
 *    f16 stay below 4 GB and hidden and inter below 2^22.
 *  - Bad expert ids (outside [0, E)) are data, not arguments: they are
 *    dropped (contribute zero) and counted into an int32 on the device.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMOE_ABI_VERSION 1

/* Status codes returned by every entry point. */
enum {
    QMOE_OK = 0,
    QMOE_ERR_NULL = 1,        /* a required pointer is NULL */
    QMOE_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
    QMOE_ERR_ALIGN = 3,       /* a pointer or stride is not 16-byte aligned */
    QMOE_ERR_UNSUPPORTED = 4, /* valid for the format, not for these kernels */
    QMOE_ERR_WORKSPACE = 5,   /* workspace missing or too small */
    QMOE_ERR_ALIAS = 6,       /* an output overlaps an input */
    QMOE_ERR_ABI = 7,         /* struct_size does not match this library */
    QMOE_ERR_HIP = 8,         /* a kernel launch failed (hipGetLastError) */
    QMOE_ERR_SCRATCH = 9      /* more than qmoe_layer_noalloc's fixed scratch */
};

/* Activation dtypes.  The dtype of x selects the path:
 *  - QMOE_F32: decode path in f32 arithmetic (GEMV kernels): every int4 code
 *    is unpacked to an exact f32, multiplied with the f32 activation and
 *    accumulated in f32 per 64-input group, the group's f32 scale applied
 *    once per group (the grouped kernel of the colibri pull request, comment
 *    "blocked by GPU driver instability"); h = silu(g) * u is kept in f32.
 *    Widths: hidden <= 8192 into gate/up, inter <= 16384 into down.  In
 *    qmoe_layer calls of more than 64 pairs with groups of 64 or more and
 *    widths that are multiples of 512 (hidden <= 6144 for gate/up, inter
 *    <= 6144 for down) the weight passes run on the matrix cores with the
 *    same arithmetic: each activation row (x, and each 64 inputs of h) is
 *    scaled by a power of two and split into three f16 parts that sum to it
 *    exactly (elements more than 2^15 below the largest keep an error below
 *    2^-39 of it), the codes are exact in f16, so every product is exact,
 *    and the sums are f32.
 *  - QMOE_F32_DIGITS: x is also f32 [tokens][H], but the activations are
 *    rounded to 18-bit block fixed point (one power-of-two exponent per
 *    64-element group of x and per 32-element chunk of h) and multiplied
 *    with the codes in integer dot products; an element far below its
 *    group's largest keeps fewer bits (error up to 2^(E-19) per element,
 *    2^(E-1) <= the group's max |x| < 2^E).  A faster variant that has to be
 *    asked for; widths: a multiple of 64 up to 12288.
 *  - QMOE_BF16: prefill path (grouped MFMA kernels).  The matrix cores take
 *    f16 operands: q * s is rounded to f16 (|s| < 8188; scales below 2^-14
 *    become f16 subnormals and lose relative precision, below about 2^-16
 *    the rounding alone approaches the 2e-3 bar), and the gated
 *    intermediate h is stored as f16 (|h| < 65504, larger values giving
 *    inf); the accumulators and every output are f32.  Experts that receive
 *    at most qmoe_prefill_pass_rows() pairs (skewed routing leaves many
 *    such experts) run as weight-streaming passes of up to 16 pairs when
 *    hidden and inter are multiples of 512 (hidden up to 6144, inter up to
 *    4608) and groups hold 64 or more inputs: the codes are exact f16 values, x16 (bf16 scaled by a
 *    power of two per token, exact in f16) and h are the other operand, and
 *    each 64-input group's f32 sums are multiplied by the f32 scale, so q * s
 *    is not rounded there; h is f16 as on the tile path.
 * A NaN or infinity in x reaches every output it feeds on the f32 and bf16
 * paths. */
enum { QMOE_F32 = 0, QMOE_BF16 = 1, QMOE_F32_DIGITS = 2 };

/* One grouped int4 matrix, or a stack of per-expert matrices of one shape.
 * q_expert_stride is the byte distance between experts' packed codes and
 * s_expert_stride the float distance between their scales (0 for a single
 * matrix).  Both must keep every expert 16-byte aligned. */
typedef struct qmoe_qmat {
    uint32_t struct_size;     /* = sizeof(qmoe_qmat) */
    int32_t rows;             /* O: output features */
    int32_t cols;             /* I: input features */
    int32_t group;            /* g: inputs per scale (64 on the pages) */
    const uint8_t *q;         /* packed codes, [E][rows][ceil(cols/2)] bytes */
    const float *s;           /* scales, [E][rows][ceil(cols/group)] f32 */
    int64_t q_expert_stride;  /* bytes between experts */
    int64_t s_expert_stride;  /* floats between experts */
} qmoe_qmat;

/* A MoE layer: E experts of hidden H and intermediate F.  gate and up are
 * [E][F][H], down is [E][H][F]. */
typedef struct qmoe_layer_desc {
    uint32_t struct_size;     /* = sizeof(qmoe_layer_desc) */
    int32_t experts;          /* E, 1..1024 */
    int32_t hidden;           /* H */
    int32_t inter;            /* F */
    int32_t group;            /* inputs per scale, = each matrix's group */
    qmoe_qmat gate, up, down;
} qmoe_layer_desc;

/* QMOE_ABI_VERSION of the loaded library; a caller built against another
 * version must not call anything else (the pull request's 7-vs-8-argument
 * upload mismatch, comment "fmt=4 CUDA attention crash", is the failure this
 * guards against). */
int qmoe_abi_version(void);

/* Static text for a status code; never NULL. */
const char *qmoe_status_str(int status);

/* rows * ceil(cols / 2): bytes of one packed matrix (pull request Summary:
 * int4 row_bytes = (I + 1) / 2).  Returns 0 for negative sizes. */
size_t qmoe_packed_bytes(int64_t rows, int64_t cols);

/* rows * ceil(cols / group): f32 scales of one matrix (pull request Summary:
 * O*ng scales instead of O).  Returns 0 for a non-positive group. */
size_t qmoe_scale_count(int64_t rows, int64_t cols, int64_t group);

/* Pack int8 codes q [rows][cols] (row-major, device) into the packed layout
 * above: byte j of row o = (q[o][2j] + 8) & 15 | ((q[o][2j+1] + 8) & 15) << 4,
 * pad nibble 8 when cols is odd.  Codes outside [-8, 7] are stored wrapped
 * and, when n_bad != NULL, counted into *n_bad (a device int32 the call
 * zeroes first).  The offset encoding is the one the container uses (nibbles
 * 0..15 standing for -8..7; comment "implementation complete but
 * system-instability").  Any rows, cols >= 0; no alignment requirement. */
int qmoe_pack(const int8_t *q, int64_t rows, int64_t cols, uint8_t *packed,
              int32_t *n_bad, void *stream);

/* Inverse of qmoe_pack: packed -> int8 codes in [-8, 7].  A test aid. */
int qmoe_unpack(const uint8_t *packed, int64_t rows, int64_t cols, int8_t *q,
                void *stream);

/* Workspace bytes qmoe_matvec needs for `batch` rows of x (0 for an invalid
 * descriptor).  When cols is not a multiple of 64 this includes a re-laid
 * copy of W (rows * cols64 / 2 bytes and its scales, cols64 = cols rounded
 * up to 64). */
size_t qmoe_matvec_workspace_bytes(const qmoe_qmat *W, int32_t batch);

/* y[b][o] = sum_i s[o][i/g] * q[o][i] * x[b][i] for b < batch: the single
 * grouped int4 matvec ("quant_matmul" with per-group scale, pull request
 * Summary).  x f32 [batch][cols], y f32 [batch][rows]; y must not overlap x,
 * W or the workspace, and the workspace must not overlap W.
 * W->q_expert_stride is ignored (expert 0).  Any cols >= 1, odd widths and a
 * last group shorter than g included (shapes the pull request's comment
 * that adds a double-precision C test for the grouped kernel covers): W is
 * then first re-laid in the workspace to a width that is a multiple of 64,
 * the added columns holding code 0 and the added groups scale 0, and x is
 * read as zero past cols. */
int qmoe_matvec(const qmoe_qmat *W, const float *x, int32_t batch, float *y,
                void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes qmoe_expert_ffn needs. */
size_t qmoe_expert_ffn_workspace_bytes(const qmoe_qmat *gate,
                                       const qmoe_qmat *up,
                                       const qmoe_qmat *down, int32_t x_dtype,
                                       int32_t batch);

/* One expert: out[b] = down(silu(gate x_b) * (up x_b)), silu(z) =
 * z / (1 + exp(-z)).  gate/up are [F][H], down is [H][F] (expert 0 of each
 * descriptor).  x is f32 or bf16 [batch][H] per x_dtype; out is f32
 * [batch][H] and must not overlap x.  Gate and up are evaluated as one fused
 * pair that loads each activation once for both matrices (pull request
 * Summary, the matmul_i4_grouped_pair entry). */
int qmoe_expert_ffn(const qmoe_qmat *gate, const qmoe_qmat *up,
                    const qmoe_qmat *down, int32_t x_dtype, const void *x,
                    int32_t batch, float *out, void *ws, size_t ws_bytes,
                    void *stream);

/* Token-to-expert table for one batched MoE layer, built entirely on the
 * device with no host round trip (pxq_llama.cpp notes, "Device-side MoE row
 * map": histogram, scan and fill).  Input topk_ids int32 [tokens][k].
 * Outputs (device int32):
 *   counts[experts]      valid pairs per expert;
 *   offsets[experts+1]   exclusive scan of counts, offsets[E] = n_valid;
 *   pairs[tokens*k]      pair ids p = t*k + j grouped by expert (ascending
 *                        expert, ascending p inside one expert), -1 after
 *                        the n_valid entries;
 *   inv[tokens*k]        position of pair p in `pairs`, -1 if dropped;
 *   n_invalid[1]         number of ids outside [0, experts).
 * The result is unique (a stable counting sort), so it is bit-exact against
 * any correct builder.  ws/ws_bytes: scratch from
 * qmoe_worklist_workspace_bytes (may be 0 bytes for small inputs). */
size_t qmoe_worklist_workspace_bytes(int32_t tokens, int32_t k,
                                     int32_t experts);
int qmoe_worklist(const int32_t *topk_ids, int32_t tokens, int32_t k,
                  int32_t experts, int32_t *counts, int32_t *offsets,
                  int32_t *pairs, int32_t *inv, int32_t *n_invalid, void *ws,
                  size_t ws_bytes, void *stream);

/* Import of the two's-complement nibble container (the layout the pages'
 * GPU upload produces; colibri pull request "cuda+engine: full fmt=4
 * (grouped int4 gs=64) support", comment "implementation complete but
 * system-instability": offset nibbles become two's complement by a byte XOR
 * of 0x88) back into the offset container this library reads: every byte
 * XOR 0x88.  twos and packed are device buffers of rows * ceil(cols/2)
 * bytes; packed == twos (in place) is allowed, any other overlap is
 * QMOE_ERR_ALIAS.  Bit-exact. */
int qmoe_import_twos(const uint8_t *twos, int64_t rows, int64_t cols, uint8_t *packed,
                     void *stream);

/* Group size of a matrix from its scale array's byte count, as the pages'
 * loader does (same pull request, quoted issue's list of CPU work,
 * detect_group_size()): the first of 16, 32, 48, 64, 96, 128, 192, 256 with
 * rows * ceil(cols / gs) * 4 == scale_bytes, or 0 when none fits.  Host
 * only; launches nothing. */
int32_t qmoe_detect_group(int64_t rows, int64_t cols, int64_t scale_bytes);

/* Expert cache: a layer whose E experts live in host memory, with a fixed
 * set of S expert slots in HBM in front of it (the VRAM tier of hot experts
 * of the colibri pull request "cuda+engine: full fmt=4 (grouped int4 gs=64)
 * support", comments on where decode wall-clock goes and on the
 * CUDA_EXPERT_GB placement curve).
 *
 * qmoe_cache_create: `host` describes the E experts (codes and scales in
 * host memory; pinned memory lets the copies run asynchronously), `dev` the
 * S slots (an ordinary device layer descriptor with experts = S, the same
 * shape and group; its memory stays the caller's).  Returns a host object in
 * *out (free it with qmoe_cache_destroy); no device work.
 *
 * qmoe_cache_prepare: for the routing ids of one call (host int32
 * [tokens][k]), keep the experts already resident, and for each missing
 * valid id pick a free slot, else the least recently used slot that neither
 * this call nor the previous prepare uses, and enqueue its six host->device
 * copies on `stream`.  Writes slot_ids (host int32 [tokens][k]): the slot of
 * each pair, -1 for ids outside [0, E).  The caller uploads slot_ids and runs
 * qmoe_layer on the slot layer `dev` with them, on `stream` or on a stream
 * that waits for it.  Because the previous call's slots are never evicted,
 * the copies for call i+1 may overlap the kernels of call i; the copies for
 * call i+2 must wait for call i's kernels.  *bytes_copied (nullable) = bytes
 * enqueued.  QMOE_ERR_SHAPE when this call's experts plus the previous call's
 * other slots exceed S.  Not thread-safe per cache object. */
typedef struct qmoe_expert_cache qmoe_expert_cache;
int qmoe_cache_create(const qmoe_layer_desc *host, const qmoe_layer_desc *dev,
                      qmoe_expert_cache **out);
void qmoe_cache_destroy(qmoe_expert_cache *cache);
int qmoe_cache_prepare(qmoe_expert_cache *cache, const int32_t *host_ids, int32_t tokens,
                       int32_t k, int32_t *slot_ids, int64_t *bytes_copied, void *stream);
/* Slot holding `expert`, or -1 (not resident or out of range). */
int32_t qmoe_cache_resident(const qmoe_expert_cache *cache, int32_t expert);

/* Device-side prepare: the same cache, deciding on the device from device
 * routing ids (as the router writes them), with no host round trip
 * (pxq_llama.cpp release notes, "Device-side MoE row map": the device builds
 * the map, no device-to-host sync).
 *
 * qmoe_cache_device_state_bytes: bytes of the caller-owned device state for
 * E experts and S slots (int32 words: tick, status, copy count, unused,
 * slot_of[E], expert_in[S], last_use[S], keep[S], copy list 2 x [S]); 0 for
 * E or S < 1.
 *
 * qmoe_cache_device_init: enqueue on `stream` the state of an empty cache
 * (no expert resident).  QMOE_ERR_UNSUPPORTED beyond 8192 experts or 1024
 * slots, QMOE_ERR_WORKSPACE when state_bytes is too small, QMOE_ERR_ALIGN
 * for a state not 4-byte aligned.
 *
 * qmoe_cache_prepare_device: for the device routing ids of one call (int32
 * [tokens][k]) enqueue on `stream` one kernel that keeps the resident experts,
 * gives each missing valid expert a slot (free slots first, then the least
 * recently used slot that neither this call nor the previous prepare uses;
 * missing experts are placed in ascending id order), updates the state and
 * writes dev_slot_ids (device int32 [tokens][k]: the slot of each pair, -1
 * for ids outside [0, E)), then a kernel that copies the placed experts' six
 * arrays from the host layer into their slots.  The host arrays must be
 * pinned host memory (QMOE_ERR_UNSUPPORTED otherwise); the GPU reads them
 * directly.  Stream rules are those of qmoe_cache_prepare: call i+1's prepare
 * may overlap call i's layer kernels, call i+2's must wait for them.  When a
 * call's experts plus the previous call's other slots exceed S, the experts
 * that found no slot keep slot id -1 (their pairs add nothing) and status
 * word 1 of the state becomes 1 (the device cannot report it synchronously;
 * read it back to check).  The state must come from qmoe_cache_device_init
 * on this cache's shape; do not mix it with qmoe_cache_prepare on one cache
 * (the two keep separate residency tables). */
size_t qmoe_cache_device_state_bytes(int32_t experts, int32_t slots);
int qmoe_cache_device_init(qmoe_expert_cache *cache, void *dev_state, size_t state_bytes,
                           void *stream);
int qmoe_cache_prepare_device(qmoe_expert_cache *cache, void *dev_state, size_t state_bytes,
                              const int32_t *dev_ids, int32_t tokens, int32_t k,
                              int32_t *dev_slot_ids, void *stream);

/* Router, the step ahead of the layer: for each token, the k experts with
 * the largest logits and their routing weights (colibri pull request
 * "cuda+engine: full fmt=4 (grouped int4 gs=64) support", the quoted issue's
 * list of CPU work: top-K with one taken flag per expert).  k passes, each
 * picking the untaken expert with the largest logit, the lowest id among
 * equal logits, NaN ranking as -infinity.  Inputs: logits f32 [tokens]
 * [experts] (device, 4-byte aligned).  Outputs (device, 4-byte aligned):
 * topk_ids int32 [tokens][k] in pick order (unique per token, bit-exact
 * against any correct implementation) and topk_w f32 [tokens][k] =
 * exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k picked logits (f32
 * arithmetic; non-finite logits give non-finite weights).  The outputs feed
 * qmoe_layer unchanged on the same stream, with no host round trip.
 * Limits: 1 <= k <= min(experts, 16), experts <= 1024 (else
 * QMOE_ERR_UNSUPPORTED); outputs may not overlap the logits or each other
 * (QMOE_ERR_ALIAS).  tokens == 0 launches nothing. */
int qmoe_route(const float *logits, int32_t tokens, int32_t experts, int32_t k,
               int32_t *topk_ids, float *topk_w, void *stream);

/* Largest number of pairs an expert may receive in a bf16 layer call and
 * still take the weight-streaming passes instead of row tiles (see
 * QMOE_BF16; 0: every expert takes tiles).  Read once per process: the
 * default, or the environment variable QMOE_PREFILL_PASS_ROWS (0 .. 256).
 * The bf16 workspace size depends on it. */
int32_t qmoe_prefill_pass_rows(void);

/* Read-stream probe, a measurement aid beside the path: reads `bytes` of
 * device memory at buf once with one of two load shapes and leaves per-block
 * sums of the dwords read (mod 2^32) in sink, so timing the call gives the
 * read rate this GPU reaches with that shape (the decode kernels' practical
 * ceiling, next to the 8 TB/s specification).
 *  - QMOE_PROBE_LINEAR: each wave instruction reads 1 KB of consecutive
 *    bytes, 16 such loads in flight per wave.
 *  - QMOE_PROBE_ROWS: rows of 2048 bytes (one 4096-input int4 row); a wave
 *    reads blocks of 16 rows x 256 consecutive bytes per row as four
 *    back-to-back 16-byte loads per lane, two blocks in flight (the weight
 *    stream of the matrix-core decode passes); bytes % 2048 == 0.
 * buf: device, 16-byte aligned, 0 < bytes <= 2^30; sink: device uint32
 * [QMOE_PROBE_SINK]; the sum of all sink entries equals the sum of the
 * buffer's dwords mod 2^32.  Errors: QMOE_ERR_NULL, QMOE_ERR_ALIGN,
 * QMOE_ERR_SHAPE, QMOE_ERR_UNSUPPORTED (other patterns), QMOE_ERR_ALIAS
 * (sink inside buf). */
enum { QMOE_PROBE_LINEAR = 0, QMOE_PROBE_ROWS = 1 };
#define QMOE_PROBE_SINK 2048
int qmoe_stream_probe(const void *buf, int64_t bytes, int32_t pattern, uint32_t *sink,
                      void *stream);

/* Workspace bytes qmoe_layer needs for these sizes and dtype. */
size_t qmoe_layer_workspace_bytes(const qmoe_layer_desc *desc, int32_t tokens,
                                  int32_t k, int32_t x_dtype);

/* The routed MoE layer:
 *   out[t] = sum_{j<k} topk_w[t][j] * ffn_{topk_ids[t][j]}(x_t)
 * x is [tokens][H] f32 (decode path) or bf16 (prefill path); topk_ids int32
 * and topk_w f32 are [tokens][k]; out is f32 [tokens][H], fully written,
 * and must not overlap x, the routing arrays or the workspace.  Routing is
 * an input: the layer does not pick experts.  Ids outside [0, E) are
 * dropped.  After the call the workspace begins with the worklist in the
 * layout of qmoe_layer_ws_view (for inspection and tests).  On the f32
 * paths an expert's tokens are taken one, two or four per weight pass; the
 * passes of one expert run side by side, so its weights come from HBM about
 * once per call and the later passes read them from the L2 cache.  With
 * QMOE_F32 and at most 64 pairs (tokens * k) the call is two kernel launches
 * (gate+up, which also groups the pairs by expert, then down); beyond that a
 * preparation kernel plans the passes once and splits x into its f16 parts
 * (three launches: faster from 128 pairs on, where every gate+up block would
 * otherwise scan all the ids), and the passes, of up to four tokens, run on
 * the matrix cores where the shapes allow (see QMOE_F32).
 * Reproducibility: the bf16 path sums each token's k expert rows in pick
 * order and gives bit-identical results from run to run; the f32 paths add
 * the k expert terms into out with f32 atomics, so their order, and the
 * last bits of out, may differ from run to run. */
int qmoe_layer(const qmoe_layer_desc *desc, int32_t x_dtype, const void *x,
               int32_t tokens, const int32_t *topk_ids, const float *topk_w,
               int32_t k, float *out, void *ws, size_t ws_bytes, void *stream);

/* The router and the layer in one call, with no host round trip: route f32
 * logits [tokens][E] with qmoe_route (top-k, softmax over the picked logits)
 * into the end of the workspace, then run qmoe_layer on those ids and
 * weights.  Workspace: qmoe_layer_logits_workspace_bytes; its first
 * qmoe_layer_workspace_bytes bytes are the layer's workspace (worklist view
 * as for qmoe_layer).  Limits are those of both calls (k <= 16, E <= 1024);
 * logits may not overlap the workspace or out. */
size_t qmoe_layer_logits_workspace_bytes(const qmoe_layer_desc *desc, int32_t tokens,
                                         int32_t k, int32_t x_dtype);
int qmoe_layer_logits(const qmoe_layer_desc *desc, int32_t x_dtype, const void *x,
                      int32_t tokens, const float *logits, int32_t k, float *out, void *ws,
                      size_t ws_bytes, void *stream);

/* qmoe_layer with phase markers: when phase_events is non-NULL it holds
 * n_events hipEvent_t handles (passed as void*, created by the caller) and the
 * call records events[0] before its first kernel and events[i] after phase i
 * on `stream`.  Phases: f32 paths 1 = worklist (+ activation digits for
 * QMOE_F32_DIGITS; for QMOE_F32 with at most 64 pairs the gate+up launch
 * builds the worklist itself and phase 1 is empty), 2 = gate+up, 3 = down and
 * combine (n_events >= 4); bf16 path 1 = worklist + activation prep,
 * 2 = gate+up, 3 = down, 4 = combine (n_events >= 5).  Fewer events =
 * QMOE_ERR_SHAPE.
 * Recording an event allocates nothing and does not synchronise.  This is
 * the per-launch event timing the maintainer asks for in the pull request
 * (data request: elapsed time around one launch per shape). */
int qmoe_layer_ex(const qmoe_layer_desc *desc, int32_t x_dtype, const void *x,
                  int32_t tokens, const int32_t *topk_ids, const float *topk_w,
                  int32_t k, float *out, void *ws, size_t ws_bytes, void *stream,
                  void *const *phase_events, int32_t n_events);

/* Byte offsets, inside a qmoe_layer workspace, of the worklist arrays the
 * call leaves behind (counts, offsets, pairs, inv, n_invalid). */
typedef struct qmoe_layer_ws_view {
    uint32_t struct_size;
    int64_t counts, offsets, pairs, inv, n_invalid;
} qmoe_layer_ws_view;
int qmoe_layer_ws_layout(const qmoe_layer_desc *desc, int32_t tokens,
                         int32_t k, int32_t x_dtype, qmoe_layer_ws_view *view);

/* Allocation-free variant of qmoe_layer, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and checks as
 * qmoe_layer, without ws/ws_bytes: the workspace is a fixed device array of
 * QMOE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  The call runs on the current device; its first call on a
 * device looks up that device's array (no allocation), later calls reuse it.
 * Nothing is allocated or freed and nothing in the array needs to start at
 * zero.  A call whose qmoe_layer_workspace_bytes exceeds the array returns
 * QMOE_ERR_SCRATCH and launches nothing (at hidden 4096, intermediate 1536
 * and top-8, the 64 MiB hold the f32 path up to 674 tokens, the digits
 * variant up to 1,546 and the bf16 path up to 668 tokens).  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one
 * GPU (different streams, or different host threads without ordering) race
 * and give wrong results; calls serialised on one stream are safe.  After a
 * call the array begins with the worklist in the layout of
 * qmoe_layer_ws_layout, as a qmoe_layer workspace does. */
#define QMOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int qmoe_layer_noalloc(const qmoe_layer_desc *desc, int32_t x_dtype, const void *x,
                       int32_t tokens, const int32_t *topk_ids, const float *topk_w,
                       int32_t k, float *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QMOE_H */
