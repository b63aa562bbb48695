// Expert cache: experts resident in host memory, only the routed ones copied
// into a fixed set of HBM slots before a layer call.
//
// The pages measure decode as expert-loading bound (colibri pull request
// "cuda+engine: full fmt=4 (grouped int4 gs=64) support", comment on where
// decode wall-clock goes: expert-disk wait 71-77 %) and describe a VRAM tier
// of hot experts in front of host memory (the CUDA_EXPERT_GB placement
// curve).  This is that tier for one layer on MI355X: the caller owns a
// pinned host copy of all E experts and a device layer of S slots; prepare()
// looks at the host routing ids of one call, keeps experts that are already
// resident, copies each missing one (six host->device copies on the given
// stream: gate, up, down codes and scales) into a free or least recently used
// slot, and writes the routing ids translated to slot ids.  The slots the
// previous prepare() used are not evicted, so the copies for call i+1 may run
// on a copy stream while the kernels of call i still read their slots.
//
// Two ways to prepare a call.  qmoe_cache_prepare decides on the host from
// host routing ids and enqueues DMA copies.  qmoe_cache_prepare_device takes
// the routing ids in device memory (as the router writes them) and decides on
// the device, with no host round trip (pxq_llama.cpp release notes,
// "Device-side MoE row map": a host-built map and its device-to-host sync
// cap the pipelining win): one single-block kernel keeps the residency
// tables in a caller-owned device state, picks the slots of the missing
// experts (free ones first, then least recently used, never one this call or
// the previous prepare uses) and writes the slot ids; a second kernel pulls
// the missing experts' bytes from the pinned host copy (mapped into the GPU's
// address space) into their slots.  Both enqueue on the given stream.
//
// The object is plain host memory; the device memory (slots, device state)
// belongs to the caller.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/qmoe.h"
#include "common.h"

struct qmoe_expert_cache {
    qmoe_layer_desc host, dev;
    int experts = 0, slots = 0;
    std::vector<int> slot_of;        // [experts] -> slot, -1 if not resident
    std::vector<int> expert_in;      // [slots] -> expert, -1 if free
    std::vector<uint64_t> last_use;  // [slots] tick of the last prepare that used it
    std::vector<char> keep;          // [slots] used by the previous prepare
    uint64_t tick = 0;
    // device-visible addresses of the six host arrays (0 until looked up)
    const void *hsrc[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
    bool hsrc_ok = false;
};

namespace {

int64_t packed_bytes(int64_t rows, int64_t cols) { return rows * ((cols + 1) / 2); }
int64_t scale_bytes(int64_t rows, int64_t cols, int64_t g) {
    return 4 * rows * ((cols + g - 1) / g);
}

bool same_shape(const qmoe_qmat &a, const qmoe_qmat &b) {
    return a.rows == b.rows && a.cols == b.cols && a.group == b.group;
}

// Host-side matrix stack: positive shape, pointers set, strides large enough.
int check_host_qmat(const qmoe_qmat &m, int experts) {
    if (m.struct_size != sizeof(qmoe_qmat)) return QMOE_ERR_ABI;
    if (m.rows <= 0 || m.cols <= 0 || m.group <= 0) return QMOE_ERR_SHAPE;
    if (!m.q || !m.s) return QMOE_ERR_NULL;
    if (experts > 1 && (m.q_expert_stride < packed_bytes(m.rows, m.cols) ||
                        4 * m.s_expert_stride < scale_bytes(m.rows, m.cols, m.group)))
        return QMOE_ERR_SHAPE;
    return QMOE_OK;
}

hipError_t copy_expert(const qmoe_expert_cache &c, int e, int slot, hipStream_t st,
                       int64_t &bytes) {
    const qmoe_qmat *hm[3] = {&c.host.gate, &c.host.up, &c.host.down};
    const qmoe_qmat *dm[3] = {&c.dev.gate, &c.dev.up, &c.dev.down};
    for (int i = 0; i < 3; i++) {
        const qmoe_qmat &h = *hm[i], &d = *dm[i];
        const int64_t qb = packed_bytes(h.rows, h.cols), sb = scale_bytes(h.rows, h.cols, h.group);
        hipError_t err = hipMemcpyAsync(const_cast<uint8_t *>(d.q) + slot * d.q_expert_stride,
                                        h.q + e * h.q_expert_stride, qb, hipMemcpyHostToDevice, st);
        if (err != hipSuccess) return err;
        err = hipMemcpyAsync(const_cast<float *>(d.s) + slot * d.s_expert_stride,
                             h.s + e * h.s_expert_stride, sb, hipMemcpyHostToDevice, st);
        if (err != hipSuccess) return err;
        bytes += qb + sb;
    }
    return hipSuccess;
}

}  // namespace

namespace {

// Device state of the device-side prepare, in int32 words:
//   [0] tick, [1] status (0, or 1 once a call's experts did not fit),
//   [2] number of experts the last prepare copies, [3] unused,
//   slot_of[E], expert_in[S], last_use[S], keep[S], copy_e[S], copy_s[S].
constexpr int CACHE_HEAD = 4;
constexpr int CACHE_MAX_SLOTS = 1024;
constexpr int CACHE_MAX_EXPERTS = 8192;
constexpr int CACHE_PLAN_THREADS = 1024;

struct DevState {
    int *head, *slot_of, *expert_in, *last_use, *keep, *copy_e, *copy_s;
};
__host__ __device__ inline DevState dev_state(void *base, int E, int S) {
    int *w = static_cast<int *>(base);
    DevState d;
    d.head = w;
    d.slot_of = w + CACHE_HEAD;
    d.expert_in = d.slot_of + E;
    d.last_use = d.expert_in + S;
    d.keep = d.last_use + S;
    d.copy_e = d.keep + S;
    d.copy_s = d.copy_e + S;
    return d;
}
__host__ __device__ inline size_t dev_state_words(int E, int S) { return (size_t)CACHE_HEAD + E + 5 * (size_t)S; }

__global__ void __launch_bounds__(256) cache_init_kernel(int *w, int E, int S) {
    const DevState d = dev_state(w, E, S);
    const int n = (int)dev_state_words(E, S);
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
        int v = 0;
        if (i >= CACHE_HEAD && i < CACHE_HEAD + E + S) v = -1;   // slot_of, expert_in
        w[i] = v;
    }
    (void)d;
}

// One block: the residency decision for one call and the routed slot ids.
__global__ void __launch_bounds__(CACHE_PLAN_THREADS)
    cache_plan_kernel(int *w, const int32_t *__restrict__ ids, int n, int E, int S,
                      int32_t *__restrict__ slot_ids) {
    __shared__ unsigned char need[CACHE_MAX_EXPERTS];
    __shared__ unsigned char used[CACHE_MAX_SLOTS];
    __shared__ unsigned long long key[CACHE_MAX_SLOTS];
    __shared__ int missing[CACHE_MAX_SLOTS];
    __shared__ int part[CACHE_PLAN_THREADS];
    __shared__ int n_missing_s, n_cand_s;
    const DevState d = dev_state(w, E, S);
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += CACHE_PLAN_THREADS) need[e] = 0;
    for (int s = tid; s < CACHE_MAX_SLOTS; s += CACHE_PLAN_THREADS) used[s] = 0;
    if (tid == 0) n_cand_s = 0;
    __syncthreads();
    for (int p = tid; p < n; p += CACHE_PLAN_THREADS) {
        const int e = ids[p];
        if (e >= 0 && e < E) need[e] = 1;
    }
    __syncthreads();
    // resident experts of this call keep their slots; the others are missing,
    // listed in ascending expert order (a block scan over expert ranges)
    const int per = (E + CACHE_PLAN_THREADS - 1) / CACHE_PLAN_THREADS;
    const int e0 = tid * per, e1 = min(E, e0 + per);
    int cnt = 0;
    for (int e = e0; e < e1; e++) {
        if (!need[e]) continue;
        const int sl = d.slot_of[e];
        if (sl >= 0 && sl < S) used[sl] = 1;
        else cnt++;
    }
    part[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < CACHE_PLAN_THREADS; off <<= 1) {   // inclusive scan
        const int v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int pos = part[tid] - cnt;
    if (tid == CACHE_PLAN_THREADS - 1) n_missing_s = part[tid];
    for (int e = e0; e < e1; e++)
        if (need[e] && !(d.slot_of[e] >= 0 && d.slot_of[e] < S)) {
            if (pos < CACHE_MAX_SLOTS) missing[pos] = e;
            pos++;
        }
    __syncthreads();
    // candidate slots, oldest first: free (key 0), else by last use; slots of
    // this call or of the previous prepare are not candidates
    for (int s = tid; s < CACHE_MAX_SLOTS; s += CACHE_PLAN_THREADS) {
        unsigned long long k = ~0ull;
        if (s < S && !used[s] && !d.keep[s]) {
            const unsigned last = (unsigned)d.last_use[s];
            const unsigned long long age =
                d.expert_in[s] < 0 ? 0ull : (unsigned long long)min(last, 0xfffffffdu) + 1ull;
            k = (age << 32) | (unsigned)s;
            atomicAdd(&n_cand_s, 1);
        }
        key[s] = k;
    }
    __syncthreads();
    for (int size = 2; size <= CACHE_MAX_SLOTS; size <<= 1)          // bitonic sort
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < CACHE_MAX_SLOTS; i += CACHE_PLAN_THREADS) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool up = (i & size) == 0;
                    const unsigned long long a = key[i], b = key[j];
                    if ((a > b) == up) {
                        key[i] = b;
                        key[j] = a;
                    }
                }
            }
            __syncthreads();
        }
    const int nm = n_missing_s, nc = n_cand_s;
    const int placed = min(nm, nc);
    for (int i = tid; i < placed; i += CACHE_PLAN_THREADS) {
        const int s = (int)(key[i] & 0xffffffffu), e = missing[i];
        const int old = d.expert_in[s];
        if (old >= 0 && old < E) d.slot_of[old] = -1;
        d.expert_in[s] = e;
        d.slot_of[e] = s;
        d.copy_e[i] = e;
        d.copy_s[i] = s;
        used[s] = 1;
    }
    __syncthreads();
    const int tick = d.head[0] + 1;
    for (int s = tid; s < S; s += CACHE_PLAN_THREADS) {
        if (used[s]) d.last_use[s] = tick;
        d.keep[s] = used[s];
    }
    if (tid == 0) {
        d.head[0] = tick;
        if (nm > nc) d.head[1] = 1;
        d.head[2] = placed;
    }
    __syncthreads();
    for (int p = tid; p < n; p += CACHE_PLAN_THREADS) {
        const int e = ids[p];
        slot_ids[p] = (e >= 0 && e < E) ? d.slot_of[e] : -1;
    }
}

// The byte ranges of the six arrays of one expert, host source and slot
// destination.  Block (x, i) copies chunk x of copy list entry i (blocks past
// the list's length, written by the plan kernel, exit).
struct CopyArrays {
    const uint8_t *src[6];
    uint8_t *dst[6];
    int64_t src_stride[6], dst_stride[6];   // bytes between experts / slots
    int64_t bytes[6];
    int64_t first_chunk[7];                 // prefix sums of the chunk counts
    int vec;                                // all bases, strides, sizes 16-byte aligned
};
constexpr int CACHE_CHUNK = 16384;

__global__ void __launch_bounds__(256) cache_copy_kernel(const int *w, int E, int S, CopyArrays a) {
    const DevState d = dev_state(const_cast<int *>(w), E, S);
    const int i = blockIdx.y;
    if (i >= d.head[2]) return;
    const int e = d.copy_e[i], s = d.copy_s[i];
    const int64_t cx = blockIdx.x;
    int arr = 0;
    while (arr < 5 && cx >= a.first_chunk[arr + 1]) arr++;
    const int64_t off = (cx - a.first_chunk[arr]) * CACHE_CHUNK;
    const int64_t len = min((int64_t)CACHE_CHUNK, a.bytes[arr] - off);
    if (len <= 0) return;
    const uint8_t *src = a.src[arr] + e * a.src_stride[arr] + off;
    uint8_t *dst = a.dst[arr] + s * a.dst_stride[arr] + off;
    if (a.vec) {
        for (int64_t b = (int64_t)threadIdx.x * 16; b < len; b += 256 * 16)
            *(qmoe::u32x4 *)(dst + b) = *(const qmoe::u32x4 *)(src + b);
    } else {
        for (int64_t b = threadIdx.x; b < len; b += 256) dst[b] = src[b];
    }
}

}  // namespace

extern "C" {

int qmoe_cache_create(const qmoe_layer_desc *host, const qmoe_layer_desc *dev,
                      qmoe_expert_cache **out) {
    if (!host || !dev || !out) return QMOE_ERR_NULL;
    *out = nullptr;
    if (host->struct_size != sizeof(qmoe_layer_desc) || dev->struct_size != sizeof(qmoe_layer_desc))
        return QMOE_ERR_ABI;
    if (host->experts < 1 || dev->experts < 1 || host->hidden != dev->hidden ||
        host->inter != dev->inter || host->group != dev->group)
        return QMOE_ERR_SHAPE;
    if (!same_shape(host->gate, dev->gate) || !same_shape(host->up, dev->up) ||
        !same_shape(host->down, dev->down))
        return QMOE_ERR_SHAPE;
    int s;
    if ((s = check_host_qmat(host->gate, host->experts))) return s;
    if ((s = check_host_qmat(host->up, host->experts))) return s;
    if ((s = check_host_qmat(host->down, host->experts))) return s;
    // the slots are an ordinary device layer: qmoe_layer validates it fully
    if ((s = check_host_qmat(dev->gate, dev->experts))) return s;
    if ((s = check_host_qmat(dev->up, dev->experts))) return s;
    if ((s = check_host_qmat(dev->down, dev->experts))) return s;
    auto *c = new (std::nothrow) qmoe_expert_cache();
    if (!c) return QMOE_ERR_HIP;
    c->host = *host;
    c->dev = *dev;
    c->experts = host->experts;
    c->slots = dev->experts;
    c->slot_of.assign(c->experts, -1);
    c->expert_in.assign(c->slots, -1);
    c->last_use.assign(c->slots, 0);
    c->keep.assign(c->slots, 0);
    *out = c;
    return QMOE_OK;
}

void qmoe_cache_destroy(qmoe_expert_cache *c) { delete c; }

int qmoe_cache_prepare(qmoe_expert_cache *c, const int32_t *host_ids, int32_t tokens, int32_t k,
                       int32_t *slot_ids, int64_t *bytes_copied, void *stream) {
    if (!c) return QMOE_ERR_NULL;
    if (tokens < 0 || k < 1) return QMOE_ERR_SHAPE;
    const int64_t n = (int64_t)tokens * k;
    if (n > 0 && (!host_ids || !slot_ids)) return QMOE_ERR_NULL;
    // experts this call needs (first appearance order) and whether they fit:
    // the slots of the previous call stay, so need + kept-but-unneeded <= slots
    std::vector<char> need(c->experts, 0);
    std::vector<int> order;
    for (int64_t p = 0; p < n; p++) {
        const int e = host_ids[p];
        if (e >= 0 && e < c->experts && !need[e]) {
            need[e] = 1;
            order.push_back(e);
        }
    }
    int kept_other = 0;
    for (int sl = 0; sl < c->slots; sl++)
        if (c->keep[sl] && !(c->expert_in[sl] >= 0 && need[c->expert_in[sl]])) kept_other++;
    if ((int64_t)order.size() + kept_other > c->slots) return QMOE_ERR_SHAPE;

    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const uint64_t now = ++c->tick;
    std::vector<char> used(c->slots, 0);
    for (int e : order)
        if (c->slot_of[e] >= 0) used[c->slot_of[e]] = 1;
    int64_t bytes = 0;
    for (int e : order) {
        int sl = c->slot_of[e];
        if (sl < 0) {
            // a free slot, else the least recently used one that neither this
            // call nor the previous one uses
            int best = -1;
            for (int i = 0; i < c->slots; i++) {
                if (used[i] || c->keep[i]) continue;
                if (c->expert_in[i] < 0) {
                    best = i;
                    break;
                }
                if (best < 0 || c->last_use[i] < c->last_use[best]) best = i;
            }
            if (best < 0) return QMOE_ERR_SHAPE;   // excluded by the count above
            sl = best;
            if (c->expert_in[sl] >= 0) c->slot_of[c->expert_in[sl]] = -1;
            c->expert_in[sl] = e;
            c->slot_of[e] = sl;
            if (copy_expert(*c, e, sl, st, bytes) != hipSuccess) {
                c->slot_of[e] = -1;   // contents unknown: forget the slot
                c->expert_in[sl] = -1;
                return QMOE_ERR_HIP;
            }
        }
        used[sl] = 1;
        c->last_use[sl] = now;
    }
    for (int64_t p = 0; p < n; p++) {
        const int e = host_ids[p];
        slot_ids[p] = (e >= 0 && e < c->experts) ? c->slot_of[e] : -1;
    }
    for (int i = 0; i < c->slots; i++) c->keep[i] = used[i];
    if (bytes_copied) *bytes_copied = bytes;
    return QMOE_OK;
}

size_t qmoe_cache_device_state_bytes(int32_t experts, int32_t slots) {
    if (experts < 1 || slots < 1) return 0;
    return dev_state_words(experts, slots) * sizeof(int32_t);
}

int qmoe_cache_device_init(qmoe_expert_cache *c, void *dev_state, size_t state_bytes,
                           void *stream) {
    if (!c || !dev_state) return QMOE_ERR_NULL;
    if (c->experts > CACHE_MAX_EXPERTS || c->slots > CACHE_MAX_SLOTS) return QMOE_ERR_UNSUPPORTED;
    if (state_bytes < qmoe_cache_device_state_bytes(c->experts, c->slots)) return QMOE_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(dev_state) % 4) return QMOE_ERR_ALIGN;
    hipLaunchKernelGGL(cache_init_kernel, dim3(64), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<int *>(dev_state),
                       c->experts, c->slots);
    return hipGetLastError() == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}

int qmoe_cache_prepare_device(qmoe_expert_cache *c, void *dev_state, size_t state_bytes,
                              const int32_t *dev_ids, int32_t tokens, int32_t k,
                              int32_t *dev_slot_ids, void *stream) {
    if (!c || !dev_state) return QMOE_ERR_NULL;
    if (tokens < 0 || k < 1) return QMOE_ERR_SHAPE;
    const int64_t n = (int64_t)tokens * k;
    if (n > 0 && (!dev_ids || !dev_slot_ids)) return QMOE_ERR_NULL;
    if (n > INT32_MAX) return QMOE_ERR_SHAPE;
    if (c->experts > CACHE_MAX_EXPERTS || c->slots > CACHE_MAX_SLOTS) return QMOE_ERR_UNSUPPORTED;
    if (state_bytes < qmoe_cache_device_state_bytes(c->experts, c->slots)) return QMOE_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(dev_state) % 4) return QMOE_ERR_ALIGN;
    const qmoe_qmat *hm[3] = {&c->host.gate, &c->host.up, &c->host.down};
    const qmoe_qmat *dm[3] = {&c->dev.gate, &c->dev.up, &c->dev.down};
    if (!c->hsrc_ok) {
        // the host arrays must be pinned (mapped into the GPU's address space)
        for (int m = 0; m < 3; m++) {
            const void *h[2] = {hm[m]->q, hm[m]->s};
            for (int j = 0; j < 2; j++) {
                void *dp = nullptr;
                if (hipHostGetDevicePointer(&dp, const_cast<void *>(h[j]), 0) != hipSuccess || !dp) {
                    (void)hipGetLastError();
                    return QMOE_ERR_UNSUPPORTED;
                }
                c->hsrc[2 * m + j] = dp;
            }
        }
        c->hsrc_ok = true;
    }
    CopyArrays a{};
    bool vec = true;
    int64_t chunks = 0;
    for (int m = 0; m < 3; m++) {
        const qmoe_qmat &h = *hm[m], &d = *dm[m];
        const int64_t b[2] = {packed_bytes(h.rows, h.cols), scale_bytes(h.rows, h.cols, h.group)};
        const int64_t hs[2] = {h.q_expert_stride, 4 * h.s_expert_stride};
        const int64_t ds[2] = {d.q_expert_stride, 4 * d.s_expert_stride};
        uint8_t *dd[2] = {const_cast<uint8_t *>(d.q), reinterpret_cast<uint8_t *>(const_cast<float *>(d.s))};
        for (int j = 0; j < 2; j++) {
            const int i = 2 * m + j;
            a.src[i] = static_cast<const uint8_t *>(c->hsrc[i]);
            a.dst[i] = dd[j];
            a.src_stride[i] = hs[j];
            a.dst_stride[i] = ds[j];
            a.bytes[i] = b[j];
            a.first_chunk[i] = chunks;
            chunks += (b[j] + CACHE_CHUNK - 1) / CACHE_CHUNK;
            vec = vec && reinterpret_cast<uintptr_t>(a.src[i]) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(a.dst[i]) % 16 == 0 && hs[j] % 16 == 0 &&
                  ds[j] % 16 == 0 && b[j] % 16 == 0;
        }
    }
    a.first_chunk[6] = chunks;
    a.vec = vec ? 1 : 0;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    int *w = static_cast<int *>(dev_state);
    if (n > 0) {
        hipLaunchKernelGGL(cache_plan_kernel, dim3(1), dim3(CACHE_PLAN_THREADS), 0, st, w,
                           dev_ids, (int)n, c->experts, c->slots, dev_slot_ids);
        // at most min(n, S) experts are copied; the plan kernel writes how many
        const int64_t maxc = n < c->slots ? n : c->slots;
        hipLaunchKernelGGL(cache_copy_kernel, dim3((unsigned)chunks, (unsigned)maxc), dim3(256), 0,
                           st, w, c->experts, c->slots, a);
    }
    return hipGetLastError() == hipSuccess ? QMOE_OK : QMOE_ERR_HIP;
}

int32_t qmoe_cache_resident(const qmoe_expert_cache *c, int32_t expert) {
    if (!c || expert < 0 || expert >= c->experts) return -1;
    return c->slot_of[expert];
}

}  // extern "C"
