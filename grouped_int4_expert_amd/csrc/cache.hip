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
// Host logic only; nothing here runs on the GPU.  The object is plain host
// memory; the device memory (slots) belongs to the caller.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/qmoe.h"

struct qmoe_expert_cache {
    qmoe_layer_desc host, dev;
    int experts = 0, slots = 0;
    std::vector<int> slot_of;        // [experts] -> slot, -1 if not resident
    std::vector<int> expert_in;      // [slots] -> expert, -1 if free
    std::vector<uint64_t> last_use;  // [slots] tick of the last prepare that used it
    std::vector<char> keep;          // [slots] used by the previous prepare
    uint64_t tick = 0;
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

int32_t qmoe_cache_resident(const qmoe_expert_cache *c, int32_t expert) {
    if (!c || expert < 0 || expert >= c->experts) return -1;
    return c->slot_of[expert];
}

}  // extern "C"
