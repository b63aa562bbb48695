// qmoe_layer_noalloc: the routed MoE layer for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The layer's workspace lives in a fixed-size
// file-scope device array instead of a caller buffer.
//
// Host code never passes the array's name to a kernel (on the host that name
// is a stand-in, not a device address): the device address is looked up once
// per device with hipGetSymbolAddress, with that device current, on the
// first call there, and only that address is used afterwards.
#include <mutex>

#include "../../include/qmoe.h"
#include "launch.h"

namespace {

static __device__ __align__(256) unsigned char scratch[QMOE_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_ptr[MAX_DEVICES];    // device address of `scratch`, per device

// Device address of this device's copy of `scratch` (nullptr on failure).
void *scratch_ptr(int dev) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" int qmoe_layer_noalloc(const qmoe_layer_desc *desc, int32_t x_dtype, const void *x,
                                  int32_t tokens, const int32_t *topk_ids, const float *topk_w,
                                  int32_t k, float *out, void *stream) {
    if (!desc) return QMOE_ERR_NULL;
    if (desc->struct_size != sizeof(qmoe_layer_desc)) return QMOE_ERR_ABI;
    if (tokens < 0 || k < 1) return QMOE_ERR_SHAPE;
    if (x_dtype != QMOE_F32 && x_dtype != QMOE_BF16 && x_dtype != QMOE_F32_DIGITS)
        return QMOE_ERR_UNSUPPORTED;
    const size_t need = qmoe_layer_workspace_bytes(desc, tokens, k, x_dtype);
    if (need > (size_t)QMOE_NOALLOC_SCRATCH_BYTES) return QMOE_ERR_SCRATCH;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return QMOE_ERR_HIP;
    void *ws = scratch_ptr(dev);
    if (!ws) return QMOE_ERR_HIP;
    return qmoe_layer(desc, x_dtype, x, tokens, topk_ids, topk_w, k, out, ws,
                      (size_t)QMOE_NOALLOC_SCRATCH_BYTES, stream);
}
