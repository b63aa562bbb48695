// Group-32 instance of the prefill gate+up kernel (mfma_gateup.h), compiled
// on its own so the two instances build in parallel.
#include "mfma_gateup.h"

namespace qmoe {

hipError_t launch_gateup_g32(const QMat &gate, const QMat &up, const uint16_t *x16,
                             const float *xinv, uint16_t *h16, const MfmaRoute &r, hipStream_t st) {
    return launch_gateup<true>(gate, up, x16, xinv, h16, r, st);
}

}  // namespace qmoe
