// Rotate + quantize for Kronecker rotations n = 64 * m (dense m x m factor).
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {

bool rq_kron_supported(const RotArgs &, int) { return false; }

hipError_t launch_rq_kron(const void *, int64_t, int64_t, const RotArgs &, int, uint8_t *, float *,
                          hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace qr
