// Entry points declared in w4.h whose kernels are not built yet.
#include "w4.h"
extern "C" {
int w4_gemv_chain(const uint32_t *const *, const uint16_t *const *, const int32_t *,
                  const int32_t *, int32_t, const uint16_t *, float *const *, void *, void *) {
    return W4_ERR_UNSUPPORTED;
}
}
