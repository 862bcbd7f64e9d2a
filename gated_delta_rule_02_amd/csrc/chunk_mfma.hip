// chunk_mfma.hip -- placeholder: the matrix-core kernel is not written yet; the
// fp32 kernels serve this configuration meanwhile.
#include "gdn_launch.h"

namespace gdn {
hipError_t launch_chunk_mfma(const Shape &sh, const void *q, const void *k, const void *v,
                             const void *g, const void *beta, const float *S0, float *o, float *ST,
                             hipStream_t s) {
  return launch_chunk_f32(sh, q, k, v, g, beta, S0, o, ST, s);
}
}  // namespace gdn
