// MFMA decode attention, instantiation for 8 query head(s) per KV head.
#include "decode_mfma.h"

namespace kvq {
hipError_t launch_decode_mfma_g8(kvq_cache* c, int layer, const void* q, int q_f32, float sigma,
                                 float* out, int S, hipStream_t stream) {
  return mfma::launch_group<8>(c, layer, q, q_f32, sigma, out, S, stream);
}
}  // namespace kvq
