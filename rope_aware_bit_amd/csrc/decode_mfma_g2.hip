// MFMA decode attention, instantiation for 2 query head(s) per KV head.
#include "decode_mfma.h"

namespace kvq {
hipError_t launch_decode_mfma_g2(kvq_cache* c, int layer, const void* q, int q_f32, float sigma,
                                 float* out, int S, const DecodeScratch& ws, const DecodeAppend& app,
                                 hipStream_t stream) {
  return mfma::launch_group<2>(c, layer, q, q_f32, sigma, out, S, ws, app, stream);
}
}  // namespace kvq
