// Dispatch of the MFMA decode-attention kernels (kernel template in decode_mfma.h).
#include "kvq_internal.h"

namespace kvq {

hipError_t launch_decode_mfma_g1(kvq_cache*, int, const void*, int, float, float*, int, const DecodeScratch&,
                                 const DecodeAppend&, hipStream_t);
hipError_t launch_decode_mfma_g2(kvq_cache*, int, const void*, int, float, float*, int, const DecodeScratch&,
                                 const DecodeAppend&, hipStream_t);
hipError_t launch_decode_mfma_g4(kvq_cache*, int, const void*, int, float, float*, int, const DecodeScratch&,
                                 const DecodeAppend&, hipStream_t);
hipError_t launch_decode_mfma_g8(kvq_cache*, int, const void*, int, float, float*, int, const DecodeScratch&,
                                 const DecodeAppend&, hipStream_t);

int auto_splits_mfma(const kvq_cache* c, int64_t len, int n_extra) {
  // one workgroup per compute unit over (splits x KV heads x sequences), counting the n_extra
  // recent-window workgroups per unit, and at least one 128-token tile per wave; `len` packed
  // positions (none: no packed split)
  if (len <= 0) return 0;
  const int64_t n_tiles = (len + kVTile - 1) / kVTile;
  const int64_t units = static_cast<int64_t>(c->cfg.batch) * c->cfg.n_kv_heads;
  const int W = decode_waves(c);
  int64_t S = (n_tiles + W - 1) / W;
  const int64_t want = (c->n_cu + units - 1) / units - n_extra;
  if (S > want) S = want;
  if (S > c->max_splits) S = c->max_splits;
  if (S < 1) S = 1;
  const int64_t tps = (n_tiles + S - 1) / S;
  S = (n_tiles + tps - 1) / tps;
  return static_cast<int>(S);
}

hipError_t launch_decode_mfma(kvq_cache* c, int layer, const void* q, int dtype, float scale,
                              float* out, int n_splits, const DecodeScratch& ws, const DecodeAppend& app,
                              hipStream_t stream) {
  const float kLog2e = 1.4426950408889634f;
  const float sigma = (scale > 0.0f ? scale : 0.08838834764831845f) * kLog2e;
  const int q_f32 = dtype == KVQ_F32;
  switch (c->group) {
    case 1: return launch_decode_mfma_g1(c, layer, q, q_f32, sigma, out, n_splits, ws, app, stream);
    case 2: return launch_decode_mfma_g2(c, layer, q, q_f32, sigma, out, n_splits, ws, app, stream);
    case 4: return launch_decode_mfma_g4(c, layer, q, q_f32, sigma, out, n_splits, ws, app, stream);
    default: return launch_decode_mfma_g8(c, layer, q, q_f32, sigma, out, n_splits, ws, app, stream);
  }
}

}  // namespace kvq
