// Decode attention that allocates nothing: the split partials, maxima words and tag bases of
// a call live in a fixed device array of this library instead of the cache's buffers, so the
// call makes no allocation of any kind (for callers under stream capture, in tight serving
// loops, or in harnesses that forbid allocation).  Same kernels and results as
// kvq_decode_attn_splits.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "kvq_internal.h"

constexpr int64_t kScratchBytes = int64_t(8) << 20;   // 8 MiB per device, held until the process ends

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on each device (host code must never use the symbol itself).
unsigned char* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

hipError_t scratch_of_current_device(unsigned char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<unsigned char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Zero n 32-bit words (a kernel, not a memset: it stays an ordinary kernel node under capture).
__global__ __launch_bounds__(256) void zero_words(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0u;
}

}  // namespace

extern "C" {

kvq_status kvq_decode_attn_noalloc(kvq_cache* c, int32_t layer, const void* q, int32_t dtype,
                                   float softmax_scale, float* out, kvq_stream stream) {
  using kvq::kVTile;
  if (!c || layer < 0 || layer >= c->cfg.n_layers || !q || !out) return KVQ_EINVAL;
  if (dtype != KVQ_F16 && dtype != KVQ_F32) return KVQ_EINVAL;
  if (reinterpret_cast<uintptr_t>(q) % 4 || reinterpret_cast<uintptr_t>(out) % 16) return KVQ_EINVAL;
  if (!(softmax_scale == softmax_scale)) return KVQ_EINVAL;
  if (!c->plan_ready[layer] || c->len[layer] == 0) return KVQ_ESTATE;
  const int64_t plen = kvq::packed_len(c, layer);
  const int64_t nb = c->len[layer] - plen;
  const int n_rwg = static_cast<int>((nb + kVTile - 1) / kVTile);
  const int S = plen == 0 ? 0 : kvq::auto_splits_mfma(c, plen, n_rwg);
  const int S_all = S + n_rwg;
  if (S_all > 256) return KVQ_EINVAL;
  // scratch: outputs [units][S][G][128] fp32, sums [units][S][G] fp32, maxima words
  // [units][S][G] (8 B), tag bases [units]; each part 256-byte aligned
  const int64_t units = static_cast<int64_t>(c->cfg.batch) * c->cfg.n_kv_heads;
  const int64_t G = c->group;
  auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
  const int64_t o_bytes = up(units * S_all * G * kvq::kHeadDim * 4), l_bytes = up(units * S_all * G * 4);
  const int64_t mt_bytes = up(units * S_all * G * 8), ep_bytes = up(units * 4);
  const int64_t need = o_bytes + l_bytes + mt_bytes + ep_bytes;
  if (need > kScratchBytes) {
    kvq::set_last_error("decode_attn_noalloc: needs " + std::to_string(need) +
                        " bytes of split scratch, more than the " + std::to_string(kScratchBytes) + " it has");
    return KVQ_EINVAL;
  }
  unsigned char* base = nullptr;
  hipError_t e = scratch_of_current_device(&base);
  if (e != hipSuccess) {
    kvq::set_last_error(std::string("decode_attn_noalloc: scratch address: ") + hipGetErrorString(e));
    return KVQ_EHIP;
  }
  float* so = reinterpret_cast<float*>(base);
  float* sl = reinterpret_cast<float*>(base + o_bytes);
  uint64_t* smt = reinterpret_cast<uint64_t*>(base + o_bytes + l_bytes);
  unsigned* sep = reinterpret_cast<unsigned*>(base + o_bytes + l_bytes + mt_bytes);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the array keeps the last call's contents: the maxima words and tag bases start at zero, so
  // no word of an earlier call carries this call's tag (tag base 0 -> tag 1)
  // (one split per unit: nothing is merged, nothing to clear)
  if (S_all > 1) {
    const int64_t zero_n = (mt_bytes + ep_bytes) / 4;
    int zb = static_cast<int>((zero_n + 255) / 256);
    if (zb > 1024) zb = 1024;
    hipLaunchKernelGGL(zero_words, dim3(zb), dim3(256), 0, s, reinterpret_cast<uint32_t*>(smt), zero_n);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    const kvq::DecodeScratch ws{so, sl, smt, sep, c->dev_status, c->merge_polls};
    e = kvq::launch_decode_mfma(c, layer, q, dtype, softmax_scale, out, S, ws,
                                 kvq::DecodeAppend{nullptr, nullptr, -1}, s);
  }
  if (e != hipSuccess) {
    kvq::set_last_error(std::string("decode_attn_noalloc launch: ") + hipGetErrorString(e));
    return KVQ_EHIP;
  }
  return KVQ_OK;
}

}  // extern "C"
