// Streaming-read probe: the per-launch HBM read ceiling that the decode kernel's effective rate
// is compared against.  Not a step of the method; a measurement aid.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace {

// Every 16-byte piece of src is read exactly once (grid-stride, eight loads in flight per
// thread); the XOR of all pieces decides one conditional store per workgroup, so no load is dead.
__global__ __launch_bounds__(256) void stream_read(const uint4* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  uint32_t acc = 0u;
  int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = src[i + k * stride];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" kvq_status kvq_probe_stream_read(const void* src, int64_t nbytes, int32_t n_blocks, uint32_t* sink,
                                            kvq_stream stream) {
  if (!src || !sink || nbytes < 16 || nbytes % 16 || n_blocks < 1 || n_blocks > 65536) return KVQ_EINVAL;
  if (reinterpret_cast<uintptr_t>(src) % 16) return KVQ_EINVAL;
  hipLaunchKernelGGL(stream_read, dim3(n_blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), nbytes / 16, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    kvq::set_last_error(std::string("probe launch: ") + hipGetErrorString(e));
    return KVQ_EHIP;
  }
  return KVQ_OK;
}
