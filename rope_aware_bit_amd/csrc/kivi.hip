// Quantize-and-append for the KIVI-style asymmetric integer codec, on gfx950.
//
// The leaderboard (KV Cache Quantization on WikiText-2 prompt 2048-token (train)) compares
// the allocation with KIVI, a streaming asymmetric quantizer (NQKV review, reference list);
// the review's ablation table gives the split of that family: keys per channel, values per
// token.  Reading (min/max integer quantizer, in IEEE order with no fused operations):
//   lo = fp16(min x), hi = fp16(max x), s = fp16(fp32(fp32(hi - lo) / (2^b - 1))),
//   is = s == 0 ? 0 : fp32(1 / s), code = clamp(rint(fp32(fp32(x - lo) * is)), 0, 2^b - 1);
//   reconstruction fp16(lo + s * code).
// A key group is one channel over a 128-position tile, a value group one position's 128
// channels.  Key tiles are quantized only once complete, so this kernel always writes whole
// tiles: one workgroup of 256 threads per (tile, KV head, sequence).
//   1. the tile's 128 K rows are copied into LDS as fp32, each position from its fp16 copy
//      in the ring or from the input;
//   2. per channel: minimum and maximum (two half-columns, then combined), the parameters;
//   3. every element's code into an LDS code image;
//   4. the K rows are assembled word by word from the code image (consecutive threads write
//      consecutive words of the tile's contiguous rows);
//   5-7. the same for V with per-position parameters, and its 512 segments of v_bits words.
#include <hip/hip_fp16.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kT = 256;                 // threads
constexpr int kXS = kHeadDim + 1;       // padded LDS row (floats)
constexpr int kCS = kHeadDim + 4;       // padded code row (bytes)

template <typename T>
__device__ inline float as_f(T v);
template <>
__device__ inline float as_f<__half>(__half v) { return __half2float(v); }
template <>
__device__ inline float as_f<float>(float v) { return v; }

struct GroupParams {
  __half s16, lo16;
  float lo32, is32;
};

// Parameters of one group from its minimum and maximum (fp32).
__device__ inline GroupParams group_params(float mn, float mx, int levels) {
  GroupParams p;
  p.lo16 = __float2half_rn(mn);
  const __half hi16 = __float2half_rn(mx);
  const float d = __fsub_rn(__half2float(hi16), __half2float(p.lo16));
  p.s16 = __float2half_rn(__fdiv_rn(d, static_cast<float>(levels - 1)));
  const float s = __half2float(p.s16);
  p.lo32 = __half2float(p.lo16);
  p.is32 = s == 0.0f ? 0.0f : __fdiv_rn(1.0f, s);
  return p;
}

__device__ inline uint32_t code_of(float x, float lo, float is, int levels) {
  const float u = __fmul_rn(__fsub_rn(x, lo), is);
  const float r = rintf(u);
  return static_cast<uint32_t>(fminf(fmaxf(r, 0.0f), static_cast<float>(levels - 1)));
}

template <typename T>
__global__ __launch_bounds__(kT) void kivi_quantize(
    const T* __restrict__ kin, const T* __restrict__ vin, int64_t in_stride, int64_t tile0,
    int64_t len_old, const __half* __restrict__ krg, const __half* __restrict__ vrg, int ring,
    int n_kv, int64_t cap, const Plan* __restrict__ plans, int plan_bs, int pairing,
    uint32_t* __restrict__ kc, uint32_t* __restrict__ vc, uint16_t* __restrict__ ks,
    uint16_t* __restrict__ vs, int kb, int vb) {
  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t tile = tile0 + blockIdx.x;
  const int64_t bh = static_cast<int64_t>(b) * n_kv + h;
  const int64_t pos0 = tile * kVTile;
  const int kL = 1 << kb, vL = 1 << vb;

  __shared__ float x_s[kVTile][kXS];
  __shared__ uint8_t c_s[kVTile][kCS];
  __shared__ float red_s[2][2][kHeadDim];   // [min, max][half][channel]
  __shared__ float lo_s[kHeadDim], is_s[kHeadDim];
  __shared__ uint8_t fdim_s[kHeadDim];

  const Plan* P = plans + static_cast<int64_t>(b) * plan_bs + h;
  if (tid < kHeadDim) fdim_s[tid] = P->fdim[tid];

  // position r of the tile: ring slot (already appended) or input row.  Thread t takes
  // channel t % 128 of rows t / 128 + 2 i, sixteen rows at a time with all sixteen loads
  // issued before the first store
  auto load_tile = [&](const T* in, const __half* rg, bool values) {
    constexpr int kU = 16;
    const int d = tid & (kHeadDim - 1);
    for (int r0 = tid >> 7; r0 < kVTile; r0 += 2 * kU) {
      // (raw loads first, conversions after, so no conversion waits between the loads)
      __half hv[kU];
      T tv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t p = pos0 + r0 + 2 * u;
        if (p < len_old) {
          const int64_t slot = p % ring;
          const int64_t off = values
              ? (((bh * (ring / kVTile) + slot / kVTile) * kHeadDim + d) * kVTile + slot % kVTile)
              : (((static_cast<int64_t>(b) * ring + slot) * n_kv + h) * kHeadDim + d);
          hv[u] = rg[off];
        } else {
          tv[u] = in[((static_cast<int64_t>(b) * in_stride + (p - len_old)) * n_kv + h) * kHeadDim + d];
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
        x_s[r0 + 2 * u][d] = pos0 + r0 + 2 * u < len_old ? __half2float(hv[u]) : as_f(tv[u]);
    }
  };

  // ---- keys: one group per channel ----
  load_tile(kin, krg, false);
  __syncthreads();
  {
    const int d = tid & (kHeadDim - 1), hf = tid >> 7;
    float mn = x_s[64 * hf][d], mx = mn;
    for (int r = 64 * hf + 1; r < 64 * hf + 64; ++r) {
      mn = fminf(mn, x_s[r][d]);
      mx = fmaxf(mx, x_s[r][d]);
    }
    red_s[0][hf][d] = mn;
    red_s[1][hf][d] = mx;
  }
  __syncthreads();
  if (tid < kHeadDim) {
    const int d = tid;
    const GroupParams gp = group_params(fminf(red_s[0][0][d], red_s[0][1][d]),
                                        fmaxf(red_s[1][0][d], red_s[1][1][d]), kL);
    lo_s[d] = gp.lo32;
    is_s[d] = gp.is32;
    // [tile][block j][s(p0), s(p1), lo(p0), lo(p1)]
    const int j = pairing == KVQ_ROPE_HALF ? d % kBlocks : d / 2;
    const int co = pairing == KVQ_ROPE_HALF ? d / kBlocks : d % 2;
    uint16_t* kp = ks + ((bh * (cap / kVTile) + tile) * kBlocks + j) * 4;
    kp[co] = __half_as_ushort(gp.s16);
    kp[2 + co] = __half_as_ushort(gp.lo16);
  }
  __syncthreads();
  {
    const int d = tid & (kHeadDim - 1);
    for (int r = tid >> 7; r < kVTile; r += 2) c_s[r][d] = static_cast<uint8_t>(code_of(x_s[r][d], lo_s[d], is_s[d], kL));
  }
  __syncthreads();
  {
    // K rows: word wi of row r holds fields f with bits [kb f, kb f + kb) meeting [32 wi, 32 wi + 32)
    const int kw = 4 * kb;
    uint32_t* dst = kc + (bh * cap + pos0) * kw;
    for (int wid = tid; wid < kVTile * kw; wid += kT) {
      const int r = wid / kw, wi = wid % kw;
      const int f0 = 32 * wi / kb, f1 = (32 * wi + 31) / kb;
      uint32_t word = 0u;
      for (int f = f0; f <= f1 && f < kHeadDim; ++f) {
        const uint32_t code = c_s[r][fdim_s[f]];
        const int sh = kb * f - 32 * wi;   // may be negative for a field straddling into this word
        word |= sh >= 0 ? code << sh : code >> -sh;
      }
      dst[wid] = word;
    }
  }
  __syncthreads();

  // ---- values: one group per position ----
  load_tile(vin, vrg, true);
  __syncthreads();
  {
    // thread pair (2 r, 2 r + 1) scans the two halves of position r's row
    const int r = tid >> 1, hf = tid & 1;
    float mn = x_s[r][64 * hf], mx = mn;
    for (int d = 64 * hf + 1; d < 64 * hf + 64; ++d) {
      mn = fminf(mn, x_s[r][d]);
      mx = fmaxf(mx, x_s[r][d]);
    }
    mn = fminf(mn, __shfl_xor(mn, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    if (hf == 0) {
      const GroupParams gp = group_params(mn, mx, vL);
      lo_s[r] = gp.lo32;
      is_s[r] = gp.is32;
      // [tile][2][128]: the tile's s, then its lo
      uint16_t* vp = vs + (bh * (cap / kVTile) + tile) * 2 * kVTile;
      vp[r] = __half_as_ushort(gp.s16);
      vp[kVTile + r] = __half_as_ushort(gp.lo16);
    }
  }
  __syncthreads();
  {
    const int d = tid & (kHeadDim - 1);
    for (int r = tid >> 7; r < kVTile; r += 2) c_s[r][d] = static_cast<uint8_t>(code_of(x_s[r][d], lo_s[r], is_s[r], vL));
  }
  __syncthreads();
  {
    // 512 segments of vb words; segment index ((dim / 16) * 4 + g) * 16 + dim % 16 holds the
    // codes of dim for positions 32 g .. 32 g + 31, position 32 g + e at bit e * vb
    uint32_t* dst = vc + (bh * (cap / kVTile) + tile) * (4 * kHeadDim * vb);
    for (int wid = tid; wid < 4 * kHeadDim * vb; wid += kT) {
      const int sg = wid / vb, wi = wid % vb;
      const int dim = (sg >> 6) * 16 + (sg & 15), g = (sg >> 4) & 3;
      const int e0 = 32 * wi / vb, e1 = (32 * wi + 31) / vb;
      uint32_t word = 0u;
      for (int e = e0; e <= e1 && e < 32; ++e) {
        const uint32_t code = c_s[32 * g + e][dim];
        const int sh = vb * e - 32 * wi;
        word |= sh >= 0 ? code << sh : code >> -sh;
      }
      dst[wid] = word;
    }
  }
}

}  // namespace

hipError_t launch_kivi_quantize(kvq_cache* c, int layer, const void* k, const void* v, int dtype,
                                int64_t in_stride, int64_t p0, int64_t n_pos, int64_t len_old,
                                hipStream_t stream) {
  const kvq_config& cfg = c->cfg;
  dim3 grid(static_cast<unsigned>(n_pos / kVTile), static_cast<unsigned>(cfg.n_kv_heads),
            static_cast<unsigned>(cfg.batch));
  const Plan* plans = c->plans + static_cast<int64_t>(layer) * c->n_plan * cfg.n_kv_heads;
  const int plan_bs = c->n_plan > 1 ? cfg.n_kv_heads : 0;
#define KVQ_LAUNCH_KIVI(T)                                                                           \
  hipLaunchKernelGGL(kivi_quantize<T>, grid, dim3(kT), 0, stream, static_cast<const T*>(k),          \
                     static_cast<const T*>(v), in_stride, p0 / kVTile, len_old, layer_k_recent(c, layer), \
                     layer_v_recent(c, layer), c->ring, cfg.n_kv_heads, c->cap, plans, plan_bs,       \
                     cfg.pairing, layer_k_codes(c, layer), layer_v_codes(c, layer),                  \
                     layer_k_scales(c, layer), layer_v_scales(c, layer), cfg.k_bits, cfg.v_bits)
  if (dtype == KVQ_F16)
    KVQ_LAUNCH_KIVI(__half);
  else
    KVQ_LAUNCH_KIVI(float);
#undef KVQ_LAUNCH_KIVI
  return hipGetLastError();
}

}  // namespace kvq
