// Quantize-and-append of new K/V rows into the packed cache, on gfx950.
//
// Row quantizer (RoPE-Aware Bit Allocation for KV-Cache Quantization,
// abstract: a TQ-MSE-based scalar quantizer under per-block widths; reading:
// per-token RMS scale after per-block gain normalisation), in IEEE order with
// no fused operations:
//   y = x * ig_j (fp32); ss = sum_i y_i^2 (fp64, i ascending);
//   s16 = fp16(fp32(sqrt(ss / 128))); is = s16 == 0 ? 0 : fp32(1 / s16);
//   u = y * is (fp32); code = number of boundaries beta_b[k] < u.
// NQKV-style codec (Pith review of NQKV, "What carries the argument" and
// referee major comment 1): per token, each run of 256 values of the
// [n_kv * 128] vector is divided by its absolute maximum and mapped to the
// 16-level Gaussian-quantile codebook.
//
// One workgroup of 128 lanes handles one 128-position V tile of one (sequence,
// KV head); lane t owns token position tile*128 + t.  K rows are written row by
// row (fields in plan order, LSB first).  V codes go through LDS so that lane i
// can assemble dim i's 128-token stream; positions outside the appended range
// keep the bits already stored (read-modify-write of partial words; a tile is
// owned by exactly one workgroup of the launch).
#include <hip/hip_fp16.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

template <typename T>
__device__ inline float load_f(const T* p);
template <>
__device__ inline float load_f<__half>(const __half* p) { return __half2float(*p); }
template <>
__device__ inline float load_f<float>(const float* p) { return *p; }

// number of entries of bd[0..n) strictly below u (bd ascending)
__device__ inline int count_below(const float* bd, int n, float u) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (bd[mid] < u) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ inline float inv_scale(__half s16) {
  const float s = __half2float(s16);
  return s == 0.0f ? 0.0f : __fdiv_rn(1.0f, s);
}

// RMS scale of a row after multiplying by the per-dim inverse gains
template <typename T>
__device__ inline __half row_rms(const T* x, const float* ig) {
  double ss = 0.0;
  for (int i = 0; i < kHeadDim; ++i) {
    const double y = static_cast<double>(__fmul_rn(load_f(x + i), ig[i]));
    ss = __dadd_rn(ss, __dmul_rn(y, y));
  }
  const float s32 = static_cast<float>(__dsqrt_rn(ss / static_cast<double>(kHeadDim)));
  return __float2half_rn(s32);
}

// absolute maximum of 256 consecutive values
template <typename T>
__device__ inline __half block_absmax(const T* x) {
  float a = 0.0f;
  for (int i = 0; i < kNfBlock; ++i) a = fmaxf(a, fabsf(load_f(x + i)));
  return __float2half_rn(a);
}

template <typename T, bool NF>
__global__ __launch_bounds__(128) void quantize_append(
    const T* __restrict__ kin, const T* __restrict__ vin, int64_t n_new, int64_t L0, int n_kv,
    int64_t cap, const Plan* __restrict__ plans, const Tables* __restrict__ tab,
    uint32_t* __restrict__ kc, uint32_t* __restrict__ vc, uint16_t* __restrict__ ks,
    uint16_t* __restrict__ vs, int k_words, int v_bits, int n_nf) {
  const int t = threadIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t tile = L0 / kVTile + blockIdx.x;
  const int64_t pos = tile * kVTile + t;
  const bool live = pos >= L0 && pos < L0 + n_new;

  __shared__ float bd_s[kMaxBits + 1][256];
  __shared__ float ig_s[kHeadDim];
  __shared__ uint8_t fdim_s[kHeadDim];
  __shared__ uint8_t fw_s[kHeadDim];
  __shared__ uint8_t vcode_s[kHeadDim][kVTile + 4];
  __shared__ int nf_s;

  const Plan* P = plans + h;
  for (int k = t; k < (kMaxBits + 1) * 256; k += blockDim.x) {
    const int bb = k >> 8, e = k & 255;
    bd_s[bb][e] = NF ? (bb == 4 && e < 16 ? tab->nf_bd[e] : INFINITY) : tab->bd[bb][e];
  }
  ig_s[t] = P->ig[t];
  fdim_s[t] = P->fdim[t];
  fw_s[t] = P->fwidth[t];
  if (t == 0) nf_s = P->n_fields;
  __syncthreads();

  if (live) {
    const int64_t src_row = (static_cast<int64_t>(b) * n_new + (pos - L0)) * n_kv + h;
    // ---- K ----
    const T* x = kin + src_row * kHeadDim;
    __half s16;
    if (NF) {
      const T* blk = kin + ((static_cast<int64_t>(b) * n_new + (pos - L0)) * n_kv) * kHeadDim +
                     static_cast<int64_t>(h / 2) * kNfBlock;
      s16 = block_absmax(blk);
    } else {
      s16 = row_rms(x, ig_s);
    }
    const float is = inv_scale(s16);
    uint32_t* row = kc + ((static_cast<int64_t>(b) * n_kv + h) * cap + pos) * k_words;
    uint64_t acc = 0;
    int nbits = 0, wo = 0;
    for (int f = 0; f < nf_s; ++f) {
      const int i = fdim_s[f], w = fw_s[f];
      const float y = NF ? load_f(x + i) : __fmul_rn(load_f(x + i), ig_s[i]);
      const float u = __fmul_rn(y, is);
      const uint32_t code = static_cast<uint32_t>(count_below(bd_s[w], (1 << w) - 1, u));
      acc |= static_cast<uint64_t>(code) << nbits;
      nbits += w;
      if (nbits >= 32) {
        row[wo++] = static_cast<uint32_t>(acc);
        acc >>= 32;
        nbits -= 32;
      }
    }
    const uint16_t sbits = __half_as_ushort(s16);
    if (NF) {
      if ((h & 1) == 0) ks[(static_cast<int64_t>(b) * cap + pos) * n_nf + h / 2] = sbits;
    } else {
      ks[(static_cast<int64_t>(b) * n_kv + h) * cap + pos] = sbits;
    }
    // ---- V ----
    const T* xv = vin + src_row * kHeadDim;
    __half sv;
    if (NF) {
      const T* blk = vin + ((static_cast<int64_t>(b) * n_new + (pos - L0)) * n_kv) * kHeadDim +
                     static_cast<int64_t>(h / 2) * kNfBlock;
      sv = block_absmax(blk);
    } else {
      double ss = 0.0;
      for (int i = 0; i < kHeadDim; ++i) {
        const double y = static_cast<double>(load_f(xv + i));
        ss = __dadd_rn(ss, __dmul_rn(y, y));
      }
      sv = __float2half_rn(static_cast<float>(__dsqrt_rn(ss / static_cast<double>(kHeadDim))));
    }
    const float isv = inv_scale(sv);
    const int vb = NF ? 4 : v_bits;
    for (int i = 0; i < kHeadDim; ++i)
      vcode_s[i][t] = static_cast<uint8_t>(
          count_below(bd_s[vb], (1 << vb) - 1, __fmul_rn(load_f(xv + i), isv)));
    const uint16_t vbits16 = __half_as_ushort(sv);
    if (NF) {
      if ((h & 1) == 0) vs[(static_cast<int64_t>(b) * cap + pos) * n_nf + h / 2] = vbits16;
    } else {
      vs[(static_cast<int64_t>(b) * n_kv + h) * cap + pos] = vbits16;
    }
  }
  __syncthreads();

  // lane i assembles dim i's four 32-token segments of this tile; segment (dim, g) is stored
  // at index ((dim / 16) * 4 + g) * 16 + dim % 16 (see the V tile layout in kvq.h)
  const int i = t;
  const int vb = NF ? 4 : v_bits;
  const int64_t lo_pos = L0 > tile * kVTile ? L0 - tile * kVTile : 0;
  const int64_t hi_pos = L0 + n_new - tile * kVTile < kVTile ? L0 + n_new - tile * kVTile : kVTile;
  uint32_t* tile_dst = vc + ((static_cast<int64_t>(b) * n_kv + h) * (cap / kVTile) + tile) * kVTile * 4 * vb;
  for (int g = 0; g < 4; ++g) {
    uint32_t* dst = tile_dst + static_cast<int64_t>(((i / 16) * 4 + g) * 16 + i % 16) * vb;
    uint64_t acc = 0, msk = 0;
    int nbits = 0, wo = 0;
    for (int e = 0; e < 32; ++e) {
      const int tau = 32 * g + e;
      const bool in = tau >= lo_pos && tau < hi_pos;
      const uint64_t code = in ? vcode_s[i][tau] : 0;
      const uint64_t m = in ? ((1ull << vb) - 1) : 0;
      acc |= code << nbits;
      msk |= m << nbits;
      nbits += vb;
      if (nbits >= 32) {
        const uint32_t nw = static_cast<uint32_t>(acc), mw = static_cast<uint32_t>(msk);
        if (mw == 0xFFFFFFFFu) dst[wo] = nw;
        else if (mw != 0u) dst[wo] = (dst[wo] & ~mw) | (nw & mw);
        ++wo;
        acc >>= 32;
        msk >>= 32;
        nbits -= 32;
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize(kvq_cache* c, int layer, const void* k, const void* v, int dtype,
                           int64_t n_new, hipStream_t stream) {
  const kvq_config& cfg = c->cfg;
  const int64_t L0 = c->len[layer];
  const int64_t first = L0 / kVTile, last = (L0 + n_new - 1) / kVTile;
  dim3 grid(static_cast<unsigned>(last - first + 1), static_cast<unsigned>(cfg.n_kv_heads),
            static_cast<unsigned>(cfg.batch));
  const bool nf = cfg.codec == KVQ_CODEC_NF16_B256;
  const Plan* plans = c->plans + static_cast<int64_t>(layer) * cfg.n_kv_heads;
#define KVQ_LAUNCH_Q(T, NF)                                                                      \
  hipLaunchKernelGGL((quantize_append<T, NF>), grid, dim3(128), 0, stream,                      \
                     static_cast<const T*>(k), static_cast<const T*>(v), n_new, L0,              \
                     cfg.n_kv_heads, c->cap, plans, c->tables, layer_k_codes(c, layer),          \
                     layer_v_codes(c, layer), layer_k_scales(c, layer), layer_v_scales(c, layer), \
                     c->k_words, cfg.v_bits, c->n_nf_blocks)
  if (dtype == KVQ_F16) {
    if (nf) KVQ_LAUNCH_Q(__half, true); else KVQ_LAUNCH_Q(__half, false);
  } else {
    if (nf) KVQ_LAUNCH_Q(float, true); else KVQ_LAUNCH_Q(float, false);
  }
#undef KVQ_LAUNCH_Q
  return hipGetLastError();
}

}  // namespace kvq
