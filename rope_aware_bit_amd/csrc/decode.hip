// Split-K grouped-query decode attention over the packed cache, on gfx950.
//
// RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: decode reads
// the packed (K3V3) cache directly.  Logits l_{h,t} = sigma * s^K_t *
// sum_i q_{h,i} g_i CB_{b_i}[code_{t,i}]; online softmax over the cached
// tokens; o_h = sum_t p_{h,t} s^V_t CB_{B_V}[code^V_{t,i}] / sum_t p_{h,t}.
// The 256-value absmax codec (NQKV review, "What carries the argument") uses
// one scale per 256 values (two KV heads share it) and its 16-level table.
//
// Pass 1 (decode_split): one workgroup per (context split, KV head, sequence)
// walks its 128-token tiles: lanes 0..127 each decode one K row and form the G
// logits (q is pre-multiplied by the gains and sigma and held in LDS), a wave
// per head updates the running max / sum, then lane i decodes dim i of the
// tile's dim-major V stream (staged in LDS) and accumulates the G outputs.
// Each split writes (m, l, unnormalised o) for its G heads.
// The last workgroup of a (sequence, KV head) to finish (an agent-scope counter)
// combines the splits in split order: m* = max m_s, l = sum exp(m_s - m*) l_s,
// o = sum exp(m_s - m*) o_s / l, and resets the counter for the next call.  Calls
// that overlap on one cache (two streams) would share the counters and must not.
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

__device__ inline float half_bits_to_float(uint16_t h) { return __half2float(__ushort_as_half(h)); }

template <typename TQ, int G, bool NF>
__global__ __launch_bounds__(256) void decode_split(
    const TQ* __restrict__ q, float sigma, int64_t len, int n_kv, int64_t cap, int tiles_per_split,
    const Plan* __restrict__ plans, const Tables* __restrict__ tab, const uint32_t* __restrict__ kc,
    const uint32_t* __restrict__ vc, const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vs,
    int k_words, int v_bits, int n_nf, int n_splits, float* __restrict__ part_o,
    float* __restrict__ part_ml, unsigned* __restrict__ counters, float* __restrict__ out) {
  const int tid = threadIdx.x;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n_q = n_kv * G;

  __shared__ float qs[kHeadDim][G];
  __shared__ float cbk_s[kMaxBits + 1][256];
  __shared__ float cbv_s[256];
  __shared__ uint8_t fdim_s[kHeadDim];
  __shared__ uint8_t fw_s[kHeadDim];
  __shared__ uint16_t foff_s[kHeadDim];
  __shared__ float logit_s[G][kVTile];
  __shared__ float pv_s[G][kVTile];
  __shared__ uint32_t vtile_s[kHeadDim * 4 * kMaxBits];
  __shared__ float alpha_s[G];
  __shared__ float m_run_s[G], l_run_s[G];
  __shared__ int nf_s;

  const Plan* P = plans + h;
  for (int k = tid; k < (kMaxBits + 1) * 256; k += blockDim.x) {
    const int bb = k >> 8, e = k & 255;
    cbk_s[bb][e] = NF ? (bb == 4 && e < 16 ? half_bits_to_float(tab->nf_cb[e]) : 0.0f)
                      : half_bits_to_float(tab->cb[bb][e]);
  }
  const int vb = NF ? 4 : v_bits;
  if (tid < 256) cbv_s[tid] = NF ? (tid < 16 ? half_bits_to_float(tab->nf_cb[tid]) : 0.0f)
                                 : half_bits_to_float(tab->cb[vb][tid]);
  if (tid < kHeadDim) {
    fdim_s[tid] = P->fdim[tid];
    fw_s[tid] = P->fwidth[tid];
    foff_s[tid] = P->foff[tid];
    const float gi = P->g[tid];
    for (int g = 0; g < G; ++g) {
      const float qv = load_f(q + (static_cast<int64_t>(b) * n_q + h * G + g) * kHeadDim + tid);
      qs[tid][g] = qv * gi * sigma;
    }
  }
  if (tid < G) {
    m_run_s[tid] = -INFINITY;
    l_run_s[tid] = 0.0f;
  }
  if (tid == 0) nf_s = P->n_fields;
  __syncthreads();

  constexpr int HPT = G >= 2 ? G / 2 : 1;  // heads per thread in the V pass
  float acc_o[HPT];
#pragma unroll
  for (int k = 0; k < HPT; ++k) acc_o[k] = 0.0f;
  const int vdim = tid & (kHeadDim - 1);
  const int vhalf = tid >> 7;
  const bool v_active = G >= 2 || vhalf == 0;

  const int64_t n_tiles = (len + kVTile - 1) / kVTile;
  const int64_t t_begin = static_cast<int64_t>(s) * tiles_per_split;
  const int64_t t_end = t_begin + tiles_per_split < n_tiles ? t_begin + tiles_per_split : n_tiles;
  const int v_words = 4 * vb;
  const int64_t bh = static_cast<int64_t>(b) * n_kv + h;

  for (int64_t tile = t_begin; tile < t_end; ++tile) {
    const int64_t tok0 = tile * kVTile;
    const int ntok = len - tok0 < kVTile ? static_cast<int>(len - tok0) : kVTile;
    // stage the tile's V streams
    const uint32_t* vsrc = vc + (bh * (cap / kVTile) + tile) * kVTile * v_words;
    for (int k = tid; k < kHeadDim * v_words; k += blockDim.x) vtile_s[k] = vsrc[k];
    // K: one row per lane
    if (tid < kVTile) {
      float acc[G];
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = 0.0f;
      if (tid < ntok) {
        const uint32_t* row = kc + (bh * cap + tok0 + tid) * k_words;
        for (int f = 0; f < nf_s; ++f) {
          const int w = fw_s[f], off = foff_s[f];
          const int wi = off >> 5, sh = off & 31;
          uint64_t win = row[wi];
          if (sh + w > 32) win |= static_cast<uint64_t>(row[wi + 1]) << 32;
          const int code = static_cast<int>((win >> sh) & ((1u << w) - 1));
          const float cval = cbk_s[w][code];
          const int i = fdim_s[f];
#pragma unroll
          for (int g = 0; g < G; ++g) acc[g] = fmaf(qs[i][g], cval, acc[g]);
        }
        const float sk = NF ? half_bits_to_float(ks[(static_cast<int64_t>(b) * cap + tok0 + tid) * n_nf + h / 2])
                            : half_bits_to_float(ks[bh * cap + tok0 + tid]);
#pragma unroll
        for (int g = 0; g < G; ++g) logit_s[g][tid] = acc[g] * sk;
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) logit_s[g][tid] = -INFINITY;
      }
    }
    __syncthreads();
    // online softmax: wave w handles heads w, w+4
    {
      const int wave = tid >> 6, lane = tid & 63;
      for (int g = wave; g < G; g += 4) {
        const float l0 = logit_s[g][lane], l1 = logit_s[g][lane + 64];
        float mx = fmaxf(l0, l1);
        for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        const float m_old = m_run_s[g];
        const float m_new = fmaxf(m_old, mx);
        const float p0 = __expf(l0 - m_new), p1 = __expf(l1 - m_new);
        const int64_t t0 = tok0 + lane, t1 = tok0 + lane + 64;
        float sv0 = 0.0f, sv1 = 0.0f;
        if (lane < ntok)
          sv0 = NF ? half_bits_to_float(vs[(static_cast<int64_t>(b) * cap + t0) * n_nf + h / 2])
                   : half_bits_to_float(vs[bh * cap + t0]);
        if (lane + 64 < ntok)
          sv1 = NF ? half_bits_to_float(vs[(static_cast<int64_t>(b) * cap + t1) * n_nf + h / 2])
                   : half_bits_to_float(vs[bh * cap + t1]);
        pv_s[g][lane] = p0 * sv0;
        pv_s[g][lane + 64] = p1 * sv1;
        float ps = p0 + p1;
        for (int o = 32; o >= 1; o >>= 1) ps += __shfl_xor(ps, o, 64);
        if (lane == 0) {
          const float alpha = __expf(m_old - m_new);
          alpha_s[g] = alpha;
          l_run_s[g] = l_run_s[g] * alpha + ps;
          m_run_s[g] = m_new;
        }
      }
    }
    __syncthreads();
    // V: lane i = dim, accumulates its heads
    if (v_active) {
      const uint32_t* words = vtile_s + vdim * v_words;
#pragma unroll
      for (int k = 0; k < HPT; ++k) acc_o[k] *= alpha_s[vhalf * HPT + k];
      const uint32_t mask = (1u << vb) - 1;
      for (int tau = 0; tau < ntok; ++tau) {
        const int bit = tau * vb;
        const int wi = bit >> 5, sh = bit & 31;
        uint64_t win = words[wi];
        if (sh + vb > 32) win |= static_cast<uint64_t>(words[wi + 1]) << 32;
        const float cval = cbv_s[(win >> sh) & mask];
#pragma unroll
        for (int k = 0; k < HPT; ++k) acc_o[k] = fmaf(pv_s[vhalf * HPT + k][tau], cval, acc_o[k]);
      }
    }
    __syncthreads();
  }

  const int64_t pbase = (bh * n_splits + s) * G;
  if (v_active) {
#pragma unroll
    for (int k = 0; k < HPT; ++k) part_o[(pbase + vhalf * HPT + k) * kHeadDim + vdim] = acc_o[k];
  }
  if (tid < G) {
    part_ml[(pbase + tid) * 2 + 0] = m_run_s[tid];
    part_ml[(pbase + tid) * 2 + 1] = l_run_s[tid];
  }

  // The last split of this (sequence, KV head) to finish combines all splits, in split
  // order: release the partials at agent scope, count, and acquire before reading.
  __shared__ bool last_s;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counters + bh, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    last_s = prev == static_cast<unsigned>(n_splits - 1);
  }
  __syncthreads();
  if (!last_s) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int idx = tid; idx < G * kHeadDim; idx += blockDim.x) {
    const int g = idx / kHeadDim, i = idx % kHeadDim;
    const int64_t p0 = bh * n_splits * G + g;
    float mstar = -INFINITY;
    for (int sp = 0; sp < n_splits; ++sp) mstar = fmaxf(mstar, part_ml[(p0 + sp * G) * 2]);
    float l = 0.0f, o = 0.0f;
    for (int sp = 0; sp < n_splits; ++sp) {
      const int64_t p = p0 + sp * G;
      const float ms = part_ml[p * 2];
      if (ms == -INFINITY) continue;
      const float wgt = __expf(ms - mstar);
      l += wgt * part_ml[p * 2 + 1];
      o += wgt * part_o[p * kHeadDim + i];
    }
    out[(static_cast<int64_t>(b) * n_q + h * G + g) * kHeadDim + i] = o / l;
  }
  if (tid == 0) counters[bh] = 0u;  // ready for the next call on this stream
}

template <typename TQ, int G>
hipError_t launch_g(kvq_cache* c, int layer, const void* q, float sigma, float* out, int S,
                    hipStream_t stream) {
  const kvq_config& cfg = c->cfg;
  const int64_t len = c->len[layer];
  const int64_t n_tiles = (len + kVTile - 1) / kVTile;
  const int tps = static_cast<int>((n_tiles + S - 1) / S);
  dim3 grid(S, cfg.n_kv_heads, cfg.batch);
  const Plan* plans = c->plans + static_cast<int64_t>(layer) * cfg.n_kv_heads;
  if (cfg.codec == KVQ_CODEC_NF16_B256)
    hipLaunchKernelGGL((decode_split<TQ, G, true>), grid, dim3(256), 0, stream,
                       static_cast<const TQ*>(q), sigma, len, cfg.n_kv_heads, c->cap, tps, plans,
                       c->tables, layer_k_codes(c, layer), layer_v_codes(c, layer),
                       layer_k_scales(c, layer), layer_v_scales(c, layer), c->k_words, cfg.v_bits,
                       c->n_nf_blocks, S, c->part_o, c->part_ml, c->split_counters, out);
  else
    hipLaunchKernelGGL((decode_split<TQ, G, false>), grid, dim3(256), 0, stream,
                       static_cast<const TQ*>(q), sigma, len, cfg.n_kv_heads, c->cap, tps, plans,
                       c->tables, layer_k_codes(c, layer), layer_v_codes(c, layer),
                       layer_k_scales(c, layer), layer_v_scales(c, layer), c->k_words, cfg.v_bits,
                       c->n_nf_blocks, S, c->part_o, c->part_ml, c->split_counters, out);
  return hipGetLastError();
}

template <typename TQ>
hipError_t launch_t(kvq_cache* c, int layer, const void* q, float sigma, float* out, int S,
                    hipStream_t stream) {
  switch (c->group) {
    case 1: return launch_g<TQ, 1>(c, layer, q, sigma, out, S, stream);
    case 2: return launch_g<TQ, 2>(c, layer, q, sigma, out, S, stream);
    case 4: return launch_g<TQ, 4>(c, layer, q, sigma, out, S, stream);
    default: return launch_g<TQ, 8>(c, layer, q, sigma, out, S, stream);
  }
}

}  // namespace

int auto_splits(const kvq_cache* c, int64_t len) {
  const int64_t n_tiles = (len + kVTile - 1) / kVTile;
  const int64_t units = static_cast<int64_t>(c->cfg.batch) * c->cfg.n_kv_heads;
  int64_t S = (1024 + units - 1) / units;
  if (S > n_tiles) S = n_tiles;
  if (S > c->max_splits) S = c->max_splits;
  if (S < 1) S = 1;
  // no empty trailing splits: S * ceil(n_tiles / S) must cover n_tiles with every split used
  const int64_t tps = (n_tiles + S - 1) / S;
  S = (n_tiles + tps - 1) / tps;
  return static_cast<int>(S);
}

hipError_t launch_decode(kvq_cache* c, int layer, const void* q, int dtype, float scale,
                         float* out, int n_splits, hipStream_t stream) {
  const float sigma = scale > 0.0f ? scale : 0.08838834764831845f;  // 1/sqrt(128)
  if (dtype == KVQ_F16) return launch_t<__half>(c, layer, q, sigma, out, n_splits, stream);
  return launch_t<float>(c, layer, q, sigma, out, n_splits, stream);
}

}  // namespace kvq
