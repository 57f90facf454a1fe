// Split-K grouped-query decode attention over the packed cache, MFMA kernel for gfx950.
//
// RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: decode reads
// the packed (K3V3) cache directly.  With sigma' = sigma * log2(e):
//   l'_{h,t} = s^K_t * sum_i (q_{h,i} g_i sigma') CB_{b_i}[code_{t,i}]   (log2 domain)
//   o_h = sum_t 2^(l'_{h,t} - m) s^V_t CB_{B_V}[code^V_{t,i}] / sum_t 2^(l'_{h,t} - m).
// The 256-value absmax codec (NQKV review, "What carries the argument") uses one
// scale per 256 values (two KV heads share it) and its 16-level table.
//
// Work decomposition.  One workgroup of 4 waves per (context split, KV head,
// sequence); each wave walks 128-token tiles of the split on its own, keeping
// its own running max / sum / output, and the waves are merged through LDS at
// the end.  Splits are merged in two levels inside the same kernel: the last
// workgroup of each group of 16 consecutive splits merges the group, and the
// last group merger merges the groups, always in split order.
//
// Keys (lane = token).  The K rows of a tile are staged in LDS word-major.  Every
// stored RoPE block contributes a pair of fields (p0, p1) of the same width w;
// the pair's 2w bits are cut out of the row with one funnel shift at a
// wave-uniform offset and looked up in an LDS table of fp16 pairs (w <= 4; two
// single lookups for w >= 5), giving two fp16 codebook values.  Two pairs form
// the 4-element B operand of a 4x4x4 (16-block) f16 MFMA whose A operand, the
// query pre-multiplied by gains and sigma' and split into fp16 hi + lo parts,
// is broadcast from one of 16 lane blocks (A-broadcast), so 64 tokens x 4
// query-head parts are produced per instruction with no data exchange.
//
// Values (lane = dim, 8 tokens).  V tiles are stored in the order of the 16x16x32
// f16 MFMA A operand: each lane loads B_V contiguous words per 16-dim slice and
// cuts 8 codes of one dim at compile-time offsets (pairs through the same LDS
// tables).  The B operand is the softmax weight p * s^V split into fp16 hi + lo,
// written by the key lanes to LDS and read back 8 tokens at a time.
//
// Cross-workgroup merging.  Split partials are written and read with agent-scope
// (device-coherent) atomic stores and loads.  A workgroup waits for its stores to
// complete (s_waitcnt) before it increments the merge counter, and the merger
// reads the partials only after it has seen the counter reach the group size,
// so no cache-wide write-back or invalidation is needed.
#pragma once

#include <hip/hip_fp16.h>

#include <type_traits>
#include <utility>

#include "kvq_internal.h"

namespace kvq {
namespace mfma {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kGroup = 16;        // splits merged per first-level merger
constexpr int kMaxGroups = 16;    // so at most kGroup * kMaxGroups = 256 splits

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1, so that MFMA broadcast
// selectors derived from I are compile-time constants.
template <typename F, int... Is>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ inline float half_bits_to_float(uint16_t h) { return __half2float(__ushort_as_half(h)); }

__device__ inline uint32_t lds_u32(const char* base, uint32_t addr) {
  return *reinterpret_cast<const uint32_t*>(base + addr);
}
__device__ inline uint32_t lds_u16(const char* base, uint32_t addr) {
  return *reinterpret_cast<const uint16_t*>(base + addr);
}

#define KVQ_DPP(v, ctrl) \
  __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false))

// Wave-wide max / sum: rotations within rows of 16 lanes, then the 4 row results
// read out to scalars; the result is the same in every lane.
__device__ inline float wave_max(float v) {
  v = fmaxf(v, KVQ_DPP(v, 0x128));
  v = fmaxf(v, KVQ_DPP(v, 0x124));
  v = fmaxf(v, KVQ_DPP(v, 0x122));
  v = fmaxf(v, KVQ_DPP(v, 0x121));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
__device__ inline float wave_sum(float v) {
  v += KVQ_DPP(v, 0x128);
  v += KVQ_DPP(v, 0x124);
  v += KVQ_DPP(v, 0x122);
  v += KVQ_DPP(v, 0x121);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// Orders a wave's LDS writes before its later LDS reads of other lanes' data (LDS
// instructions of one wave execute in issue order; this keeps the compiler from moving
// them across).
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Device-coherent (agent-scope) stores / loads of split partials.
__device__ inline void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Count this workgroup in a merge counter after all of its partial stores have
// completed; returns (in every thread) whether it was the last of `expected`.
__device__ inline bool arrive(unsigned* counter, unsigned expected, bool* flag_s) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);   // all outstanding memory operations of this wave
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag_s = prev == expected - 1u;
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return *flag_s;
}

// fp16 pairs (CB[c0], CB[c1]) of one K block for two tokens.  The block's 2w-bit field
// starts at bit `off` of every row.  K rows of the 128-token tile are staged in LDS
// word-major: kr[(d + 1) * 128 + tau] is word d of token tau's row, rows 0 and
// k_words + 1 are zero.  The lane reads tokens `lane` and `lane + 64`.  off and w are
// wave-uniform.
__device__ inline void k_pair2(const uint32_t* kr, int lane, int off, int w, const char* tab,
                               uint32_t& v0, uint32_t& v1) {
  if (w <= 4) {
    const int a = off + 30;  // field lands at bit 2 of the window
    const uint32_t* p = kr + (a >> 5) * kVTile + lane;
    const uint32_t x0 = __builtin_amdgcn_alignbit(p[kVTile], p[0], a & 31);
    const uint32_t x1 = __builtin_amdgcn_alignbit(p[kVTile + 64], p[64], a & 31);
    const uint32_t m = (((1u << (2 * w)) - 1u)) << 2;
    const uint32_t pb = static_cast<uint32_t>(pair_table_base(w));
    v0 = lds_u32(tab, (x0 & m) | pb);
    v1 = lds_u32(tab, (x1 & m) | pb);
  } else {
    const int a = off + 31;  // first field at bit 1, second at bit 1 + w (2w <= 16 bits)
    const uint32_t* p = kr + (a >> 5) * kVTile + lane;
    const uint32_t x0 = __builtin_amdgcn_alignbit(p[kVTile], p[0], a & 31);
    const uint32_t x1 = __builtin_amdgcn_alignbit(p[kVTile + 64], p[64], a & 31);
    const uint32_t m = ((1u << w) - 1u) << 1;
    const uint32_t sb = static_cast<uint32_t>(single_table_base(w));
    v0 = lds_u16(tab, (x0 & m) | sb) | (lds_u16(tab, ((x0 >> w) & m) | sb) << 16);
    v1 = lds_u16(tab, (x1 & m) | sb) | (lds_u16(tab, ((x1 >> w) & m) | sb) << 16);
  }
}

// fp16 pair of V codes e, e+1 (e even) of a 32-code segment held in S[0..VB) (S[-1] and
// S[VB] are zero words).
template <int VB>
__device__ inline uint32_t v_pair(const uint32_t* S, int e, const char* tab) {
  if constexpr (VB <= 4) {
    constexpr uint32_t mask = ((1u << (2 * VB)) - 1u) << 2;
    const int a = e * VB + 30;
    const uint32_t x = __builtin_amdgcn_alignbit(S[(a >> 5)], S[(a >> 5) - 1], a & 31);
    return lds_u32(tab, (x & mask) | static_cast<uint32_t>(pair_table_base(VB)));
  } else {
    constexpr uint32_t mask = ((1u << VB) - 1u) << 1;
    const int a0 = e * VB + 31, a1 = (e + 1) * VB + 31;
    const uint32_t x0 = __builtin_amdgcn_alignbit(S[(a0 >> 5)], S[(a0 >> 5) - 1], a0 & 31);
    const uint32_t x1 = __builtin_amdgcn_alignbit(S[(a1 >> 5)], S[(a1 >> 5) - 1], a1 & 31);
    constexpr uint32_t sb = static_cast<uint32_t>(single_table_base(VB));
    return lds_u16(tab, (x0 & mask) | sb) | (lds_u16(tab, (x1 & mask) | sb) << 16);
  }
}

// Merge `count` (1..kGroup) consecutive split partials of one (sequence, KV head):
// partial e holds, per head g, (m, l) at ml[(e*G + g)*2 + {0,1}] and the unnormalised
// output at o[(e*G + g)*128 + i].  m* = max_e m_e, l = sum_e 2^(m_e - m*) l_e and
// o = sum_e 2^(m_e - m*) o_e, in e order.  Writes either the merged partial or, if
// `final_out`, o / l to dst_o[g*128 + i].  All loads are issued before any result is
// needed, so the merge costs one round of memory latency.
template <int G>
__device__ inline void merge_level(const float* __restrict__ src_o, const float* __restrict__ src_ml,
                                   int count, float* mw, int tid, float* __restrict__ dst_o,
                                   float* __restrict__ dst_ml, bool final_out) {
  constexpr int NOUT = G * kHeadDim;
  constexpr int OPT = (NOUT + 255) / 256;
  float ov[OPT][kGroup];
#pragma unroll
  for (int k = 0; k < OPT; ++k) {
    const int idx = (tid + 256 * k) % NOUT;
    const int g = idx / kHeadDim, i = idx % kHeadDim;
#pragma unroll
    for (int e = 0; e < kGroup; ++e) {
      const int ee = e < count ? e : count - 1;   // loads stay in range; weight 0 below
      ov[k][e] = ld_coh(src_o + (ee * G + g) * kHeadDim + i);
    }
  }
  float* wv = mw;                       // [kGroup][G] maxima, then weights
  float* lv = mw + kGroup * G;          // [kGroup][G] sums
  float* ms = lv + kGroup * G;          // [G] merged max
  float* ls = ms + G;                   // [G] merged sum
  if (tid < kGroup * G) {
    const int e = tid / G, g = tid % G;
    const int ee = e < count ? e : count - 1;
    const float m = ld_coh(src_ml + (ee * G + g) * 2);
    const float l = ld_coh(src_ml + (ee * G + g) * 2 + 1);
    wv[tid] = e < count ? m : -INFINITY;
    lv[tid] = l;
  }
  __syncthreads();
  if (tid < G) {
    float m = -INFINITY;
    for (int e = 0; e < kGroup; ++e) m = fmaxf(m, wv[e * G + tid]);
    float l = 0.0f;
    for (int e = 0; e < kGroup; ++e) {
      const float me = wv[e * G + tid];
      const float w = me == -INFINITY ? 0.0f : exp2f(me - m);
      l += w * lv[e * G + tid];
      wv[e * G + tid] = w;
    }
    ms[tid] = m;
    ls[tid] = l;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < OPT; ++k) {
    const int idx = tid + 256 * k;
    if (idx >= NOUT) break;
    const int g = idx / kHeadDim, i = idx % kHeadDim;
    float o = 0.0f;
#pragma unroll
    for (int e = 0; e < kGroup; ++e) o += wv[e * G + g] * ov[k][e];
    if (final_out) {
      dst_o[g * kHeadDim + i] = o / ls[g];
    } else {
      st_coh(dst_o + g * kHeadDim + i, o);
      if (i == 0) {
        st_coh(dst_ml + g * 2 + 0, ms[g]);
        st_coh(dst_ml + g * 2 + 1, ls[g]);
      }
    }
  }
}

template <int G, int VB, bool NF>
__global__ __launch_bounds__(256) void decode_mfma(
    const void* __restrict__ qv, int q_f32, float sigma, int64_t len, int n_kv, int64_t cap,
    int tiles_per_split, const Plan* __restrict__ plans, const Tables* __restrict__ tabg,
    const uint32_t* __restrict__ kc, const uint32_t* __restrict__ vc, const uint16_t* __restrict__ ks,
    const uint16_t* __restrict__ vs, int k_words, int n_nf, int n_splits, float* __restrict__ part_o,
    float* __restrict__ part_ml, float* __restrict__ gpart_o, float* __restrict__ gpart_ml,
    unsigned* __restrict__ counters, float* __restrict__ out) {
  constexpr int HP = 2 * G;                     // query-head parts (hi, lo)
  constexpr int HG = (HP + 3) / 4;              // 4-row groups of parts for the 4x4x4 MFMA
  constexpr int NA = (32 * HG + 15) / 16;       // A-operand registers (16 broadcast blocks each)
  constexpr int PCOLS = HP;                     // P columns: hi of heads 0..G-1, then lo
  constexpr int KWV = 4 * VB;                   // words per dim per V tile

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n_q = n_kv * G;
  const int64_t bh = static_cast<int64_t>(b) * n_kv + h;

  __shared__ __attribute__((aligned(16))) char tab_s[kLdsTableBytes];
  __shared__ __attribute__((aligned(16))) _Float16 p_s[kWaves][PCOLS][kVTile];
  __shared__ float qs_s[G][kHeadDim];
  __shared__ uint8_t fdim_s[kHeadDim];
  __shared__ uint32_t pd_s[kBlocks];
  __shared__ float comb_m[kWaves][G], comb_l[kWaves][G];
  __shared__ bool flag_s;
  extern __shared__ __attribute__((aligned(16))) uint32_t kr_dyn[];   // [kWaves][k_words + 2][128]
  uint32_t* kr = kr_dyn + wave * (k_words + 2) * kVTile;

  const int64_t n_tiles = (len + kVTile - 1) / kVTile;
  const int64_t t_begin = static_cast<int64_t>(s) * tiles_per_split;
  const int64_t t_end = t_begin + tiles_per_split < n_tiles ? t_begin + tiles_per_split : n_tiles;
  const Plan* P = plans + h;

  // ---- per-tile loads (issued for the first tile before the setup work) ----
  uint32_t vseg[8][VB + 2];
  uint4 ka[4], kb2[4];
  float sk0 = 0.f, sk1 = 0.f, sv0 = 0.f, sv1 = 0.f;
  auto load_k = [&](int64_t tile) {
    const int64_t tok0 = tile * kVTile;
    const uint4* krow0 = reinterpret_cast<const uint4*>(kc + (bh * cap + tok0 + lane) * k_words);
    const uint4* krow1 = reinterpret_cast<const uint4*>(kc + (bh * cap + tok0 + 64 + lane) * k_words);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (4 * k < k_words) {
        ka[k] = krow0[k];
        kb2[k] = krow1[k];
      }
    }
  };
  auto load_scales = [&](int64_t tile) {
    const int64_t t0i = tile * kVTile + lane, t1i = t0i + 64;
    if (NF) {
      sk0 = half_bits_to_float(ks[(static_cast<int64_t>(b) * cap + t0i) * n_nf + h / 2]);
      sk1 = half_bits_to_float(ks[(static_cast<int64_t>(b) * cap + t1i) * n_nf + h / 2]);
      sv0 = half_bits_to_float(vs[(static_cast<int64_t>(b) * cap + t0i) * n_nf + h / 2]);
      sv1 = half_bits_to_float(vs[(static_cast<int64_t>(b) * cap + t1i) * n_nf + h / 2]);
    } else {
      sk0 = half_bits_to_float(ks[bh * cap + t0i]);
      sk1 = half_bits_to_float(ks[bh * cap + t1i]);
      sv0 = half_bits_to_float(vs[bh * cap + t0i]);
      sv1 = half_bits_to_float(vs[bh * cap + t1i]);
    }
  };
  auto load_v = [&](int64_t tile) {
    const uint32_t* vt = vc + (bh * (cap / kVTile) + tile) * (kVTile * KWV);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int k = 0; k < VB; ++k) vseg[dt][k + 1] = vt[(dt * 64 + lane) * VB + k];
    }
  };
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) vseg[dt][0] = vseg[dt][VB + 1] = 0u;
  if (t_begin + wave < t_end) {
    load_k(t_begin + wave);
    load_scales(t_begin + wave);
    load_v(t_begin + wave);
  }

  // ---- setup: decode tables, scaled query, field dims, pair descriptors into LDS ----
  {
    const uint4* img = reinterpret_cast<const uint4*>(tabg->lds_image[NF ? 1 : 0]);
    if (tid < kLdsTableBytes / 16) reinterpret_cast<uint4*>(tab_s)[tid] = img[tid];
  }
  for (int k = tid; k < G * kHeadDim; k += blockDim.x) {
    const int hd = k / kHeadDim, i = k % kHeadDim;
    const int64_t qi = (static_cast<int64_t>(b) * n_q + h * G + hd) * kHeadDim + i;
    const float qraw = q_f32 ? static_cast<const float*>(qv)[qi]
                             : __half2float(static_cast<const __half*>(qv)[qi]);
    qs_s[hd][i] = qraw * P->g[i] * sigma;
  }
  const int n_pairs = __builtin_amdgcn_readfirstlane(P->n_fields) >> 1;
  if (tid < kHeadDim) fdim_s[tid] = P->fdim[tid];
  // blocks past the stored ones get a harmless width-1 descriptor (their query part is zero)
  if (tid < kBlocks) pd_s[tid] = tid < n_pairs ? P->pdesc[tid] : (1u << 16);
  kr[lane] = kr[64 + lane] = 0u;
  kr[(k_words + 1) * kVTile + lane] = kr[(k_words + 1) * kVTile + 64 + lane] = 0u;
  __syncthreads();

  // ---- A operands: q' split into hi/lo fp16, laid out for A-broadcast ----
  h4 areg[NA];
  {
    const int blk = lane >> 2, i = lane & 3;
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      const int mi = a * 16 + blk;
      const int st = mi / HG, g = mi % HG;
      const int hp = 4 * g + i;
      const int head = hp >> 1, part = hp & 1;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 2 * st + (k >> 1);
        float qq = 0.0f;
        if (st < 32 && head < G && r < n_pairs) qq = qs_s[head][fdim_s[2 * r + (k & 1)]];
        const _Float16 hi = static_cast<_Float16>(qq);
        areg[a][k] = part ? static_cast<_Float16>(qq - static_cast<float>(hi)) : hi;
      }
    }
  }

  // ---- per-wave state ----
  float m_run[G], l_lane[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_lane[g] = 0.0f;
  }
  f4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f4{0.f, 0.f, 0.f, 0.f};

  for (int64_t tile = t_begin + wave; tile < t_end; tile += kWaves) {
    const int64_t tok0 = tile * kVTile;
    const int64_t next = tile + kWaves;
    const bool ok0 = tok0 + lane < len, ok1 = tok0 + 64 + lane < len;
    // positions past the sequence end get weight 0 below; their stored scales are not used
    const float tk0 = sk0, tk1 = sk1, tv0 = ok0 ? sv0 : 0.f, tv1 = ok1 ? sv1 : 0.f;
    // -- stage the K rows in LDS word-major, then start the next tile's K rows and scales --
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (4 * k < k_words) {
        uint32_t* dst = kr + (4 * k + 1) * kVTile + lane;
        dst[0] = ka[k].x; dst[kVTile] = ka[k].y; dst[2 * kVTile] = ka[k].z; dst[3 * kVTile] = ka[k].w;
        dst[64] = kb2[k].x; dst[kVTile + 64] = kb2[k].y; dst[2 * kVTile + 64] = kb2[k].z;
        dst[3 * kVTile + 64] = kb2[k].w;
      }
    }
    for (int k = 4; 4 * k < k_words; ++k) {   // rows longer than 16 words (more than 4 bits)
      const uint4* krow0 = reinterpret_cast<const uint4*>(kc + (bh * cap + tok0 + lane) * k_words);
      const uint4* krow1 = reinterpret_cast<const uint4*>(kc + (bh * cap + tok0 + 64 + lane) * k_words);
      const uint4 a = krow0[k], c = krow1[k];
      uint32_t* dst = kr + (4 * k + 1) * kVTile + lane;
      dst[0] = a.x; dst[kVTile] = a.y; dst[2 * kVTile] = a.z; dst[3 * kVTile] = a.w;
      dst[64] = c.x; dst[kVTile + 64] = c.y; dst[2 * kVTile + 64] = c.z; dst[3 * kVTile + 64] = c.w;
    }
    if (next < t_end) {
      load_k(next);
      load_scales(next);
    }
    // -- keys: logits of the two 64-token halves --
    f4 acc0[HG], acc1[HG];
#pragma unroll
    for (int g = 0; g < HG; ++g) acc0[g] = acc1[g] = f4{0.f, 0.f, 0.f, 0.f};
    static_for<32>([&](auto stc) {
      constexpr int st = decltype(stc)::value;
      // pair descriptors (bit offset | width << 16) are wave-uniform
      const uint32_t d0 = __builtin_amdgcn_readfirstlane(pd_s[2 * st]);
      const uint32_t d1 = __builtin_amdgcn_readfirstlane(pd_s[2 * st + 1]);
      uint32_t b00, b10, b01, b11;
      k_pair2(kr, lane, static_cast<int>(d0 & 0xFFFFu), static_cast<int>(d0 >> 16), tab_s, b00, b10);
      k_pair2(kr, lane, static_cast<int>(d1 & 0xFFFFu), static_cast<int>(d1 >> 16), tab_s, b01, b11);
      h4 bv0, bv1;
      const uint32_t u0[2] = {b00, b01}, u1[2] = {b10, b11};
      __builtin_memcpy(&bv0, u0, 8);
      __builtin_memcpy(&bv1, u1, 8);
      static_for<HG>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        constexpr int mi = st * HG + g;
        acc0[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(areg[mi / 16], bv0, acc0[g], 4, mi % 16, 0);
        acc1[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(areg[mi / 16], bv1, acc1[g], 4, mi % 16, 0);
      });
    });
    float lg0[G], lg1[G];
#pragma unroll
    for (int hd = 0; hd < G; ++hd) {
      const int hp = 2 * hd;
      lg0[hd] = ok0 ? (acc0[hp / 4][hp % 4] + acc0[hp / 4][hp % 4 + 1]) * tk0 : -INFINITY;
      lg1[hd] = ok1 ? (acc1[hp / 4][hp % 4] + acc1[hp / 4][hp % 4 + 1]) * tk1 : -INFINITY;
    }
    // -- online softmax over the 128-token tile --
    bool rescale = false;
    float al_h[G];
#pragma unroll
    for (int hd = 0; hd < G; ++hd) {
      const float mt = wave_max(fmaxf(lg0[hd], lg1[hd]));
      const float mn = fmaxf(m_run[hd], mt);
      const float al = exp2f(m_run[hd] - mn);
      rescale |= al != 1.0f;
      al_h[hd] = al;
      m_run[hd] = mn;
      const float p0 = exp2f(lg0[hd] - mn), p1 = exp2f(lg1[hd] - mn);
      l_lane[hd] = l_lane[hd] * al + p0 + p1;
      const float q0 = p0 * tv0, q1 = p1 * tv1;
      const _Float16 q0h = static_cast<_Float16>(q0), q1h = static_cast<_Float16>(q1);
      p_s[wave][hd][lane] = q0h;
      p_s[wave][hd][64 + lane] = q1h;
      p_s[wave][G + hd][lane] = static_cast<_Float16>(q0 - static_cast<float>(q0h));
      p_s[wave][G + hd][64 + lane] = static_cast<_Float16>(q1 - static_cast<float>(q1h));
    }
    wave_sync();
    if (rescale) {
      // output column n = lane % 16 belongs to head n % G (columns >= 2G are unused)
      const int col = lane & 15;
      float al = 1.0f;
#pragma unroll
      for (int hd = 0; hd < G; ++hd)
        if (col < PCOLS && col % G == hd) al = al_h[hd];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[dt] *= al;
    }
    // -- values: O^T[dim][col] += V^T[dim][tok] P^T[tok][col] over 4 chunks of 32 tokens --
    {
      const int col = lane & 15, grp = lane >> 4;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        h8 bp;
        if (col < PCOLS) {
          bp = *reinterpret_cast<const h8*>(&p_s[wave][col][32 * grp + 8 * c]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) bp[e] = static_cast<_Float16>(0.0f);
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          uint32_t pr[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) pr[e] = v_pair<VB>(&vseg[dt][1], 8 * c + 2 * e, tab_s);
          h8 av;
          __builtin_memcpy(&av, pr, 16);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bp, oacc[dt], 0, 0, 0);
        }
      }
    }
    wave_sync();
    if (next < t_end) load_v(next);
  }

  // ---- merge the 4 waves of this workgroup ----
  float lw[G];
#pragma unroll
  for (int hd = 0; hd < G; ++hd) lw[hd] = wave_sum(l_lane[hd]);
  if (lane == 0) {
#pragma unroll
    for (int hd = 0; hd < G; ++hd) {
      comb_m[wave][hd] = m_run[hd];
      comb_l[wave][hd] = lw[hd];
    }
  }
  // O^T layout: lane holds rows 4*(lane/16)+r of dim-slice dt for column lane%16;
  // add the lo column (col + G) into the hi column (col)
  float* o_s = reinterpret_cast<float*>(&p_s[0][0][0]);   // reuse: [kWaves][G][128] floats
  __syncthreads();
  {
    const int col = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float other = __shfl(oacc[dt][r], (lane & ~15) | ((col + G) & 15), 64);
        if (col < G) o_s[(wave * G + col) * kHeadDim + dt * 16 + 4 * grp + r] = oacc[dt][r] + other;
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * kHeadDim; idx += blockDim.x) {
    const int hd = idx / kHeadDim, i = idx % kHeadDim;
    float ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) ms = fmaxf(ms, comb_m[w][hd]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = comb_m[w][hd];
      if (mw == -INFINITY) continue;
      const float sc = exp2f(mw - ms);
      o += sc * o_s[(w * G + hd) * kHeadDim + i];
      l += sc * comb_l[w][hd];
    }
    const int64_t p = (bh * n_splits + s) * G + hd;
    st_coh(part_o + p * kHeadDim + i, o);
    if (i == 0) {
      st_coh(part_ml + p * 2 + 0, ms);
      st_coh(part_ml + p * 2 + 1, l);
    }
  }

  // ---- split merge, two levels ----
  const int grp = s / kGroup;
  const int n_groups = (n_splits + kGroup - 1) / kGroup;
  const int gsize = n_splits - grp * kGroup < kGroup ? n_splits - grp * kGroup : kGroup;
  unsigned* cnt = counters + bh * (kMaxGroups + 1);
  float* mw_s = reinterpret_cast<float*>(kr_dyn);   // merge scratch: 2 x [kGroup][G] + 2 x [G]
  if (!arrive(cnt + grp, static_cast<unsigned>(gsize), &flag_s)) return;
  {
    const int64_t src = (bh * n_splits + grp * kGroup) * G;
    if (n_groups == 1) {
      merge_level<G>(part_o + src * kHeadDim, part_ml + src * 2, gsize, mw_s, tid,
                     out + (static_cast<int64_t>(b) * n_q + h * G) * kHeadDim, nullptr, true);
      if (tid == 0) __hip_atomic_store(cnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    const int64_t dst = (bh * kMaxGroups + grp) * G;
    merge_level<G>(part_o + src * kHeadDim, part_ml + src * 2, gsize, mw_s, tid,
                   gpart_o + dst * kHeadDim, gpart_ml + dst * 2, false);
  }
  if (tid == 0) __hip_atomic_store(cnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!arrive(cnt + kMaxGroups, static_cast<unsigned>(n_groups), &flag_s)) return;
  {
    const int64_t src = bh * kMaxGroups * G;
    merge_level<G>(gpart_o + src * kHeadDim, gpart_ml + src * 2, n_groups, mw_s, tid,
                   out + (static_cast<int64_t>(b) * n_q + h * G) * kHeadDim, nullptr, true);
  }
  if (tid == 0) __hip_atomic_store(cnt + kMaxGroups, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int G, int VB>
hipError_t launch_gv(kvq_cache* c, int layer, const void* q, int q_f32, float sigma, float* out,
                     int S, hipStream_t stream) {
  const kvq_config& cfg = c->cfg;
  const int64_t len = c->len[layer];
  const int64_t n_tiles = (len + kVTile - 1) / kVTile;
  const int tps = static_cast<int>((n_tiles + S - 1) / S);
  dim3 grid(S, cfg.n_kv_heads, cfg.batch);
  const size_t dyn = static_cast<size_t>(kWaves) * (c->k_words + 2) * kVTile * sizeof(uint32_t);
  const Plan* plans = c->plans + static_cast<int64_t>(layer) * cfg.n_kv_heads;
  const bool nf = cfg.codec == KVQ_CODEC_NF16_B256;
  if constexpr (VB == 4) {
    if (nf) {
      hipLaunchKernelGGL((decode_mfma<G, 4, true>), grid, dim3(256), dyn, stream, q, q_f32, sigma, len,
                         cfg.n_kv_heads, c->cap, tps, plans, c->tables, layer_k_codes(c, layer),
                         layer_v_codes(c, layer), layer_k_scales(c, layer), layer_v_scales(c, layer),
                         c->k_words, c->n_nf_blocks, S, c->part_o, c->part_ml, c->gpart_o, c->gpart_ml,
                         c->split_counters, out);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_mfma<G, VB, false>), grid, dim3(256), dyn, stream, q, q_f32, sigma, len,
                     cfg.n_kv_heads, c->cap, tps, plans, c->tables, layer_k_codes(c, layer),
                     layer_v_codes(c, layer), layer_k_scales(c, layer), layer_v_scales(c, layer),
                     c->k_words, c->n_nf_blocks, S, c->part_o, c->part_ml, c->gpart_o, c->gpart_ml,
                     c->split_counters, out);
  return hipGetLastError();
}

template <int G>
hipError_t launch_group(kvq_cache* c, int layer, const void* q, int q_f32, float sigma, float* out,
                        int S, hipStream_t stream) {
  const int vb = c->cfg.codec == KVQ_CODEC_NF16_B256 ? 4 : c->cfg.v_bits;
  switch (vb) {
    case 1: return launch_gv<G, 1>(c, layer, q, q_f32, sigma, out, S, stream);
    case 2: return launch_gv<G, 2>(c, layer, q, q_f32, sigma, out, S, stream);
    case 3: return launch_gv<G, 3>(c, layer, q, q_f32, sigma, out, S, stream);
    case 4: return launch_gv<G, 4>(c, layer, q, q_f32, sigma, out, S, stream);
    case 5: return launch_gv<G, 5>(c, layer, q, q_f32, sigma, out, S, stream);
    case 6: return launch_gv<G, 6>(c, layer, q, q_f32, sigma, out, S, stream);
    case 7: return launch_gv<G, 7>(c, layer, q, q_f32, sigma, out, S, stream);
    default: return launch_gv<G, 8>(c, layer, q, q_f32, sigma, out, S, stream);
  }
}

}  // namespace mfma
}  // namespace kvq
