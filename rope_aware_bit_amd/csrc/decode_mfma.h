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

#include "kvq_internal.h"

namespace kvq {
namespace mfma {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) void* glb_ptr;
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kGroup = 16;        // splits merged per first-level merger
constexpr int kMaxGroups = 16;    // so at most kGroup * kMaxGroups = 256 splits
constexpr int kKS = 144;          // LDS row stride (words) of a staged K tile: 128 tokens + 16
constexpr int kPS = 136;          // LDS row stride (halves) of the softmax weights: 128 + 8
constexpr int kOS = 10;           // LDS stride (floats) per dim of a wave's merge share: G <= 8, + 2
constexpr int kAS = 40;           // LDS row stride (halves) of the query operand: 32 + 8
// LDS table region (bytes).  Pair tables hold fp16x2 (CB_w[c0], CB_w[c1]) at index c0 | c1 << w.
// Random lookups into the larger tables would collide in LDS banks, so they are replicated:
// the width-4 table 16 times (entry p of copy k at (p << 6) + 4 k, lane l reads copy l % 16)
// and the width-3 table 32 times (entry p of copy k at (p << 7) + 4 k, lane l reads copy
// l % 32).  The width-5 table is a single copy (entry p at p << 2), built per workgroup when
// the plan uses it.  The prebuilt image holds the pair tables of widths 1..4 and the single
// tables of widths 1..8.  Every base is a multiple of its table's extent, so an entry address
// is "(p << shift) | copy offset | base".  Blocks of 6..8 bits use two single lookups.
constexpr int kRep4Base = 0;           // 16 KB
constexpr int kRep3Base = 16384;       // 8 KB
constexpr int kPair5Base = 24576;      // 4 KB
constexpr int kImageBase = 28672;      // 2.5 KB
constexpr int kTableRegion = kImageBase + kLdsTableBytes;

// Lookup parameters of a pair of width w: base (without the lane's copy offset) | copy kind
// << 16 (0 single, 1 sixteen copies, 2 thirty-two copies) | extract width << 24.  For widths of
// 6..8 the pair lookup stays inside the width-5 table and its result is replaced.
__device__ inline uint32_t pair_lookup_params(uint32_t w) {
  uint32_t base, kind = 0u;
  if (w == 4u) { base = kRep4Base; kind = 1u; }
  else if (w == 3u) { base = kRep3Base; kind = 2u; }
  else if (w >= 5u) base = kPair5Base;
  else base = kImageBase + static_cast<uint32_t>(pair_table_base(static_cast<int>(w)));
  const uint32_t bw = w <= 5u ? 2u * w : 10u;
  return base | (kind << 16) | (bw << 24);
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

// Max / sum over the 16 lanes of a row (lanes 16 r .. 16 r + 15); the result is in every
// lane of the row.
__device__ inline float row_max16(float v) {
  v = fmaxf(v, KVQ_DPP(v, 0x128));
  v = fmaxf(v, KVQ_DPP(v, 0x124));
  v = fmaxf(v, KVQ_DPP(v, 0x122));
  v = fmaxf(v, KVQ_DPP(v, 0x121));
  return v;
}
__device__ inline float row_sum16(float v) {
  v += KVQ_DPP(v, 0x128);
  v += KVQ_DPP(v, 0x124);
  v += KVQ_DPP(v, 0x122);
  v += KVQ_DPP(v, 0x121);
  return v;
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
__device__ __attribute__((always_inline)) inline bool arrive(unsigned* counter, unsigned expected, bool* flag_s) {
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

// fp16 pair of V codes e, e+1 (e even) of a 32-code segment held in S[0..VB) (S[VB] is a
// zero word).  `tab` is the table region, `lb` the lane's replica offset (lane % 32) * 4 (the
// sixteen-copy table uses its low six bits).
template <int VB>
__device__ inline uint32_t v_pair(const uint32_t* S, int e, const char* tab, uint32_t lb) {
  if constexpr (VB <= 4) {
    const int off = e * VB, w0 = off >> 5, sh = off & 31;
    uint32_t code;
    if (sh + 2 * VB <= 32) code = __builtin_amdgcn_ubfe(S[w0], sh, 2 * VB);
    else code = __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(S[w0 + 1], S[w0], sh), 0, 2 * VB);
    if constexpr (VB == 4) {
      return lds_u32(tab, (code << 6) | (lb & 63u) | kRep4Base);
    } else if constexpr (VB == 3) {
      return lds_u32(tab, (code << 7) | lb | kRep3Base);
    } else {
      return lds_u32(tab + kImageBase, (code << 2) | static_cast<uint32_t>(pair_table_base(VB)));
    }
  } else {
    constexpr uint32_t mask = ((1u << VB) - 1u) << 1;
    const int a0 = e * VB + 31, a1 = (e + 1) * VB + 31;
    const uint32_t x0 = __builtin_amdgcn_alignbit(S[(a0 >> 5)], S[(a0 >> 5) - 1], a0 & 31);
    const uint32_t x1 = __builtin_amdgcn_alignbit(S[(a1 >> 5)], S[(a1 >> 5) - 1], a1 & 31);
    constexpr uint32_t sb = static_cast<uint32_t>(single_table_base(VB));
    return lds_u16(tab + kImageBase, (x0 & mask) | sb) | (lds_u16(tab + kImageBase, (x1 & mask) | sb) << 16);
  }
}

// Merge `count` (1..kGroup) consecutive split partials of one (sequence, KV head):
// partial e holds, per head g, (m, l) at ml[(e*G + g)*2 + {0,1}] and the unnormalised
// output at o[(e*G + g)*128 + i].  m* = max_e m_e, l = sum_e 2^(m_e - m*) l_e and
// o = sum_e 2^(m_e - m*) o_e, in e order.  Writes either the merged partial or, if
// `final_out`, o / l to dst_o[g*128 + i].  All loads are issued before any result is
// needed, so the merge costs one round of memory latency.
template <int G, int NT>
__device__ __attribute__((always_inline)) inline void merge_level(const float* __restrict__ src_o, const float* __restrict__ src_ml,
                                   int count, float* mw, int tid, float* __restrict__ dst_o,
                                   float* __restrict__ dst_ml, bool final_out) {
  constexpr int NOUT = G * kHeadDim;
  constexpr int OPT = (NOUT + NT - 1) / NT;
  float ov[OPT][kGroup];
#pragma unroll
  for (int k = 0; k < OPT; ++k) {
    const int idx = (tid + NT * k) % NOUT;
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
    const int idx = tid + NT * k;
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

// One chunk of the key product for lane (n, g): the query operand, the lookup parameters of
// the lane's four pairs (plan ranks 16 c + 4 g .. + 3) and the two 32-bit row windows (pairs
// 0-1 and 2-3) of each of its 8 tokens 16 tg + n.
struct KChunk {
  h8 aq;
  uint32_t shA, shB, rel1, rel3, baseA, baseB;
  uint32_t wp[4], bw[4], pb[4], ps[4];
  uint32_t la[8], ha[8], lb[8], hb[8];
};

__device__ __attribute__((always_inline)) inline KChunk k_chunk_params(
    int c, int g, int n, const uint32_t* pd_s, const uint32_t* px_s, const _Float16 (*a_s)[16][kAS],
    uint32_t lane_copy, const uint32_t* kr) {
  KChunk k;
  k.aq = *reinterpret_cast<const h8*>(&a_s[c][n][8 * g]);
  const int grp = 4 * c + g;
  const uint4 dd = *reinterpret_cast<const uint4*>(&pd_s[4 * grp]);
  const uint4 xx = *reinterpret_cast<const uint4*>(&px_s[4 * grp]);
  const uint32_t d4[4] = {dd.x, dd.y, dd.z, dd.w}, x4[4] = {xx.x, xx.y, xx.z, xx.w};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    k.wp[p] = d4[p] >> 16;
    k.bw[p] = x4[p] >> 24;
    const uint32_t kind = (x4[p] >> 16) & 3u;
    k.pb[p] = (x4[p] & 0xFFFFu) | (kind == 2u ? lane_copy : kind == 1u ? (lane_copy & 63u) : 0u);
    k.ps[p] = kind == 2u ? 7u : kind == 1u ? 6u : 2u;
  }
  const uint32_t offA = d4[0] & 0xFFFFu, offB = d4[2] & 0xFFFFu;
  k.shA = offA & 31u;
  k.shB = offB & 31u;
  k.rel1 = 2u * k.wp[0];
  k.rel3 = 2u * k.wp[2];
  k.baseA = (offA >> 5) * kKS + n;
  k.baseB = (offB >> 5) * kKS + n;
  return k;
}

__device__ __attribute__((always_inline)) inline void k_chunk_windows(KChunk& k, const uint32_t* kr) {
#pragma unroll
  for (int tg = 0; tg < 8; ++tg) {
    k.la[tg] = kr[k.baseA + 16 * tg];
    k.ha[tg] = kr[k.baseA + 16 * tg + kKS];
    k.lb[tg] = kr[k.baseB + 16 * tg];
    k.hb[tg] = kr[k.baseB + 16 * tg + kKS];
  }
}

// Decode kernel.  W waves per workgroup (one or two per SIMD).  Every wave owns a region of
// `region_words` LDS words that holds, in turn, its staged K tile, its softmax weights and its
// share of the wave merge (and, during set-up, wave 0's region holds the scaled query).
template <int G, int VB, bool NF, int W>
__global__ __launch_bounds__(64 * W, W / 4) void decode_mfma(
    const void* __restrict__ qv, int q_f32, float sigma, int64_t len, int n_kv, int64_t cap,
    int tiles_per_split, const Plan* __restrict__ plans, const Tables* __restrict__ tabg,
    const uint32_t* __restrict__ kc, const uint32_t* __restrict__ vc, const uint16_t* __restrict__ ks,
    const uint16_t* __restrict__ vs, int k_words, int n_nf, int n_splits, int region_words,
    int v_early, int v_off, float* __restrict__ part_o, float* __restrict__ part_ml, float* __restrict__ gpart_o,
    float* __restrict__ gpart_ml, unsigned* __restrict__ counters, float* __restrict__ out) {
  constexpr int NT = 64 * W;
  constexpr bool kPipe = W == 4;                      // one wave per SIMD: prefetch and pipeline
  constexpr int PCOLS = 2 * G;                        // P columns: hi of heads 0..G-1, then lo
  constexpr int KWV = 4 * VB;                         // words per dim per V tile
  constexpr int QPT = (G * kHeadDim + 255) / 256;     // query values per set-up thread

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, g = lane >> 4;             // MFMA column and row group of this lane
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n_q = n_kv * G;
  const int64_t bh = static_cast<int64_t>(b) * n_kv + h;

  __shared__ __attribute__((aligned(16))) char tab_s[kTableRegion];
  __shared__ __attribute__((aligned(16))) _Float16 a_s[4][16][kAS];
  __shared__ uint8_t fdim_s[kHeadDim];
  __shared__ __attribute__((aligned(16))) uint32_t pd_s[kBlocks];
  __shared__ __attribute__((aligned(16))) uint32_t px_s[kBlocks];
  __shared__ float comb_m[W][G], comb_l[W][G];
  __shared__ float alpha_s[W][G];
  __shared__ bool flag_s;
  __shared__ uint64_t wide_s;
  __shared__ float sc_s[W][G], ms_s[G], ls_s[G];
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn_s[];   // [W][region_words]
  uint32_t* kr = dyn_s + wave * region_words;                         // [k_words + 1][kKS]
  _Float16* pw = reinterpret_cast<_Float16*>(kr);                     // [PCOLS][kPS], after keys
  uint32_t* vbuf = kr + v_off;                                        // [512][VB] V tile
  float (*qs_s)[kHeadDim] = reinterpret_cast<float (*)[kHeadDim]>(dyn_s);   // set-up only

  const int64_t n_tiles = (len + kVTile - 1) / kVTile;
  const int64_t t_begin = static_cast<int64_t>(s) * tiles_per_split;
  const int64_t t_end = t_begin + tiles_per_split < n_tiles ? t_begin + tiles_per_split : n_tiles;
  const Plan* P = plans + h;

  // ---- set-up loads first (small and shared by every workgroup), then the first tile's.
  //      Waves 0..3 do the set-up; a wave-uniform branch lets the others skip it. ----
  const bool setup_wave = __builtin_amdgcn_readfirstlane(wave) < 4;
  const uint8_t* gimg = tabg->lds_image[NF ? 1 : 0];
  const int n_pairs = __builtin_amdgcn_readfirstlane(P->n_fields) >> 1;
  uint4 timg = make_uint4(0u, 0u, 0u, 0u);
  float qr[QPT], gr[QPT];
  uint32_t fd_r = 0u, pd_r = 0u, rep4v = 0u, rep3v = 0u, hi5 = 0u;
  uint2 lo5 = make_uint2(0u, 0u);
  if (setup_wave) {
    if (tid < kLdsTableBytes / 16) timg = reinterpret_cast<const uint4*>(gimg)[tid];
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int k = tid + 256 * j;
      qr[j] = gr[j] = 0.0f;
      if (k < G * kHeadDim) {
        const int64_t qi = (static_cast<int64_t>(b) * n_q + h * G) * kHeadDim + k;
        qr[j] = q_f32 ? static_cast<const float*>(qv)[qi] : __half2float(static_cast<const __half*>(qv)[qi]);
        gr[j] = P->g[k % kHeadDim];
      }
    }
    if (tid < kHeadDim) fd_r = P->fdim[tid];
    pd_r = P->pdesc[lane];   // descriptor of pair `lane`
    // sources of the per-workgroup pair tables (see below)
    rep4v = reinterpret_cast<const uint32_t*>(gimg + pair_table_base(4))[tid];
    rep3v = reinterpret_cast<const uint32_t*>(gimg + pair_table_base(3))[tid & 63];
    const uint16_t* cb5 = reinterpret_cast<const uint16_t*>(gimg + single_table_base(5));
    hi5 = cb5[tid >> 3];
    lo5 = *reinterpret_cast<const uint2*>(cb5 + ((4 * tid) & 31));
  }

  // K rows of tokens lane and lane + 64 (first 16 words), scales of tokens 16 tg + n, V segments
  uint4 ka[4], kb2[4];
  float skr[8], svr[8];
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
#pragma unroll
    for (int tg = 0; tg < 8; ++tg) {
      const int64_t t = tile * kVTile + 16 * tg + n;
      if (NF) {
        skr[tg] = half_bits_to_float(ks[(static_cast<int64_t>(b) * cap + t) * n_nf + h / 2]);
        svr[tg] = half_bits_to_float(vs[(static_cast<int64_t>(b) * cap + t) * n_nf + h / 2]);
      } else {
        skr[tg] = half_bits_to_float(ks[bh * cap + t]);
        svr[tg] = half_bits_to_float(vs[bh * cap + t]);
      }
    }
  };
  // the V tile (512 segments x VB words, contiguous in HBM) goes straight into this wave's LDS
  // area: 2 VB copies of 64 lanes x 16 bytes, waited for with s_waitcnt vmcnt(0) before use
  auto dma_v = [&](int64_t tile) {
    const uint32_t* vt = vc + (bh * (cap / kVTile) + tile) * (kVTile * KWV);
#pragma unroll
    for (int i = 0; i < 2 * VB; ++i)
      __builtin_amdgcn_global_load_lds((glb_ptr)(vt + 256 * i + 4 * lane), (lds_ptr)(vbuf + 256 * i), 16, 0, 0);
  };
  if (t_begin + wave < t_end) {
    load_k(t_begin + wave);
    load_scales(t_begin + wave);
    if (v_early) dma_v(t_begin + wave);
  }

  // ---- set-up: tables, scaled query, field dims and pair descriptors into LDS ----
  if (setup_wave) {
    if (tid < kLdsTableBytes / 16) reinterpret_cast<uint4*>(tab_s + kImageBase)[tid] = timg;
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int k = tid + 256 * j;
      if (k < G * kHeadDim) qs_s[k / kHeadDim][k % kHeadDim] = qr[j] * gr[j] * sigma;
    }
    if (tid < kHeadDim) fdim_s[tid] = static_cast<uint8_t>(fd_r);
    if (tid < kBlocks) {
      pd_s[tid] = pd_r;
      px_s[tid] = pair_lookup_params(pd_r >> 16);
    }
    // replicas of the width-4 (16 copies) and width-3 (32 copies) pair tables: thread t writes
    // all copies of entry t (rotating the 16-byte pieces over the lanes spreads the banks)
    {
      const uint4 v4 = make_uint4(rep4v, rep4v, rep4v, rep4v), v3 = make_uint4(rep3v, rep3v, rep3v, rep3v);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int jj = (j + tid) & 3;
        *reinterpret_cast<uint4*>(tab_s + kRep4Base + (tid << 6) + 16 * jj) = v4;
      }
      if (tid < 64) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int jj = (j + tid) & 7;
          *reinterpret_cast<uint4*>(tab_s + kRep3Base + (tid << 7) + 16 * jj) = v3;
        }
      }
    }
    // pair table of width 5 when the plan stores such blocks: entry (c1 << 5) | c0 holds
    // (CB_5[c0], CB_5[c1]); thread t fills 4 consecutive c0 of one c1
    const uint64_t uses5 = __ballot((pd_r >> 16) == 5u);
    const uint64_t wide = __ballot((pd_r >> 16) >= 6u);
    if (tid == 0) wide_s = wide;
    if (uses5) {
      const uint32_t hi = hi5 << 16;
      const uint4 v = make_uint4((lo5.x & 0xFFFFu) | hi, (lo5.x >> 16) | hi, (lo5.y & 0xFFFFu) | hi, (lo5.y >> 16) | hi);
      *reinterpret_cast<uint4*>(tab_s + kPair5Base + 4 * (4 * tid)) = v;
    }
  }
  __syncthreads();
  // query operand of the key product: a_s[c][m][k] = hi (m even) or lo (m odd) fp16 part of
  // q'[m / 2][dim of field 32 c + k]; rows of heads >= G and fields past the stored ones are 0.
  // Thread t < 256 fills field t % 128 for heads t / 128, t / 128 + 2, ...
  if (setup_wave) {
    const int f = tid & 127, c = f >> 5, k = f & 31;
    const bool live = f < 2 * n_pairs;
    const int dim = fdim_s[f];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hh = 2 * j + (tid >> 7);
      const float qq = (hh < G && live) ? qs_s[hh < G ? hh : 0][dim] : 0.0f;
      const _Float16 hi = static_cast<_Float16>(qq);
      a_s[c][2 * hh][k] = hi;
      a_s[c][2 * hh + 1][k] = static_cast<_Float16>(qq - static_cast<float>(hi));
    }
  }
  const uint32_t lb = (lane & 31u) << 2;   // this lane's replica offset
  __syncthreads();
  const uint64_t uses_wide = wide_s;       // pairs (plan ranks) with blocks of 6..8 bits

  // ---- per-wave state: lane (n, g) keeps heads 2g, 2g + 1 ----
  const int h0 = 2 * g, h1 = 2 * g + 1;
  const bool vh0 = h0 < G, vh1 = h1 < G;
  float m0 = -INFINITY, m1 = -INFINITY, l0 = 0.0f, l1 = 0.0f;
  f4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f4{0.f, 0.f, 0.f, 0.f};

  for (int64_t tile = t_begin + wave; tile < t_end; tile += W) {
    const int64_t tok0 = tile * kVTile;
    const int64_t next = tile + W;
    if constexpr (!kPipe) {
      if (tile != t_begin + wave) {   // later tiles: loaded here (the other wave hides the wait)
        load_k(tile);
        load_scales(tile);
        if (v_early) dma_v(tile);
      }
    }
    // -- stage the K rows in LDS word-major (kr[d * kKS + tau] = word d of token tau), then a
    //    zero row after them (the area held the previous tile's softmax weights) --
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (4 * k < k_words) {
        uint32_t* dst = kr + 4 * k * kKS + lane;
        dst[0] = ka[k].x; dst[kKS] = ka[k].y; dst[2 * kKS] = ka[k].z; dst[3 * kKS] = ka[k].w;
        dst[64] = kb2[k].x; dst[kKS + 64] = kb2[k].y; dst[2 * kKS + 64] = kb2[k].z; dst[3 * kKS + 64] = kb2[k].w;
      }
    }
    for (int k = 4; 4 * k < k_words; ++k) {   // rows longer than 16 words (more than 4 bits)
      const uint4* krow0 = reinterpret_cast<const uint4*>(kc + (bh * cap + tok0 + lane) * k_words);
      const uint4* krow1 = reinterpret_cast<const uint4*>(kc + (bh * cap + tok0 + 64 + lane) * k_words);
      const uint4 x0 = krow0[k], x1 = krow1[k];
      uint32_t* dst = kr + 4 * k * kKS + lane;
      dst[0] = x0.x; dst[kKS] = x0.y; dst[2 * kKS] = x0.z; dst[3 * kKS] = x0.w;
      dst[64] = x1.x; dst[kKS + 64] = x1.y; dst[2 * kKS + 64] = x1.z; dst[3 * kKS + 64] = x1.w;
    }
    kr[k_words * kKS + lane] = kr[k_words * kKS + 64 + lane] = 0u;
    wave_sync();
    if constexpr (kPipe) {
      if (next < t_end) load_k(next);
    }

    // -- keys: D[part][token] = sum over fields of q'[part][field] * CB[code[token][field]],
    //    one 16x16x32 product per (chunk of 16 pairs, group of 16 tokens).  Chunks past the
    //    stored pairs have zero descriptors and a zero query operand, so all four are processed
    //    without branches. --
    f4 dacc[8];
#pragma unroll
    for (int tg = 0; tg < 8; ++tg) dacc[tg] = f4{0.f, 0.f, 0.f, 0.f};
    auto k_lookups = [&](const KChunk& cur, int c, uint32_t (&u)[8][4]) {
#pragma unroll
      for (int tg = 0; tg < 8; ++tg) {
        const uint32_t xa = __builtin_amdgcn_alignbit(cur.ha[tg], cur.la[tg], cur.shA);
        const uint32_t xb = __builtin_amdgcn_alignbit(cur.hb[tg], cur.lb[tg], cur.shB);
        u[tg][0] = lds_u32(tab_s, (__builtin_amdgcn_ubfe(xa, 0u, cur.bw[0]) << cur.ps[0]) | cur.pb[0]);
        u[tg][1] = lds_u32(tab_s, (__builtin_amdgcn_ubfe(xa, cur.rel1, cur.bw[1]) << cur.ps[1]) | cur.pb[1]);
        u[tg][2] = lds_u32(tab_s, (__builtin_amdgcn_ubfe(xb, 0u, cur.bw[2]) << cur.ps[2]) | cur.pb[2]);
        u[tg][3] = lds_u32(tab_s, (__builtin_amdgcn_ubfe(xb, cur.rel3, cur.bw[3]) << cur.ps[3]) | cur.pb[3]);
      }
      if ((uses_wide >> (16 * c)) & 0xFFFFull) {
        // blocks of 6..8 bits: two single lookups (lanes whose pair is narrower skip)
        const char* tabi = tab_s + kImageBase;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          if (cur.wp[p] >= 6u) {
            const uint32_t sb = static_cast<uint32_t>(kLdsTableBytes) - (4u << cur.wp[p]);
            const uint32_t rel = (p & 1) ? (p == 1 ? cur.rel1 : cur.rel3) : 0u;
#pragma unroll
            for (int tg = 0; tg < 8; ++tg) {
              const uint32_t x = (p < 2) ? __builtin_amdgcn_alignbit(cur.ha[tg], cur.la[tg], cur.shA)
                                         : __builtin_amdgcn_alignbit(cur.hb[tg], cur.lb[tg], cur.shB);
              const uint32_t f0 = __builtin_amdgcn_ubfe(x, rel, cur.wp[p]);
              const uint32_t f1 = __builtin_amdgcn_ubfe(x, rel + cur.wp[p], cur.wp[p]);
              u[tg][p] = lds_u16(tabi, (f0 << 1) | sb) | (lds_u16(tabi, (f1 << 1) | sb) << 16);
            }
          }
        }
      }
    };
    auto k_products = [&](const KChunk& cur, const uint32_t (&u)[8][4]) {
#pragma unroll
      for (int tg = 0; tg < 8; ++tg) {
        h8 bk;
        __builtin_memcpy(&bk, u[tg], 16);
        dacc[tg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur.aq, bk, dacc[tg], 0, 0, 0);
      }
    };
    if constexpr (kPipe) {
      // software pipeline: chunk c + 1's descriptors and row windows are read while chunk c's
      // lookups and products run
      KChunk cur = k_chunk_params(0, g, n, pd_s, px_s, a_s, lb, kr);
      k_chunk_windows(cur, kr);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        KChunk nxt;
        if (c + 1 < 4) nxt = k_chunk_params(c + 1, g, n, pd_s, px_s, a_s, lb, kr);
        uint32_t u[8][4];
        k_lookups(cur, c, u);
        if (c + 1 < 4) k_chunk_windows(nxt, kr);
        k_products(cur, u);
        if (c + 1 < 4) cur = nxt;
      }
    } else {
#pragma unroll 1
      for (int c = 0; c < 4; ++c) {
        KChunk cur = k_chunk_params(c, g, n, pd_s, px_s, a_s, lb, kr);
        k_chunk_windows(cur, kr);
        uint32_t u[8][4];
        k_lookups(cur, c, u);
        k_products(cur, u);
      }
    }
    wave_sync();   // the key rows are read; the area takes the softmax weights (and V) next
    if (!v_early) dma_v(tile);

    // -- online softmax: lane (n, g) holds heads 2g and 2g + 1 of tokens 16 tg + n --
    float L0[8], L1[8];
    float mt0 = -INFINITY, mt1 = -INFINITY;
#pragma unroll
    for (int tg = 0; tg < 8; ++tg) {
      const bool ok = tok0 + 16 * tg + n < len;
      L0[tg] = ok ? (dacc[tg][0] + dacc[tg][1]) * skr[tg] : -INFINITY;
      L1[tg] = ok ? (dacc[tg][2] + dacc[tg][3]) * skr[tg] : -INFINITY;
      mt0 = fmaxf(mt0, L0[tg]);
      mt1 = fmaxf(mt1, L1[tg]);
    }
    mt0 = row_max16(mt0);
    mt1 = row_max16(mt1);
    const float mn0 = fmaxf(m0, mt0), mn1 = fmaxf(m1, mt1);
    // hardware 2^x: arguments are <= 0 and results below the fp32 normal range only
    // ever meet sums >= 1, so flushing them changes nothing that is kept
    const float al0 = __builtin_amdgcn_exp2f(m0 - mn0), al1 = __builtin_amdgcn_exp2f(m1 - mn1);
    m0 = mn0;
    m1 = mn1;
    l0 *= al0;
    l1 *= al1;
#pragma unroll
    for (int tg = 0; tg < 8; ++tg) {
      const bool ok = tok0 + 16 * tg + n < len;
      const float sv = ok ? svr[tg] : 0.0f;   // stored scales past the sequence end are not used
      const float p0 = __builtin_amdgcn_exp2f(L0[tg] - mn0), p1 = __builtin_amdgcn_exp2f(L1[tg] - mn1);
      l0 += p0;
      l1 += p1;
      const float q0 = p0 * sv, q1 = p1 * sv;
      const _Float16 q0h = static_cast<_Float16>(q0), q1h = static_cast<_Float16>(q1);
      const int t = 16 * tg + n;
      if (vh0) {
        pw[h0 * kPS + t] = q0h;
        pw[(G + h0) * kPS + t] = static_cast<_Float16>(q0 - static_cast<float>(q0h));
      }
      if (vh1) {
        pw[h1 * kPS + t] = q1h;
        pw[(G + h1) * kPS + t] = static_cast<_Float16>(q1 - static_cast<float>(q1h));
      }
    }
    if (n == 0) {
      if (vh0) alpha_s[wave][h0] = al0;
      if (vh1) alpha_s[wave][h1] = al1;
    }
    const bool rescale = __ballot((vh0 && al0 != 1.0f) || (vh1 && al1 != 1.0f)) != 0ull;
    if constexpr (kPipe) {
      if (next < t_end) load_scales(next);
    }
    wave_sync();
    if (rescale) {
      // output column n belongs to head n % G (columns >= 2G are unused)
      const float al = n < PCOLS ? alpha_s[wave][n % G] : 1.0f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[dt] *= al;
    }
    // -- values: O^T[dim][col] += V^T[dim][tok] P^T[tok][col] over 4 chunks of 32 tokens --
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the V tile copy has landed
    wave_sync();
    uint32_t vseg[8][VB + 2];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      vseg[dt][0] = vseg[dt][VB + 1] = 0u;
#pragma unroll
      for (int k = 0; k < VB; ++k) vseg[dt][k + 1] = vbuf[(dt * 64 + lane) * VB + k];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      h8 bp;
      if (n < PCOLS) {
        bp = *reinterpret_cast<const h8*>(&pw[n * kPS + 32 * g + 8 * c]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) bp[e] = static_cast<_Float16>(0.0f);
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        uint32_t pr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[e] = v_pair<VB>(&vseg[dt][1], 8 * c + 2 * e, tab_s, lb);
        h8 av;
        __builtin_memcpy(&av, pr, 16);
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bp, oacc[dt], 0, 0, 0);
      }
    }
    wave_sync();
    if constexpr (kPipe) {
      if (v_early && next < t_end) dma_v(next);
    }
  }

  // ---- merge the W waves of this workgroup ----
  l0 = row_sum16(l0);
  l1 = row_sum16(l1);
  if (n == 0) {
    if (vh0) {
      comb_m[wave][h0] = m0;
      comb_l[wave][h0] = l0;
    }
    if (vh1) {
      comb_m[wave][h1] = m1;
      comb_l[wave][h1] = l1;
    }
  }
  // O^T layout: lane holds rows 4 g + r of dim slice dt for column n; add the lo column
  // (n + G) into the hi column (n), into this wave's region as [128][kOS] floats (the padded
  // stride keeps the 32 writing lanes on distinct banks)
  float* ow = reinterpret_cast<float*>(kr);
  __syncthreads();
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float other = __shfl(oacc[dt][r], (lane & ~15) | ((n + G) & 15), 64);
      if (n < G) ow[(dt * 16 + 4 * g + r) * kOS + n] = oacc[dt][r] + other;
    }
  }
  __syncthreads();
  // scale of each wave's share per head: 2^(m_w - max_w m_w), 0 for waves without tokens
  if (tid < G) {
    float ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) ms = fmaxf(ms, comb_m[w][tid]);
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = comb_m[w][tid];
      const float sc = mw == -INFINITY ? 0.0f : exp2f(mw - ms);
      sc_s[w][tid] = sc;
      l += sc * comb_l[w][tid];
    }
    ms_s[tid] = ms;
    ls_s[tid] = l;
  }
  __syncthreads();
  for (int idx = tid; idx < G * kHeadDim; idx += NT) {
    const int hd = idx / kHeadDim, i = idx % kHeadDim;
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w)
      o += sc_s[w][hd] * reinterpret_cast<const float*>(dyn_s + w * region_words)[i * kOS + hd];
    const int64_t p = (bh * n_splits + s) * G + hd;
    st_coh(part_o + p * kHeadDim + i, o);
    if (i == 0) {
      st_coh(part_ml + p * 2 + 0, ms_s[hd]);
      st_coh(part_ml + p * 2 + 1, ls_s[hd]);
    }
  }

  // ---- split merge, two levels ----
  const int grp = s / kGroup;
  const int n_groups = (n_splits + kGroup - 1) / kGroup;
  const int gsize = n_splits - grp * kGroup < kGroup ? n_splits - grp * kGroup : kGroup;
  unsigned* cnt = counters + bh * (kMaxGroups + 1);
  float* mw_s = reinterpret_cast<float*>(dyn_s);   // merge scratch: 2 x [kGroup][G] + 2 x [G]
  if (!arrive(cnt + grp, static_cast<unsigned>(gsize), &flag_s)) return;
  {
    const int64_t src = (bh * n_splits + grp * kGroup) * G;
    if (n_groups == 1) {
      merge_level<G, NT>(part_o + src * kHeadDim, part_ml + src * 2, gsize, mw_s, tid,
                         out + (static_cast<int64_t>(b) * n_q + h * G) * kHeadDim, nullptr, true);
      if (tid == 0) __hip_atomic_store(cnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    const int64_t dst = (bh * kMaxGroups + grp) * G;
    merge_level<G, NT>(part_o + src * kHeadDim, part_ml + src * 2, gsize, mw_s, tid,
                       gpart_o + dst * kHeadDim, gpart_ml + dst * 2, false);
  }
  if (tid == 0) __hip_atomic_store(cnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!arrive(cnt + kMaxGroups, static_cast<unsigned>(n_groups), &flag_s)) return;
  {
    const int64_t src = bh * kMaxGroups * G;
    merge_level<G, NT>(gpart_o + src * kHeadDim, gpart_ml + src * 2, n_groups, mw_s, tid,
                       out + (static_cast<int64_t>(b) * n_q + h * G) * kHeadDim, nullptr, true);
  }
  if (tid == 0) __hip_atomic_store(cnt + kMaxGroups, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int G, int VB, int W>
hipError_t launch_gvw(kvq_cache* c, int layer, const void* q, int q_f32, float sigma, float* out,
                      int S, const DecodeShape& sh, hipStream_t stream) {
  const kvq_config& cfg = c->cfg;
  const int64_t len = c->len[layer];
  const int64_t n_tiles = (len + kVTile - 1) / kVTile;
  const int tps = static_cast<int>((n_tiles + S - 1) / S);
  dim3 grid(S, cfg.n_kv_heads, cfg.batch);
  const size_t dyn = static_cast<size_t>(W) * sh.region_words * sizeof(uint32_t);
  const Plan* plans = c->plans + static_cast<int64_t>(layer) * cfg.n_kv_heads;
  const bool nf = cfg.codec == KVQ_CODEC_NF16_B256;
  if constexpr (VB == 4) {
    if (nf) {
      hipLaunchKernelGGL((decode_mfma<G, 4, true, W>), grid, dim3(64 * W), dyn, stream, q, q_f32, sigma,
                         len, cfg.n_kv_heads, c->cap, tps, plans, c->tables, layer_k_codes(c, layer),
                         layer_v_codes(c, layer), layer_k_scales(c, layer), layer_v_scales(c, layer),
                         c->k_words, c->n_nf_blocks, S, sh.region_words, sh.v_early, sh.v_off, c->part_o,
                         c->part_ml, c->gpart_o, c->gpart_ml, c->split_counters, out);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_mfma<G, VB, false, W>), grid, dim3(64 * W), dyn, stream, q, q_f32, sigma,
                     len, cfg.n_kv_heads, c->cap, tps, plans, c->tables, layer_k_codes(c, layer),
                     layer_v_codes(c, layer), layer_k_scales(c, layer), layer_v_scales(c, layer),
                     c->k_words, c->n_nf_blocks, S, sh.region_words, sh.v_early, sh.v_off, c->part_o,
                     c->part_ml, c->gpart_o, c->gpart_ml, c->split_counters, out);
  return hipGetLastError();
}

template <int G, int VB>
hipError_t launch_gv(kvq_cache* c, int layer, const void* q, int q_f32, float sigma, float* out,
                     int S, hipStream_t stream) {
  const DecodeShape sh = decode_shape(c);
  if (sh.waves == 8) return launch_gvw<G, VB, 8>(c, layer, q, q_f32, sigma, out, S, sh, stream);
  return launch_gvw<G, VB, 4>(c, layer, q, q_f32, sigma, out, S, sh, stream);
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
