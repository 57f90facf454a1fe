// Split-K grouped-query decode attention over the packed cache, MFMA kernel for gfx950.
//
// RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: decode reads
// the packed (K3V3) cache directly.  With sigma' = sigma * log2(e):
//   l'_{h,t} = s^K_t * sum_i (q_{h,i} g_i sigma') CB_{b_i}[code_{t,i}]   (log2 domain)
//   o_h = sum_t 2^(l'_{h,t} - m) s^V_t CB_{B_V}[code^V_{t,i}] / sum_t 2^(l'_{h,t} - m).
// The 256-value absmax codec (NQKV review, "What carries the argument") uses one
// scale per 256 values (two KV heads share it) and its 16-level table.
//
// Work decomposition.  One workgroup of W waves (8: two per SIMD, or 4) per (context split,
// KV head, sequence); each wave walks 128-token tiles of the split on its own, keeping its own
// running max / sum / output, and the waves are merged through LDS at the end.  The last
// splits of each (sequence, KV head) to finish merge the splits, each one slice of the
// outputs, always in split order.
//
// Keys (lane = token).  The K rows of a tile are staged in LDS word-major.  Every stored RoPE
// block contributes a pair of fields of the same width w; a lane cuts two pairs out of a 32-bit
// row window with one funnel shift and looks each up in an LDS table of fp16 pairs (w <= 4;
// two single lookups for w >= 5).  Four pairs of a token form 8 fp16 values of the B operand
// of a 16x16x32 f16 MFMA whose A operand is the query, pre-multiplied by gains and sigma' and
// split into fp16 hi + lo parts (16 rows = 8 heads x 2 parts).
//
// Values (lane = dim, 8 tokens).  V tiles are stored in the order of the 16x16x32 f16 MFMA A
// operand and copied into LDS by global-to-LDS loads: each lane reads B_V words per 16-dim
// slice and cuts 8 codes of one dim at compile-time offsets (pairs through the same tables).
// The B operand is the softmax weight p * s^V split into fp16 hi + lo, written by the key
// lanes to LDS and read back 8 tokens at a time.
//
// Cross-workgroup merging.  Split partials are written with agent-scope (device-coherent)
// stores.  Once they have completed (s_waitcnt), the split stores its maxima together with a
// per-call tag as 64-bit words; the merging workgroups poll those words, so no counter and no
// cache-wide write-back or invalidation is needed.
#pragma once

#include <hip/hip_fp16.h>

#include "kvq_internal.h"

namespace kvq {
namespace mfma {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// fp16x2 a * b + c with one rounding per half (the asymmetric integer codec's reconstruction
// lo + s * code of two values at once)
__device__ inline uint32_t fma_h2(uint32_t a, uint32_t b, uint32_t c) {
  h2 x, y, z;
  __builtin_memcpy(&x, &a, 4);
  __builtin_memcpy(&y, &b, 4);
  __builtin_memcpy(&z, &c, 4);
  const h2 r = __builtin_elementwise_fma(x, y, z);
  uint32_t o;
  __builtin_memcpy(&o, &r, 4);
  return o;
}
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) void* glb_ptr;
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kCohAux = 16;         // buffer-load cache policy sc1: coherent at device scope
constexpr int kRawBuffer = 0x00020000;   // buffer descriptor word 3: raw 32-bit data
constexpr int kKS = 144;          // LDS row stride (words) of a staged K tile: 128 tokens + 16
constexpr int kPS = 136;          // LDS row stride (halves) of the softmax weights: 128 + 8
constexpr int kOS = 10;           // LDS stride (floats) per dim of a wave's merge share: G <= 8, + 2
constexpr int kAS = 40;           // LDS row stride (halves) of the query operand: 32 + 8
// LDS table region (bytes).  Pair tables hold fp16x2 (CB_w[c0], CB_w[c1]) at index c0 | c1 << w.
// Random lookups into the larger tables would collide in LDS banks, so they are replicated:
// the width-4 pair table 16 times (entry p of copy k at (p << 6) + 4 k, lane l reads copy
// l % 16) and the width-3 pair table 32 times (entry p of copy k at (p << 7) + 4 k, lane l
// reads copy l % 32).  Widths 6..8 use single tables (one fp16 in the low half of a 32-bit
// slot, the high half zero), built per workgroup when the plan uses them: width 6
// replicated 32 times the same way, widths 7 and 8 once (few blocks are that wide); a pair
// costs two lookups in the same table.  Width 5 has a pair table of its own (1024 fp16 pairs,
// not replicated), so its pairs cost one lookup.  The prebuilt image holds the pair tables of
// widths 1..4 and the fp16 single tables of widths 1..8.  Every base is a multiple of its
// table's extent, so an entry address is "(p << shift) | copy offset | base".
constexpr int kRep4Base = 0;           // 16 KB
constexpr int kRep3Base = 16384;       // 8 KB
constexpr int kSing6Base = 24576;      // 8 KB
constexpr int kPair5Base = 32768;      // 4 KB
constexpr int kImageBase = 36864;      // 2.5 KB
constexpr int kSing7Base = 39424;      // 512 B
constexpr int kSing8Base = 39936;      // 1 KB
constexpr int kTableRegion = 40960;
static_assert(kImageBase + kLdsTableBytes <= kSing7Base, "table region overlap");

// Pairs of plan ranks go to the product slots in pairs of pairs: in chunk c, lane group g
// handles ranks 16 c + 2 g, + 1 (positions 0, 1: one row window) and 16 c + 8 + 2 g, + 1
// (positions 2, 3: the other window).  The widest pairs (lowest ranks) thus share positions
// 0 and 1 across the lane groups.  Field f of the plan sits in chunk f / 32 at slot
// k = 8 g + 2 p + (f % 2) of the 32-field product.
__host__ __device__ constexpr int slot_field(int c, int k) {
  return 32 * c + 4 * (k >> 3) + 2 * ((k >> 1) & 1) + 16 * ((k >> 2) & 1) + (k & 1);
}
// Key-product parameters of one (chunk c, lane group g): its four pairs, held in LDS as 24 words
//   [0..3]  table base of pair p (with the part of the lane's replica offset fixed by g)
//   [4..7]  mask applied to 4 n (the rest of the replica offset; 0 for single tables)
//   [8..11] extract width (2 w for pair tables, widths up to 5; w for widths 6..8, whose
//           first field is looked up here)
//   [12..15] left shift of the extracted code (2 single copy, 6 sixteen copies, 32: 7)
//   [16..19] bit shift of window A (pairs 0, 1) and B (pairs 2, 3); bit offset of pairs 1, 3
//   [20..21] byte offset of the first word of windows A and B in a staged K tile
//   [22]    block width of pair p in byte p
constexpr int kParamWords = 24;
__device__ inline void write_pair_params(uint32_t* kp, int r, uint32_t desc) {
  const int c = r >> 4, g = (r & 7) >> 1, p = (r & 1) | (((r >> 3) & 1) << 1);
  const uint32_t w = desc >> 16, off = desc & 0xFFFFu;
  uint32_t base, mask = 0u, shift = 2u;
  if (w == 4u) {
    base = kRep4Base;
    mask = 0x3Cu;
    shift = 6u;
  } else if (w == 3u) {
    base = kRep3Base | (64u * (g & 1));   // lane & 31 = n + 16 (g & 1)
    mask = 0x3Cu;
    shift = 7u;
  } else if (w == 6u) {
    base = kSing6Base | (64u * (g & 1));
    mask = 0x3Cu;
    shift = 7u;
  } else if (w >= 7u) {
    base = w == 7u ? kSing7Base : kSing8Base;
  } else if (w == 5u) {
    base = kPair5Base;
  } else {
    base = kImageBase + static_cast<uint32_t>(pair_table_base(static_cast<int>(w)));
  }
  uint32_t* blk = kp + (4 * c + g) * kParamWords;
  blk[p] = base;
  blk[4 + p] = mask;
  blk[8 + p] = w <= 5u ? 2u * w : w;
  blk[12 + p] = shift;
  reinterpret_cast<uint8_t*>(blk + 22)[p] = static_cast<uint8_t>(w);
  if ((p & 1) == 0) {
    const int k = p >> 1;   // window A or B
    blk[16 + k] = off & 31u;
    blk[18 + k] = 2u * w;
    blk[20 + k] = (off >> 5) * kKS * 4u;
  }
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

// Global-to-LDS copy of 16 bytes per lane to the LDS bytes lds + 16 lane .. + 15 (lds is
// wave-uniform).  Issued from assembly, so the compiler neither counts it nor waits for it
// before other LDS accesses (it cannot prove them disjoint); the wave that reads the copy waits
// for it with s_waitcnt vmcnt(0).  Only safe where the compiler has no loads of its own in
// flight whose completion it would then count wrongly, and M0 is declared written.
__device__ inline void dma16(const void* g, const void* lds) {
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t base =
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<size_t>((lds_char*)lds)));
  uint32_t m0;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               : "={m0}"(m0)
               : "v"(g), "s"(base)
               : "memory");
}

// Max / sum over the 64 lanes of a wave (rows through DPP, then the four row results).
__device__ inline float wave_max(float v) {
  v = row_max16(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
__device__ inline float wave_sum(float v) {
  v = row_sum16(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// Orders a wave's LDS writes before its later LDS reads of other lanes' data: LDS
// instructions of one wave execute in issue order, so only the compiler must be kept from
// moving memory accesses across.  (A memory-model fence would also wait for the wave's
// global-to-LDS copies in flight.)
__device__ inline void wave_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier for LDS data: this wave's LDS accesses complete (lgkmcnt(0)), then all
// waves meet.  LDS has no caches, so the data written before is visible after.  Unlike
// __syncthreads it does not wait for global loads or global-to-LDS copies in flight; LDS
// written by such copies must be waited for (vmcnt) by the wave that reads it.
__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Device-coherent (agent-scope) stores / loads of split partials.
__device__ inline void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Four consecutive floats (16-byte aligned) at byte offset `off` of the buffer `r`, read at
// device scope (sc1) with one 16-byte buffer load (buffer stores with the same policy write
// them coherently).
__device__ inline float4 ld_coh4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned u4 __attribute__((ext_vector_type(4)));
  const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCohAux);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
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

// Merge of the S split partials of one (sequence, KV head), restricted to outputs
// [first, first + count) of the G x 128 (head-major) outputs; count is a power of two.
// Split e publishes, per head hd, its unnormalised output at o[(e G + hd) 128 + i] and its
// sum at l[e G + hd], and only once those stores have completed, its maximum together with
// the tag `want` as one 64-bit word at mt[e G + hd].  Wave hh polls the words of head
// hd0 + hh until every split carries the tag (bounded), which also hands it the maxima; with
// m* = max_e m_e and w_e = 2^(m_e - m*), out = sum_e w_e o_e / sum_e w_e l_e.  `bump`, if
// not null, receives `want` once every split is seen (the next call's tag base).  `smem`
// holds nh S + 4 NT + nh floats (+3 alignment; nh = heads covered); S <= 256.
//
// The wait is bounded by `max_polls`.  A merger that gives up, or that finds the sticky error
// word `status` already set (an earlier merge of this cache gave up; its partial words may be
// stale), writes NaN over its slice and sets bit 0 of `status`; the tag base is then not
// advanced.  The host clears the word, the maxima words and the tag bases after a device-wide
// synchronization (kvq_cache_status).
template <int G, int NT>
__device__ __attribute__((always_inline)) inline void merge_slice(
    const float* __restrict__ src_o, const float* __restrict__ src_l, const uint64_t* __restrict__ src_mt,
    unsigned want, unsigned* bump, unsigned* status, int max_polls, int S, int first, int count,
    float* smem, int tid, float* __restrict__ dst) {
  constexpr int kPre = 8;
  __shared__ unsigned merge_fail;
  const int hd0 = first / kHeadDim;
  const int nh = count > kHeadDim ? count / kHeadDim : 1;
  float* wv = smem;                               // [nh][S] weights
  const int wave = tid >> 6, lane = tid & 63;
  const unsigned sticky = __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) merge_fail = sticky;
  __syncthreads();
  for (int hh = wave; hh < nh; hh += NT / 64) {
    const uint64_t* mt = src_mt + hd0 + hh;
    float mr[4];
    bool ok[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ok[k] = lane + 64 * k >= S;
      mr[k] = -INFINITY;
    }
    bool seen_all = false;
    for (int polls = sticky ? max_polls : 0; polls < max_polls; ++polls) {
      bool mine = true;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (!ok[k]) {
          const uint64_t v = __hip_atomic_load(mt + (lane + 64 * k) * G, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (static_cast<unsigned>(v >> 32) == want) {
            ok[k] = true;
            mr[k] = __uint_as_float(static_cast<unsigned>(v));
          } else {
            mine = false;
          }
        }
      }
      if (__ballot(!mine) == 0ull) {
        seen_all = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!seen_all) {
      if (lane == 0) merge_fail = 1u;
      continue;
    }
    if (hh == 0 && lane == 0 && bump) __hip_atomic_store(bump, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float m = wave_max(fmaxf(fmaxf(mr[0], mr[1]), fmaxf(mr[2], mr[3])));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = lane + 64 * k;
      if (e < S) wv[hh * S + e] = mr[k] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mr[k] - m);
    }
  }
  __syncthreads();
  if (merge_fail) {
    for (int i = tid; i < count; i += NT) dst[first + i] = __builtin_nanf("");
    if (tid == 0) __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // outputs in groups of four (one 16-byte load per split and group)
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(src_o), 0, S * G * kHeadDim * 4, kRawBuffer);
  const int P4 = count / 4 < NT ? count / 4 : NT;   // groups per pass
  const int R = NT / P4;                              // threads per group
  const int j4 = tid % P4, e0 = tid / P4;
  float4* red = reinterpret_cast<float4*>(smem + ((nh * S + 3) & ~3));   // [NT]
  float* Ls = reinterpret_cast<float*>(red + NT);                        // [nh] merged sums
  for (int pass = 0; pass * 4 * P4 < count; ++pass) {
    const int oi = first + 4 * (pass * P4 + j4);    // first output of the group (head-major)
    const int hh = oi / kHeadDim - hd0;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    auto add = [&](float w, float4 o) {
      acc.x += w * o.x; acc.y += w * o.y; acc.z += w * o.z; acc.w += w * o.w;
    };
    int e = e0;
    if (pass == 0) {
      float4 ov[kPre];
#pragma unroll
      for (int k = 0; k < kPre; ++k) {
        const int ek = e0 + R * k;
        ov[k] = ek < S ? ld_coh4(ro, 4u * static_cast<uint32_t>(ek * G * kHeadDim + oi)) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      if (wave < nh) {   // merged sum of head hd0 + wave
        float l = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int ek = lane + 64 * k;
          if (ek < S) l += wv[wave * S + ek] * ld_coh(src_l + ek * G + hd0 + wave);
        }
        l = wave_sum(l);
        if (lane == 0) Ls[wave] = l;
      }
#pragma unroll
      for (int k = 0; k < kPre; ++k, e += R)
        if (e < S) add(wv[hh * S + e], ov[k]);
    }
    for (; e < S; e += R) add(wv[hh * S + e], ld_coh4(ro, 4u * static_cast<uint32_t>(e * G * kHeadDim + oi)));
    if (P4 < 64) {
      // the R threads of a group sit at lanes j4 + P4 k of each wave: sum them across lanes
      // first, then the waves' sums through LDS
      for (int off = P4; off < 64; off <<= 1) {
        acc.x += __shfl_xor(acc.x, off);
        acc.y += __shfl_xor(acc.y, off);
        acc.z += __shfl_xor(acc.z, off);
        acc.w += __shfl_xor(acc.w, off);
      }
      if (lane < P4) red[wave * P4 + lane] = acc;
      __syncthreads();
      if (tid < P4) {
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int r = 0; r < NT / 64; ++r) {
          const float4 t = red[tid + P4 * r];
          o.x += t.x; o.y += t.y; o.z += t.z; o.w += t.w;
        }
        const float inv = 1.0f / Ls[hh];
        *reinterpret_cast<float4*>(dst + oi) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
      }
    } else {
      red[tid] = acc;
      __syncthreads();
      if (tid < P4) {
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int r = 0; r < R; ++r) {
          const float4 t = red[tid + P4 * r];
          o.x += t.x; o.y += t.y; o.z += t.z; o.w += t.w;
        }
        const float inv = 1.0f / Ls[hh];
        *reinterpret_cast<float4*>(dst + oi) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
      }
    }
    __syncthreads();
  }
}

// Key product of lane (n, g) in chunk c: the query operand, the lookup parameters of the
// lane's four pairs (positions 0..3, see slot_field); and, per half of the tile, the two 32-bit
// row windows (pairs 0-1 and 2-3) of its four tokens 16 tg + n, tg = 4 half .. 4 half + 3.
struct KPar {
  h8 aq;
  uint32_t shA, shB, rel1, rel3, baseA, baseB, wid;
  uint32_t bw[4], pb[4], ps[4];
};
struct KWin {
  uint32_t la[4], ha[4], lb[4], hb[4];
};

__device__ __attribute__((always_inline)) inline KPar k_params(int c, int g, int n, const uint32_t* kp_s,
                                                              const _Float16 (*a_s)[16][kAS]) {
  KPar k;
  k.aq = *reinterpret_cast<const h8*>(&a_s[c][n][8 * g]);
  const uint32_t* blk = kp_s + (4 * c + g) * kParamWords;
  const uint4 b4 = *reinterpret_cast<const uint4*>(blk);
  const uint4 m4 = *reinterpret_cast<const uint4*>(blk + 4);
  const uint4 w4 = *reinterpret_cast<const uint4*>(blk + 8);
  const uint4 s4 = *reinterpret_cast<const uint4*>(blk + 12);
  const uint4 x4 = *reinterpret_cast<const uint4*>(blk + 16);
  const uint4 y4 = *reinterpret_cast<const uint4*>(blk + 20);
  const uint32_t n4 = 4u * static_cast<uint32_t>(n);
  k.pb[0] = (n4 & m4.x) | b4.x;
  k.pb[1] = (n4 & m4.y) | b4.y;
  k.pb[2] = (n4 & m4.z) | b4.z;
  k.pb[3] = (n4 & m4.w) | b4.w;
  k.bw[0] = w4.x; k.bw[1] = w4.y; k.bw[2] = w4.z; k.bw[3] = w4.w;
  k.ps[0] = s4.x; k.ps[1] = s4.y; k.ps[2] = s4.z; k.ps[3] = s4.w;
  k.shA = x4.x;
  k.shB = x4.y;
  k.rel1 = x4.z;
  k.rel3 = x4.w;
  k.baseA = y4.x + n4;
  k.baseB = y4.y + n4;
  k.wid = y4.z;
  return k;
}

__device__ __attribute__((always_inline)) inline KWin k_windows(const KPar& k, const uint32_t* kr, int half) {
  const char* kb = reinterpret_cast<const char*>(kr) + 256 * half;   // 64 tokens x 4 bytes
  KWin w;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    w.la[t] = lds_u32(kb, k.baseA + 64 * t);
    w.ha[t] = lds_u32(kb, k.baseA + 64 * t + 4 * kKS);
    w.lb[t] = lds_u32(kb, k.baseB + 64 * t);
    w.hb[t] = lds_u32(kb, k.baseB + 64 * t + 4 * kKS);
  }
  return w;
}

// Decode kernel.  W waves per workgroup (one or two per SIMD).  Every wave owns a region of
// `region_words` LDS words that holds, in turn, its staged K tile, its softmax weights and its
// share of the wave merge (and, during set-up, wave 0's region holds the scaled query).
template <int G, int VB, bool NF, int W, bool KV, bool APP, bool LV>
__global__ __launch_bounds__(64 * W, W / 4) void decode_mfma(
    const void* __restrict__ qv, int q_f32, float sigma, int64_t len, int n_packed_splits,
    const __half* __restrict__ rk, const __half* __restrict__ rv, int R, int64_t n_recent,
    const int8_t* __restrict__ rot, int rot_groups, int n_kv, int64_t cap,
    int tiles_per_split, const Plan* __restrict__ plans, int plan_bs, const Tables* __restrict__ tabg,
    const uint32_t* __restrict__ kc, const uint32_t* __restrict__ vc, const uint16_t* __restrict__ ks,
    const uint16_t* __restrict__ vs, int k_words, int n_nf, int n_splits, int n_mergers, int region_words,
    int v_early, int v_off, float* __restrict__ part_o, float* __restrict__ part_l,
    uint64_t* __restrict__ part_mt, unsigned* __restrict__ epochs, unsigned* status, int max_polls,
    const void* __restrict__ app_k, const void* __restrict__ app_v, int64_t app_pos, uint32_t* app_kc,
    uint32_t* app_vc, uint16_t* app_ks, uint16_t* app_vs, float* __restrict__ out) {
  constexpr int NT = 64 * W;
  constexpr bool kPipe = W == 4;                      // one wave per SIMD: prefetch and pipeline
  // 8 waves with a static V tile area each, copied at tile start (else: the V tile shares the
  // wave's region, copied after the key product, LV with 8 waves or 4 waves without v_early)
  constexpr bool kStaticV = W == 8 && !LV;
  // 8 waves, at most 4-bit values, attention only: each lane loads its own V words straight into
  // registers (the tile is stored in the value product's operand order, so a lane's 8 x VB
  // words are its own), after the key product (late V) or once the tile's K rows are staged
  // (static V areas, several tiles per wave); no LDS copy, the LDS V areas stay unused.  (The
  // fused-append instantiation keeps the LDS copy: with the V words in registers its append
  // code no longer fits the register budget.)
  constexpr bool kRegV = (LV || kStaticV) && VB <= 4 && !kPipe && !APP;
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
  __shared__ __attribute__((aligned(16))) uint32_t kp_s[16 * kParamWords];
  __shared__ __attribute__((aligned(16))) float comb_m[G][W];
  __shared__ __attribute__((aligned(16))) float comb_l[G][W];
  __shared__ float alpha_s[W][G];
  __shared__ float ms_s[G];
  __shared__ uint64_t wide_s;
  // fused append: the new position's key row, value codes, scales (fp16 bits) and inverse
  // scales, and its gain-normalised rows (keys) / rows (values) in fp32
  __shared__ uint32_t app_kw[32];
  __shared__ uint8_t app_vcode[kHeadDim];
  __shared__ uint32_t app_s16[2];
  __shared__ float app_is[2];
  __shared__ float app_y[2][kHeadDim];
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn_s[];   // [W][region_words]
  uint32_t* kr = dyn_s + wave * region_words;                         // [k_words + 1][kKS]
  _Float16* pw = reinterpret_cast<_Float16*>(kr);                     // [PCOLS][kPS], after keys
  // [512][VB] V tile, written by global-to-LDS loads.  With 8 waves it is an LDS object of its
  // own, so the compiler need not wait for those loads before reading the K tile.
  uint32_t* vbuf;
  if constexpr (kStaticV && !kRegV) {
    __shared__ __attribute__((aligned(16))) uint32_t vbuf_s[W][kVTile * 4 * VB];
    vbuf = vbuf_s[wave];
  } else {
    vbuf = kr + v_off;
  }
  // asymmetric integer codec: the wave's tile parameters, [0, 64) key block j (s pair, lo
  // pair), [64, 128) value positions (s of the 128 positions, then their lo)
  uint2* kvp = nullptr;
  if constexpr (KV) {
    __shared__ __attribute__((aligned(16))) uint2 kvp_s[W][2 * kBlocks];
    kvp = kvp_s[wave];
  }
  float (*qs_s)[kHeadDim] = reinterpret_cast<float (*)[kHeadDim]>(dyn_s);   // set-up only

  // `len` packed positions in 128-token tiles; workgroups from n_packed_splits on read the
  // n_recent positions of the recent window instead (one 128-slot ring tile per wave)
  const bool recent_wg = s >= n_packed_splits;
  // tag base of this call's split partials: read first (its round trip overlaps the set-up);
  // only a merger of this same call advances it, after every split has published, so every
  // workgroup of the call reads the same value
  const unsigned epoch = __hip_atomic_load(epochs + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int64_t n_tiles = (len + kVTile - 1) / kVTile;
  const int64_t t_begin = recent_wg ? n_tiles : static_cast<int64_t>(s) * tiles_per_split;
  const int64_t t_end = recent_wg ? n_tiles : (t_begin + tiles_per_split < n_tiles ? t_begin + tiles_per_split : n_tiles);
  const Plan* P = plans + static_cast<int64_t>(b) * plan_bs + h;   // plan of (sequence, head)

  // ---- set-up loads first (small and shared by every workgroup), then the first tile's.
  //      Every load is unconditional (clamped indices; waves 4..7 repeat those of waves 0..3
  //      and discard them) and nothing loaded is used before all are issued, so they share
  //      one round of memory latency. ----
  const bool setup_wave = __builtin_amdgcn_readfirstlane(wave) < 4;
  const int st = tid & 255;   // set-up thread
  const uint8_t* gimg = tabg->lds_image[KV ? 2 : NF ? 1 : 0];
  const uint16_t* gimg16 = reinterpret_cast<const uint16_t*>(gimg);
  uint4 timg = make_uint4(0u, 0u, 0u, 0u);
  uint32_t qraw[QPT];
  float gr[QPT];
  uint32_t fd_r = 0u, pd_r = 0u, rep4v = 0u, rep3v = 0u, cb6 = 0u, cb8 = 0u, cb7 = 0u, cb5lo = 0u;
  uint32_t cb5hi[4] = {0u, 0u, 0u, 0u};
  int nf_r = 0;
  // rotation inside equal-width groups: the chunk (start | size << 8) of field st % 128 and the
  // sign of dim st % 128
  uint32_t rg_chunk = 0u;
  float rg_sign = 1.0f;
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
    qraw[j] = 0u;
    gr[j] = 0.0f;
  }
  if (setup_wave) {   // (with 8 waves, waves 4..7 load nothing of the set-up)
    timg = reinterpret_cast<const uint4*>(gimg)[st < kLdsTableBytes / 16 ? st : kLdsTableBytes / 16 - 1];
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int k = st + 256 * j < G * kHeadDim ? st + 256 * j : G * kHeadDim - 1;
      const int64_t qi = (static_cast<int64_t>(b) * n_q + h * G) * kHeadDim + k;
      // fp32: the element; fp16: the aligned 32-bit word holding it (q is 4-byte aligned)
      const int64_t byte = q_f32 ? 4 * qi : (2 * qi) & ~static_cast<int64_t>(3);
      qraw[j] = *reinterpret_cast<const uint32_t*>(static_cast<const char*>(qv) + byte);
      gr[j] = P->g[k % kHeadDim];
    }
    fd_r = P->fdim[st & (kHeadDim - 1)];
    pd_r = P->pdesc[lane];   // descriptor of pair `lane`
    nf_r = P->n_fields;
    // sources of the per-workgroup tables (see below)
    rep4v = reinterpret_cast<const uint32_t*>(gimg + pair_table_base(4))[st];
    rep3v = reinterpret_cast<const uint32_t*>(gimg + pair_table_base(3))[st & 63];
    cb6 = gimg16[single_table_base(6) / 2 + (st & 63)];
    cb8 = gimg16[single_table_base(8) / 2 + st];
    cb7 = gimg16[single_table_base(7) / 2 + (st & 127)];
    // width-5 pair entries st + 256 i: CB_5[st % 32] and CB_5[st / 32 + 8 i]
    cb5lo = gimg16[single_table_base(5) / 2 + (st & 31)];
#pragma unroll
    for (int i = 0; i < 4; ++i) cb5hi[i] = gimg16[single_table_base(5) / 2 + (st >> 5) + 8 * i];
    if (rot_groups && rot != nullptr) {
      rg_chunk = static_cast<uint32_t>(P->cstart[st & 127]) | (static_cast<uint32_t>(P->csize[st & 127]) << 8);
      rg_sign = static_cast<float>(rot[h * kHeadDim + (st & 127)]);
    }
  }

  // The sequence's last tile is taken by wave 0 of its split, the oldest wave, which finishes its
  // tiles first (slot s of a split is tiles t_begin + s, + W, ...; wave w takes slot
  // (w + last - t_begin) mod W there, slot w elsewhere).
  const int64_t last_tile = n_tiles - 1;
  const int wslot = __builtin_amdgcn_readfirstlane(
      !recent_wg && t_begin <= last_tile && last_tile < t_end
          ? static_cast<int>((static_cast<int64_t>(wave) + last_tile - t_begin) & (W - 1))
          : wave);

  // ---- fused append of one new position app_pos (a decode step; it is the sequence's last
  //      position): rows [batch][n_kv][128] in q's precision.  The workgroup whose tiles hold
  //      app_pos quantizes that position with the row quantizer of the append (codes and scales
  //      identical to it), stores it in HBM and puts the same codes and scales into its own copy
  //      of the tile, so nothing waits for the stores.  Wave 0, which holds that tile, does all of
  //      it after the set-up, so no other wave waits for it; its rows are loaded with the set-up. ----
  const int64_t app_tile = app_pos >= 0 ? app_pos / kVTile : -1;
  const bool app_wg = APP && !NF && !KV && app_pos >= 0 && !recent_wg && t_begin <= app_tile && app_tile < t_end;
  // (in the tile loop: the tile to patch, -1 for none, and the position's index in it)
  const int app_t32 = app_wg ? static_cast<int>(app_tile) : -1;
  const int app_tau = static_cast<int>(app_pos & (kVTile - 1));
  const bool app_w0 = app_wg && __builtin_amdgcn_readfirstlane(wave) == 0;
  float ax0 = 0.0f, ax1 = 0.0f, bx0 = 0.0f, bx1 = 0.0f, ag0 = 1.0f, ag1 = 1.0f;
  if (app_w0) {   // key and value dims lane and lane + 64, and their inverse gains
    const int64_t e = bh * kHeadDim + lane;
    if (q_f32) {
      ax0 = static_cast<const float*>(app_k)[e];
      ax1 = static_cast<const float*>(app_k)[e + 64];
      bx0 = static_cast<const float*>(app_v)[e];
      bx1 = static_cast<const float*>(app_v)[e + 64];
    } else {
      ax0 = __half2float(static_cast<const __half*>(app_k)[e]);
      ax1 = __half2float(static_cast<const __half*>(app_k)[e + 64]);
      bx0 = __half2float(static_cast<const __half*>(app_v)[e]);
      bx1 = __half2float(static_cast<const __half*>(app_v)[e + 64]);
    }
    ag0 = P->ig[lane];
    ag1 = P->ig[lane + 64];
  }

  // K rows of tokens lane and lane + 64 (first 16 words), scales of tokens 16 tg + n, V segments
  uint4 ka[4], kb2[4];
  auto load_k = [&](int64_t tile) {
    const int64_t tok0 = tile * kVTile;
    const uint4* krow0 = reinterpret_cast<const uint4*>(kc + (bh * cap + tok0 + lane) * k_words);
    const uint4* krow1 = reinterpret_cast<const uint4*>(kc + (bh * cap + tok0 + 64 + lane) * k_words);
    const int last = (k_words >> 2) - 1;   // rows are whole 16-byte units; shorter rows repeat
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ka[k] = krow0[k < last ? k : last];
      kb2[k] = krow1[k < last ? k : last];
    }
  };
  uint32_t vreg[8][kRegV ? VB : 1];   // lane's words of the 8 16-dim slices (dims 16 dt + n % 16,
                                     // tokens 32 ((lane / 16) % 4) .. + 31 of the tile)
  auto load_v = [&](int64_t tile) {
    if constexpr (kRegV) {
      const uint32_t* vt = vc + (bh * (cap / kVTile) + tile) * (kVTile * KWV) + lane * VB;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
        for (int k = 0; k < VB; ++k) vreg[dt][k] = vt[dt * 64 * VB + k];
      }
    }
  };
  uint32_t skr[8], svr[8];   // fp16 bits of the scales of tokens 16 tg + n
  uint2 kpr, vpr;            // asymmetric integer codec: this lane's 8 bytes of each tile parameter set
  auto load_scales = [&](int64_t tile) {
    if constexpr (KV) {
      // [tile][64 blocks][s(p0), s(p1), lo(p0), lo(p1)] and [tile][2][128]: 512 bytes each
      const int64_t tb = (bh * (cap / kVTile) + tile) * kBlocks + lane;
      kpr = reinterpret_cast<const uint2*>(ks)[tb];
      vpr = reinterpret_cast<const uint2*>(vs)[tb];
      return;
    }
#pragma unroll
    for (int tg = 0; tg < 8; ++tg) {
      const int64_t t = tile * kVTile + 16 * tg + n;
      if (NF) {
        skr[tg] = ks[(static_cast<int64_t>(b) * cap + t) * n_nf + h / 2];
        svr[tg] = vs[(static_cast<int64_t>(b) * cap + t) * n_nf + h / 2];
      } else {
        skr[tg] = ks[bh * cap + t];
        svr[tg] = vs[bh * cap + t];
      }
    }
  };
  // after the K staging (which waits for the tile's K rows and scales), the scales are packed
  // two per register for the rest of the tile
  uint32_t skp[4], svp[4];
  auto pack_scales = [&]() {
    if constexpr (KV) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      skp[j] = (skr[2 * j] & 0xFFFFu) | (skr[2 * j + 1] << 16);
      svp[j] = (svr[2 * j] & 0xFFFFu) | (svr[2 * j + 1] << 16);
    }
  };
  auto scale_of = [](const uint32_t (&pk)[4], int tg) {
    return half_bits_to_float(static_cast<uint16_t>(pk[tg >> 1] >> (16 * (tg & 1))));
  };
  // the V tile (512 segments x VB words, contiguous in HBM) goes straight into this wave's LDS
  // area: 2 VB copies of 64 lanes x 16 bytes, waited for with s_waitcnt vmcnt(0) before use
  auto dma_v = [&](int64_t tile) {
    const uint32_t* vt = vc + (bh * (cap / kVTile) + tile) * (kVTile * KWV);
    // 8 waves: every load of this wave has been consumed by now; saying so keeps the compiler
    // from waiting later (for loads it would believe in flight, and so for the copy)
    if constexpr (kStaticV) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
#pragma unroll
    for (int i = 0; i < 2 * VB; ++i) {
      if constexpr (kStaticV)
        dma16(vt + 256 * i + 4 * lane, vbuf + 256 * i);
      else
        __builtin_amdgcn_global_load_lds((glb_ptr)(vt + 256 * i + 4 * lane), (lds_ptr)(vbuf + 256 * i), 16, 0, 0);
    }
  };
  // the first tile's K rows and scales are loaded unconditionally (a wave without a tile of
  // its own reads the split's last tile and discards it); its V tile is copied once the
  // set-up data has been used, so waiting for the set-up loads never waits for it
  const int64_t t0 = t_begin + wslot < t_end ? t_begin + wslot : (t_end > 0 ? t_end - 1 : 0);
  // with 8 waves, the older four (one per SIMD) ask for their tiles first; the younger four
  // ask once the set-up has landed
  const bool late_tile = W == 8 && !setup_wave;
  if (!late_tile) {
    load_k(t0);
    load_scales(t0);
  }

  // ---- set-up: tables, scaled query, field dims and pair descriptors into LDS ----
  if (setup_wave) {
    if (tid < kLdsTableBytes / 16) reinterpret_cast<uint4*>(tab_s + kImageBase)[tid] = timg;
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int k = tid + 256 * j;
      const float qf = q_f32 ? __uint_as_float(qraw[j])
                             : half_bits_to_float(static_cast<uint16_t>(qraw[j] >> (16 * (k & 1))));
      // the recent window holds the keys as given: no gains there
      if (k < G * kHeadDim) qs_s[k / kHeadDim][k % kHeadDim] = qf * (recent_wg ? 1.0f : gr[j]) * sigma;
    }
    if (tid < kHeadDim) fdim_s[tid] = static_cast<uint8_t>(fd_r);
    if (tid < kBlocks) {
      pd_s[tid] = pd_r;
      write_pair_params(kp_s, tid, pd_r);
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
    // tables of widths 5..8 when the plan stores such blocks: the width-5 pair table (thread t
    // writes entries t + 256 i), 32 copies of the width-6 single table (thread t < 64 writes
    // the copies of entry t), and for widths 7 and 8 thread t writes CB_8[t] and (t < 128)
    // CB_7[t].  Pairs of 6 bits or more take two single lookups in the key product.
    const uint32_t pw = pd_r >> 16;
    const uint64_t wide = __ballot(pw >= 6u);
    const uint64_t w5 = __ballot(pw == 5u);
    const uint64_t w6 = __ballot(pw == 6u);
    const uint64_t w78 = __ballot(pw >= 7u);
    if (tid == 0) wide_s = wide;
    if (w5) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint32_t*>(tab_s + kPair5Base + 4 * (tid + 256 * i)) = cb5lo | (cb5hi[i] << 16);
    }
    if (w6 && tid < 64) {
      const uint4 v = make_uint4(cb6, cb6, cb6, cb6);
      char* row = tab_s + kSing6Base + (tid << 7);
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4*>(row + 16 * ((j + tid) & 7)) = v;
    }
    if (w78) {
      *reinterpret_cast<uint32_t*>(tab_s + kSing8Base + 4 * tid) = cb8;
      if (tid < 128) *reinterpret_cast<uint32_t*>(tab_s + kSing7Base + 4 * tid) = cb7;
    }
  }
  lds_barrier();
  if (late_tile) {
    load_k(t0);
    load_scales(t0);
  }
  // rotated keys (randomized Hadamard R = H D / sqrt(128)): <q, R^T y> = <R q, y>, so the
  // packed splits rotate the scaled query (fast Walsh-Hadamard stages in fp32); the recent
  // window holds unrotated keys
  if (rot != nullptr && !recent_wg && rot_groups) {
    // rotation inside equal-width groups: <q, g * R^T y> = <R (g * q), y>.  In plan field
    // order, chunk (start, m) of each equal-width run gets the signs, the butterflies of
    // H_m (stage h pairs fields f, f + h with (f - start) & h == 0) and 1/sqrt(m), in fp32,
    // on the gain-scaled query held by dim
    // (set-up thread t handles dim t % 128 for the signs and field t % 128 for the chunks; the
    // signs of dims whose blocks are not stored are applied too, and never read)
    const int nfs = __builtin_amdgcn_readfirstlane(nf_r);
    const int c_start = static_cast<int>(rg_chunk & 0xFFu), c_size = static_cast<int>(rg_chunk >> 8);
    if (setup_wave) {
      for (int k = tid; k < G * kHeadDim; k += 256) qs_s[k / kHeadDim][k % kHeadDim] *= rg_sign;
    }
    lds_barrier();
    for (int hb = 1; hb < kHeadDim; hb <<= 1) {
      if (setup_wave) {
        for (int k = tid; k < G * kHeadDim; k += 256) {
          const int hh = k / kHeadDim, f = k % kHeadDim;
          if (hb < c_size && ((f - c_start) & hb) == 0) {
            const int d0 = fdim_s[f], d1 = fdim_s[f + hb];
            const float a = qs_s[hh][d0], bq = qs_s[hh][d1];
            qs_s[hh][d0] = a + bq;
            qs_s[hh][d1] = a - bq;
          }
        }
      }
      lds_barrier();
    }
    if (setup_wave) {
      for (int k = tid; k < G * kHeadDim; k += 256) {
        const int f = k % kHeadDim;
        if (f < nfs) qs_s[k / kHeadDim][fdim_s[f]] *= 1.0f / sqrtf(static_cast<float>(c_size));
      }
    }
    lds_barrier();
  } else if (rot != nullptr && !recent_wg) {
    if (setup_wave) {
      for (int k = tid; k < G * kHeadDim; k += 256)
        qs_s[k / kHeadDim][k % kHeadDim] *= static_cast<float>(rot[h * kHeadDim + k % kHeadDim]);
    }
    lds_barrier();
    for (int hb = 1; hb < kHeadDim; hb <<= 1) {
      if (setup_wave) {
        for (int p = tid; p < G * kHeadDim / 2; p += 256) {
          const int hh = p / (kHeadDim / 2), jj = p % (kHeadDim / 2);
          const int i0 = (jj / hb) * 2 * hb + jj % hb, i1 = i0 + hb;
          const float a = qs_s[hh][i0], bq = qs_s[hh][i1];
          const float sc = hb == kHeadDim / 2 ? 0.08838834764831845f : 1.0f;   // 1/sqrt(128) at the end
          qs_s[hh][i0] = (a + bq) * sc;
          qs_s[hh][i1] = (a - bq) * sc;
        }
      }
      lds_barrier();
    }
  }
  if (W == 4 && v_early) dma_v(t0);   // (8 waves: copied after the tile's K rows are staged)
  // query operand of the key product: a_s[c][m][k] = hi (m even) or lo (m odd) fp16 part of
  // q'[m / 2][dim of field 32 c + k]; rows of heads >= G and fields past the stored ones are 0.
  // Thread t < 256 fills field t % 128 for heads t / 128, t / 128 + 2, ...
  if (setup_wave) {
    // (recent window: natural dim order, every dim stored)
    const int c = (tid >> 5) & 3, k = tid & 31, f = slot_field(c, k);
    const bool live = recent_wg || f < (__builtin_amdgcn_readfirstlane(nf_r) & ~1);
    const int dim = recent_wg ? 32 * c + k : fdim_s[f];
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
  lds_barrier();
  const uint64_t uses_wide = wide_s;       // pairs (plan ranks) with blocks of 6..8 bits
  // wave 0 of the appending workgroup: the new position's key row y = x * ig_i (fp32) and value
  // row x into LDS; lanes 0 and 1 take the key and the value scale, fp16(fp32(sqrt(sum y_i^2 /
  // 128))) with the fp64 sum in dim order (y_i^2 is exact in fp64, so each fused multiply-add
  // rounds as the addition of the square), and the inverse scale fp32(1 / scale) (0 for a zero
  // scale); then lane l codes key fields l, l + 64 and value dims l, l + 64: u = y * is, and the
  // code is the number of boundaries below u, the boundary between centroids k and k + 1 being
  // their midpoint (exact in fp32 for fp16 centroids).  Field f is coordinate f % 2 of plan pair
  // f / 2 (offset | width << 16): at the pair's offset, plus its width for the second.
  auto app_quantize = [&]() __attribute__((always_inline)) {
    app_y[0][lane] = __fmul_rn(ax0, ag0);
    app_y[0][lane + 64] = __fmul_rn(ax1, ag1);
    app_y[1][lane] = bx0;
    app_y[1][lane + 64] = bx1;
    if (lane < 32) app_kw[lane] = 0u;
    wave_sync();
    if (lane < 2) {
      const float* yr = app_y[lane];
      double ss = 0.0;
#pragma unroll 16
      for (int i = 0; i < kHeadDim; ++i) {
        const double y = static_cast<double>(yr[i]);
        ss = __fma_rn(y, y, ss);
      }
      const __half s16 = __float2half_rn(static_cast<float>(__dsqrt_rn(ss / static_cast<double>(kHeadDim))));
      const float sf = __half2float(s16);
      app_s16[lane] = __half_as_ushort(s16);
      app_is[lane] = sf == 0.0f ? 0.0f : __fdiv_rn(1.0f, sf);
    }
    wave_sync();
    const int nfs = __builtin_amdgcn_readfirstlane(nf_r);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool key = e < 2;
      const int idx = lane + 64 * (e & 1);
      if (key && idx >= nfs) continue;
      uint32_t w = VB, off = 0u;
      int dim = idx;
      if (key) {
        const uint32_t pd = pd_s[idx >> 1];
        w = pd >> 16;
        off = (pd & 0xFFFFu) + (idx & 1 ? w : 0u);
        dim = fdim_s[idx];
      }
      const float u = __fmul_rn(app_y[key ? 0 : 1][dim], app_is[key ? 0 : 1]);
      const _Float16* cbw = reinterpret_cast<const _Float16*>(tab_s + kImageBase + single_table_base(static_cast<int>(w)));
      uint32_t code = 0u;
      for (int sh = static_cast<int>(w) - 1; sh >= 0; --sh) {
        const uint32_t step = 1u << sh, k = code + step - 1u;
        const float bk = __fmul_rn(0.5f, __fadd_rn(static_cast<float>(cbw[k]), static_cast<float>(cbw[k + 1])));
        code += bk < u ? step : 0u;
      }
      if (key) {
        const uint32_t wd = off >> 5, sb = off & 31u;
        atomicOr(&app_kw[wd], code << sb);
        if (sb + w > 32u) atomicOr(&app_kw[wd + 1], code >> (32u - sb));
      } else {
        app_vcode[idx] = static_cast<uint8_t>(code);
      }
    }
    wave_sync();
  };
  if (app_w0) app_quantize();
  // the new position into HBM (wave 0, once its tile's value copy has landed, so that no wait of
  // the tile loop also waits for these stores): its key row whole, its value codes OR-ed into
  // their segment words (the position's bits are still zero there), its scales
  auto app_store = [&]() __attribute__((always_inline)) {
    if (lane < k_words) app_kc[(bh * cap + app_pos) * k_words + lane] = app_kw[lane];
    const int gq = app_tau >> 5;
    const uint32_t bit = static_cast<uint32_t>(app_tau & 31) * VB, wd = bit >> 5, sb = bit & 31u;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = lane + 64 * jj;
      const uint32_t a_vcode = app_vcode[j];
      if (a_vcode != 0u) {
        uint32_t* seg = app_vc + (bh * (cap / kVTile) + app_t32) * (kVTile * KWV) +
                        ((((j >> 4) << 2) + gq) * 16 + (j & 15)) * VB;
        atomicOr(seg + wd, a_vcode << sb);
        if (sb + VB > 32u && (a_vcode >> (32u - sb))) atomicOr(seg + wd + 1, a_vcode >> (32u - sb));
      }
    }
    if (lane == 0) {
      app_ks[bh * cap + app_pos] = static_cast<uint16_t>(app_s16[0]);
      app_vs[bh * cap + app_pos] = static_cast<uint16_t>(app_s16[1]);
    }
  };

  // ---- per-wave state: lane (n, g) keeps heads 2g, 2g + 1 ----
  const int h0 = 2 * g, h1 = 2 * g + 1;
  const bool vh0 = h0 < G, vh1 = h1 < G;
  float m0 = -INFINITY, m1 = -INFINITY, l0 = 0.0f, l1 = 0.0f;
  f4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f4{0.f, 0.f, 0.f, 0.f};

  // one 128-token tile of this wave; the first is peeled out of the loop, so that the compiler
  // counts its loads in flight exactly (no merge at a loop header)
  auto tile_body = [&](int64_t tile, bool first) __attribute__((always_inline)) {
    const int64_t tok0 = tile * kVTile;
    const int64_t next = tile + W;
    if constexpr (!kPipe) {
      if (!first) {   // later tiles: loaded here (the other wave hides the wait)
        load_k(tile);
        load_scales(tile);
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
#pragma unroll
    for (int k = 4; k < 8; ++k) {   // rows longer than 16 words (more than 4 bits)
      if (4 * k >= k_words) break;
      const uint4* krow0 = reinterpret_cast<const uint4*>(kc + (bh * cap + tok0 + lane) * k_words);
      const uint4* krow1 = reinterpret_cast<const uint4*>(kc + (bh * cap + tok0 + 64 + lane) * k_words);
      const uint4 x0 = krow0[k], x1 = krow1[k];
      uint32_t* dst = kr + 4 * k * kKS + lane;
      dst[0] = x0.x; dst[kKS] = x0.y; dst[2 * kKS] = x0.z; dst[3 * kKS] = x0.w;
      dst[64] = x1.x; dst[kKS + 64] = x1.y; dst[2 * kKS + 64] = x1.z; dst[3 * kKS + 64] = x1.w;
    }
    kr[k_words * kKS + lane] = kr[k_words * kKS + 64 + lane] = 0u;
    if (APP && static_cast<int>(tile) == app_t32) {   // the appended position: row and scales from above
      const int tau = app_tau;
      if (lane < k_words) kr[lane * kKS + tau] = app_kw[lane];
      // (selected by masks, not by conditional writes, which the compiler would merge into one
      // write at a variable index and so move the scale registers to memory)
      const uint32_t hit = n == (tau & 15) ? 0xFFFFFFFFu : 0u;
      const uint32_t nk = app_s16[0], nv = app_s16[1];
#pragma unroll
      for (int tg = 0; tg < 8; ++tg) {
        const uint32_t m = tg == (tau >> 4) ? hit : 0u;
        skr[tg] = (skr[tg] & ~m) | (nk & m);
        svr[tg] = (svr[tg] & ~m) | (nv & m);
      }
    }
    pack_scales();
    if constexpr (KV) {
      kvp[lane] = kpr;
      kvp[kBlocks + lane] = vpr;
    }
    wave_sync();
    // 8 waves: the V tile is copied now, when no other load of this wave is in flight, and
    // arrives during the key product
    if constexpr (kStaticV) {
      if constexpr (kRegV) load_v(tile);
      else dma_v(tile);
    }
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
    auto k_lookups = [&](const KPar& P, const KWin& Wn, int c, uint32_t (&u)[4][4]) {
      uint32_t xa[4], xb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        xa[t] = __builtin_amdgcn_alignbit(Wn.ha[t], Wn.la[t], P.shA);
        xb[t] = __builtin_amdgcn_alignbit(Wn.hb[t], Wn.lb[t], P.shB);
        u[t][0] = lds_u32(tab_s, (__builtin_amdgcn_ubfe(xa[t], 0u, P.bw[0]) << P.ps[0]) | P.pb[0]);
        u[t][1] = lds_u32(tab_s, (__builtin_amdgcn_ubfe(xa[t], P.rel1, P.bw[1]) << P.ps[1]) | P.pb[1]);
        u[t][2] = lds_u32(tab_s, (__builtin_amdgcn_ubfe(xb[t], 0u, P.bw[2]) << P.ps[2]) | P.pb[2]);
        u[t][3] = lds_u32(tab_s, (__builtin_amdgcn_ubfe(xb[t], P.rel3, P.bw[3]) << P.ps[3]) | P.pb[3]);
      }
      if ((uses_wide >> (16 * c)) & 0xFFFFull) {
        // blocks of 6..8 bits, without branches per lane: the first field was looked up above;
        // the second comes from the same single table (same shift and base) into the high
        // half.  Lanes whose pair is narrower read a placeholder and keep their value.  Pair
        // position p of the chunk holds ranks 16 c + 8 (p / 2) + (p % 2) + 2 g: positions with
        // no such pair in any lane group are skipped.
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          if (!((uses_wide >> (16 * c + 8 * (p >> 1) + (p & 1))) & 0x55ull)) continue;
          const uint32_t w = (P.wid >> (8 * p)) & 0xFFu;
          const uint32_t rel = (p & 1) ? (p == 1 ? P.rel1 : P.rel3) : 0u;
          const bool wide = w >= 6u;
          uint32_t v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t f1 = __builtin_amdgcn_ubfe(p < 2 ? xa[t] : xb[t], rel + w, w);
            v[t] = lds_u32(tab_s, wide ? (f1 << P.ps[p]) | P.pb[p] : static_cast<uint32_t>(kImageBase));
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) u[t][p] = wide ? u[t][p] | (v[t] << 16) : u[t][p];
        }
      }
    };
    auto k_products = [&](const KPar& P, const uint32_t (&u)[4][4], int half) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        h8 bk;
        __builtin_memcpy(&bk, u[t], 16);
        dacc[4 * half + t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P.aq, bk, dacc[4 * half + t], 0, 0, 0);
      }
    };
    // per chunk: parameters, then the first half's row windows; the second half's windows are
    // read before the first half's lookups
    // asymmetric integer codec: the lookups give the codes as fp16 integers; each pair becomes
    // fp16(lo + s * code) with its block's parameters (pair p of chunk c is plan rank
    // 16 c + 8 (p >> 1) + 2 g + (p & 1), which is block index for the codec's uniform plan)
    auto k_dequant = [&](const uint2 (&sm)[4], uint32_t (&u)[4][4]) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
#pragma unroll
        for (int t = 0; t < 4; ++t) u[t][p] = fma_h2(u[t][p], sm[p].x, sm[p].y);
      }
    };
#pragma unroll 1
    for (int c = 0; c < 4; ++c) {
      const KPar P = k_params(c, g, n, kp_s, a_s);
      const KWin W0 = k_windows(P, kr, 0);
      const KWin W1 = k_windows(P, kr, 1);
      uint2 sm[4];
      if constexpr (KV) {
#pragma unroll
        for (int p = 0; p < 4; ++p) sm[p] = kvp[16 * c + 8 * (p >> 1) + 2 * g + (p & 1)];
      }
      uint32_t u[4][4];
      k_lookups(P, W0, c, u);
      if constexpr (KV) k_dequant(sm, u);
      k_products(P, u, 0);
      k_lookups(P, W1, c, u);
      if constexpr (KV) k_dequant(sm, u);
      k_products(P, u, 1);
    }
    wave_sync();   // the key rows are read; the area takes the softmax weights (and V) next
    if constexpr (kRegV && LV) load_v(tile);   // the V words land in registers during the softmax
    else if (!kStaticV && !v_early) dma_v(tile);

    // -- online softmax: lane (n, g) holds heads 2g and 2g + 1 of tokens 16 tg + n --
    float L0[8], L1[8];
    float mt0 = -INFINITY, mt1 = -INFINITY;
    const int rem = len - tok0 < kVTile ? static_cast<int>(len - tok0) : kVTile;   // valid packed tokens
#pragma unroll
    for (int tg = 0; tg < 8; ++tg) {
      const float bias = 16 * tg + n < rem ? 0.0f : -INFINITY;
      const float sk = KV ? 1.0f : scale_of(skp, tg);
      L0[tg] = fmaf(dacc[tg][0] + dacc[tg][1], sk, bias);
      L1[tg] = fmaf(dacc[tg][2] + dacc[tg][3], sk, bias);
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
      // tokens past the sequence end have p = 0; their stored scales are finite (zero-filled)
      const float sv = KV ? 1.0f : scale_of(svp, tg);
      const float p0 = __builtin_amdgcn_exp2f(L0[tg] - mn0), p1 = __builtin_amdgcn_exp2f(L1[tg] - mn1);
      l0 += p0;
      l1 += p1;
      // weight p s^V as fp16 hi + lo: hi = fp16(p s^V), lo = fp16(p s^V - hi) with the product
      // kept exact inside one fused operation (one mixed-precision instruction each)
      const _Float16 q0h = static_cast<_Float16>(p0 * sv), q1h = static_cast<_Float16>(p1 * sv);
      const int t = 16 * tg + n;
      if (vh0) {
        pw[h0 * kPS + t] = q0h;
        pw[(G + h0) * kPS + t] = static_cast<_Float16>(__builtin_fmaf(p0, sv, -static_cast<float>(q0h)));
      }
      if (vh1) {
        pw[h1 * kPS + t] = q1h;
        pw[(G + h1) * kPS + t] = static_cast<_Float16>(__builtin_fmaf(p1, sv, -static_cast<float>(q1h)));
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
    if constexpr (!kRegV) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the V tile copy has landed
    wave_sync();
    if (APP && static_cast<int>(tile) == app_t32) {   // the appended position's value codes into the copy
      const int tau = app_tau;
      const int bit = (tau & 31) * VB, wd = bit >> 5, sb = bit & 31;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = lane + 64 * jj;
        const uint32_t code = app_vcode[j];
        uint32_t* seg = vbuf + ((((j >> 4) << 2) + (tau >> 5)) * 16 + (j & 15)) * VB;
        seg[wd] |= code << sb;
        if (sb + VB > 32) seg[wd + 1] |= code >> (32 - sb);
      }
      wave_sync();
    }
    if (APP && static_cast<int>(tile) == app_t32) app_store();
    uint32_t vseg[8][VB + 2];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      vseg[dt][0] = vseg[dt][VB + 1] = 0u;
#pragma unroll
      for (int k = 0; k < VB; ++k) vseg[dt][k + 1] = kRegV ? vreg[dt][kRegV ? k : 0] : vbuf[(dt * 64 + lane) * VB + k];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // asymmetric integer codec: s and lo pairs of this lane's tokens 32 g + 8 c + 2 e, +1
      uint4 vsc, vlo;
      if constexpr (KV) {
        const uint32_t* vp = reinterpret_cast<const uint32_t*>(kvp + kBlocks);
        vsc = *reinterpret_cast<const uint4*>(vp + 16 * g + 4 * c);
        vlo = *reinterpret_cast<const uint4*>(vp + kBlocks + 16 * g + 4 * c);
      }
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
        if constexpr (KV) {
          pr[0] = fma_h2(pr[0], vsc.x, vlo.x);
          pr[1] = fma_h2(pr[1], vsc.y, vlo.y);
          pr[2] = fma_h2(pr[2], vsc.z, vlo.z);
          pr[3] = fma_h2(pr[3], vsc.w, vlo.w);
        }
        h8 av;
        __builtin_memcpy(&av, pr, 16);
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bp, oacc[dt], 0, 0, 0);
      }
    }
    wave_sync();
    if constexpr (kPipe) {
      if (v_early && next < t_end) dma_v(next);
    }
  };
  if (t_begin + wslot < t_end) {
    tile_body(t_begin + wslot, true);
    for (int64_t tile = t_begin + wslot + W; tile < t_end; tile += W) tile_body(tile, false);
  }
  if (recent_wg) {
    // ---- recent window: fp16 keys [R][n_kv][128] and values in dim-major 128-slot tiles, no
    //      scales.  Recent workgroup j takes ring tile j (its first min(128, n_recent - 128 j)
    //      slots hold window positions; the order of positions does not matter to the
    //      softmax), on wave 0: the tile's 64 KB of fp16 operands are as much as one compute
    //      unit reads for a packed split.  Same products as a packed tile, with the operands
    //      loaded straight from the ring. ----
    const int64_t j = s - n_packed_splits;
    const int64_t nv64 = n_recent - 128 * j;
    // window positions len .. len + n_recent - 1 sit in slots p mod R; the j-th 128 of them
    // fill ring tile (len / 128 + j) mod (R / 128) from its first slot on (len is a multiple of
    // 128, or the window is full and every tile is)
    const int64_t jt = ((len >> 7) + j) % (R >> 7);
    if (wave == 0) {
      const int nv = nv64 < 128 ? static_cast<int>(nv64) : 128;
      const __half* kt = rk + ((static_cast<int64_t>(b) * R + 128 * jt) * n_kv + h) * kHeadDim;
      const __half* vt = rv + ((bh * (R / 128) + jt) * kHeadDim) * 128;
      f4 dacc[8];
#pragma unroll
      for (int tg = 0; tg < 8; ++tg) dacc[tg] = f4{0.f, 0.f, 0.f, 0.f};
      // all of the tile's key operands are loaded at once (one round of memory latency)
      h8 bk[4][8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int tg = 0; tg < 8; ++tg) {
          const int t = 16 * tg + n < nv ? 16 * tg + n : 0;   // slots past the window: slot 0, masked
          bk[c][tg] = *reinterpret_cast<const h8*>(kt + static_cast<int64_t>(t) * n_kv * kHeadDim + 32 * c + 8 * g);
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const h8 aq = *reinterpret_cast<const h8*>(&a_s[c][n][8 * g]);
#pragma unroll
        for (int tg = 0; tg < 8; ++tg) dacc[tg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, bk[c][tg], dacc[tg], 0, 0, 0);
      }
      // and the value operands, in flight during the softmax
      // (slots past the window hold zeros or stale values with p = 0: finite either way)
      h8 av[4][8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          av[c][dt] = *reinterpret_cast<const h8*>(vt + static_cast<int64_t>(16 * dt + n) * 128 + 32 * g + 8 * c);
      }
      float L0[8], L1[8];
      float mt0 = -INFINITY, mt1 = -INFINITY;
#pragma unroll
      for (int tg = 0; tg < 8; ++tg) {
        const float bias = 16 * tg + n < nv ? 0.0f : -INFINITY;
        L0[tg] = dacc[tg][0] + dacc[tg][1] + bias;
        L1[tg] = dacc[tg][2] + dacc[tg][3] + bias;
        mt0 = fmaxf(mt0, L0[tg]);
        mt1 = fmaxf(mt1, L1[tg]);
      }
      mt0 = row_max16(mt0);
      mt1 = row_max16(mt1);
      // first (and only) tile of this wave: m starts at -inf, so no rescale of o or l
      m0 = mt0;
      m1 = mt1;
#pragma unroll
      for (int tg = 0; tg < 8; ++tg) {
        const float p0 = __builtin_amdgcn_exp2f(L0[tg] - m0), p1 = __builtin_amdgcn_exp2f(L1[tg] - m1);
        l0 += p0;
        l1 += p1;
        const _Float16 p0h = static_cast<_Float16>(p0), p1h = static_cast<_Float16>(p1);
        const int t = 16 * tg + n;
        if (vh0) {
          pw[h0 * kPS + t] = p0h;
          pw[(G + h0) * kPS + t] = static_cast<_Float16>(p0 - static_cast<float>(p0h));
        }
        if (vh1) {
          pw[h1 * kPS + t] = p1h;
          pw[(G + h1) * kPS + t] = static_cast<_Float16>(p1 - static_cast<float>(p1h));
        }
      }
      wave_sync();
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
        for (int dt = 0; dt < 8; ++dt) oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[c][dt], bp, oacc[dt], 0, 0, 0);
      }
      wave_sync();
    }
  }


  // ---- merge the W waves of this workgroup: each wave adds its lo columns (n + G) into its
  //      hi columns (n) and writes them, with its (m, l), to LDS; after one barrier every
  //      thread combines the waves for its outputs ----
  l0 = row_sum16(l0);
  l1 = row_sum16(l1);
  float* ow = reinterpret_cast<float*>(kr);   // [128][kOS]: dim-major, padded (distinct banks)
  if (n == 0) {
    if (vh0) {
      comb_m[h0][wave] = m0;
      comb_l[h0][wave] = l0;
    }
    if (vh1) {
      comb_m[h1][wave] = m1;
      comb_l[h1][wave] = l1;
    }
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // lane n reads lane (n + G) mod 16 of its row
      const float other = KVQ_DPP(oacc[dt][r], 0x120 + (16 - G) % 16);
      if (n < G) ow[(dt * 16 + 4 * g + r) * kOS + n] = oacc[dt][r] + other;
    }
  }
  lds_barrier();
  const int64_t out_base = (static_cast<int64_t>(b) * n_q + h * G) * kHeadDim;
  // thread q combines outputs 4 i .. 4 i + 3 of head hd = q % G (i = q / G: the lanes of a
  // wave read distinct LDS banks) and stores them as one 16-byte word
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
      part_o + (bh * n_splits + s) * G * kHeadDim, 0, G * kHeadDim * 4, kRawBuffer);
  for (int q = tid; q < G * kHeadDim / 4; q += NT) {
    const int hd = q % G, i0 = 4 * (q / G);
    float mw[W], lw[W], sc[W];
#pragma unroll
    for (int w = 0; w < W; w += 4) {
      const float4 m4 = *reinterpret_cast<const float4*>(&comb_m[hd][w]);
      const float4 l4 = *reinterpret_cast<const float4*>(&comb_l[hd][w]);
      mw[w] = m4.x; mw[w + 1] = m4.y; mw[w + 2] = m4.z; mw[w + 3] = m4.w;
      lw[w] = l4.x; lw[w + 1] = l4.y; lw[w + 2] = l4.z; lw[w + 3] = l4.w;
    }
    float ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) ms = fmaxf(ms, mw[w]);
    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f}, l = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      // 0 for waves without tokens; hardware 2^x (weights far below 1 only meet sums >= 1)
      sc[w] = mw[w] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw[w] - ms);
      l += sc[w] * lw[w];
      const float* ow_w = reinterpret_cast<const float*>(dyn_s + w * region_words);
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] += sc[w] * ow_w[(i0 + j) * kOS + hd];
    }
    if (n_splits == 1) {
      const float inv = 1.0f / l;
      *reinterpret_cast<float4*>(out + out_base + hd * kHeadDim + i0) =
          make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    } else {
      typedef float fv4 __attribute__((ext_vector_type(4)));
      __builtin_amdgcn_raw_buffer_store_b128(fv4{o[0], o[1], o[2], o[3]}, rp,
                                             4u * static_cast<uint32_t>(hd * kHeadDim + i0), 0, kCohAux);
      if (i0 == 0) {
        st_coh(part_l + (bh * n_splits + s) * G + hd, l);
        ms_s[hd] = ms;
      }
    }
  }
  if (n_splits == 1) return;

  // ---- split merge.  Each split publishes its maxima with this call's tag once its output
  //      and sum stores have completed; the last n_mergers splits of this (sequence, KV head)
  //      each merge one slice of the outputs, waiting (bounded) for every split's tag ----
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);   // this wave's partial stores have completed
  __syncthreads();
  const unsigned tag = epoch + 1u;
  if (tid < G) {
    const uint64_t v = (static_cast<uint64_t>(tag) << 32) | __float_as_uint(ms_s[tid]);
    __hip_atomic_store(part_mt + (bh * n_splits + s) * G + tid, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int rank = s - (n_splits - n_mergers);
  if (rank < 0) return;
  const int count = G * kHeadDim / n_mergers;
  merge_slice<G, NT>(part_o + bh * n_splits * G * kHeadDim, part_l + bh * n_splits * G,
                     part_mt + bh * n_splits * G, tag, rank == 0 ? epochs + bh : nullptr, status, max_polls,
                     n_splits, rank * count, count, reinterpret_cast<float*>(dyn_s), tid, out + out_base);
}

// Merge of the split partials by a kernel of its own, for launches whose mergers would not fit
// beside the splits they wait for (as many (sequence, KV head) units as compute units): the
// decode kernel only publishes partials, and this kernel, enqueued after it on the same stream,
// merges each unit's splits in one workgroup.  Every tag is then already published; the tag
// base is the one the decode kernel read, advanced here.
template <int G>
__global__ __launch_bounds__(256) void decode_merge(
    const float* __restrict__ part_o, const float* __restrict__ part_l, const uint64_t* __restrict__ part_mt,
    unsigned* __restrict__ epochs, unsigned* status, int max_polls, int n_splits, int n_kv,
    float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) float msm[];
  const int h = blockIdx.x, b = blockIdx.y;
  const int64_t bh = static_cast<int64_t>(b) * n_kv + h;
  const unsigned want = __hip_atomic_load(epochs + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  merge_slice<G, 256>(part_o + bh * n_splits * G * kHeadDim, part_l + bh * n_splits * G, part_mt + bh * n_splits * G,
                      want, epochs + bh, status, max_polls, n_splits, 0, G * kHeadDim, msm, threadIdx.x,
                      out + bh * G * kHeadDim);
}

template <int G, int VB, int W>
hipError_t launch_gvw(kvq_cache* c, int layer, const void* q, int q_f32, float sigma, float* out,
                      int S, const DecodeShape& sh, const DecodeScratch& ws, const DecodeAppend& app,
                      hipStream_t stream) {
  const kvq_config& cfg = c->cfg;
  // S packed splits over the packed positions, plus one workgroup for the recent window
  const int64_t plen = packed_len(c, layer);
  const int64_t n_recent = c->len[layer] - plen;
  const int64_t n_tiles = (plen + kVTile - 1) / kVTile;
  const int tps = S > 0 ? static_cast<int>((n_tiles + S - 1) / S) : 0;
  // one ring tile of the window per recent workgroup
  const int S_all = S + static_cast<int>((n_recent + 127) / 128);
  const __half* rk = n_recent > 0 ? layer_k_recent(c, layer) : nullptr;
  const __half* rv = n_recent > 0 ? layer_v_recent(c, layer) : nullptr;
  const int R = c->ring;
  const int8_t* rot = codec_rotates(cfg.codec) ? c->rot_signs + static_cast<int64_t>(layer) * cfg.n_kv_heads * kHeadDim : nullptr;
  const int rot_groups = cfg.codec == KVQ_CODEC_BGTQ_ROT ? 1 : 0;
  dim3 grid(S_all, cfg.n_kv_heads, cfg.batch);
  // 8 waves: the V tile in the wave's region when no wave has more than one tile (the static V
  // areas only pay when a wave's next tile can be copied during its key product)
  const bool lv = W == 8 && sh.lv_region > 0 && (!sh.v_early || tps <= W);
  const int region_words = lv ? sh.lv_region : sh.region_words;
  const int v_early = lv ? 0 : sh.v_early, v_off = lv ? sh.lv_off : sh.v_off;
  const size_t dyn = static_cast<size_t>(W) * region_words * sizeof(uint32_t);
  const Plan* plans = c->plans + static_cast<int64_t>(layer) * c->n_plan * cfg.n_kv_heads;
  const int plan_bs = c->n_plan > 1 ? cfg.n_kv_heads : 0;
  const int mergers = decode_split_mergers(S_all, static_cast<int64_t>(cfg.batch) * cfg.n_kv_heads, c->n_cu);
#define KVQ_LAUNCH_DEC_(NF, KV, APP, LV)                                                               \
  hipLaunchKernelGGL((decode_mfma<G, VB, NF, W, KV, APP, LV>), grid, dim3(64 * W), dyn, stream, q, q_f32, sigma, \
                     plen, S, rk, rv, R, n_recent, rot, rot_groups, cfg.n_kv_heads, c->cap, tps, plans, plan_bs, \
                     c->tables, layer_k_codes(c, layer), layer_v_codes(c, layer), layer_k_scales(c, layer), \
                     layer_v_scales(c, layer), c->k_words, c->n_nf_blocks, S_all, mergers, region_words,     \
                     v_early, v_off, ws.o, ws.l, ws.mt, ws.epochs, ws.status, ws.max_polls, app.k, app.v,        \
                     app.pos, layer_k_codes(c, layer), layer_v_codes(c, layer), layer_k_scales(c, layer),         \
                     layer_v_scales(c, layer), out)
  // 8 waves: a static V tile area per wave (v_early) or the V tile in the wave's region (LV)
#define KVQ_LAUNCH_DEC(NF, KV, APP)                                        \
  do {                                                                     \
    if constexpr (W == 8) {                                                \
      if (lv) {                                                            \
        KVQ_LAUNCH_DEC_(NF, KV, APP, true);                                \
      } else {                                                             \
        if constexpr (VB <= 4) KVQ_LAUNCH_DEC_(NF, KV, APP, false);        \
      }                                                                    \
    } else {                                                               \
      KVQ_LAUNCH_DEC_(NF, KV, APP, false);                                 \
    }                                                                      \
  } while (0)
  bool launched = false;
  if constexpr (VB == 4) {
    if (cfg.codec == KVQ_CODEC_NF16_B256) {
      KVQ_LAUNCH_DEC(true, false, false);
      launched = true;
    }
  }
  if constexpr (VB <= 4) {
    if (!launched && cfg.codec == KVQ_CODEC_KIVI) {
      KVQ_LAUNCH_DEC(false, true, false);
      launched = true;
    }
  }
  // a decode step's append (Block-GTQ / uniform codecs only) runs in an instantiation of its own
  if (!launched && app.pos >= 0) KVQ_LAUNCH_DEC(false, false, true);
  else if (!launched) KVQ_LAUNCH_DEC(false, false, false);
#undef KVQ_LAUNCH_DEC
#undef KVQ_LAUNCH_DEC_
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S_all <= 1 || mergers > 0) return e;
  // no room for in-kernel mergers: merge in a kernel of its own
  const size_t msm = sizeof(float) * ((static_cast<size_t>(G) * S_all + 3) / 4 * 4 + 4 * 256 + G);
  hipLaunchKernelGGL((decode_merge<G>), dim3(cfg.n_kv_heads, cfg.batch), dim3(256), msm, stream, ws.o, ws.l, ws.mt,
                     ws.epochs, ws.status, ws.max_polls, S_all, cfg.n_kv_heads, out);
  return hipGetLastError();
}

template <int G, int VB>
hipError_t launch_gv(kvq_cache* c, int layer, const void* q, int q_f32, float sigma, float* out,
                     int S, const DecodeScratch& ws, const DecodeAppend& app, hipStream_t stream) {
  const DecodeShape sh = decode_shape(c);
  if (sh.waves == 8) return launch_gvw<G, VB, 8>(c, layer, q, q_f32, sigma, out, S, sh, ws, app, stream);
  if (sh.waves != 4) return hipErrorInvalidConfiguration;
  return launch_gvw<G, VB, 4>(c, layer, q, q_f32, sigma, out, S, sh, ws, app, stream);
}

template <int G>
hipError_t launch_group(kvq_cache* c, int layer, const void* q, int q_f32, float sigma, float* out,
                        int S, const DecodeScratch& ws, const DecodeAppend& app, hipStream_t stream) {
  const int vb = c->cfg.codec == KVQ_CODEC_NF16_B256 ? 4 : c->cfg.v_bits;
  switch (vb) {
    case 1: return launch_gv<G, 1>(c, layer, q, q_f32, sigma, out, S, ws, app, stream);
    case 2: return launch_gv<G, 2>(c, layer, q, q_f32, sigma, out, S, ws, app, stream);
    case 3: return launch_gv<G, 3>(c, layer, q, q_f32, sigma, out, S, ws, app, stream);
    case 4: return launch_gv<G, 4>(c, layer, q, q_f32, sigma, out, S, ws, app, stream);
    case 5: return launch_gv<G, 5>(c, layer, q, q_f32, sigma, out, S, ws, app, stream);
    case 6: return launch_gv<G, 6>(c, layer, q, q_f32, sigma, out, S, ws, app, stream);
    case 7: return launch_gv<G, 7>(c, layer, q, q_f32, sigma, out, S, ws, app, stream);
    default: return launch_gv<G, 8>(c, layer, q, q_f32, sigma, out, S, ws, app, stream);
  }
}

}  // namespace mfma
}  // namespace kvq
