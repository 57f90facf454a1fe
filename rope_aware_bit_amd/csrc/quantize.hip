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
// One workgroup of 256 threads handles 8 consecutive positions of one (sequence, KV head):
//   1. the group's K and V rows (for the 256-value codec both heads of the block) are copied
//      into LDS with coalesced 16-byte loads;
//   2. one lane per token computes the token's scales in the order above;
//   3. every thread quantizes four K (token, field) and four V (token, dim) elements with
//      branchless binary searches over the width's boundaries, all eight in lock step, and ORs
//      each code into the LDS image of its K row word and V segment word;
//   4. the group's K rows are stored as one contiguous run, and its V segment words are
//      OR-ed into HBM with atomics: a 32-position V segment is shared by four workgroups,
//      and positions at or past the sequence length are still zero (the cache is zero-filled
//      at creation and only appended to), so the ORs compose.
#include <hip/hip_fp16.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kGroupTok = 8;    // positions per workgroup
constexpr int kThreads = 256;

template <typename T>
__device__ inline float to_f(T v);
template <>
__device__ inline float to_f<__half>(__half v) { return __half2float(v); }
template <>
__device__ inline float to_f<float>(float v) { return v; }

__device__ inline float inv_scale(__half s16) {
  const float s = __half2float(s16);
  return s == 0.0f ? 0.0f : __fdiv_rn(1.0f, s);
}

// RM: key rotation, 0 none, 1 the whole row (uniform codec), 2 inside equal-width groups
template <typename T, bool NF, int RM>
__global__ __launch_bounds__(kThreads) void quantize_append(
    const T* __restrict__ kin, const T* __restrict__ vin, int64_t n_new, int64_t in_stride, int ring_R, int64_t L0, int n_kv,
    int64_t cap, const Plan* __restrict__ plans, int plan_bs, const Tables* __restrict__ tab,
    uint32_t* __restrict__ kc, uint32_t* __restrict__ vc, uint16_t* __restrict__ ks,
    uint16_t* __restrict__ vs, int k_words, int v_bits, int n_nf, const int8_t* __restrict__ rot) {
  constexpr int kVec = 16 / sizeof(T);            // elements per 16-byte load
  constexpr int kRowW = kHeadDim * static_cast<int>(sizeof(T)) / 4 + 1;   // odd: no bank conflicts
  constexpr int kHeads = NF ? 2 : 1;              // heads staged per tensor
  constexpr int kEl = kHeadDim * kGroupTok / kThreads;   // K (and V) elements per thread
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t g0 = (L0 / kGroupTok + blockIdx.x) * kGroupTok;   // first position of the group
  // appended positions of the group: [lo, hi) relative to g0
  const int lo = static_cast<int>(L0 > g0 ? L0 - g0 : 0);
  const int hi = static_cast<int>(L0 + n_new - g0 < kGroupTok ? L0 + n_new - g0 : kGroupTok);
  const int vb = NF ? 4 : v_bits;
  const int eb = static_cast<int>(g0 % 32);       // first position inside its V segment
  const int vw0 = eb * vb / 32;                   // first segment word the group touches
  const int nvw = ((eb + kGroupTok) * vb + 31) / 32 - vw0;   // segment words it touches (<= 3)

  __shared__ uint32_t x_s[2][kHeads][kGroupTok][kRowW];   // [K, V][head][token] rows of T
  auto xval = [&](int tsr, int hh, int r, int i) {
    return to_f(reinterpret_cast<const T*>(&x_s[tsr][hh][r][0])[i]);
  };
  __shared__ float bd_s[(kMaxBits + 1) * 256];
  __shared__ float ig_s[kHeadDim];
  __shared__ uint8_t fdim_s[kHeadDim], fw_s[kHeadDim];
  __shared__ uint16_t foff_s[kHeadDim];
  __shared__ __attribute__((aligned(16))) uint32_t krow_s[kGroupTok * 4 * kMaxBits];
  __shared__ uint32_t vw_s[kHeadDim][4];           // the group's V segment words, per dim
  __shared__ float isk_s[kGroupTok], isv_s[kGroupTok];
  __shared__ int nf_s;

  // ---- 1. stage rows, tables and plan; clear the word images ----
  const int h0 = NF ? (h & ~1) : h;   // first head of the staged block
  for (int k = tid; k < 2 * kHeads * kGroupTok * (kHeadDim / kVec); k += kThreads) {
    const int q = k % (kHeadDim / kVec);
    const int r = (k / (kHeadDim / kVec)) % kGroupTok;
    const int hh = (k / (kHeadDim / kVec * kGroupTok)) % kHeads;
    const int tsr = k / (kHeadDim / kVec * kGroupTok * kHeads);   // 0: K, 1: V
    if (r >= lo && r < hi) {
      uint4 v4;
      if (ring_R == 0) {
        const int64_t src = ((static_cast<int64_t>(b) * in_stride + (g0 + r - L0)) * n_kv + h0 + hh) * kHeadDim + q * kVec;
        v4 = *reinterpret_cast<const uint4*>((tsr ? vin : kin) + src);
      } else {
        // recent-window rings (fp16): keys [batch][R][n_kv][128], values in dim-major 128-slot
        // tiles [batch][n_kv][R / 128][128][128]; position p sits in slot p mod R
        const int64_t slot = (g0 + r) % ring_R;
        if (tsr == 0) {
          v4 = *reinterpret_cast<const uint4*>(kin + ((static_cast<int64_t>(b) * ring_R + slot) * n_kv + h0 + hh) * kHeadDim + q * kVec);
        } else {
          const T* vt = vin + (((static_cast<int64_t>(b) * n_kv + h0 + hh) * (ring_R / 128) + slot / 128) * kHeadDim + q * kVec) * 128 + slot % 128;
          T e8[kVec];
#pragma unroll
          for (int e = 0; e < kVec; ++e) e8[e] = vt[e * 128];
          __builtin_memcpy(&v4, e8, 16);
        }
      }
      uint32_t* d = &x_s[tsr][hh][r][q * 4];
      d[0] = v4.x;
      d[1] = v4.y;
      d[2] = v4.z;
      d[3] = v4.w;
    }
  }
  const Plan* P = plans + static_cast<int64_t>(b) * plan_bs + h;   // plan of (sequence, head)
  for (int k = tid; k < (kMaxBits + 1) * 256; k += kThreads) {
    const int bb = k >> 8, e = k & 255;
    bd_s[k] = NF ? (bb == 4 && e < 16 ? tab->nf_bd[e] : INFINITY) : tab->bd[bb][e];
  }
  if (tid < kHeadDim) {
    ig_s[tid] = P->ig[tid];
    fdim_s[tid] = P->fdim[tid];
    fw_s[tid] = P->fwidth[tid];
    foff_s[tid] = P->foff[tid];
    vw_s[tid][0] = vw_s[tid][1] = vw_s[tid][2] = vw_s[tid][3] = 0u;
  }
  // rotation inside equal-width groups: field f's chunk, and each dim's chunk size (0: the
  // dim's block is not stored)
  __shared__ uint8_t cst_s[RM == 2 ? kHeadDim : 1], csz_s[RM == 2 ? kHeadDim : 1], dsz_s[RM == 2 ? kHeadDim : 1];
  if constexpr (RM == 2) {
    if (tid < kHeadDim) {
      cst_s[tid] = P->cstart[tid];
      csz_s[tid] = P->csize[tid];
      dsz_s[tid] = 0;
    }
  }
  for (int k = tid; k < kGroupTok * k_words; k += kThreads) krow_s[k] = 0u;
  if (tid == 0) nf_s = P->n_fields;
  __syncthreads();

  // ---- 1b. rotated keys (randomized Hadamard): y = fp32(H (s * x) / sqrt(128)), the fast
  //      Walsh-Hadamard stages in fp64 (exact for fp16 keys), one rounding at the division and
  //      one to fp32; the K rows below are then read from ky_s ----
  // (only the rotating instantiation carries these buffers)
  __shared__ double rw_s[RM ? kGroupTok : 1][RM ? kHeadDim : 1];
  __shared__ float ky_s[RM ? kGroupTok : 1][RM ? kHeadDim : 1];
  if constexpr (RM == 2) {
    // gain-normalised rows v = fp32(x * ig), signs on the stored dims, then in plan field
    // order the butterflies of each power-of-two chunk of an equal-width run (stage h pairs
    // fields f, f + h with (f - chunk start) & h == 0), fp64, and the division by sqrt(m)
    const int8_t* sg = rot + h * kHeadDim;
    if (tid < nf_s) dsz_s[fdim_s[tid]] = csz_s[tid];
    __syncthreads();
    for (int e = tid; e < kGroupTok * kHeadDim; e += kThreads) {
      const int r = e / kHeadDim, i = e % kHeadDim;
      const double v = static_cast<double>(__fmul_rn(xval(0, 0, r, i), ig_s[i]));
      rw_s[r][i] = dsz_s[i] ? v * static_cast<double>(sg[i]) : v;
    }
    __syncthreads();
    for (int hb = 1; hb < kHeadDim; hb <<= 1) {
      for (int e = tid; e < kGroupTok * kHeadDim; e += kThreads) {
        const int r = e / kHeadDim, f = e % kHeadDim;
        if (hb < csz_s[f] && ((f - cst_s[f]) & hb) == 0) {
          const int d0 = fdim_s[f], d1 = fdim_s[f + hb];
          const double a = rw_s[r][d0], b = rw_s[r][d1];
          rw_s[r][d0] = __dadd_rn(a, b);
          rw_s[r][d1] = __dsub_rn(a, b);
        }
      }
      __syncthreads();
    }
    for (int e = tid; e < kGroupTok * kHeadDim; e += kThreads) {
      const int r = e / kHeadDim, i = e % kHeadDim;
      const int m = dsz_s[i];
      ky_s[r][i] = m ? static_cast<float>(__ddiv_rn(rw_s[r][i], __dsqrt_rn(static_cast<double>(m))))
                     : static_cast<float>(rw_s[r][i]);
    }
    if (tid < kHeadDim) ig_s[tid] = 1.0f;   // the gains are inside the rotated rows now
    __syncthreads();
  }
  if constexpr (RM == 1) {
    const int8_t* sg = rot + h * kHeadDim;
    for (int e = tid; e < kGroupTok * kHeadDim; e += kThreads) {
      const int r = e / kHeadDim, i = e % kHeadDim;
      rw_s[r][i] = static_cast<double>(xval(0, 0, r, i)) * static_cast<double>(sg[i]);
    }
    __syncthreads();
    for (int hb = 1; hb < kHeadDim; hb <<= 1) {
      for (int p = tid; p < kGroupTok * kHeadDim / 2; p += kThreads) {
        const int r = p / (kHeadDim / 2), jj = p % (kHeadDim / 2);
        const int i0 = (jj / hb) * 2 * hb + jj % hb, i1 = i0 + hb;
        const double a = rw_s[r][i0], b = rw_s[r][i1];
        rw_s[r][i0] = __dadd_rn(a, b);
        rw_s[r][i1] = __dsub_rn(a, b);
      }
      __syncthreads();
    }
    const double sq = __dsqrt_rn(static_cast<double>(kHeadDim));
    for (int e = tid; e < kGroupTok * kHeadDim; e += kThreads) {
      const int r = e / kHeadDim, i = e % kHeadDim;
      ky_s[r][i] = static_cast<float>(__ddiv_rn(rw_s[r][i], sq));
    }
    __syncthreads();
  }
  // K value i of staged row r of this head (rotated when the codec rotates)
  auto kval = [&](int r, int i) {
    if constexpr (RM != 0) return ky_s[r][i];
    else return xval(0, NF ? (h - h0) : 0, r, i);
  };

  // ---- 2. scales: lanes 0..7 K, 8..15 V (one token each, in the quantizer's order) ----
  const int hsel = h - h0;   // this head's staged rows
  if (tid < 2 * kGroupTok) {
    const int tsr = tid / kGroupTok, r = tid % kGroupTok;
    __half s16 = __float2half_rn(0.0f);
    if (NF) {
      float a = 0.0f;
      for (int hh = 0; hh < kHeads; ++hh)
        for (int i = 0; i < kHeadDim; ++i) a = fmaxf(a, fabsf(xval(tsr, hh, r, i)));
      s16 = __float2half_rn(a);
    } else {
      // one code path for K and V lanes (no branch per element), so the LDS reads of a batch
      // are issued together and only the fp64 sum is a dependent chain
      double ss = 0.0;
      const float* krot = nullptr;
      if constexpr (RM != 0) krot = &ky_s[r][0];
#pragma unroll 16
      for (int i = 0; i < kHeadDim; ++i) {
        const float x = (RM != 0 && tsr == 0) ? krot[i] : xval(tsr, hsel, r, i);
        const double y = static_cast<double>(__fmul_rn(x, tsr == 0 ? ig_s[i] : 1.0f));
        ss = __dadd_rn(ss, __dmul_rn(y, y));
      }
      s16 = __float2half_rn(static_cast<float>(__dsqrt_rn(ss / static_cast<double>(kHeadDim))));
    }
    (tsr == 0 ? isk_s : isv_s)[r] = inv_scale(s16);
    if (r >= lo && r < hi) {
      const int64_t pos = g0 + r;
      const uint16_t bits = __half_as_ushort(s16);
      uint16_t* sc = tsr == 0 ? ks : vs;
      if (NF) {
        if ((h & 1) == 0) sc[(static_cast<int64_t>(b) * cap + pos) * n_nf + h / 2] = bits;
      } else {
        sc[(static_cast<int64_t>(b) * n_kv + h) * cap + pos] = bits;
      }
    }
  }
  __syncthreads();

  // ---- 3. codes.  K: wave w takes the plan's fields 32 w .. 32 w + 31 (fields are in plan
  //      order, widest first), lane l fields 32 w + l / 8 + 8 m and token l % 8, so the wave's
  //      searches need only as many steps as its first field's width.  V: element e = tid +
  //      256 m is dim e / 8, token e % 8 (v_bits steps).  The four searches of a thread of each
  //      kind advance in lock step. ----
  const int nfld = nf_s;
  const int wv = tid >> 6, ln = tid & 63;
  uint32_t pos[2 * kEl], tb[2 * kEl];
  int wd[2 * kEl], fk[kEl];
  float u[2 * kEl];
#pragma unroll
  for (int m = 0; m < kEl; ++m) {
    const int f = 32 * wv + (ln >> 3) + 8 * m, r = ln & 7;   // K element
    const bool kl = r >= lo && r < hi && f < nfld;
    const int i = kl ? fdim_s[f] : 0;
    const int w = kl ? fw_s[f] : 0;
    const float x = kval(r, i);
    const float y = NF ? x : __fmul_rn(x, ig_s[i]);
    u[m] = __fmul_rn(y, isk_s[r]);
    wd[m] = w;
    fk[m] = f;
    tb[m] = static_cast<uint32_t>(w) * 256u;
    pos[m] = 0u;
    const int e = tid + kThreads * m, fv = e / kGroupTok, rv = e % kGroupTok;   // V element
    const bool vl = rv >= lo && rv < hi;
    u[kEl + m] = __fmul_rn(xval(1, hsel, rv, fv), isv_s[rv]);
    wd[kEl + m] = vl ? vb : 0;
    tb[kEl + m] = static_cast<uint32_t>(vb) * 256u;
    pos[kEl + m] = 0u;
  }
  auto search = [&](int m0, int steps) {
    for (int st = 0; st < steps; ++st) {
#pragma unroll
      for (int m = m0; m < m0 + kEl; ++m) {
        const int sh = wd[m] - 1 - st;
        const uint32_t step = sh >= 0 ? 1u << sh : 0u;
        const float bdv = bd_s[tb[m] + pos[m] + (step ? step : 1u) - 1u];
        pos[m] += (step != 0u && bdv < u[m]) ? step : 0u;
      }
    }
  };
  search(0, 32 * wv < nfld ? fw_s[32 * wv] : 0);   // wave-uniform: the widest field of the wave
  search(kEl, vb);
#pragma unroll
  for (int m = 0; m < kEl; ++m) {
    if (wd[m] > 0) {   // K code into its row word(s)
      const int f = fk[m], r = ln & 7;
      const int off = foff_s[f], w = wd[m];
      const int word = off >> 5, sh = off & 31;
      atomicOr(&krow_s[r * k_words + word], pos[m] << sh);
      if (sh + w > 32) atomicOr(&krow_s[r * k_words + word + 1], pos[m] >> (32 - sh));
    }
    if (wd[kEl + m] > 0) {   // V code into its segment word(s)
      const int e = tid + kThreads * m, fv = e / kGroupTok, rv = e % kGroupTok;
      const int bit = (eb + rv) * vb - 32 * vw0, word = bit >> 5, sh = bit & 31;
      const uint32_t code = pos[kEl + m];
      atomicOr(&vw_s[fv][word], code << sh);
      if (sh + vb > 32) atomicOr(&vw_s[fv][word + 1], code >> (32 - sh));
    }
  }
  __syncthreads();

  // ---- 4. stores ----
  {
    uint32_t* dst = kc + ((static_cast<int64_t>(b) * n_kv + h) * cap + g0) * k_words;
    for (int k = tid + lo * k_words; k < hi * k_words; k += kThreads) dst[k] = krow_s[k];
  }
  {
    const int64_t tile = g0 / kVTile;
    const int gq = static_cast<int>((g0 % kVTile) / 32);   // segment group in the tile
    uint32_t* tile_dst = vc + ((static_cast<int64_t>(b) * n_kv + h) * (cap / kVTile) + tile) * kVTile * 4 * vb;
    for (int k = tid; k < kHeadDim * nvw; k += kThreads) {
      const int i = k / nvw, w = k % nvw;
      const uint32_t bits = vw_s[i][w];
      if (bits) atomicOr(tile_dst + static_cast<int64_t>(((i / 16) * 4 + gq) * 16 + i % 16) * vb + vw0 + w, bits);
    }
  }
}

}  // namespace

hipError_t launch_quantize(kvq_cache* c, int layer, const void* k, const void* v, int dtype,
                           int64_t n_new, int64_t in_stride, int ring_R, int64_t L0, hipStream_t stream) {
  const kvq_config& cfg = c->cfg;
  const int64_t first = L0 / kGroupTok, last = (L0 + n_new - 1) / kGroupTok;
  dim3 grid(static_cast<unsigned>(last - first + 1), static_cast<unsigned>(cfg.n_kv_heads),
            static_cast<unsigned>(cfg.batch));
  const bool nf = cfg.codec == KVQ_CODEC_NF16_B256;
  const int rm = cfg.codec == KVQ_CODEC_UNIFORM_ROT ? 1 : cfg.codec == KVQ_CODEC_BGTQ_ROT ? 2 : 0;
  const Plan* plans = c->plans + static_cast<int64_t>(layer) * c->n_plan * cfg.n_kv_heads;
  const int plan_bs = c->n_plan > 1 ? cfg.n_kv_heads : 0;
#define KVQ_LAUNCH_Q(T, NF, RM)                                                                  \
  hipLaunchKernelGGL((quantize_append<T, NF, RM>), grid, dim3(kThreads), 0, stream,             \
                     static_cast<const T*>(k), static_cast<const T*>(v), n_new, in_stride, ring_R, L0, \
                     cfg.n_kv_heads, c->cap, plans, plan_bs, c->tables, layer_k_codes(c, layer), \
                     layer_v_codes(c, layer), layer_k_scales(c, layer), layer_v_scales(c, layer), \
                     c->k_words, cfg.v_bits, c->n_nf_blocks,                                      \
                     rm ? c->rot_signs + static_cast<int64_t>(layer) * cfg.n_kv_heads * kHeadDim : nullptr)
  if (dtype == KVQ_F16) {
    if (nf) KVQ_LAUNCH_Q(__half, true, 0);
    else if (rm == 1) KVQ_LAUNCH_Q(__half, false, 1);
    else if (rm == 2) KVQ_LAUNCH_Q(__half, false, 2);
    else KVQ_LAUNCH_Q(__half, false, 0);
  } else {
    if (nf) KVQ_LAUNCH_Q(float, true, 0);
    else if (rm == 1) KVQ_LAUNCH_Q(float, false, 1);
    else if (rm == 2) KVQ_LAUNCH_Q(float, false, 2);
    else KVQ_LAUNCH_Q(float, false, 0);
  }
#undef KVQ_LAUNCH_Q
  return hipGetLastError();
}

namespace {

// Copies `count` new positions (input rows row0 .. row0 + count - 1 of a [batch][in_stride]
// [n_kv][128] tensor, positions pos0 ..) into the recent-window rings at slot position mod R,
// rounding fp32 inputs to fp16 (nearest even): keys as [batch][R][n_kv][128], values in
// dim-major 128-slot tiles [batch][n_kv][R / 128][128 dims][128 slots] (the value product's
// operand order).  One workgroup per (position, sequence); thread i copies element i of every
// head.
template <typename T>
__global__ __launch_bounds__(256) void recent_write(const T* __restrict__ kin, const T* __restrict__ vin,
                                                   int64_t in_stride, int64_t row0, int64_t pos0, int n_kv,
                                                   int R, __half* __restrict__ kr, __half* __restrict__ vr) {
  const int64_t i = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t slot = (pos0 + i) % R;
  const int64_t src = (static_cast<int64_t>(b) * in_stride + row0 + i) * n_kv * kHeadDim;
  const int64_t dst = (static_cast<int64_t>(b) * R + slot) * n_kv * kHeadDim;
  for (int e = threadIdx.x; e < n_kv * kHeadDim; e += 256) {
    const int hh = e / kHeadDim, d = e % kHeadDim;
    kr[dst + e] = __float2half_rn(static_cast<float>(kin[src + e]));
    const int64_t vdst = (((static_cast<int64_t>(b) * n_kv + hh) * (R / 128) + slot / 128) * kHeadDim + d) * 128 + slot % 128;
    vr[vdst] = __float2half_rn(static_cast<float>(vin[src + e]));
  }
}

}  // namespace

hipError_t launch_recent_write(kvq_cache* c, int layer, const void* k, const void* v, int dtype,
                               int64_t in_stride, int64_t row0, int64_t pos0, int64_t count,
                               hipStream_t stream) {
  const kvq_config& cfg = c->cfg;
  dim3 grid(static_cast<unsigned>(count), static_cast<unsigned>(cfg.batch));
  if (dtype == KVQ_F16)
    hipLaunchKernelGGL(recent_write<__half>, grid, dim3(256), 0, stream, static_cast<const __half*>(k),
                       static_cast<const __half*>(v), in_stride, row0, pos0, cfg.n_kv_heads,
                       c->ring, layer_k_recent(c, layer), layer_v_recent(c, layer));
  else
    hipLaunchKernelGGL(recent_write<float>, grid, dim3(256), 0, stream, static_cast<const float*>(k),
                       static_cast<const float*>(v), in_stride, row0, pos0, cfg.n_kv_heads,
                       c->ring, layer_k_recent(c, layer), layer_v_recent(c, layer));
  return hipGetLastError();
}

}  // namespace kvq
