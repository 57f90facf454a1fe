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
  __shared__ __attribute__((aligned(16))) float bd_s[(kMaxBits + 1) * 256];
  __shared__ float ig_s[kHeadDim];
  __shared__ uint8_t fdim_s[kHeadDim], fw_s[kHeadDim];
  __shared__ uint16_t foff_s[kHeadDim];
  __shared__ __attribute__((aligned(16))) uint32_t krow_s[kGroupTok * 4 * kMaxBits];
  __shared__ uint32_t vw_s[kHeadDim][4];           // the group's V segment words, per dim
  __shared__ float isk_s[kGroupTok], isv_s[kGroupTok];
  __shared__ int nf_s;

  // ---- 1. every load of the workgroup first (rows, tables, plan: one round of memory
  //      latency; nothing loaded is used before all are issued), then the LDS images.  Rows
  //      outside [lo, hi) read the nearest row inside (their images are never used). ----
  const int h0 = NF ? (h & ~1) : h;   // first head of the staged block
  constexpr int kPieces = kHeadDim / kVec;                                 // 16-byte pieces per row
  constexpr int kRowIt = 2 * kHeads * kGroupTok * kPieces / kThreads;      // pieces per thread
  constexpr int kBd4 = (kMaxBits + 1) * 256 / 4;
  constexpr int kBdIt = (kBd4 + kThreads - 1) / kThreads;
  uint4 xr[kRowIt];
#pragma unroll
  for (int it = 0; it < kRowIt; ++it) {
    const int k = tid + kThreads * it;
    const int q = k % kPieces;
    const int r = (k / kPieces) % kGroupTok;
    const int hh = (k / (kPieces * kGroupTok)) % kHeads;
    const int tsr = k / (kPieces * kGroupTok * kHeads);   // 0: K, 1: V
    const int rc = r < lo ? lo : r >= hi ? hi - 1 : r;
    if (ring_R == 0) {
      const int64_t src = ((static_cast<int64_t>(b) * in_stride + (g0 + rc - L0)) * n_kv + h0 + hh) * kHeadDim + q * kVec;
      xr[it] = *reinterpret_cast<const uint4*>((tsr ? vin : kin) + src);
    } else {
      // recent-window rings (fp16): keys [batch][R][n_kv][128], values in dim-major 128-slot
      // tiles [batch][n_kv][R / 128][128][128]; position p sits in slot p mod R
      const int64_t slot = (g0 + rc) % ring_R;
      if (tsr == 0) {
        xr[it] = *reinterpret_cast<const uint4*>(kin + ((static_cast<int64_t>(b) * ring_R + slot) * n_kv + h0 + hh) * kHeadDim + q * kVec);
      } else {
        const T* vt = vin + (((static_cast<int64_t>(b) * n_kv + h0 + hh) * (ring_R / 128) + slot / 128) * kHeadDim + q * kVec) * 128 + slot % 128;
        T e8[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) e8[e] = vt[e * 128];
        __builtin_memcpy(&xr[it], e8, 16);
      }
    }
  }
  uint4 bdr[NF ? 1 : kBdIt];
  float nfb = 0.0f;
  if constexpr (NF) {
    nfb = tab->nf_bd[tid & 15];
  } else {
#pragma unroll
    for (int j = 0; j < kBdIt; ++j) {
      const int q = tid + kThreads * j;
      bdr[j] = reinterpret_cast<const uint4*>(&tab->bd[0][0])[q < kBd4 ? q : kBd4 - 1];
    }
  }
  const Plan* P = plans + static_cast<int64_t>(b) * plan_bs + h;   // plan of (sequence, head)
  const int pi = tid & (kHeadDim - 1);
  const float igv = P->ig[pi];
  const uint32_t fdv = P->fdim[pi], fwv = P->fwidth[pi], fov = P->foff[pi];
  uint32_t cstv = 0u, cszv = 0u;
  if constexpr (RM == 2) {
    cstv = P->cstart[pi];
    cszv = P->csize[pi];
  }
  float sgv = 1.0f;   // rotating codecs: the sign of dim pi
  if constexpr (RM != 0) sgv = static_cast<float>(rot[h * kHeadDim + pi]);
  const int nfv = P->n_fields;
#pragma unroll
  for (int it = 0; it < kRowIt; ++it) {
    const int k = tid + kThreads * it;
    const int q = k % kPieces;
    const int r = (k / kPieces) % kGroupTok;
    const int hh = (k / (kPieces * kGroupTok)) % kHeads;
    const int tsr = k / (kPieces * kGroupTok * kHeads);
    uint32_t* d = &x_s[tsr][hh][r][q * 4];
    d[0] = xr[it].x;
    d[1] = xr[it].y;
    d[2] = xr[it].z;
    d[3] = xr[it].w;
  }
  // (the table stores are unconditional: threads past it rewrite its last piece with the same
  // value, so the compiler has no reason to move their loads down to a conditional store)
  if constexpr (NF) {
#pragma unroll
    for (int j = 0; j < (kMaxBits + 1); ++j) {
      const int k = tid + kThreads * j, bb = k >> 8, e = k & 255;
      bd_s[k] = bb == 4 && e < 16 ? nfb : INFINITY;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kBdIt; ++j) {
      const int q = tid + kThreads * j;
      reinterpret_cast<uint4*>(bd_s)[q < kBd4 ? q : kBd4 - 1] = bdr[j];
    }
  }
  // (the plan's entries are written by both halves of the workgroup, with the same values, so
  // that their loads are not moved down to a conditional store either)
  ig_s[pi] = igv;
  fdim_s[pi] = static_cast<uint8_t>(fdv);
  fw_s[pi] = static_cast<uint8_t>(fwv);
  foff_s[pi] = static_cast<uint16_t>(fov);
  if (tid < kHeadDim) vw_s[tid][0] = vw_s[tid][1] = vw_s[tid][2] = vw_s[tid][3] = 0u;
  // rotation inside equal-width groups: field f's chunk, and each dim's chunk size (0: the
  // dim's block is not stored)
  __shared__ uint8_t cst_s[RM == 2 ? kHeadDim : 1], csz_s[RM == 2 ? kHeadDim : 1], dsz_s[RM == 2 ? kHeadDim : 1];
  __shared__ float sg_s[RM ? kHeadDim : 1];
  if constexpr (RM != 0) sg_s[pi] = sgv;
  if constexpr (RM == 2) {
    cst_s[pi] = static_cast<uint8_t>(cstv);
    csz_s[pi] = static_cast<uint8_t>(cszv);
    if (tid < kHeadDim) dsz_s[tid] = 0;
  }
  for (int k = tid; k < kGroupTok * k_words; k += kThreads) krow_s[k] = 0u;
  if (tid == 0) nf_s = nfv;
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
    if (tid < nf_s) dsz_s[fdim_s[tid]] = csz_s[tid];
    __syncthreads();
    for (int e = tid; e < kGroupTok * kHeadDim; e += kThreads) {
      const int r = e / kHeadDim, i = e % kHeadDim;
      const double v = static_cast<double>(__fmul_rn(xval(0, 0, r, i), ig_s[i]));
      rw_s[r][i] = dsz_s[i] ? v * static_cast<double>(sg_s[i]) : v;
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
    for (int e = tid; e < kGroupTok * kHeadDim; e += kThreads) {
      const int r = e / kHeadDim, i = e % kHeadDim;
      rw_s[r][i] = static_cast<double>(xval(0, 0, r, i)) * static_cast<double>(sg_s[i]);
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
  // 256-value absmax codec: the absolute maximum of each staged (tensor, token) block by all
  // threads, 16 lanes per block with 16 values each, then across those lanes (a maximum does not
  // depend on the order in which it is taken)
  __shared__ float amax_s[NF ? 2 * kGroupTok : 1];
  if constexpr (NF) {
    const int blk = tid >> 4, sub = tid & 15;   // block tensor * 8 + token
    const int tsr = blk / kGroupTok, r = blk % kGroupTok;
    float a = 0.0f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int v = sub + 16 * u;                // value v: head v / 128, dim v % 128
      a = fmaxf(a, fabsf(xval(tsr, v >> 7, r, v & (kHeadDim - 1))));
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    if (sub == 0) amax_s[blk] = a;
    __syncthreads();
  }
  if (tid < 2 * kGroupTok) {
    const int tsr = tid / kGroupTok, r = tid % kGroupTok;
    __half s16 = __float2half_rn(0.0f);
    if (NF) {
      s16 = __float2half_rn(amax_s[tid]);
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

// Many new positions (a prefill), for the codecs without rotation or absmax blocks, from the
// caller's rows: the same row quantizer as quantize_append, one workgroup per 32 consecutive
// positions (one V segment) of one (sequence, KV head), 8 waves.
//   - One wave runs the 64 scale sums (32 key and 32 value rows, one lane each, dim order).
//   - Keys: thread t quantizes fields 8 (t / 32) .. + 7 of position t % 32, so the 32 lanes
//     that share a field hold 32 different rows and OR into 32 different row words (the LDS row
//     image has an odd stride: no two lanes of a field share a bank); wave w holds fields
//     16 w .. 16 w + 15.
//   - Values: thread t quantizes dim t / 4 at the 8 positions 8 (t % 4) .. + 7, packs their
//     codes into words in registers and ORs a handful of words into the segment image.
//   - The searches take one step size per step for a whole wave (the widest field of the wave,
//     or the value width): a narrower field's boundaries are followed by +inf in the table,
//     which no value exceeds, so the extra steps leave its code unchanged.
//   - A segment whose 32 positions are all new is stored with plain stores (no other position
//     shares its words); the first and last segments of a call are OR-ed in.
constexpr int kBulkTok = 32;
constexpr int kBulkThreads = 512;   // 8 waves per workgroup

template <typename T, int VB>
__global__ __launch_bounds__(kBulkThreads) void quantize_bulk(
    const T* __restrict__ kin, const T* __restrict__ vin, int64_t n_new, int64_t in_stride, int64_t L0, int n_kv,
    int64_t cap, const Plan* __restrict__ plans, int plan_bs, const Tables* __restrict__ tab,
    uint32_t* __restrict__ kc, uint32_t* __restrict__ vc, uint16_t* __restrict__ ks,
    uint16_t* __restrict__ vs, int k_words) {
  constexpr int kVec = 16 / sizeof(T);
  constexpr int kRowW = kHeadDim * static_cast<int>(sizeof(T)) / 4 + 1;   // odd: no bank conflicts
  constexpr int kBd4 = (kMaxBits + 1) * 256 / 4;
  constexpr int kVW = VB | 1;                     // odd stride of the segment image rows (>= VB words)
  constexpr int kBT = kBulkThreads;
  constexpr int kE = kBulkTok * kHeadDim / kBT;   // key (and value) elements per thread: 8
  constexpr int kVPer = kBulkTok / kE;             // threads per value dim: 4
  constexpr int kLW = (kE * VB + 31) / 32;         // words of one thread's value codes
  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t g0 = (L0 / kBulkTok + blockIdx.x) * kBulkTok;   // first position of the segment
  const int lo = static_cast<int>(L0 > g0 ? L0 - g0 : 0);
  const int hi = static_cast<int>(L0 + n_new - g0 < kBulkTok ? L0 + n_new - g0 : kBulkTok);
  const int ks_stride = k_words | 1;               // odd stride of the K row image

  __shared__ uint32_t x_s[2][kBulkTok][kRowW];   // [K, V][position] rows of T
  auto xval = [&](int tsr, int r, int i) { return to_f(reinterpret_cast<const T*>(&x_s[tsr][r][0])[i]); };
  __shared__ __attribute__((aligned(16))) float bd_s[(kMaxBits + 1) * 256];
  // gains of the key rows (ig) and of the value rows (1), indexed by tensor
  __shared__ __attribute__((aligned(16))) float g2_s[2][kHeadDim];
  float* ig_s = g2_s[0];
  __shared__ uint8_t fdim_s[kHeadDim], fw_s[kHeadDim];
  __shared__ uint16_t foff_s[kHeadDim];
  // the K row image, 32 rows of k_words | 1 words and a spare word, in dynamic LDS sized by the
  // launch (so that narrow rows leave room for a fifth workgroup per compute unit)
  extern __shared__ uint32_t krow_s[];
  __shared__ uint32_t vw_s[kHeadDim * kVW];       // the segment's words, per dim
  __shared__ __attribute__((aligned(16))) float isk_s[kBulkTok];
  __shared__ __attribute__((aligned(16))) float isv_s[kBulkTok];
  __shared__ int nf_s;

  // ---- 1. every load of the workgroup first (rows, boundaries, plan: one round of memory
  //      latency; nothing loaded is used before all are issued), then the LDS images.  Rows
  //      outside [lo, hi) read the nearest row inside (their images are never used). ----
  constexpr int kPieces = kHeadDim / kVec;                     // 16-byte pieces per row
  constexpr int kRowIt = 2 * kBulkTok * kPieces / kBT;    // pieces per thread
  constexpr int kBdIt = (kBd4 + kBT - 1) / kBT;
  uint4 xr[kRowIt], bdr[kBdIt];
#pragma unroll
  for (int i = 0; i < kRowIt; ++i) {
    const int k = tid + kBT * i;
    const int q = k % kPieces, r = (k / kPieces) % kBulkTok, tsr = k / (kPieces * kBulkTok);
    const int rc = r < lo ? lo : r >= hi ? hi - 1 : r;
    const int64_t src = ((static_cast<int64_t>(b) * in_stride + (g0 + rc - L0)) * n_kv + h) * kHeadDim + q * kVec;
    xr[i] = *reinterpret_cast<const uint4*>((tsr ? vin : kin) + src);
  }
#pragma unroll
  for (int j = 0; j < kBdIt; ++j) {
    const int q = tid + kBT * j;
    bdr[j] = reinterpret_cast<const uint4*>(&tab->bd[0][0])[q < kBd4 ? q : kBd4 - 1];
  }
  const Plan* P = plans + static_cast<int64_t>(b) * plan_bs + h;
  const int pi = tid & (kHeadDim - 1);
  const float igv = P->ig[pi];
  const uint32_t fdv = P->fdim[pi], fwv = P->fwidth[pi], fov = P->foff[pi];
  const int nfv = P->n_fields;
  for (int k = tid; k < kBulkTok * ks_stride + 1; k += kBT) krow_s[k] = 0u;
  for (int k = tid; k < kHeadDim * kVW; k += kBT) vw_s[k] = 0u;
#pragma unroll
  for (int i = 0; i < kRowIt; ++i) {
    const int k = tid + kBT * i;
    const int q = k % kPieces, r = (k / kPieces) % kBulkTok, tsr = k / (kPieces * kBulkTok);
    uint32_t* d = &x_s[tsr][r][q * 4];
    d[0] = xr[i].x;
    d[1] = xr[i].y;
    d[2] = xr[i].z;
    d[3] = xr[i].w;
  }
  // (unconditional: threads past the table rewrite its last piece with the same value, so the
  // compiler has no reason to move their loads down to a conditional store)
#pragma unroll
  for (int j = 0; j < kBdIt; ++j) {
    const int q = tid + kBT * j;
    reinterpret_cast<uint4*>(bd_s)[q < kBd4 ? q : kBd4 - 1] = bdr[j];
  }
  if (tid < kHeadDim) {
    g2_s[0][tid] = igv;
    g2_s[1][tid] = 1.0f;
    fdim_s[tid] = static_cast<uint8_t>(fdv);
    fw_s[tid] = static_cast<uint8_t>(fwv);
    foff_s[tid] = static_cast<uint16_t>(fov);
  }
  if (tid == 0) nf_s = nfv;
  __syncthreads();

  // ---- 2. scales (wave 0: lane l < 32 key row l, lane 32 + l value row l, the quantizer's
  //      order); the other waves meanwhile read their elements ----
  const int wv = tid >> 6;
  const int nfld = nf_s;
  const int kr_ = tid & 31, fg = tid >> 5;        // key: position kr_, fields kE fg .. kE fg + kE - 1
  const int vd = tid / kVPer, r0 = kE * (tid % kVPer);   // value: dim vd, positions r0 .. r0 + kE - 1
  float uk[kE], uv[kE];
  auto gather = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kE; ++j) {
      const int f = kE * fg + j;
      const int d = fdim_s[f];
      uk[j] = __fmul_rn(xval(0, kr_, d), ig_s[d]);   // y = x * ig
      uv[j] = xval(1, r0 + j, vd);
    }
  };
  if (wv != 0) gather();
  if (wv == 0) {
    const int tsr = tid / kBulkTok, r = tid % kBulkTok;
    const float* gp = g2_s[tsr];   // keys: y = x * ig_i; values: y = x * 1
    double ss = 0.0;
    // the sum in dim order; each square y_i^2 is exact in fp64 (a product of two fp32 values), so
    // one fused multiply-add ss + y_i * y_i rounds exactly as the addition of the square does
    for (int i0 = 0; i0 < kHeadDim; i0 += 16) {
      double yd[16];
#pragma unroll
      for (int u = 0; u < 16; u += 4) {
        const float4 g4 = *reinterpret_cast<const float4*>(gp + i0 + u);
        const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          float x0, x1;
          if constexpr (sizeof(T) == 2) {   // one 32-bit word holds the fp16 pair i, i + 1
            const uint32_t w = x_s[tsr][r][(i0 + u + e) >> 1];
            x0 = __half2float(__ushort_as_half(static_cast<uint16_t>(w & 0xFFFFu)));
            x1 = __half2float(__ushort_as_half(static_cast<uint16_t>(w >> 16)));
          } else {
            x0 = __uint_as_float(x_s[tsr][r][i0 + u + e]);
            x1 = __uint_as_float(x_s[tsr][r][i0 + u + e + 1]);
          }
          yd[u + e] = static_cast<double>(__fmul_rn(x0, gv[e]));
          yd[u + e + 1] = static_cast<double>(__fmul_rn(x1, gv[e + 1]));
        }
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) ss = __fma_rn(yd[u], yd[u], ss);
    }
    const __half s16 = __float2half_rn(static_cast<float>(__dsqrt_rn(ss / static_cast<double>(kHeadDim))));
    (tsr == 0 ? isk_s : isv_s)[r] = inv_scale(s16);
    if (r >= lo && r < hi) (tsr == 0 ? ks : vs)[(static_cast<int64_t>(b) * n_kv + h) * cap + g0 + r] = __half_as_ushort(s16);
  }
  __syncthreads();
  if (wv == 0) gather();

  // ---- 3. codes: u = y * is; the count of boundaries below u by a search of S steps ----
  {
    const float isk = isk_s[kr_];
#pragma unroll
    for (int j = 0; j < kE; ++j) uk[j] = __fmul_rn(uk[j], isk);
#pragma unroll
    for (int j = 0; j < kE; j += 4) {
      const float4 iv = *reinterpret_cast<const float4*>(&isv_s[r0 + j]);
      uv[j] = __fmul_rn(uv[j], iv.x);
      uv[j + 1] = __fmul_rn(uv[j + 1], iv.y);
      uv[j + 2] = __fmul_rn(uv[j + 2], iv.z);
      uv[j + 3] = __fmul_rn(uv[j + 3], iv.w);
    }
  }
  // search state as byte addresses into the boundary table: row w (1 KB) plus 4 x code, so that
  // with the steps unrolled each probe is one LDS read at a constant offset from it
  const char* bdb = reinterpret_cast<const char*>(bd_s);
  uint32_t pk[kE], pv[kE];
#pragma unroll
  for (int j = 0; j < kE; ++j) {
    pk[j] = static_cast<uint32_t>(fw_s[kE * fg + j]) * 1024u;
    pv[j] = static_cast<uint32_t>(VB) * 1024u;
  }
  // wave-uniform step counts: the wave's widest field (fields are widest first) and the value width
  const int ksteps = __builtin_amdgcn_readfirstlane(2 * kE * wv < nfld ? fw_s[2 * kE * wv] : 0);
#pragma unroll
  for (int st = kMaxBits - 1; st >= 0; --st) {
    if (st >= ksteps) continue;
    constexpr uint32_t one = 1u;
    const uint32_t step4 = (one << st) * 4u;
#pragma unroll
    for (int j = 0; j < kE; ++j) {
      const float bdv = *reinterpret_cast<const float*>(bdb + pk[j] + (step4 - 4u));
      pk[j] = bdv < uk[j] ? pk[j] + step4 : pk[j];
    }
  }
#pragma unroll
  for (int st = VB - 1; st >= 0; --st) {
    const uint32_t step4 = (1u << st) * 4u;
#pragma unroll
    for (int j = 0; j < kE; ++j) {
      const float bdv = *reinterpret_cast<const float*>(bdb + pv[j] + (step4 - 4u));
      pv[j] = bdv < uv[j] ? pv[j] + step4 : pv[j];
    }
  }
#pragma unroll
  for (int j = 0; j < kE; ++j) {   // back to codes
    pk[j] = (pk[j] >> 2) & 255u;
    pv[j] = (pv[j] >> 2) & 255u;
  }
  // key codes into the row image (position kr_, lanes of one field on distinct rows), without
  // branches: fields past the stored ones have width 0, offset 0 and code 0 (they OR nothing),
  // rows outside [lo, hi) are never stored, and a field's bits are OR-ed into its word and the
  // next (zero when it does not straddle; the image has a spare word after its last row)
  {
    uint32_t* row = krow_s + kr_ * ks_stride;
#pragma unroll
    for (int j = 0; j < kE; ++j) {
      const int f = kE * fg + j;
      const int off = foff_s[f];
      const uint64_t bits = static_cast<uint64_t>(pk[j]) << (off & 31);
      atomicOr(&row[off >> 5], static_cast<uint32_t>(bits));
      atomicOr(&row[(off >> 5) + 1], static_cast<uint32_t>(bits >> 32));
    }
  }
  // value codes: this thread's kE positions of dim vd as a bit string in registers, then OR-ed
  // into the segment image at bit r0 VB (positions outside [lo, hi) contribute 0)
  {
    uint32_t lw[kLW + 1];
#pragma unroll
    for (int i = 0; i <= kLW; ++i) lw[i] = 0u;
#pragma unroll
    for (int j = 0; j < kE; ++j) {
      const uint32_t code = (r0 + j >= lo && r0 + j < hi) ? pv[j] : 0u;
      const int bit = j * VB, word = bit >> 5, sh = bit & 31;
      lw[word] |= code << sh;
      if (sh + VB > 32) lw[word + 1] |= code >> (32 - sh);
    }
    const int base = r0 * VB, bw = base >> 5, bs = base & 31;
    uint32_t* row = vw_s + vd * kVW;
#pragma unroll
    for (int i = 0; i < kLW; ++i) {
      if (lw[i] == 0u) continue;
      atomicOr(&row[bw + i], lw[i] << bs);
      if (bs != 0 && (lw[i] >> (32 - bs)) != 0u) atomicOr(&row[bw + i + 1], lw[i] >> (32 - bs));
    }
  }
  __syncthreads();

  // ---- 4. stores ----
  {
    // half-wave per row (k_words <= 32): rows 2 w + (lane / 32), + 8, ...; no division
    uint32_t* dst = kc + ((static_cast<int64_t>(b) * n_kv + h) * cap + g0) * k_words;
    const int wl = tid & 31;
    for (int r = (tid >> 5); r < kBulkTok; r += kBT / 32)
      if (r >= lo && r < hi && wl < k_words) dst[r * k_words + wl] = krow_s[r * ks_stride + wl];
  }
  {
    const int gq = static_cast<int>((g0 % kVTile) / kBulkTok);
    uint32_t* tile_dst = vc + ((static_cast<int64_t>(b) * n_kv + h) * (cap / kVTile) + g0 / kVTile) * kVTile * 4 * VB;
    const bool whole = lo == 0 && hi == kBulkTok;
    for (int k = tid; k < kHeadDim * VB; k += kBT) {
      const int i = k / VB, w = k % VB;
      const uint32_t bits = vw_s[i * kVW + w];
      uint32_t* d = tile_dst + static_cast<int64_t>(((i / 16) * 4 + gq) * 16 + i % 16) * VB + w;
      if (whole) *d = bits;
      else if (bits) atomicOr(d, bits);
    }
  }
}

// A few new positions (a decode step's), one workgroup per (KV head, sequence): the same row
// quantizer as quantize_append, arranged for latency.  Every load of the call (rows, plan,
// boundary tables) is issued in one round; the squares y_i^2 of all rows are formed in parallel
// (exact in fp64), so the scale lane of each row only runs the sum's dependent chain; every
// thread then quantizes one (position, element) at a time; K rows are stored whole and V codes
// OR-ed into their segment words in HBM.  No fp16 window, no rotation, not the 256-value codec.
constexpr int kSmallMax = 4;   // positions per call handled this way

template <typename T>
__global__ __launch_bounds__(kThreads) void quantize_small(
    const T* __restrict__ kin, const T* __restrict__ vin, int n_new, int64_t L0, int n_kv, int64_t cap,
    const Plan* __restrict__ plans, int plan_bs, const Tables* __restrict__ tab, uint32_t* __restrict__ kc,
    uint32_t* __restrict__ vc, uint16_t* __restrict__ ks, uint16_t* __restrict__ vs, int k_words, int v_bits) {
  constexpr int kVec = 16 / sizeof(T);                       // elements per 16-byte load
  constexpr int kRowVec = kHeadDim / kVec;                   // 16-byte pieces per row
  constexpr int kBd4 = (kMaxBits + 1) * 256 / 4;             // boundary table in 16-byte pieces
  const int tid = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  const Plan* P = plans + static_cast<int64_t>(b) * plan_bs + h;

  __shared__ __attribute__((aligned(16))) float bd_s[(kMaxBits + 1) * 256];
  __shared__ __attribute__((aligned(16))) T x_s[2][kSmallMax][kHeadDim];      // [K, V][position][dim]
  __shared__ __attribute__((aligned(16))) double sq_s[2 * kSmallMax][kHeadDim];
  __shared__ float ig_s[kHeadDim];
  __shared__ uint8_t fdim_s[kHeadDim], fw_s[kHeadDim];
  __shared__ uint16_t foff_s[kHeadDim];
  __shared__ float is_s[2 * kSmallMax];
  __shared__ uint32_t krow_s[kSmallMax * 4 * kMaxBits];

  // ---- one round of loads: boundary tables, rows, plan ----
  uint4 bdv[(kBd4 + kThreads - 1) / kThreads];
#pragma unroll
  for (int j = 0; j < (kBd4 + kThreads - 1) / kThreads; ++j) {
    const int q = tid + kThreads * j;
    bdv[j] = reinterpret_cast<const uint4*>(&tab->bd[0][0])[q < kBd4 ? q : kBd4 - 1];
  }
  // row piece tid: tensor tid / (kSmallMax kRowVec), position, 16-byte piece
  const int rt = tid / (kSmallMax * kRowVec), rp = (tid / kRowVec) % kSmallMax, rq = tid % kRowVec;
  const bool rl = rt < 2 && rp < n_new;
  uint4 xv = make_uint4(0u, 0u, 0u, 0u);
  if (rl) {
    const T* src = (rt ? vin : kin) + ((static_cast<int64_t>(b) * n_new + rp) * n_kv + h) * kHeadDim + rq * kVec;
    xv = *reinterpret_cast<const uint4*>(src);
  }
  float igv = 1.0f;
  uint32_t fdv = 0u, fwv = 0u, fov = 0u;
  if (tid < kHeadDim) {
    igv = P->ig[tid];
    fdv = P->fdim[tid];
    fwv = P->fwidth[tid];
    fov = P->foff[tid];
  }
  const int nfld = P->n_fields;
#pragma unroll
  for (int j = 0; j < (kBd4 + kThreads - 1) / kThreads; ++j) {
    const int q = tid + kThreads * j;
    if (q < kBd4) reinterpret_cast<uint4*>(bd_s)[q] = bdv[j];
  }
  if (rl) *reinterpret_cast<uint4*>(&x_s[rt][rp][rq * kVec]) = xv;
  if (tid < kHeadDim) {
    ig_s[tid] = igv;
    fdim_s[tid] = static_cast<uint8_t>(fdv);
    fw_s[tid] = static_cast<uint8_t>(fwv);
    foff_s[tid] = static_cast<uint16_t>(fov);
  }
  for (int k = tid; k < kSmallMax * k_words; k += kThreads) krow_s[k] = 0u;
  __syncthreads();

  // ---- squares y_i^2 in fp64 (exact), all rows at once: y = x * ig for K, x for V ----
  for (int e = tid; e < 2 * n_new * kHeadDim; e += kThreads) {
    const int c = e / kHeadDim, i = e % kHeadDim;           // chain c: K of position c, or V of c - n_new
    const int t = c < n_new ? 0 : 1, p = c < n_new ? c : c - n_new;
    const float x = to_f(x_s[t][p][i]);
    const double y = static_cast<double>(t == 0 ? __fmul_rn(x, ig_s[i]) : x);
    sq_s[c][i] = __dmul_rn(y, y);
  }
  __syncthreads();
  // ---- scales: the sum of squares in dim order, one lane per row ----
  if (tid < 2 * n_new) {
    const int c = tid, t = c < n_new ? 0 : 1, p = c < n_new ? c : c - n_new;
    double ss = 0.0;
#pragma unroll 16
    for (int i = 0; i < kHeadDim; ++i) ss = __dadd_rn(ss, sq_s[c][i]);
    const __half s16 = __float2half_rn(static_cast<float>(__dsqrt_rn(ss / static_cast<double>(kHeadDim))));
    is_s[c] = inv_scale(s16);
    (t == 0 ? ks : vs)[(static_cast<int64_t>(b) * n_kv + h) * cap + L0 + p] = __half_as_ushort(s16);
  }
  __syncthreads();

  // ---- codes: element e = (position, K field or V dim); binary search over the width's
  //      boundaries (a u on a boundary takes the lower code) ----
  for (int e = tid; e < 2 * n_new * kHeadDim; e += kThreads) {
    const int c = e / kHeadDim, j = e % kHeadDim;
    const bool key = c < n_new;
    const int p = key ? c : c - n_new;
    int w;
    float u;
    if (key) {
      if (j >= nfld) continue;
      const int i = fdim_s[j];
      w = fw_s[j];
      u = __fmul_rn(__fmul_rn(to_f(x_s[0][p][i]), ig_s[i]), is_s[c]);
    } else {
      w = v_bits;
      u = __fmul_rn(to_f(x_s[1][p][j]), is_s[c]);
    }
    uint32_t code = 0u;
    const float* bw = bd_s + 256 * w;
    for (int sh = w - 1; sh >= 0; --sh) {
      const uint32_t step = 1u << sh;
      code += bw[code + step - 1u] < u ? step : 0u;
    }
    if (key) {
      const int off = foff_s[j], word = off >> 5, sb = off & 31;
      atomicOr(&krow_s[p * k_words + word], code << sb);
      if (sb + w > 32) atomicOr(&krow_s[p * k_words + word + 1], code >> (32 - sb));
    } else {
      const int64_t pos = L0 + p;
      const int gq = static_cast<int>((pos % kVTile) / 32), bit = static_cast<int>(pos % 32) * w;
      uint32_t* seg = vc + ((static_cast<int64_t>(b) * n_kv + h) * (cap / kVTile) + pos / kVTile) * kVTile * 4 * w +
                      static_cast<int64_t>(((j / 16) * 4 + gq) * 16 + j % 16) * w;
      const int word = bit >> 5, sb = bit & 31;
      if (code) {
        atomicOr(seg + word, code << sb);
        if (sb + w > 32 && (code >> (32 - sb))) atomicOr(seg + word + 1, code >> (32 - sb));
      }
    }
  }
  __syncthreads();
  uint32_t* dst = kc + ((static_cast<int64_t>(b) * n_kv + h) * cap + L0) * k_words;
  for (int k = tid; k < n_new * k_words; k += kThreads) dst[k] = krow_s[k];
}

}  // namespace

hipError_t launch_quantize(kvq_cache* c, int layer, const void* k, const void* v, int dtype,
                           int64_t n_new, int64_t in_stride, int ring_R, int64_t L0, hipStream_t stream) {
  const kvq_config& cfg = c->cfg;
  if (n_new <= kSmallMax && ring_R == 0 && in_stride == n_new &&
      (cfg.codec == KVQ_CODEC_BGTQ || cfg.codec == KVQ_CODEC_UNIFORM)) {
    const Plan* plans = c->plans + static_cast<int64_t>(layer) * c->n_plan * cfg.n_kv_heads;
    const int plan_bs = c->n_plan > 1 ? cfg.n_kv_heads : 0;
    dim3 grid(static_cast<unsigned>(cfg.n_kv_heads), static_cast<unsigned>(cfg.batch));
    if (dtype == KVQ_F16)
      hipLaunchKernelGGL(quantize_small<__half>, grid, dim3(kThreads), 0, stream, static_cast<const __half*>(k),
                         static_cast<const __half*>(v), static_cast<int>(n_new), L0, cfg.n_kv_heads, c->cap, plans,
                         plan_bs, c->tables, layer_k_codes(c, layer), layer_v_codes(c, layer),
                         layer_k_scales(c, layer), layer_v_scales(c, layer), c->k_words, cfg.v_bits);
    else
      hipLaunchKernelGGL(quantize_small<float>, grid, dim3(kThreads), 0, stream, static_cast<const float*>(k),
                         static_cast<const float*>(v), static_cast<int>(n_new), L0, cfg.n_kv_heads, c->cap, plans,
                         plan_bs, c->tables, layer_k_codes(c, layer), layer_v_codes(c, layer),
                         layer_k_scales(c, layer), layer_v_scales(c, layer), c->k_words, cfg.v_bits);
    return hipGetLastError();
  }
  if (n_new >= kBulkTok && ring_R == 0 && (cfg.codec == KVQ_CODEC_BGTQ || cfg.codec == KVQ_CODEC_UNIFORM)) {
    const Plan* plans = c->plans + static_cast<int64_t>(layer) * c->n_plan * cfg.n_kv_heads;
    const int plan_bs = c->n_plan > 1 ? cfg.n_kv_heads : 0;
    const int64_t first = L0 / kBulkTok, last = (L0 + n_new - 1) / kBulkTok;
    dim3 grid(static_cast<unsigned>(last - first + 1), static_cast<unsigned>(cfg.n_kv_heads),
              static_cast<unsigned>(cfg.batch));
    const size_t krow_bytes = (static_cast<size_t>(kBulkTok) * (c->k_words | 1) + 1) * sizeof(uint32_t);
#define KVQ_LAUNCH_BULK(T, VB)                                                                        \
  hipLaunchKernelGGL((quantize_bulk<T, VB>), grid, dim3(kBulkThreads), krow_bytes, stream, static_cast<const T*>(k), \
                     static_cast<const T*>(v), n_new, in_stride, L0, cfg.n_kv_heads, c->cap, plans, plan_bs, \
                     c->tables, layer_k_codes(c, layer), layer_v_codes(c, layer), layer_k_scales(c, layer), \
                     layer_v_scales(c, layer), c->k_words)
#define KVQ_LAUNCH_BULK_T(T)                  \
  switch (cfg.v_bits) {                       \
    case 1: KVQ_LAUNCH_BULK(T, 1); break;     \
    case 2: KVQ_LAUNCH_BULK(T, 2); break;     \
    case 3: KVQ_LAUNCH_BULK(T, 3); break;     \
    case 4: KVQ_LAUNCH_BULK(T, 4); break;     \
    case 5: KVQ_LAUNCH_BULK(T, 5); break;     \
    case 6: KVQ_LAUNCH_BULK(T, 6); break;     \
    case 7: KVQ_LAUNCH_BULK(T, 7); break;     \
    default: KVQ_LAUNCH_BULK(T, 8); break;    \
  }
    if (dtype == KVQ_F16) {
      KVQ_LAUNCH_BULK_T(__half);
    } else {
      KVQ_LAUNCH_BULK_T(float);
    }
#undef KVQ_LAUNCH_BULK_T
#undef KVQ_LAUNCH_BULK
    return hipGetLastError();
  }
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
