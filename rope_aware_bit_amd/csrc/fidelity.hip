// Key-cache fidelity diagnostics on gfx950: attention-logit MAE and softmax KL of the stored
// keys against the keys as given.
//
// RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: the allocation is judged by
// how well the stored keys preserve the query-key logits (per-layer mean absolute error,
// keys only); KV Cache Quantization on WikiText-2 prompt 2048-token (train), evaluation
// results: the softmax KL divergence of the attention distributions.  For query head h of
// sequence b, over the cached positions t:
//   a_t = sigma <q_h, k_t>,   a^_t = sigma <q_h, k^_t>,  k^ = the cache's keys dequantized
//   (s_t g_i CB_{b_i}[code], or s_t NF[code] for the 256-value codec; the fp16 copies for
//   positions in the recent window), all in fp64;
//   mae = mean_t |a_t - a^_t|,  kl = KL(softmax(a) || softmax(a^)).
//
// Kernel 1 (fidelity_partials): one 256-lane workgroup per (split, KV head, sequence).  It
// stages 64 positions at a time (the given keys with 16-byte loads, the packed rows, the
// scales).  Wave w takes positions 16 w .. 16 w + 15 of a round and forms both sets of logits
// as fp64 16x16x4 matrix products (positions x dims times dims x query heads, 32 steps of 4
// dims): each lane supplies one element of the position operand per step (a given key value,
// or a stored one decoded from its packed field, its codebook entry and scales) and one of the
// query operand.  The lane holding column h then keeps running statistics of head h over its
// four positions per round: sum |a - a^|, and for each distribution a running maximum M, the
// sum Z = sum e^(x - M) and (for a) W = sum e^(a - M_a) (a - a^).  The lanes' statistics are
// merged within each wave, then across the four waves, and the split's six numbers per head
// are stored.
// Kernel 2 (fidelity_merge): one wave per (sequence, query head) merges the splits and
// writes mae = sum |a - a^| / T and kl = W / Z_a - M_a - ln Z_a + M_b + ln Z_b.
#include <hip/hip_fp16.h>

#include <cmath>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kFidTok = 64;       // positions staged per round
typedef double d4 __attribute__((ext_vector_type(4)));
constexpr int kFidStats = 6;      // sum|d|, M_a, Z_a, W_a, M_b, Z_b

template <typename T>
__device__ inline double to_d(T v);
template <>
__device__ inline double to_d<__half>(__half v) { return static_cast<double>(__half2float(v)); }
template <>
__device__ inline double to_d<float>(float v) { return static_cast<double>(v); }

struct Stats {
  double abs_sum, ma, za, wa, mb, zb;
};

__device__ inline void stats_init(Stats& s) {
  s.abs_sum = 0.0;
  s.ma = s.mb = -INFINITY;
  s.za = s.wa = s.zb = 0.0;
}

// adds one position with logits a (reference) and b (stored keys)
__device__ inline void stats_add(Stats& s, double a, double b) {
  s.abs_sum += fabs(a - b);
  if (a > s.ma) {
    const double r = exp(s.ma - a);   // 0 for the first position
    s.za = s.za * r + 1.0;
    s.wa = s.wa * r + (a - b);
    s.ma = a;
  } else {
    const double e = exp(a - s.ma);
    s.za += e;
    s.wa += e * (a - b);
  }
  if (b > s.mb) {
    s.zb = s.zb * exp(s.mb - b) + 1.0;
    s.mb = b;
  } else {
    s.zb += exp(b - s.mb);
  }
}

// merges o into s (either may be empty: M = -inf, Z = 0)
__device__ inline void stats_merge(Stats& s, const Stats& o) {
  s.abs_sum += o.abs_sum;
  if (o.za > 0.0) {
    if (s.za == 0.0) {
      s.ma = o.ma;
      s.za = o.za;
      s.wa = o.wa;
    } else {
      const double m = fmax(s.ma, o.ma);
      const double r1 = exp(s.ma - m), r2 = exp(o.ma - m);
      s.za = s.za * r1 + o.za * r2;
      s.wa = s.wa * r1 + o.wa * r2;
      s.ma = m;
    }
  }
  if (o.zb > 0.0) {
    if (s.zb == 0.0) {
      s.mb = o.mb;
      s.zb = o.zb;
    } else {
      const double m = fmax(s.mb, o.mb);
      s.zb = s.zb * exp(s.mb - m) + o.zb * exp(o.mb - m);
      s.mb = m;
    }
  }
}

__device__ inline Stats stats_shfl_xor(const Stats& s, int mask) {
  Stats o;
  o.abs_sum = __shfl_xor(s.abs_sum, mask);
  o.ma = __shfl_xor(s.ma, mask);
  o.za = __shfl_xor(s.za, mask);
  o.wa = __shfl_xor(s.wa, mask);
  o.mb = __shfl_xor(s.mb, mask);
  o.zb = __shfl_xor(s.zb, mask);
  return o;
}

template <typename T, int G>
__global__ __launch_bounds__(256, 2) void fidelity_partials(
    const T* __restrict__ q, const T* __restrict__ keys, int64_t len, int n_kv, int64_t cap,
    double sigma, int64_t tok_per_split, const Plan* __restrict__ plans, int plan_bs, const Tables* __restrict__ tab,
    const uint32_t* __restrict__ kc, const uint16_t* __restrict__ ks, int k_words, int n_nf, int nf,
    int kivi, int pairing, int rot_groups,
    int64_t plen, const __half* __restrict__ rk, int R, const int8_t* __restrict__ rot,
    double* __restrict__ part, int S) {
  constexpr int kVec = 16 / sizeof(T);
  constexpr int kRow = kHeadDim + kVec;            // padded key row (elements)
  const int tid = threadIdx.x;
  const int wave = tid >> 6, mi = tid & 15, kq = (tid & 63) >> 4;   // MFMA row / column, k slot
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = static_cast<int64_t>(b) * n_kv + h;
  const int64_t t_begin = s * tok_per_split;
  const int64_t t_end = t_begin + tok_per_split < len ? t_begin + tok_per_split : len;

  __shared__ double q_s[kMaxGroup][kHeadDim];
  __shared__ double qr_s[kMaxGroup][kHeadDim];   // rotated query (packed keys of the rotated codec)
  __shared__ double g_s[kHeadDim];
  __shared__ uint16_t cb_s[kMaxBits + 1][256];
  __shared__ uint8_t fdim_s[kHeadDim], fw_s[kHeadDim];
  __shared__ uint16_t foff_s[kHeadDim];
  __shared__ __attribute__((aligned(16))) T x_s[kFidTok][kRow];
  __shared__ uint32_t kr_s[kFidTok][4 * kMaxBits + 1];
  __shared__ __attribute__((aligned(16))) __half xr_s[kFidTok][kHeadDim + 8];   // recent-window rows
  __shared__ double sc_s[kFidTok];
  __shared__ __half ksc_s[kHeadDim], klo_s[kHeadDim];   // asymmetric integer codec: the tile's channel parameters
  __shared__ int nf_s;

  const Plan* P = plans + static_cast<int64_t>(b) * plan_bs + h;   // plan of (sequence, head)
  for (int k = tid; k < G * kHeadDim; k += 256)
    q_s[k / kHeadDim][k % kHeadDim] = to_d(q[(static_cast<int64_t>(b) * n_kv * G + h * G) * kHeadDim + k]);
  for (int k = tid; k < (kMaxBits + 1) * 256; k += 256) {
    const int w = k >> 8, c = k & 255;
    cb_s[w][c] = nf ? (w == 4 && c < 16 ? tab->nf_cb[c] : 0) : (w >= 1 ? tab->cb[w][c] : 0);
  }
  __shared__ uint16_t dfo_s[kHeadDim];   // bit offset of dim d's field in the packed row
  __shared__ uint8_t dfw_s[kHeadDim];    // its width (0: the dim is not stored)
  if (tid < kHeadDim) {
    dfw_s[tid] = 0;
    dfo_s[tid] = 0;
    g_s[tid] = nf ? 1.0 : static_cast<double>(P->g[tid]);
    fdim_s[tid] = P->fdim[tid];
    fw_s[tid] = P->fwidth[tid];
    foff_s[tid] = P->foff[tid];
  }
  if (tid == 0) nf_s = P->n_fields;
  __syncthreads();
  const int n_fields = nf_s;
  if (tid < n_fields) {
    dfw_s[fdim_s[tid]] = fw_s[tid];
    dfo_s[fdim_s[tid]] = foff_s[tid];
  }
  // rotated codecs: <q, R^T y> = <R q, y>.  Inside equal-width groups (fp64): R (g * q), chunk
  // by chunk in plan field order (signs, butterflies, 1/sqrt(m)); the gains are then inside
  // the rotated query
  if (rot != nullptr && rot_groups) {
    __shared__ uint8_t cst_s[kHeadDim], csz_s[kHeadDim];
    if (tid < kHeadDim) {
      cst_s[tid] = P->cstart[tid];
      csz_s[tid] = P->csize[tid];
    }
    for (int k = tid; k < G * kHeadDim; k += 256) {
      const int d = k % kHeadDim;
      qr_s[k / kHeadDim][d] = q_s[k / kHeadDim][d] * g_s[d];
    }
    __syncthreads();
    for (int k = tid; k < G * kHeadDim; k += 256) {
      const int f = k % kHeadDim;
      if (f < n_fields) qr_s[k / kHeadDim][fdim_s[f]] *= static_cast<double>(rot[h * kHeadDim + fdim_s[f]]);
    }
    __syncthreads();
    for (int hb = 1; hb < kHeadDim; hb <<= 1) {
      for (int k = tid; k < G * kHeadDim; k += 256) {
        const int hh = k / kHeadDim, f = k % kHeadDim;
        if (hb < csz_s[f] && ((f - cst_s[f]) & hb) == 0) {
          const int d0 = fdim_s[f], d1 = fdim_s[f + hb];
          const double a = qr_s[hh][d0], bq = qr_s[hh][d1];
          qr_s[hh][d0] = a + bq;
          qr_s[hh][d1] = a - bq;
        }
      }
      __syncthreads();
    }
    for (int k = tid; k < G * kHeadDim; k += 256) {
      const int f = k % kHeadDim;
      if (f < n_fields) qr_s[k / kHeadDim][fdim_s[f]] /= sqrt(static_cast<double>(csz_s[f]));
    }
    __syncthreads();
    if (tid < kHeadDim) g_s[tid] = 1.0;
  } else if (rot != nullptr) {
    for (int k = tid; k < G * kHeadDim; k += 256)
      qr_s[k / kHeadDim][k % kHeadDim] = q_s[k / kHeadDim][k % kHeadDim] * static_cast<double>(rot[h * kHeadDim + k % kHeadDim]);
    __syncthreads();
    for (int hb = 1; hb < kHeadDim; hb <<= 1) {
      for (int p = tid; p < G * kHeadDim / 2; p += 256) {
        const int hh = p / (kHeadDim / 2), jj = p % (kHeadDim / 2);
        const int i0 = (jj / hb) * 2 * hb + jj % hb, i1 = i0 + hb;
        const double a = qr_s[hh][i0], bq = qr_s[hh][i1];
        qr_s[hh][i0] = a + bq;
        qr_s[hh][i1] = a - bq;
      }
      __syncthreads();
    }
    const double sq = sqrt(static_cast<double>(kHeadDim));
    for (int k = tid; k < G * kHeadDim; k += 256) qr_s[k / kHeadDim][k % kHeadDim] /= sq;
  } else {
    for (int k = tid; k < G * kHeadDim; k += 256) qr_s[k / kHeadDim][k % kHeadDim] = q_s[k / kHeadDim][k % kHeadDim];
  }
  __syncthreads();

  Stats st;   // head mi's statistics over this lane's positions
  stats_init(st);
  // which rows of the product this lane's four results belong to: one product of the row
  // numbers (A[i][0] = i + 1) with ones (B[0][j] = 1) tells, whatever the register layout
  int prow[4];
  {
    const d4 z = {0.0, 0.0, 0.0, 0.0};
    const d4 pr = __builtin_amdgcn_mfma_f64_16x16x4f64(kq == 0 ? static_cast<double>(mi + 1) : 0.0,
                                                       kq == 0 ? 1.0 : 0.0, z, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) prow[r] = static_cast<int>(pr[r]) - 1;
  }
  for (int64_t r0 = t_begin; r0 < t_end; r0 += kFidTok) {
    const int nr = t_end - r0 < kFidTok ? static_cast<int>(t_end - r0) : kFidTok;
    // stage the given keys (16-byte pieces), the packed rows and the scales: the loads of the
    // keys and rows are all issued first (indices clamped to the round; the packed words of
    // window positions are zero, within capacity, and never read), then the scales, then the
    // stores, so the round waits for memory once
    constexpr int kXIt = kFidTok * (kHeadDim / kVec) / 256;
    constexpr int kKIt = kFidTok * 4 * kMaxBits / 256;
    uint4 xv[kXIt];
    uint32_t kw[kKIt];
#pragma unroll
    for (int i = 0; i < kXIt; ++i) {
      const int k = tid + 256 * i, r = k / (kHeadDim / kVec), c = k % (kHeadDim / kVec);
      const int rc = r < nr ? r : nr - 1;
      xv[i] = *reinterpret_cast<const uint4*>(keys + ((static_cast<int64_t>(b) * len + r0 + rc) * n_kv + h) * kHeadDim + c * kVec);
    }
    const int nkw = nr * k_words;
#pragma unroll
    for (int i = 0; i < kKIt; ++i) {
      const int k = tid + 256 * i;
      kw[i] = kc[(bh * cap + r0) * k_words + (k < nkw ? k : nkw - 1)];
    }
    if (!kivi && tid < nr && r0 + tid < plen) {
      const uint16_t sb = nf ? ks[(static_cast<int64_t>(b) * cap + r0 + tid) * n_nf + h / 2] : ks[bh * cap + r0 + tid];
      sc_s[tid] = static_cast<double>(__half2float(__ushort_as_half(sb)));
    }
#pragma unroll
    for (int i = 0; i < kXIt; ++i) {
      const int k = tid + 256 * i, r = k / (kHeadDim / kVec), c = k % (kHeadDim / kVec);
      *reinterpret_cast<uint4*>(&x_s[r][c * kVec]) = xv[i];
    }
    // stored rows: packed below plen, fp16 ring copies (slot p mod R) from plen on
#pragma unroll
    for (int i = 0; i < kKIt; ++i) {
      const int k = tid + 256 * i, kk = k < nkw ? k : nkw - 1;
      kr_s[kk / k_words][kk % k_words] = kw[i];
    }
    for (int k = tid; k < nr * (kHeadDim / 8); k += 256) {
      const int r = k / (kHeadDim / 8), c = k % (kHeadDim / 8);
      if (r0 + r >= plen) {
        const int64_t slot = (r0 + r) % R;
        *reinterpret_cast<uint4*>(&xr_s[r][8 * c]) =
            *reinterpret_cast<const uint4*>(rk + ((static_cast<int64_t>(b) * R + slot) * n_kv + h) * kHeadDim + 8 * c);
      }
    }
    if (kivi && tid < kHeadDim && r0 < plen) {
      // [tile][block j][s(p0), s(p1), lo(p0), lo(p1)]; the round lies inside one 128-position tile
      const int j = pairing == KVQ_ROPE_HALF ? tid % kBlocks : tid / 2;
      const int co = pairing == KVQ_ROPE_HALF ? tid / kBlocks : tid % 2;
      const uint16_t* kp = ks + ((bh * (cap / kVTile) + r0 / kVTile) * kBlocks + j) * 4;
      ksc_s[tid] = __ushort_as_half(kp[co]);
      klo_s[tid] = __ushort_as_half(kp[2 + co]);
    }
    if (tid < kFidTok) kr_s[tid][k_words] = 0u;   // zero word after the row (fields read two words)
    __syncthreads();
    // wave w: positions 16 w .. 16 w + 15 of the round as fp64 16x16x4 products, rows =
    // positions, columns = query heads (G of 16 used), 4 dims per step:
    //   a = <x_t, q_h> (given keys), a_hat = <k_hat_t, q'_h> (stored keys; q' = q rotated,
    //   with the gains inside for the group rotation), plus <window row, q_h> for recent rows
    // lane l gives A[l % 16][l / 16] and B[l / 16][l % 16] and holds D[prow[r]][l % 16]
    {
      const int tl = 16 * wave + mi;                   // this lane's A row (staged position)
      const bool valid = tl < nr;
      const bool packed = valid && r0 + tl < plen;
      const bool ring = valid && r0 + tl >= plen;
      const bool any_packed = r0 + 16 * wave < plen && 16 * wave < nr;
      const bool any_ring = r0 + 16 * wave + 15 >= plen && 16 * wave < nr;
      const double s16 = packed ? sc_s[tl] : 0.0;
      d4 da = {0.0, 0.0, 0.0, 0.0}, db = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
      for (int kk = 0; kk < kHeadDim / 4; ++kk) {
        const int d = 4 * kk + kq;
        const double bq = mi < G ? q_s[mi][d] : 0.0;
        const double ag = valid ? to_d(x_s[tl][d]) : 0.0;
        da = __builtin_amdgcn_mfma_f64_16x16x4f64(ag, bq, da, 0, 0, 0);
        if (any_packed) {
          double ap = 0.0;
          const int w = dfw_s[d];
          if (packed && w > 0) {
            const int off = dfo_s[d];
            const uint64_t two = static_cast<uint64_t>(kr_s[tl][off >> 5]) |
                                 (static_cast<uint64_t>(kr_s[tl][(off >> 5) + 1]) << 32);
            const uint32_t code = static_cast<uint32_t>(two >> (off & 31)) & ((1u << w) - 1u);
            // asymmetric integer codec: fp16(lo + s * code) with one rounding
            ap = kivi ? static_cast<double>(__half2float(__hfma(ksc_s[d], __float2half_rn(static_cast<float>(code)), klo_s[d])))
                      : (s16 * g_s[d]) * static_cast<double>(__half2float(__ushort_as_half(cb_s[w][code])));
          }
          const double br = mi < G ? qr_s[mi][d] : 0.0;
          db = __builtin_amdgcn_mfma_f64_16x16x4f64(ap, br, db, 0, 0, 0);
        }
        if (any_ring) {
          // recent window: the stored key is the fp16 copy, against the plain query
          const double ar = ring ? static_cast<double>(__half2float(xr_s[tl][d])) : 0.0;
          db = __builtin_amdgcn_mfma_f64_16x16x4f64(ar, bq, db, 0, 0, 0);
        }
      }
      if (mi < G) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (16 * wave + prow[r] < nr) stats_add(st, sigma * da[r], sigma * db[r]);
        }
      }
    }
    __syncthreads();
  }
  // merge the lanes of one head (l % 16) in the wave, then the four waves through LDS
  __shared__ double wst_s[4][kMaxGroup][kFidStats];
  for (int m = 16; m <= 32; m <<= 1) {
    const Stats o = stats_shfl_xor(st, m);
    stats_merge(st, o);
  }
  if (kq == 0 && mi < G) {
    double* d = wst_s[wave][mi];
    d[0] = st.abs_sum;
    d[1] = st.ma;
    d[2] = st.za;
    d[3] = st.wa;
    d[4] = st.mb;
    d[5] = st.zb;
  }
  __syncthreads();
  if (tid < G) {
    Stats acc;
    stats_init(acc);
    for (int w = 0; w < 4; ++w) {
      const double* d = wst_s[w][tid];
      const Stats o{d[0], d[1], d[2], d[3], d[4], d[5]};
      stats_merge(acc, o);
    }
    double* p = part + ((bh * G + tid) * S + s) * kFidStats;
    p[0] = acc.abs_sum;
    p[1] = acc.ma;
    p[2] = acc.za;
    p[3] = acc.wa;
    p[4] = acc.mb;
    p[5] = acc.zb;
  }
}

__global__ __launch_bounds__(64) void fidelity_merge(const double* __restrict__ part, int S, int64_t len,
                                                     double* __restrict__ mae, double* __restrict__ kl) {
  const int lane = threadIdx.x;
  const int64_t hq = blockIdx.x;   // sequence * n_q + query head
  Stats st;
  stats_init(st);
  for (int s = lane; s < S; s += 64) {
    const double* p = part + (hq * S + s) * kFidStats;
    Stats o{p[0], p[1], p[2], p[3], p[4], p[5]};
    stats_merge(st, o);
  }
  for (int m = 32; m >= 1; m >>= 1) {
    const Stats o = stats_shfl_xor(st, m);
    stats_merge(st, o);
  }
  if (lane == 0) {
    mae[hq] = st.abs_sum / static_cast<double>(len);
    kl[hq] = st.wa / st.za - st.ma - log(st.za) + st.mb + log(st.zb);
  }
}

}  // namespace

hipError_t launch_fidelity(kvq_cache* c, int layer, const void* q, const void* keys, int dtype,
                           float scale, double* mae, double* kl, hipStream_t stream) {
  const kvq_config& cfg = c->cfg;
  const int64_t len = c->len[layer], plen = packed_len(c, layer);
  const int H = cfg.n_kv_heads, B = cfg.batch, G = c->group;
  const int64_t units = static_cast<int64_t>(B) * H;
  // about four workgroups per compute unit, at least 256 positions each
  int64_t S = (4LL * c->n_cu + units - 1) / units;
  const int64_t by_len = (len + 255) / 256;
  if (S > by_len) S = by_len;
  if (S > c->fid_max_splits) S = c->fid_max_splits;
  if (S < 1) S = 1;
  const int64_t per = ((len + S - 1) / S + kFidTok - 1) / kFidTok * kFidTok;
  S = (len + per - 1) / per;
  const double sigma = scale > 0.0f ? static_cast<double>(scale) : 1.0 / std::sqrt(static_cast<double>(kHeadDim));
  const bool nf = cfg.codec == KVQ_CODEC_NF16_B256;
  const Plan* plans = c->plans + static_cast<int64_t>(layer) * c->n_plan * H;
  const int plan_bs = c->n_plan > 1 ? H : 0;
  dim3 grid(static_cast<unsigned>(S), static_cast<unsigned>(H), static_cast<unsigned>(B));
#define KVQ_FID(T, GG)                                                                              \
  hipLaunchKernelGGL((fidelity_partials<T, GG>), grid, dim3(256), 0, stream, static_cast<const T*>(q), \
                     static_cast<const T*>(keys), len, H, c->cap, sigma, per, plans, plan_bs, c->tables, \
                     layer_k_codes(c, layer), layer_k_scales(c, layer), c->k_words, c->n_nf_blocks,   \
                     nf ? 1 : 0, cfg.codec == KVQ_CODEC_KIVI ? 1 : 0, cfg.pairing,                  \
                     cfg.codec == KVQ_CODEC_BGTQ_ROT ? 1 : 0, plen, plen < len ? layer_k_recent(c, layer) : nullptr,       \
                     c->ring > 0 ? c->ring : 1,                                                   \
                     codec_rotates(cfg.codec) ? c->rot_signs + static_cast<int64_t>(layer) * H * kHeadDim : nullptr, \
                     c->fid_part, static_cast<int>(S))
#define KVQ_FID_G(T)                  \
  switch (G) {                        \
    case 1: KVQ_FID(T, 1); break;     \
    case 2: KVQ_FID(T, 2); break;     \
    case 4: KVQ_FID(T, 4); break;     \
    default: KVQ_FID(T, 8); break;    \
  }
  if (dtype == KVQ_F16) {
    KVQ_FID_G(__half)
  } else {
    KVQ_FID_G(float)
  }
#undef KVQ_FID_G
#undef KVQ_FID
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fidelity_merge, dim3(static_cast<unsigned>(units * G)), dim3(64), 0, stream, c->fid_part,
                     static_cast<int>(S), len, mae, kl);
  return hipGetLastError();
}

}  // namespace kvq
