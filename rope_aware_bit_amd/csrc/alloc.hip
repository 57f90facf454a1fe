// Per-(layer, KV head) RoPE-block bit allocation on gfx950.
//
// RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: each 2-D RoPE
// frequency block of each (layer, KV head) gets an energy score computed from
// keys alone; integer widths are then raised greedily by marginal gain.
//
// Kernel 1 (energy_chunks): one 64-lane wave per (256-token chunk, KV head);
// lane j sums the block's squared norm over the chunk in token order (fp64;
// each term x0*x0 + x1*x1 with exact squares and one rounding).
// Kernel 2 (greedy_plan): one wave per KV head; lane j adds the chunk partials
// in chunk order, divides by 2T, then runs the (k_bits - b_min) * 64 greedy
// steps with a wave-wide argmax (ties to the lowest lane = smallest block),
// derives gains sqrt(m_j / mean m) and writes the plan (field order: blocks by
// width descending then index, coordinate p0 then p1).
#include <hip/hip_fp16.h>

#include <cmath>

#include "kvq_internal.h"

namespace kvq {
namespace {

template <typename T>
__device__ inline float load_f(const T* p);
template <>
__device__ inline float load_f<__half>(const __half* p) { return __half2float(*p); }
template <>
__device__ inline float load_f<float>(const float* p) { return *p; }

template <typename T>
__global__ __launch_bounds__(64) void energy_chunks(const T* __restrict__ keys, int64_t n_tok,
                                                    int n_kv, int pairing, double* __restrict__ scratch,
                                                    int64_t n_chunks) {
  const int j = threadIdx.x;
  const int h = blockIdx.y;
  const int64_t c = blockIdx.x;
  const int p0 = pairing == KVQ_ROPE_HALF ? j : 2 * j;
  const int p1 = pairing == KVQ_ROPE_HALF ? j + kBlocks : 2 * j + 1;
  const int64_t t0 = c * kEnergyChunk;
  const int64_t t1 = t0 + kEnergyChunk < n_tok ? t0 + kEnergyChunk : n_tok;
  double acc = 0.0;
  for (int64_t t = t0; t < t1; ++t) {
    const T* row = keys + (t * n_kv + h) * kHeadDim;
    const double x0 = static_cast<double>(load_f(row + p0));
    const double x1 = static_cast<double>(load_f(row + p1));
    acc = __dadd_rn(acc, __dadd_rn(__dmul_rn(x0, x0), __dmul_rn(x1, x1)));
  }
  scratch[(static_cast<int64_t>(h) * n_chunks + c) * kBlocks + j] = acc;
}

__global__ __launch_bounds__(64) void greedy_plan(const double* __restrict__ scratch, int64_t n_chunks,
                                                  int64_t n_tok, const double* __restrict__ weight,
                                                  int k_bits, int b_min, int b_max, int codec,
                                                  int pairing, const Tables* __restrict__ tab,
                                                  Plan* __restrict__ plans) {
  const int j = threadIdx.x;
  const int h = blockIdx.x;
  __shared__ double m_s[kBlocks];
  __shared__ int w_s[kBlocks];
  __shared__ double mbar_s;
  __shared__ int nf_s;

  const bool bgtq = codec == KVQ_CODEC_BGTQ;
  double m = 0.0;
  if (bgtq) {
    double S = 0.0;
    for (int64_t c = 0; c < n_chunks; ++c)
      S = __dadd_rn(S, scratch[(static_cast<int64_t>(h) * n_chunks + c) * kBlocks + j]);
    m = __ddiv_rn(S, 2.0 * static_cast<double>(n_tok));
  }
  // equal scores make the greedy hand out a uniform width (UNIFORM and NF16 plans)
  const double s = bgtq ? (weight ? __dmul_rn(m, weight[h * kBlocks + j]) : m) : 1.0;

  int b = b_min;
  const int steps = (k_bits - b_min) * kBlocks;
  for (int it = 0; it < steps; ++it) {
    double bv = b < b_max ? __dmul_rn(s, static_cast<double>(tab->delta[b])) : -INFINITY;
    int bi = j;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi == j) ++b;
  }

  m_s[j] = m;
  w_s[j] = b;
  __syncthreads();
  if (j == 0) {
    double t = 0.0;
    int nf = 0;
    for (int k = 0; k < kBlocks; ++k) {
      t = __dadd_rn(t, m_s[k]);
      nf += w_s[k] > 0 ? 2 : 0;
    }
    mbar_s = __ddiv_rn(t, static_cast<double>(kBlocks));
    nf_s = nf;
  }
  __syncthreads();

  float g = 1.0f, ig = 1.0f;
  if (bgtq && mbar_s != 0.0) {
    if (m == 0.0) {
      g = ig = 0.0f;
    } else {
      const double r = __dsqrt_rn(__ddiv_rn(m, mbar_s));
      g = static_cast<float>(r);
      ig = static_cast<float>(__ddiv_rn(1.0, r));
    }
  }

  // rank in plan order and bit offset of the block's first field
  int rank = 0, off = 0;
  for (int k = 0; k < kBlocks; ++k) {
    const int wk = w_s[k];
    if (wk > b || (wk == b && k < j)) {
      ++rank;
      off += 2 * wk;
    }
  }
  const int p0 = pairing == KVQ_ROPE_HALF ? j : 2 * j;
  const int p1 = pairing == KVQ_ROPE_HALF ? j + kBlocks : 2 * j + 1;
  Plan* P = plans + h;
  // fields past n_fields are zero: every lane first clears two slots, then writes its own
  P->fdim[2 * j] = P->fdim[2 * j + 1] = 0;
  P->fwidth[2 * j] = P->fwidth[2 * j + 1] = 0;
  P->foff[2 * j] = P->foff[2 * j + 1] = 0;
  P->pdesc[j] = 0u;
  __syncthreads();
  if (b > 0) {
    P->fdim[2 * rank] = static_cast<uint8_t>(p0);
    P->fdim[2 * rank + 1] = static_cast<uint8_t>(p1);
    P->fwidth[2 * rank] = P->fwidth[2 * rank + 1] = static_cast<uint8_t>(b);
    P->foff[2 * rank] = static_cast<uint16_t>(off);
    P->foff[2 * rank + 1] = static_cast<uint16_t>(off + b);
    P->pdesc[rank] = static_cast<uint32_t>(off) | (static_cast<uint32_t>(b) << 16);
  }
  P->g[p0] = P->g[p1] = g;
  P->ig[p0] = P->ig[p1] = ig;
  P->dwidth[p0] = P->dwidth[p1] = static_cast<uint8_t>(b);
  P->bwidth[j] = static_cast<int8_t>(b);
  if (j == 0) {
    P->n_fields = nf_s;
    P->pad[0] = P->pad[1] = P->pad[2] = 0;
  }
}

}  // namespace

hipError_t launch_alloc(kvq_cache* c, int layer, const void* keys, int dtype, int64_t n_tok,
                        const double* block_weight, hipStream_t stream) {
  const kvq_config& cfg = c->cfg;
  const int H = cfg.n_kv_heads;
  const bool bgtq = cfg.codec == KVQ_CODEC_BGTQ;
  const int64_t n_chunks = bgtq ? (n_tok + kEnergyChunk - 1) / kEnergyChunk : 0;
  if (bgtq) {
    dim3 grid(static_cast<unsigned>(n_chunks), static_cast<unsigned>(H));
    if (dtype == KVQ_F16)
      hipLaunchKernelGGL(energy_chunks<__half>, grid, dim3(64), 0, stream,
                         static_cast<const __half*>(keys), n_tok, H, cfg.pairing, c->energy_scratch,
                         n_chunks);
    else
      hipLaunchKernelGGL(energy_chunks<float>, grid, dim3(64), 0, stream,
                         static_cast<const float*>(keys), n_tok, H, cfg.pairing, c->energy_scratch,
                         n_chunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int k_bits = cfg.codec == KVQ_CODEC_NF16_B256 ? 4 : cfg.k_bits;
  const int b_min = bgtq ? cfg.b_min : 0;
  const int b_max = bgtq ? cfg.b_max : kMaxBits;
  hipLaunchKernelGGL(greedy_plan, dim3(H), dim3(64), 0, stream, c->energy_scratch, n_chunks, n_tok,
                     block_weight, k_bits, b_min, b_max, cfg.codec, cfg.pairing, c->tables,
                     c->plans + static_cast<int64_t>(layer) * H);
  return hipGetLastError();
}

}  // namespace kvq
