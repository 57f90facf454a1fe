// Per-(layer, KV head) RoPE-block bit allocation on gfx950.
//
// RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: each 2-D RoPE
// frequency block of each (layer, KV head) gets an energy score computed from
// keys alone; integer widths are then raised greedily by marginal gain.
//
// With per-sequence plans every sequence's calibration keys give a plan of their own: the
// kernels below run once per (sequence, KV head) instead of once per KV head.
//
// Kernel 1 (energy_chunks): one workgroup per (256-token chunk, KV head).  The
// chunk's keys of that head are first copied into LDS with coalesced loads (one
// round of memory latency); lane j then sums block j's squared norm over the
// chunk in token order (fp64; each term x0*x0 + x1*x1 with exact squares and one
// rounding).
// Kernel 2 (greedy_plan): one workgroup per KV head.  Lane j adds the chunk
// partials in chunk order and divides by 2T.  The greedy raises, (k_bits - b_min)
// * 64 times, the block with the largest s_j * delta(b_j) (ties to the smallest
// block).  delta is strictly decreasing, so block j's candidate gains
// s_j * delta(b), b = b_min .. b_max - 1, decrease in b and the greedy takes the
// candidates of all blocks in the order (gain descending, block ascending, b
// ascending): the width of block j is b_min plus the number of its candidates
// among the first N of that order.  A bitonic sort of the 512 candidates in LDS
// gives that order, hence the same widths as the sequential steps.
// Gains sqrt(m_j / mean m) and the plan (field order: blocks by width
// descending then index, coordinate p0 then p1) follow.
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

constexpr int kEnergyTok = 128;   // tokens staged in LDS at a time (a chunk is 1 or 2 stages)

template <typename T>
__global__ __launch_bounds__(256) void energy_chunks(const T* __restrict__ keys, int64_t n_tok,
                                                     int n_kv, int pairing, double* __restrict__ scratch,
                                                     int64_t n_chunks) {
  const int tid = threadIdx.x, j = tid;
  const int h = blockIdx.y;
  const int64_t c = blockIdx.x;
  const int64_t u = static_cast<int64_t>(blockIdx.z) * n_kv + h;   // (sequence, head) unit
  keys += static_cast<int64_t>(blockIdx.z) * n_tok * n_kv * kHeadDim;
  const int p0 = pairing == KVQ_ROPE_HALF ? j : 2 * j;
  const int p1 = pairing == KVQ_ROPE_HALF ? j + kBlocks : 2 * j + 1;
  __shared__ T x_s[kEnergyTok][kHeadDim + 16 / sizeof(T)];   // padded rows
  constexpr int kVec = 16 / sizeof(T);                       // elements per 16-byte load
  double acc = 0.0;
  for (int64_t s0 = c * kEnergyChunk; s0 < (c + 1) * kEnergyChunk && s0 < n_tok; s0 += kEnergyTok) {
    const int64_t ns = n_tok - s0 < kEnergyTok ? n_tok - s0 : kEnergyTok;
    // stage: thread t copies 16-byte pieces t, t + 256, ... of the stage's rows, all loads
    // issued before the first store (rows past the stage's end repeat its last row, unused)
    constexpr int kIt = kEnergyTok * kHeadDim / kVec / 256;
    uint4 v[kIt];
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int k = tid + 256 * i, r = k / (kHeadDim / kVec), q = k % (kHeadDim / kVec);
      const int64_t rc = r < ns ? r : ns - 1;
      v[i] = *reinterpret_cast<const uint4*>(keys + ((s0 + rc) * n_kv + h) * kHeadDim + q * kVec);
    }
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int k = tid + 256 * i, r = k / (kHeadDim / kVec), q = k % (kHeadDim / kVec);
      *reinterpret_cast<uint4*>(&x_s[r][q * kVec]) = v[i];
    }
    __syncthreads();
    if (j < kBlocks) {
      for (int r = 0; r < ns; ++r) {
        const double x0 = static_cast<double>(load_f(&x_s[r][p0]));
        const double x1 = static_cast<double>(load_f(&x_s[r][p1]));
        acc = __dadd_rn(acc, __dadd_rn(__dmul_rn(x0, x0), __dmul_rn(x1, x1)));
      }
    }
    __syncthreads();
  }
  if (j < kBlocks) scratch[(u * n_chunks + c) * kBlocks + j] = acc;
}

__global__ __launch_bounds__(512) void greedy_plan(const double* __restrict__ scratch, int64_t n_chunks,
                                                   int64_t n_tok, const double* __restrict__ weight,
                                                   int k_bits, int b_min, int b_max, int codec,
                                                   int pairing, const Tables* __restrict__ tab,
                                                   Plan* __restrict__ plans) {
  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const int64_t u = static_cast<int64_t>(blockIdx.y) * gridDim.x + h;   // (sequence, head) unit
  __shared__ double m_s[kBlocks];
  __shared__ int w_s[kBlocks];
  __shared__ double cand_s[kBlocks * kMaxBits];   // candidate gains, then sorted
  __shared__ int cid_s[kBlocks * kMaxBits];       // candidate j * 8 + b, sorted alongside
  __shared__ int cnt_s[kBlocks];
  __shared__ double mbar_s;
  __shared__ int nf_s;

  const bool bgtq = codec_allocates(codec);
  if (tid < kBlocks) {
    const int j = tid;
    double m = 0.0;
    if (bgtq) {
      double S = 0.0;
      for (int64_t c = 0; c < n_chunks; ++c)
        S = __dadd_rn(S, scratch[(u * n_chunks + c) * kBlocks + j]);
      m = __ddiv_rn(S, 2.0 * static_cast<double>(n_tok));
    }
    m_s[j] = m;
    cnt_s[j] = 0;
  }
  __syncthreads();
  // candidate (j, b) for b in [b_min, b_max): gain s_j * delta(b); others are absent (-inf,
  // sorted last)
  {
    const int j = tid >> 3, b = tid & 7;
    const double m = m_s[j];
    // equal scores make the greedy hand out a uniform width (UNIFORM and NF16 plans)
    const double sj = bgtq ? (weight ? __dmul_rn(m, weight[u * kBlocks + j]) : m) : 1.0;
    cand_s[tid] = (b >= b_min && b < b_max) ? __dmul_rn(sj, static_cast<double>(tab->delta[b])) : -INFINITY;
    cid_s[tid] = tid;
  }
  __syncthreads();
  // bitonic sort of the 512 candidates into the greedy's order: gain descending, then
  // (block, step) ascending; "a before b" is a total order, so the sort is unique
  for (int k = 2; k <= kBlocks * kMaxBits; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      const int i = tid, pr = i ^ jj;
      if (pr > i) {
        const double va = cand_s[i], vb = cand_s[pr];
        const int ia = cid_s[i], ib = cid_s[pr];
        const bool a_first = va > vb || (va == vb && ia < ib);
        const bool up = (i & k) == 0;   // this half of the bitonic block in "before" order
        if (a_first != up) {
          cand_s[i] = vb;
          cand_s[pr] = va;
          cid_s[i] = ib;
          cid_s[pr] = ia;
        }
      }
      __syncthreads();
    }
  }
  // the greedy's (k_bits - b_min) * 64 steps take the first candidates of that order
  if (tid < (k_bits - b_min) * kBlocks) atomicAdd(&cnt_s[cid_s[tid] >> 3], 1);
  __syncthreads();
  // threads 0..63 finish block j = tid; all threads keep meeting at the barriers
  const bool act = tid < kBlocks;
  const int j = act ? tid : 0;
  const double m = m_s[j];
  const int b = b_min + cnt_s[j];
  if (act) w_s[j] = b;
  __syncthreads();
  if (tid == 0) {
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

  // rank in plan order and bit offset of the block's first field; the blocks of equal width
  // form the run of fields [2 n_wider, 2 (n_wider + n_equal)) in plan order
  int rank = 0, off = 0, n_wider = 0, n_equal = 0;
  for (int k = 0; k < kBlocks; ++k) {
    const int wk = w_s[k];
    if (wk > b || (wk == b && k < j)) {
      ++rank;
      off += 2 * wk;
    }
    n_wider += wk > b ? 1 : 0;
    n_equal += wk == b ? 1 : 0;
  }
  const int p0 = pairing == KVQ_ROPE_HALF ? j : 2 * j;
  const int p1 = pairing == KVQ_ROPE_HALF ? j + kBlocks : 2 * j + 1;
  Plan* P = plans + u;
  // fields past n_fields are zero: every lane first clears two slots, then writes its own
  if (act) {
    P->cstart[2 * j] = P->cstart[2 * j + 1] = 0;
    P->csize[2 * j] = P->csize[2 * j + 1] = 0;
    P->fdim[2 * j] = P->fdim[2 * j + 1] = 0;
    P->fwidth[2 * j] = P->fwidth[2 * j + 1] = 0;
    P->foff[2 * j] = P->foff[2 * j + 1] = 0;
    P->pdesc[j] = 0u;
  }
  __syncthreads();
  if (!act) return;
  if (b > 0) {
    P->fdim[2 * rank] = static_cast<uint8_t>(p0);
    P->fdim[2 * rank + 1] = static_cast<uint8_t>(p1);
    P->fwidth[2 * rank] = P->fwidth[2 * rank + 1] = static_cast<uint8_t>(b);
    P->foff[2 * rank] = static_cast<uint16_t>(off);
    P->foff[2 * rank + 1] = static_cast<uint16_t>(off + b);
    P->pdesc[rank] = static_cast<uint32_t>(off) | (static_cast<uint32_t>(b) << 16);
    // rotation chunks: the run's power-of-two pieces, largest first
    for (int e = 0; e < 2; ++e) {
      const int f = 2 * rank + e;
      int start = 2 * n_wider, o = f - start, n = 2 * n_equal;
      for (int bit = 7; bit >= 0; --bit) {
        const int m = 1 << bit;
        if (!(n & m)) continue;
        if (o < m) {
          P->cstart[f] = static_cast<uint8_t>(start);
          P->csize[f] = static_cast<uint8_t>(m);
          break;
        }
        o -= m;
        start += m;
      }
    }
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
  const bool bgtq = codec_allocates(cfg.codec);
  const int64_t n_chunks = bgtq ? (n_tok + kEnergyChunk - 1) / kEnergyChunk : 0;
  if (bgtq) {
    dim3 grid(static_cast<unsigned>(n_chunks), static_cast<unsigned>(H), static_cast<unsigned>(c->n_plan));
    if (dtype == KVQ_F16)
      hipLaunchKernelGGL(energy_chunks<__half>, grid, dim3(256), 0, stream,
                         static_cast<const __half*>(keys), n_tok, H, cfg.pairing, c->energy_scratch,
                         n_chunks);
    else
      hipLaunchKernelGGL(energy_chunks<float>, grid, dim3(256), 0, stream,
                         static_cast<const float*>(keys), n_tok, H, cfg.pairing, c->energy_scratch,
                         n_chunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int k_bits = cfg.codec == KVQ_CODEC_NF16_B256 ? 4 : cfg.k_bits;
  const int b_min = bgtq ? cfg.b_min : 0;
  const int b_max = bgtq ? cfg.b_max : kMaxBits;
  hipLaunchKernelGGL(greedy_plan, dim3(H, c->n_plan), dim3(kBlocks * kMaxBits), 0, stream, c->energy_scratch, n_chunks, n_tok,
                     block_weight, k_bits, b_min, b_max, cfg.codec, cfg.pairing, c->tables,
                     c->plans + static_cast<int64_t>(layer) * c->n_plan * H);
  return hipGetLastError();
}

}  // namespace kvq
