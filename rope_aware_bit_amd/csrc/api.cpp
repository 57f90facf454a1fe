// Host side of the libkvq C ABI: validation, cache memory, bookkeeping, launches.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "kvq_internal.h"

using kvq::kBlocks;
using kvq::kHeadDim;
using kvq::kMaxBits;
using kvq::kVTile;

namespace {

thread_local std::string g_last_error;

kvq_status hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return KVQ_EHIP;
}

bool config_valid(const kvq_config* c) {
  if (!c) return false;
  if (c->n_layers < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1 || c->batch < 1) return false;
  if (c->head_dim != kHeadDim) return false;
  if (c->max_tokens < 1 || c->max_tokens > (int64_t(1) << 40)) return false;
  if (c->n_q_heads % c->n_kv_heads != 0) return false;
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  if (c->codec < KVQ_CODEC_BGTQ || c->codec > KVQ_CODEC_BGTQ_ROT) return false;
  if (c->recent_window < 0 || c->recent_window > kvq::kMaxRecent || c->recent_window % 128) return false;
  if (c->pairing != KVQ_ROPE_HALF && c->pairing != KVQ_ROPE_INTERLEAVED) return false;
  if (c->per_sequence_plans != 0 && c->per_sequence_plans != 1) return false;
  if (c->v_bits < 1 || c->v_bits > kMaxBits) return false;
  if (c->b_min < 0 || c->b_max > kMaxBits || c->b_min > c->b_max) return false;
  if (c->k_bits < 1 || c->k_bits < c->b_min || c->k_bits > c->b_max) return false;
  if (c->codec == KVQ_CODEC_KIVI && (c->k_bits > 4 || c->v_bits > 4)) return false;
  if (c->codec == KVQ_CODEC_NF16_B256) {
    if (c->k_bits != 4 || c->v_bits != 4) return false;
    if ((c->n_kv_heads * kHeadDim) % kvq::kNfBlock != 0) return false;
  }
  return true;
}

bool layer_ok(const kvq_cache* c, int32_t layer) {
  return c && layer >= 0 && layer < c->cfg.n_layers;
}

void free_device(kvq_cache* c) {
  void* ptrs[] = {c->k_codes, c->v_codes, c->k_scales, c->v_scales, c->plans,
                  c->tables,  c->part_o,  c->part_l,  c->part_mt, c->energy_scratch, c->split_epochs,
                  c->fid_part, c->k_recent, c->v_recent, c->rot_signs, c->dev_status};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
}

kvq_status dev_alloc(void** p, size_t bytes, const char* what) {
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    g_last_error = std::string("hipMalloc ") + what + ": " + hipGetErrorString(e);
    *p = nullptr;
    return e == hipErrorOutOfMemory ? KVQ_ENOMEM : KVQ_EHIP;
  }
  return KVQ_OK;
}

}  // namespace

namespace kvq {
void set_last_error(const std::string& what) { g_last_error = what; }
}  // namespace kvq

extern "C" {

const char* kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_EINVAL: return "KVQ_EINVAL";
    case KVQ_ENOMEM: return "KVQ_ENOMEM";
    case KVQ_ECAPACITY: return "KVQ_ECAPACITY";
    case KVQ_ESTATE: return "KVQ_ESTATE";
    case KVQ_EHIP: return "KVQ_EHIP";
  }
  return "KVQ_UNKNOWN";
}

const char* kvq_last_error(void) { return g_last_error.c_str(); }

kvq_status kvq_codebook(int32_t bits, uint16_t* centroids, float* boundaries) {
  if (bits < 1 || bits > kMaxBits) return KVQ_EINVAL;
  kvq::Tables t;
  kvq::build_tables(&t);
  const int L = 1 << bits;
  if (centroids) std::memcpy(centroids, t.cb[bits], sizeof(uint16_t) * L);
  if (boundaries) std::memcpy(boundaries, t.bd[bits], sizeof(float) * (L - 1));
  return KVQ_OK;
}

kvq_status kvq_delta(float* delta) {
  if (!delta) return KVQ_EINVAL;
  kvq::Tables t;
  kvq::build_tables(&t);
  std::memcpy(delta, t.delta, sizeof(t.delta));
  return KVQ_OK;
}

kvq_status kvq_nf16_codebook(uint16_t* levels, float* boundaries) {
  kvq::Tables t;
  kvq::build_tables(&t);
  if (levels) std::memcpy(levels, t.nf_cb, sizeof(t.nf_cb));
  if (boundaries) std::memcpy(boundaries, t.nf_bd, sizeof(float) * 15);
  return KVQ_OK;
}

kvq_status kvq_cache_create(const kvq_config* cfg, kvq_cache** out) {
  if (!out || !config_valid(cfg)) return KVQ_EINVAL;
  kvq_cache* c = new (std::nothrow) kvq_cache();
  if (!c) return KVQ_ENOMEM;
  std::memset(static_cast<void*>(c), 0, sizeof(kvq_cache));
  c->cfg = *cfg;
  c->group = cfg->n_q_heads / cfg->n_kv_heads;
  c->n_plan = cfg->per_sequence_plans ? cfg->batch : 1;
  // KIVI packs whole 128-position key tiles: its fp16 ring also holds the last partial tile
  const bool kivi = cfg->codec == KVQ_CODEC_KIVI;
  c->ring = cfg->recent_window + (kivi ? kVTile : 0);
  c->pack_group = kivi ? kVTile : 1;
  c->cap = (cfg->max_tokens + kVTile - 1) / kVTile * kVTile;
  const bool nf = cfg->codec == KVQ_CODEC_NF16_B256;
  c->k_words = 4 * (nf ? 4 : cfg->k_bits);
  c->v_words = 4 * (nf ? 4 : cfg->v_bits);
  c->n_nf_blocks = cfg->n_kv_heads * kHeadDim / kvq::kNfBlock;
  c->len = static_cast<int64_t*>(std::calloc(cfg->n_layers, sizeof(int64_t)));
  c->plan_ready = static_cast<uint8_t*>(std::calloc(cfg->n_layers, 1));
  c->rot_ready = static_cast<uint8_t*>(std::calloc(cfg->n_layers, 1));
  if (!c->len || !c->plan_ready || !c->rot_ready) {
    std::free(c->len);
    std::free(c->plan_ready);
    std::free(c->rot_ready);
    delete c;
    return KVQ_ENOMEM;
  }
  kvq::build_tables(&c->host_tables);

  const int64_t B = cfg->batch, H = cfg->n_kv_heads, L = cfg->n_layers, cap = c->cap;
  c->k_codes_layer = B * H * cap * c->k_words * 4;
  c->v_codes_layer = B * H * cap * c->v_words * 4;  // (cap/128) tiles * 128 dims * v_words words
  // KIVI: 2 fp16 per channel per 128-position tile (K), 2 fp16 per position (V)
  c->k_scales_layer = nf ? B * cap * c->n_nf_blocks * 2 : B * H * cap * (kivi ? 4 : 2);
  c->v_scales_layer = c->k_scales_layer;
  c->recent_layer = B * c->ring * H * kHeadDim * 2;
  // split partials: at most 256 splits per (sequence, head), at most 256 MiB of partials
  int64_t per_split = B * H * c->group * (kHeadDim + 2) * 4;
  int64_t ms = (int64_t(256) << 20) / per_split;
  if (ms > 256) ms = 256;
  if (ms < 1) ms = 1;
  c->max_splits = static_cast<int>(ms);

  hipError_t e = hipGetDevice(&c->device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&c->n_cu, hipDeviceAttributeMultiprocessorCount, c->device);
  kvq_status st = e == hipSuccess ? KVQ_OK : hip_fail(e, "hipGetDevice");
  if (st == KVQ_OK) st = dev_alloc(reinterpret_cast<void**>(&c->k_codes), c->k_codes_layer * L, "K codes");
  if (st == KVQ_OK) st = dev_alloc(reinterpret_cast<void**>(&c->v_codes), c->v_codes_layer * L, "V codes");
  if (st == KVQ_OK) st = dev_alloc(reinterpret_cast<void**>(&c->k_scales), c->k_scales_layer * L, "K scales");
  if (st == KVQ_OK) st = dev_alloc(reinterpret_cast<void**>(&c->v_scales), c->v_scales_layer * L, "V scales");
  if (st == KVQ_OK && c->recent_layer > 0) {
    st = dev_alloc(reinterpret_cast<void**>(&c->k_recent), c->recent_layer * L, "recent K");
    if (st == KVQ_OK) st = dev_alloc(reinterpret_cast<void**>(&c->v_recent), c->recent_layer * L, "recent V");
  }
  if (st == KVQ_OK) st = dev_alloc(reinterpret_cast<void**>(&c->plans), sizeof(kvq::Plan) * L * c->n_plan * H, "plans");
  if (st == KVQ_OK && kvq::codec_rotates(cfg->codec))
    st = dev_alloc(reinterpret_cast<void**>(&c->rot_signs), L * H * kHeadDim, "rotation signs");
  if (st == KVQ_OK) st = dev_alloc(reinterpret_cast<void**>(&c->tables), sizeof(kvq::Tables), "tables");
  if (st == KVQ_OK)
    st = dev_alloc(reinterpret_cast<void**>(&c->part_o), per_split / (kHeadDim + 2) * kHeadDim * ms, "partials");
  if (st == KVQ_OK)
    st = dev_alloc(reinterpret_cast<void**>(&c->part_l), per_split / (kHeadDim + 2) * ms, "partials");
  if (st == KVQ_OK)
    st = dev_alloc(reinterpret_cast<void**>(&c->part_mt), per_split / (kHeadDim + 2) * 2 * ms, "partials");
  if (st == KVQ_OK)
    st = dev_alloc(reinterpret_cast<void**>(&c->split_epochs), sizeof(unsigned) * B * H, "split tags");
  if (st == KVQ_OK) st = dev_alloc(reinterpret_cast<void**>(&c->dev_status), sizeof(unsigned), "status word");
  // bound on a split merger's wait (a test hook: a small bound makes the wait give up at once)
  c->merge_polls = kvq::kMaxMergePolls;
  if (const char* ev = std::getenv("KVQ_MERGE_POLL_LIMIT")) {
    const long v = std::strtol(ev, nullptr, 10);
    if (v >= 0 && v <= kvq::kMaxMergePolls) c->merge_polls = static_cast<int>(v);
  }
  // fidelity diagnostics: about four workgroups per compute unit over the (sequence, KV head)
  // units, six fp64 statistics per query head and split
  c->fid_max_splits = static_cast<int>((4LL * c->n_cu + B * H - 1) / (B * H));
  if (st == KVQ_OK)
    st = dev_alloc(reinterpret_cast<void**>(&c->fid_part),
                   sizeof(double) * 6 * B * H * c->group * c->fid_max_splits, "fidelity statistics");
  if (st == KVQ_OK) {
    const hipError_t es[] = {
        hipMemset(c->split_epochs, 0, sizeof(unsigned) * B * H),
        hipMemset(c->dev_status, 0, sizeof(unsigned)),
        hipMemset(c->part_mt, 0, per_split / (kHeadDim + 2) * 2 * ms),
        hipMemset(c->k_codes, 0, c->k_codes_layer * L),
        hipMemset(c->v_codes, 0, c->v_codes_layer * L),
        hipMemset(c->k_scales, 0, c->k_scales_layer * L),
        hipMemset(c->v_scales, 0, c->v_scales_layer * L),
        c->k_recent ? hipMemset(c->k_recent, 0, c->recent_layer * L) : hipSuccess,
        c->v_recent ? hipMemset(c->v_recent, 0, c->recent_layer * L) : hipSuccess,
        hipMemset(c->plans, 0, sizeof(kvq::Plan) * L * c->n_plan * H),
        hipMemcpy(c->tables, &c->host_tables, sizeof(kvq::Tables), hipMemcpyHostToDevice),
        hipDeviceSynchronize()};
    for (hipError_t x : es)
      if (x != hipSuccess && st == KVQ_OK) st = hip_fail(x, "cache init");
  }
  if (st != KVQ_OK) {
    free_device(c);
    std::free(c->len);
    std::free(c->plan_ready);
    std::free(c->rot_ready);
    delete c;
    return st;
  }
  *out = c;
  return KVQ_OK;
}

void kvq_cache_destroy(kvq_cache* c) {
  if (!c) return;
  (void)hipDeviceSynchronize();
  free_device(c);
  std::free(c->len);
  std::free(c->plan_ready);
  std::free(c->rot_ready);
  delete c;
}

kvq_status kvq_alloc_bits(kvq_cache* c, int32_t layer, const void* keys, int32_t dtype,
                          int64_t n_tok, const double* block_weight, kvq_stream stream) {
  if (!layer_ok(c, layer)) return KVQ_EINVAL;
  if (dtype != KVQ_F16 && dtype != KVQ_F32) return KVQ_EINVAL;
  const bool bgtq = kvq::codec_allocates(c->cfg.codec);
  if (bgtq && (!keys || n_tok < 1)) return KVQ_EINVAL;
  if (bgtq && reinterpret_cast<uintptr_t>(keys) % 16) {
    g_last_error = "alloc_bits: keys must be 16-byte aligned";
    return KVQ_EINVAL;
  }
  if (bgtq && n_tok * c->n_plan > (int64_t(1) << 31)) return KVQ_EINVAL;
  if (c->len[layer] > 0) return KVQ_ESTATE;
  if (bgtq) {
    const int64_t n_chunks = (n_tok + kvq::kEnergyChunk - 1) / kvq::kEnergyChunk;
    if (n_chunks > c->energy_scratch_chunks) {
      // the scratch grows to the largest calibration seen; earlier work on any stream may
      // still read the old buffer, so wait for the device before freeing it
      if (c->energy_scratch) {
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
        (void)hipFree(c->energy_scratch);
        c->energy_scratch = nullptr;
        c->energy_scratch_chunks = 0;
      }
      kvq_status st = dev_alloc(reinterpret_cast<void**>(&c->energy_scratch),
                                sizeof(double) * n_chunks * c->n_plan * c->cfg.n_kv_heads * kBlocks, "energy scratch");
      if (st != KVQ_OK) return st;
      c->energy_scratch_chunks = n_chunks;
    }
  }
  hipError_t e = kvq::launch_alloc(c, layer, keys, dtype, bgtq ? n_tok : 0, block_weight,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "alloc launch");
  c->plan_ready[layer] = 1;
  return KVQ_OK;
}

kvq_status kvq_get_plan(const kvq_cache* c, int32_t layer, int8_t* bits, float* gains) {
  if (!layer_ok(c, layer) || !bits) return KVQ_EINVAL;
  if (!c->plan_ready[layer]) return KVQ_ESTATE;
  const int H = c->n_plan * c->cfg.n_kv_heads;   // (sequence,) head units of the layer
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  for (int h = 0; h < H; ++h) {
    kvq::Plan p;
    e = hipMemcpy(&p, c->plans + static_cast<int64_t>(layer) * H + h, sizeof(p), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "plan copy");
    std::memcpy(bits + h * kBlocks, p.bwidth, kBlocks);
    if (gains) {
      for (int j = 0; j < kBlocks; ++j) {
        const int d0 = c->cfg.pairing == KVQ_ROPE_HALF ? j : 2 * j;
        gains[h * kBlocks + j] = p.g[d0];
      }
    }
  }
  return KVQ_OK;
}

kvq_status kvq_quantize_append(kvq_cache* c, int32_t layer, const void* k, const void* v,
                               int32_t dtype, int64_t n_new, kvq_stream stream) {
  if (!layer_ok(c, layer)) return KVQ_EINVAL;
  if (dtype != KVQ_F16 && dtype != KVQ_F32) return KVQ_EINVAL;
  if (n_new < 0) return KVQ_EINVAL;
  if (n_new == 0) return KVQ_OK;
  if (!k || !v) return KVQ_EINVAL;
  if (reinterpret_cast<uintptr_t>(k) % 16 || reinterpret_cast<uintptr_t>(v) % 16) {
    g_last_error = "quantize_append: k and v must be 16-byte aligned";
    return KVQ_EINVAL;
  }
  if (!c->plan_ready[layer]) return KVQ_ESTATE;
  if (kvq::codec_rotates(c->cfg.codec) && !c->rot_ready[layer]) return KVQ_ESTATE;
  if (c->len[layer] + n_new > c->cfg.max_tokens) return KVQ_ECAPACITY;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t len = c->len[layer], R = c->cfg.recent_window;
  hipError_t e = hipSuccess;
  if (c->cfg.codec == KVQ_CODEC_KIVI) {
    // whole key tiles [p_old, p_new) are quantized, each position from its fp16 copy in the
    // ring (positions before len) or from the input; new positions after p_new go to the ring
    // (after the quantization: they may reuse the slots it reads)
    const int64_t p_old = kvq::packed_len_at(c, len), p_new = kvq::packed_len_at(c, len + n_new);
    if (p_new > p_old) e = kvq::launch_kivi_quantize(c, layer, k, v, dtype, n_new, p_old, p_new - p_old, len, s);
    const int64_t w0 = p_new > len ? p_new : len;
    if (e == hipSuccess && w0 < len + n_new)
      e = kvq::launch_recent_write(c, layer, k, v, dtype, n_new, w0 - len, w0, len + n_new - w0, s);
  } else if (R == 0) {
    e = kvq::launch_quantize(c, layer, k, v, dtype, n_new, n_new, 0, len, s);
  } else {
    // positions [p_old, p_new) leave the window for the packed storage: first those already
    // buffered (from their fp16 copies in the rings), then new ones that arrive already
    // outside the window; the remaining new positions are copied into the rings (after the
    // evictions: they reuse the evicted slots)
    const int64_t p_old = len > R ? len - R : 0, p_new = len + n_new > R ? len + n_new - R : 0;
    const int64_t e_end = p_new < len ? p_new : len;
    if (e_end > p_old)
      e = kvq::launch_quantize(c, layer, kvq::layer_k_recent(c, layer), kvq::layer_v_recent(c, layer), KVQ_F16,
                               e_end - p_old, 0, static_cast<int>(R), p_old, s);
    if (e == hipSuccess && p_new > len) e = kvq::launch_quantize(c, layer, k, v, dtype, p_new - len, n_new, 0, len, s);
    const int64_t w0 = p_new > len ? p_new : len;
    if (e == hipSuccess && w0 < len + n_new)
      e = kvq::launch_recent_write(c, layer, k, v, dtype, n_new, w0 - len, w0, len + n_new - w0, s);
  }
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  c->len[layer] += n_new;
  return KVQ_OK;
}

kvq_status kvq_decode_attn_splits(kvq_cache* c, int32_t layer, const void* q, int32_t dtype,
                                  float softmax_scale, float* out, int32_t n_splits,
                                  kvq_stream stream) {
  if (!layer_ok(c, layer) || !q || !out) return KVQ_EINVAL;
  if (dtype != KVQ_F16 && dtype != KVQ_F32) return KVQ_EINVAL;
  if (reinterpret_cast<uintptr_t>(q) % 4 || reinterpret_cast<uintptr_t>(out) % 16) {
    g_last_error = "decode: q must be 4-byte and out 16-byte aligned";
    return KVQ_EINVAL;
  }
  if (!(softmax_scale == softmax_scale)) return KVQ_EINVAL;  // NaN
  if (!c->plan_ready[layer] || c->len[layer] == 0) return KVQ_ESTATE;
  // S splits of the packed positions, plus one workgroup for the recent window if any
  const int64_t plen = kvq::packed_len(c, layer);
  const int64_t nb = c->len[layer] - plen;
  const int n_rwg = static_cast<int>((nb + 127) / 128);   // recent-window workgroups (one ring tile each)
  const int S = plen == 0 ? 0 : n_splits > 0 ? n_splits : kvq::auto_splits_mfma(c, plen, n_rwg);
  const int S_all = S + n_rwg;
  if (S_all > c->max_splits) return KVQ_EINVAL;
  // (with as many (sequence, KV head) units as compute units the splits are merged by a
  // second kernel instead of in the decode kernel)
  const kvq::DecodeScratch ws{c->part_o, c->part_l, c->part_mt, c->split_epochs, c->dev_status, c->merge_polls};
  hipError_t e = kvq::launch_decode_mfma(c, layer, q, dtype, softmax_scale, out, S, ws,
                                         kvq::DecodeAppend{nullptr, nullptr, -1}, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return KVQ_OK;
}

kvq_status kvq_decode_step(kvq_cache* c, int32_t layer, const void* k_new, const void* v_new, const void* q,
                           int32_t dtype, float softmax_scale, float* out, kvq_stream stream) {
  if (!layer_ok(c, layer) || !k_new || !v_new || !q || !out) return KVQ_EINVAL;
  if (dtype != KVQ_F16 && dtype != KVQ_F32) return KVQ_EINVAL;
  // every check of both calls comes first, so that a rejected call appends nothing
  if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16) {
    g_last_error = "decode_step: k_new and v_new must be 16-byte aligned";
    return KVQ_EINVAL;
  }
  if (reinterpret_cast<uintptr_t>(q) % 4 || reinterpret_cast<uintptr_t>(out) % 16) {
    g_last_error = "decode_step: q must be 4-byte and out 16-byte aligned";
    return KVQ_EINVAL;
  }
  if (!(softmax_scale == softmax_scale)) return KVQ_EINVAL;  // NaN
  if (!c->plan_ready[layer]) return KVQ_ESTATE;
  const kvq_config& cfg = c->cfg;
  if (kvq::codec_rotates(cfg.codec) && !c->rot_ready[layer]) return KVQ_ESTATE;
  if (c->len[layer] + 1 > cfg.max_tokens) return KVQ_ECAPACITY;
  if (!((cfg.codec == KVQ_CODEC_BGTQ || cfg.codec == KVQ_CODEC_UNIFORM) && cfg.recent_window == 0)) {
    // the other codecs and the recent window: the append, then the attention
    const kvq_status st = kvq_quantize_append(c, layer, k_new, v_new, dtype, 1, stream);
    if (st != KVQ_OK) return st;
    return kvq_decode_attn(c, layer, q, dtype, softmax_scale, out, stream);
  }
  const int64_t pos = c->len[layer];
  c->len[layer] = pos + 1;
  const int S = kvq::auto_splits_mfma(c, kvq::packed_len(c, layer), 0);
  if (S > c->max_splits) {
    c->len[layer] = pos;
    return KVQ_EINVAL;
  }
  const kvq::DecodeScratch ws{c->part_o, c->part_l, c->part_mt, c->split_epochs, c->dev_status, c->merge_polls};
  const hipError_t e = kvq::launch_decode_mfma(c, layer, q, dtype, softmax_scale, out, S, ws,
                                               kvq::DecodeAppend{k_new, v_new, pos}, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    c->len[layer] = pos;
    return hip_fail(e, "decode step launch");
  }
  return KVQ_OK;
}

kvq_status kvq_decode_attn(kvq_cache* c, int32_t layer, const void* q, int32_t dtype,
                           float softmax_scale, float* out, kvq_stream stream) {
  return kvq_decode_attn_splits(c, layer, q, dtype, softmax_scale, out, 0, stream);
}

kvq_status kvq_key_fidelity(kvq_cache* c, int32_t layer, const void* q, const void* keys,
                            int32_t dtype, float softmax_scale, double* mae, double* kl,
                            kvq_stream stream) {
  if (!layer_ok(c, layer) || !q || !keys || !mae || !kl) return KVQ_EINVAL;
  if (dtype != KVQ_F16 && dtype != KVQ_F32) return KVQ_EINVAL;
  const size_t el = dtype == KVQ_F16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(q) % el || reinterpret_cast<uintptr_t>(keys) % 16 ||
      reinterpret_cast<uintptr_t>(mae) % 8 || reinterpret_cast<uintptr_t>(kl) % 8) {
    g_last_error = "fidelity: keys must be 16-byte, mae and kl 8-byte aligned";
    return KVQ_EINVAL;
  }
  if (!(softmax_scale == softmax_scale)) return KVQ_EINVAL;  // NaN
  if (!c->plan_ready[layer] || c->len[layer] == 0) return KVQ_ESTATE;
  hipError_t e = kvq::launch_fidelity(c, layer, q, keys, dtype, softmax_scale, mae, kl,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fidelity launch");
  return KVQ_OK;
}

kvq_status kvq_set_rotation(kvq_cache* c, int32_t layer, const int8_t* signs) {
  if (!layer_ok(c, layer) || !signs || !kvq::codec_rotates(c->cfg.codec)) return KVQ_EINVAL;
  const int64_t n = static_cast<int64_t>(c->cfg.n_kv_heads) * kHeadDim;
  for (int64_t i = 0; i < n; ++i)
    if (signs[i] != 1 && signs[i] != -1) return KVQ_EINVAL;
  if (c->len[layer] > 0) return KVQ_ESTATE;
  hipError_t e = hipMemcpy(c->rot_signs + layer * n, signs, n, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "set rotation");
  c->rot_ready[layer] = 1;
  return KVQ_OK;
}

kvq_status kvq_cache_status(kvq_cache* c) {
  if (!c) return KVQ_EINVAL;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  unsigned word = 0;
  e = hipMemcpy(&word, c->dev_status, sizeof(word), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "status read");
  if (word == 0) return KVQ_OK;
  // nothing is in flight: clear the word, the split maxima words and the tag bases, so the
  // next decode starts from a clean state
  const int64_t units = static_cast<int64_t>(c->cfg.batch) * c->cfg.n_kv_heads;
  const hipError_t es[] = {hipMemset(c->dev_status, 0, sizeof(unsigned)),
                           hipMemset(c->part_mt, 0, sizeof(uint64_t) * units * c->group * c->max_splits),
                           hipMemset(c->split_epochs, 0, sizeof(unsigned) * units), hipDeviceSynchronize()};
  for (hipError_t x : es)
    if (x != hipSuccess) return hip_fail(x, "status reset");
  g_last_error = "decode: a split merge gave up waiting for the partials of other splits; the outputs it "
                 "covered (and those of later merged decodes until this call) were written as NaN";
  return KVQ_EHIP;
}

static_assert(sizeof(kvq::Plan) == KVQ_PLAN_BYTES, "plan record size");
static_assert(offsetof(kvq::Plan, g) == KVQ_PLAN_OFF_GAIN, "plan gains");
static_assert(offsetof(kvq::Plan, fdim) == KVQ_PLAN_OFF_FIELD_DIM, "plan field dims");
static_assert(offsetof(kvq::Plan, fwidth) == KVQ_PLAN_OFF_FIELD_WIDTH, "plan field widths");
static_assert(offsetof(kvq::Plan, bwidth) == KVQ_PLAN_OFF_BLOCK_WIDTH, "plan block widths");
static_assert(offsetof(kvq::Plan, n_fields) == KVQ_PLAN_OFF_N_FIELDS, "plan field count");

kvq_status kvq_cache_view(const kvq_cache* c, int32_t layer, kvq_view* v) {
  if (!layer_ok(c, layer) || !v) return KVQ_EINVAL;
  kvq_cache* m = const_cast<kvq_cache*>(c);
  const int64_t H = c->cfg.n_kv_heads, cap = c->cap;
  std::memset(v, 0, sizeof(*v));
  v->k_codes = kvq::layer_k_codes(m, layer);
  v->k_codes_strides[0] = H * cap * c->k_words;
  v->k_codes_strides[1] = cap * c->k_words;
  v->k_codes_strides[2] = c->k_words;
  v->v_codes = kvq::layer_v_codes(m, layer);
  v->v_codes_strides[0] = H * cap * c->v_words;
  v->v_codes_strides[1] = cap * c->v_words;
  v->v_codes_strides[2] = kVTile * c->v_words;
  v->k_scales = kvq::layer_k_scales(m, layer);
  v->v_scales = kvq::layer_v_scales(m, layer);
  if (c->cfg.codec == KVQ_CODEC_NF16_B256) {
    v->scale_strides[0] = cap * c->n_nf_blocks;
    v->scale_strides[1] = c->n_nf_blocks;
    v->scale_strides[2] = 1;
  } else if (c->cfg.codec == KVQ_CODEC_KIVI) {
    v->scale_strides[0] = H * (cap / kVTile) * 256;
    v->scale_strides[1] = (cap / kVTile) * 256;
    v->scale_strides[2] = 256;
  } else {
    v->scale_strides[0] = H * cap;
    v->scale_strides[1] = cap;
    v->scale_strides[2] = 1;
  }
  if (c->recent_layer > 0) {
    v->k_recent = reinterpret_cast<const uint16_t*>(kvq::layer_k_recent(m, layer));
    v->v_recent = reinterpret_cast<const uint16_t*>(kvq::layer_v_recent(m, layer));
  }
  v->plans = c->plans + static_cast<int64_t>(layer) * c->n_plan * H;
  v->n_plans = static_cast<int32_t>(c->n_plan * H);
  v->plan_bytes = static_cast<int32_t>(sizeof(kvq::Plan));
  v->capacity = cap;
  v->len = c->len[layer];
  v->packed_len = kvq::packed_len(c, layer);
  return KVQ_OK;
}

kvq_status kvq_seq_len(const kvq_cache* c, int32_t layer, int64_t* len) {
  if (!layer_ok(c, layer) || !len) return KVQ_EINVAL;
  *len = c->len[layer];
  return KVQ_OK;
}

kvq_status kvq_layer_info_get(const kvq_cache* c, int32_t layer, kvq_layer_info* info) {
  if (!layer_ok(c, layer) || !info) return KVQ_EINVAL;
  info->capacity = c->cap;
  info->len = c->len[layer];
  info->k_row_words = c->k_words;
  info->v_dim_words = c->v_words;
  info->k_codes_bytes = c->k_codes_layer;
  info->v_codes_bytes = c->v_codes_layer;
  info->k_scales_bytes = c->k_scales_layer;
  info->v_scales_bytes = c->v_scales_layer;
  info->plan_ready = c->plan_ready[layer];
  info->recent_window = c->cfg.recent_window;
  info->packed_len = kvq::packed_len(c, layer);
  info->recent_bytes = c->recent_layer;
  info->ring_slots = c->ring;
  return KVQ_OK;
}

kvq_status kvq_read_cache(const kvq_cache* c, int32_t layer, int32_t part, int64_t offset,
                          int64_t nbytes, void* dst) {
  if (!layer_ok(c, layer) || !dst || offset < 0 || nbytes < 0) return KVQ_EINVAL;
  const char* base = nullptr;
  int64_t size = 0;
  kvq_cache* m = const_cast<kvq_cache*>(c);
  switch (part) {
    case KVQ_PART_K_CODES: base = reinterpret_cast<const char*>(kvq::layer_k_codes(m, layer)); size = c->k_codes_layer; break;
    case KVQ_PART_V_CODES: base = reinterpret_cast<const char*>(kvq::layer_v_codes(m, layer)); size = c->v_codes_layer; break;
    case KVQ_PART_K_SCALES: base = reinterpret_cast<const char*>(kvq::layer_k_scales(m, layer)); size = c->k_scales_layer; break;
    case KVQ_PART_V_SCALES: base = reinterpret_cast<const char*>(kvq::layer_v_scales(m, layer)); size = c->v_scales_layer; break;
    case KVQ_PART_K_RECENT: base = reinterpret_cast<const char*>(kvq::layer_k_recent(m, layer)); size = c->recent_layer; break;
    case KVQ_PART_V_RECENT: base = reinterpret_cast<const char*>(kvq::layer_v_recent(m, layer)); size = c->recent_layer; break;
    default: return KVQ_EINVAL;
  }
  if (offset + nbytes > size) return KVQ_EINVAL;
  if (nbytes == 0) return KVQ_OK;
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(dst, base + offset, nbytes, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "read cache");
  return KVQ_OK;
}

}  // extern "C"
