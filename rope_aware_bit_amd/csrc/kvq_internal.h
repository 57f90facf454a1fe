// Internal definitions shared by the libkvq host code and its gfx950 kernels.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kBlocks = 64;          // 2-D RoPE blocks per head
constexpr int kMaxBits = 8;
constexpr int kVTile = 128;          // tokens per dim-major V tile
constexpr int kEnergyChunk = 256;    // tokens per sequential energy partial sum
constexpr int kMaxGroup = 8;         // query heads per KV head supported
constexpr int kNfBlock = 256;        // values per absmax block of the NF16 codec
constexpr int kMaxRecent = 4096;     // largest recent window (tokens)
constexpr int kMaxMergePolls = 1 << 22;   // default bound on a split merger's wait for partials

// Byte layout of the decode lookup tables that every decode workgroup copies into LDS.
// Pair tables (widths 1..4) hold fp16x2 (CB[c0], CB[c1]) at index c0 | c1 << w; single
// tables (widths 1..8) hold fp16 CB[c] at 2560 - 2^(w+2); width 0 addresses zero bytes at
// the end.  Each base is a multiple of its table's size, so "(field << 2) | base" (pairs)
// and "(field << 1) | base" (singles) address an entry.
__host__ __device__ constexpr int pair_table_base(int w) {
  return w == 4 ? 0 : w == 3 ? 1024 : w == 2 ? 1280 : 1344;
}
constexpr int kLdsTableBytes = 2560;
__host__ __device__ constexpr int single_table_base(int w) { return kLdsTableBytes - (4 << w); }

// Constant tables, built on the host at cache creation and copied to the device.
struct Tables {
  uint16_t cb[kMaxBits + 1][256];    // fp16 bit patterns of CB_b[k], b = 1..8 (row 0 unused)
  float bd[kMaxBits + 1][256];       // fp32 boundaries beta_b[k], k < 2^b - 1; +inf after them (row 0: all +inf)
  float delta[kMaxBits];             // greedy gain delta(b) = c(b) - c(b+1), fp32
  uint16_t nf_cb[16];                // fp16 levels of the 16-level Gaussian-quantile codebook
  float nf_bd[16];                   // 15 boundaries; [15] = +inf
  // decode lookup tables in their LDS layout: [0] Lloyd-Max codebooks, [1] the same with
  // the width-4 tables holding the 16-level Gaussian-quantile codebook, [2] the integers
  // 0 .. 2^b - 1 as fp16 (codes of the asymmetric integer codec)
  alignas(16) uint8_t lds_image[3][kLdsTableBytes];
};

// Per-(layer, KV head) plan written by the allocation kernel.
struct alignas(16) Plan {
  float g[kHeadDim];                 // per-dim gain (its block's g_j)
  float ig[kHeadDim];                // per-dim inverse gain
  uint16_t foff[kHeadDim];           // bit offset of field f within the K row
  uint8_t fdim[kHeadDim];            // dim of field f, plan order
  uint8_t fwidth[kHeadDim];          // width of field f
  uint8_t dwidth[kHeadDim];          // width of dim i
  int8_t bwidth[kBlocks];            // width of block j
  uint32_t pdesc[kBlocks];           // stored block (pair) r in plan order: bit offset | width << 16
  uint8_t cstart[kHeadDim];          // field f's rotation chunk (power-of-two piece of its
  uint8_t csize[kHeadDim];           //   equal-width run): first field and size; 0 past n_fields
  int32_t n_fields;                  // stored fields (2 x blocks with width > 0)
  int32_t pad[3];
};

// Codecs whose K widths come from the allocation, and codecs that rotate keys.
__host__ __device__ inline bool codec_allocates(int codec) { return codec == KVQ_CODEC_BGTQ || codec == KVQ_CODEC_BGTQ_ROT; }
__host__ __device__ inline bool codec_rotates(int codec) { return codec == KVQ_CODEC_UNIFORM_ROT || codec == KVQ_CODEC_BGTQ_ROT; }

// Host-side tables builder (independent implementation of the codebook definitions).
void build_tables(Tables* t);

}  // namespace kvq

struct kvq_cache {
  kvq_config cfg;
  int device;
  int n_cu;                    // compute units of the device
  int64_t cap;                 // token capacity per sequence, multiple of kVTile
  int group;                   // n_q / n_kv
  int k_words;                 // 32-bit words per K row
  int v_words;                 // 32-bit words per dim per V tile
  int n_nf_blocks;             // NF16 scale blocks per token (n_kv*128/256)
  int64_t* len;                // per layer
  uint8_t* plan_ready;         // per layer
  // device memory
  uint32_t* k_codes;           // [L][B][H][cap][k_words]
  uint32_t* v_codes;           // [L][B][H][cap/128][128][v_words]
  uint16_t* k_scales;          // BGTQ/UNI [L][B][H][cap]; NF16 [L][B][cap][nnf]
  uint16_t* v_scales;
  __half* k_recent;            // recent-window rings [L][B][ring][H][128] fp16 (ring > 0)
  __half* v_recent;
  int ring;                    // ring slots: R, or R + 128 for KIVI (its last partial key tile)
  int pack_group;              // positions are packed in whole groups of this many (KIVI: 128)
  kvq::Plan* plans;            // [L][n_plan][H]
  int n_plan;                  // plans per (layer, KV head): batch with per-sequence plans, else 1
  int8_t* rot_signs;           // key-rotation signs [L][H][128] (codecs UNIFORM_ROT, BGTQ_ROT)
  uint8_t* rot_ready;          // per layer: signs set
  kvq::Tables* tables;         // device copy
  kvq::Tables host_tables;
  float* part_o;               // split partials [B][H][max_splits][G][128]
  float* part_l;               // split softmax sums [B][H][max_splits][G]
  uint64_t* part_mt;           // split maxima | publication tag << 32 [B][H][max_splits][G]
  unsigned* split_epochs;      // [B][H] tag base of the next call's split partials
  unsigned* dev_status;        // sticky device error word (bit 0: a split merge gave up waiting)
  int merge_polls;             // bound on a merger's polls (KVQ_MERGE_POLL_LIMIT, else kMaxMergePolls)
  int max_splits;
  double* energy_scratch;      // [H][n_chunks][64]
  double* fid_part;            // fidelity split statistics [B][n_q][fid_max_splits][6]
  int fid_max_splits;
  int64_t energy_scratch_chunks;
  // byte sizes per layer
  int64_t k_codes_layer, v_codes_layer, k_scales_layer, v_scales_layer, recent_layer;
};

namespace kvq {

// Records the text kvq_last_error() returns to this thread.
void set_last_error(const std::string& what);

// Kernel launchers (defined in the .hip sources).  All enqueue on `stream` and
// return the launch status; arguments are validated by the caller.
hipError_t launch_alloc(kvq_cache* c, int layer, const void* keys, int dtype, int64_t n_tok,
                        const double* block_weight, hipStream_t stream);
// Quantizes positions L0 .. L0 + n_new - 1 of every sequence into the packed storage, from
// rows 0 .. n_new - 1 of [batch][in_stride][n_kv][128] K and V inputs, or (ring_R > 0) from
// the recent-window rings of R = ring_R slots (fp16).
hipError_t launch_quantize(kvq_cache* c, int layer, const void* k, const void* v, int dtype,
                           int64_t n_new, int64_t in_stride, int ring_R, int64_t L0, hipStream_t stream);
// KIVI: quantizes the n_pos positions from p0 (whole 128-position tiles) of every sequence;
// position p < len_old comes from its fp16 copy in the ring, others from input row p - len_old
// of [batch][in_stride][n_kv][128] K and V.
hipError_t launch_kivi_quantize(kvq_cache* c, int layer, const void* k, const void* v, int dtype,
                                int64_t in_stride, int64_t p0, int64_t n_pos, int64_t len_old,
                                hipStream_t stream);
hipError_t launch_recent_write(kvq_cache* c, int layer, const void* k, const void* v, int dtype,
                               int64_t in_stride, int64_t row0, int64_t pos0, int64_t count,
                               hipStream_t stream);
// Split partials and merge bookkeeping of one decode call: outputs [units][S][G][128], sums
// [units][S][G], maxima | tag << 32 [units][S][G], one tag base per unit, the sticky error word
// and the bound on a merger's polls.  The cache's own buffers, or a caller's.
struct DecodeScratch {
  float* o;
  float* l;
  uint64_t* mt;
  unsigned* epochs;
  unsigned* status;
  int max_polls;
};
// A decode step's new position, appended by the decode launch itself: rows k and v
// [batch][n_kv][128] in the query's precision, quantized into position pos (pos < 0: none).
// Only for codecs without rotation, not the 256-value or asymmetric integer codecs, and no
// recent window.
struct DecodeAppend {
  const void* k;
  const void* v;
  int64_t pos;
};
hipError_t launch_decode_mfma(kvq_cache* c, int layer, const void* q, int dtype, float scale,
                              float* out, int n_splits, const DecodeScratch& ws, const DecodeAppend& app,
                              hipStream_t stream);
hipError_t launch_fidelity(kvq_cache* c, int layer, const void* q, const void* keys, int dtype,
                           float scale, double* mae, double* kl, hipStream_t stream);
int auto_splits_mfma(const kvq_cache* c, int64_t len, int n_extra);

// Launch shape of the decode kernel for a cache: waves per workgroup (8 = two per SIMD, or 4),
// whether each wave's V tile has an LDS area of its own (copied at tile start; a static array
// with 8 waves) or reuses the K area after the key product, the dynamic LDS words of each
// wave's region and the V area's offset in it.
struct DecodeShape {
  int waves, v_early, region_words, v_off;
  // 8 waves: the region and V offset when each V tile is copied into the wave's region after the
  // key product (0 when that does not fit).  Launches of at most one tile per wave use it; the
  // static V areas (v_early) serve launches of several tiles per wave, whose copies then overlap
  // the key products
  int lv_region, lv_off;
};
inline DecodeShape decode_shape(const kvq_cache* c) {
  constexpr int kKS = 144, kPS = 136, kOS = 10, kLds = 163840;
  // tables, query operand, field dims, pair descriptors, pair parameters, small words
  constexpr int kStaticBase0 = 40960 + 4 * 16 * 40 * 2 + 128 + 64 * 4 + 16 * 24 * 4 + 64;
  // caches whose decode step may append inside the decode launch reserve that instantiation's
  // row image (1 KB rows + 128 B key row + 128 B value codes + scales), so both launches of
  // such a cache have the same shape
  const bool fusable = (c->cfg.codec == KVQ_CODEC_BGTQ || c->cfg.codec == KVQ_CODEC_UNIFORM) &&
                       c->cfg.recent_window == 0;
  const int kStaticBase = kStaticBase0 + (fusable ? 1024 + 128 + 128 + 16 : 0);
  const int G = c->group;
  const int vb = c->cfg.codec == KVQ_CODEC_NF16_B256 ? 4 : c->cfg.v_bits;
  int kpart = (c->k_words + 1) * kKS;
  if (kpart < G * kPS) kpart = G * kPS;
  if (kpart < 128 * kOS) kpart = 128 * kOS;
  if (kpart < G * 128) kpart = G * 128;
  if (kpart < G * 192) kpart = G * 192;   // recent window: q * sigma' and one chunk's weights
  kpart = (kpart + 3) & ~3;
  const int vwords = 512 * vb;
  // asymmetric integer codec: 1 KB of tile parameters per wave
  const int kvx = c->cfg.codec == KVQ_CODEC_KIVI ? 1024 : 0;
  // 8 waves, each V tile copied into its wave's region (after the softmax weights) once the key
  // product is done
  int late = ((G * kPS + 3) & ~3) + vwords;
  if (late < kpart) late = kpart;
  const bool lv_ok = kStaticBase + 16 * 8 * G + 64 * G + 8 * kvx + 4 * 8 * late <= kLds;
  const int lv_region = lv_ok ? late : 0, lv_off = (G * kPS + 3) & ~3;
  if (vb <= 4) {   // 8 waves, each with a static V tile area copied at tile start
    const int stat = kStaticBase + 16 * 8 * G + 64 * G + 4 * 8 * vwords + 8 * kvx;
    if (stat + 4 * 8 * kpart <= kLds) return {8, 1, kpart, 0, lv_region, lv_off};
  }
  if (lv_ok) return {8, 0, late, lv_off, lv_region, lv_off};
  const int stat = kStaticBase + 16 * 4 * G + 64 * G + 4 * kvx;
  if (stat + 4 * 4 * (kpart + vwords) <= kLds) return {4, 1, kpart + vwords, kpart, 0, 0};
  return {4, 0, late, lv_off, 0, 0};
}
inline int decode_waves(const kvq_cache* c) { return decode_shape(c).waves; }

// Workgroups that merge the S splits of one (sequence, KV head) in the decode kernel: a power
// of two, at most 32 and at most S, small enough that the waiting mergers of all units occupy
// fewer than all compute units (units x K < CUs), so the splits they wait for can always be
// scheduled.  0: no such count (the call is rejected).
inline int decode_split_mergers(int S, int64_t units, int n_cu) {
  int k = 32;
  while (k > 1 && (k > S || units * k >= n_cu)) k >>= 1;
  return units * k < n_cu ? k : 0;
}

// Offsets of one layer's storage.
inline uint32_t* layer_k_codes(kvq_cache* c, int layer) {
  return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(c->k_codes) + c->k_codes_layer * layer);
}
inline uint32_t* layer_v_codes(kvq_cache* c, int layer) {
  return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(c->v_codes) + c->v_codes_layer * layer);
}
inline uint16_t* layer_k_scales(kvq_cache* c, int layer) {
  return reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(c->k_scales) + c->k_scales_layer * layer);
}
inline __half* layer_k_recent(kvq_cache* c, int layer) {
  return reinterpret_cast<__half*>(reinterpret_cast<char*>(c->k_recent) + c->recent_layer * layer);
}
inline __half* layer_v_recent(kvq_cache* c, int layer) {
  return reinterpret_cast<__half*>(reinterpret_cast<char*>(c->v_recent) + c->recent_layer * layer);
}
// Positions of `layer` held by the packed storage (the rest are in the recent window).
inline int64_t packed_len_at(const kvq_cache* c, int64_t len) {
  const int64_t R = c->cfg.recent_window;
  const int64_t p = len > R ? len - R : 0;
  return p / c->pack_group * c->pack_group;
}
inline int64_t packed_len(const kvq_cache* c, int layer) { return packed_len_at(c, c->len[layer]); }
inline uint16_t* layer_v_scales(kvq_cache* c, int layer) {
  return reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(c->v_scales) + c->v_scales_layer * layer);
}

}  // namespace kvq
