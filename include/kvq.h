/*
 * kvq.h — C ABI of libkvq: low-bit KV-cache quantization with RoPE-aware
 * per-block bit allocation, and decode attention that reads the packed cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * Sources.  The method is that of "RoPE-Aware Bit Allocation for KV-Cache
 * Quantization" (Liang, Zhang, Jia; arXiv 2606.24033), abstract: a key's
 * contribution to a future logit decomposes over two-dimensional RoPE
 * frequency blocks; for each layer and KV head a label-free energy score is
 * computed per block and integer bit widths are allocated greedily by marginal
 * gain under a bits-per-dimension budget (KxVy); the quantizer is built on
 * TQ-MSE; decode runs over a packed cache.  The comparison codec is NQKV's
 * per-block Gaussian-quantile quantizer ("NQKV: A KV Cache Quantization Scheme
 * Based on Normal Distribution Characteristics", Pith review: "What carries
 * the argument", referee major comment 1; block size 256 from "Assumptions &
 * free parameters"), with append-only encoding ("Assumptions", third item).
 *
 * Conventions shared by every call.
 *  - head_dim is 128; each KV head has 64 RoPE blocks.
 *  - Tensor arguments are device pointers owned by the caller, C-contiguous,
 *    on the device that was current when the cache was created.  The library
 *    never keeps them after the call returns (work already enqueued on
 *    `stream` may still read them until it completes).
 *  - The cache owns all of its own device memory; kvq_cache_destroy frees it.
 *  - Calls validate their arguments synchronously on the host and return a
 *    status without enqueuing anything when validation fails; a failed call
 *    leaves the cache unchanged.  Valid calls enqueue kernels on `stream` and
 *    return without waiting (except the calls documented as synchronizing).
 *  - KVQ_EHIP reports a HIP runtime error seen at launch; a device-side fault
 *    surfaces at the caller's next synchronization.
 *  - A cache must not be mutated from two host threads at once.
 *  - Every sequence of the batch has the same length; kvq_quantize_append
 *    advances the length of one layer.
 *  - The library never applies RoPE: keys and queries arrive rotated.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvq_cache kvq_cache;
typedef void* kvq_stream; /* a hipStream_t; NULL is the default stream */

typedef enum {
  KVQ_OK = 0,
  KVQ_EINVAL = 1,    /* bad argument: null pointer, out-of-range layer/size/budget, bad config */
  KVQ_ENOMEM = 2,    /* device or host allocation failed */
  KVQ_ECAPACITY = 3, /* an append would exceed max_tokens */
  KVQ_ESTATE = 4,    /* call out of order: append before alloc, re-alloc after append,
                        decode of an empty layer */
  KVQ_EHIP = 5       /* HIP runtime error (kvq_last_error() has the text) */
} kvq_status;

typedef enum { KVQ_F16 = 0, KVQ_F32 = 1 } kvq_dtype;

typedef enum {
  KVQ_CODEC_BGTQ = 0,       /* Block-GTQ: per-block widths from kvq_alloc_bits, per-block gains */
  KVQ_CODEC_UNIFORM = 1,    /* uniform TQ-MSE-style baseline: every block k_bits, no gains */
  KVQ_CODEC_UNIFORM_ROT = 3, /* uniform baseline on randomly rotated keys: K rows pass through
                                R = H D / sqrt(128) (Sylvester-Hadamard H, caller signs D, see
                                kvq_set_rotation) before the uniform quantizer; V as UNIFORM */
  KVQ_CODEC_NF16_B256 = 2,  /* NQKV-style: 4-bit 16-level Gaussian quantiles, absmax scale per
                               256 consecutive values of a token's [n_kv_heads*128] vector */
  KVQ_CODEC_BGTQ_ROT = 5,   /* Block-GTQ with rotations inside equal-width groups: in plan field order
                               each run of equal-width fields is cut into power-of-two chunks (largest
                               first) and every chunk of m fields rotated by H_m D / sqrt(m) (caller
                               signs D per dim, see kvq_set_rotation) after the gain normalisation;
                               decode rotates g * q instead; V as BGTQ */
  KVQ_CODEC_KIVI = 4        /* KIVI-style asymmetric integers (the leaderboard's third method; NQKV
                               review, ablation table: keys per channel, values per token): a key
                               group is one channel over a 128-position tile, a value group is one
                               position's 128 channels; per group lo = fp16(min), s = fp16(fp32(
                               fp32(fp16(max) - lo) / (2^b - 1))), code = clamp(rint(fp32(fp32(x - lo)
                               * fp32(1/s))), 0, 2^b - 1), reconstruction fp16(lo + s * code).  Key
                               tiles are quantized once complete: the positions after the last
                               whole tile (and the window, if any) stay in fp16 */
} kvq_codec;

typedef enum {
  KVQ_ROPE_HALF = 0,        /* block j pairs dims (j, j+64) */
  KVQ_ROPE_INTERLEAVED = 1  /* block j pairs dims (2j, 2j+1) */
} kvq_pairing;

typedef struct {
  int32_t n_layers;    /* >= 1 */
  int32_t n_kv_heads;  /* >= 1 */
  int32_t n_q_heads;   /* multiple of n_kv_heads; group size n_q/n_kv in {1, 2, 4, 8} */
  int32_t head_dim;    /* must be 128 */
  int32_t batch;       /* sequences, >= 1 */
  int64_t max_tokens;  /* capacity per sequence and layer, >= 1 */
  int32_t k_bits;      /* K budget in bits per dim, in [max(1,b_min), b_max] */
  int32_t v_bits;      /* V width in bits per dim, in [1, 8] */
  int32_t b_min;       /* smallest per-block K width, >= 0 (default 0) */
  int32_t b_max;       /* largest per-block K width, <= 8 (default 8) */
  int32_t codec;       /* kvq_codec; NF16_B256 needs k_bits = v_bits = 4 and
                          n_kv_heads*128 divisible by 256 */
  int32_t pairing;     /* kvq_pairing */
  int32_t recent_window; /* R in [0, 4096], a multiple of 128: the most recent min(len, R) tokens of each
                            sequence and layer are kept in fp16 (K and V) instead of the
                            packed cache; 0 = none.  The paper reports its results with no such
                            fp16 buffer of recent keys (RoPE-aware bit allocation page,
                            abstract); the leaderboard's buffer-setting column is this option. */
  int32_t per_sequence_plans; /* 0: one plan per (layer, KV head), shared by the batch; 1: one
                            plan per (layer, sequence, KV head), each from that sequence's own
                            calibration keys (see kvq_alloc_bits) */
} kvq_config;

/* Layout facts of one layer's packed storage, for parity dumps (see kvq_read_cache). */
typedef struct {
  int64_t capacity;        /* token capacity per sequence (max_tokens rounded up to 128) */
  int64_t len;             /* tokens appended so far */
  int32_t k_row_words;     /* 32-bit words per K row = 4*k_bits */
  int32_t v_dim_words;     /* 32-bit words per dim per 128-token V tile = 4*v_bits */
  int64_t k_codes_bytes;   /* bytes of one layer's K rows: [batch][n_kv][capacity][k_row_words]; a row
                              is the stored fields in plan order (blocks by width descending, then
                              block index; coordinate p0 then p1), LSB first */
  int64_t v_codes_bytes;   /* bytes of one layer's V tiles: [batch][n_kv][capacity/128][512][v_bits].
                              A tile is 512 segments of v_bits words; segment (dim, g) holds the codes
                              of that dim for tile tokens 32g .. 32g+31, LSB first (token 32g+e at bit
                              e*v_bits), stored at index ((dim/16)*4 + g)*16 + dim%16 */
  int64_t k_scales_bytes;  /* fp16 K scales: BGTQ/UNIFORM [batch][n_kv][capacity];
                              NF16 [batch][capacity][n_kv*128/256];
                              KIVI [batch][n_kv][capacity/128][64 blocks][s(p0), s(p1), lo(p0), lo(p1)] */
  int64_t v_scales_bytes;  /* fp16 V scales, same shapes as K scales;
                              KIVI [batch][n_kv][capacity/128][2][128]: the tile's s, then its lo */
  int32_t plan_ready;      /* 1 once kvq_alloc_bits has run for this layer */
  int32_t recent_window;   /* R of the config */
  int64_t packed_len;      /* positions held by the packed storage: max(0, len - R) (KIVI: rounded
                              down to a multiple of 128); positions packed_len .. len-1 are in the
                              recent window */
  int64_t recent_bytes;    /* bytes of one layer's recent-window K (or V) ring of ring_slots slots,
                              fp16, position p in slot p mod ring_slots: K [batch][ring_slots][n_kv][128];
                              V in dim-major 128-slot tiles [batch][n_kv][ring_slots/128][128 dims][128 slots] */
  int32_t ring_slots;      /* R, or R + 128 for KIVI (whose window also holds the last partial tile) */
} kvq_layer_info;

typedef enum {
  KVQ_PART_K_CODES = 0,
  KVQ_PART_V_CODES = 1,
  KVQ_PART_K_SCALES = 2,
  KVQ_PART_V_SCALES = 3,
  KVQ_PART_K_RECENT = 4,   /* recent-window rings (see kvq_layer_info) */
  KVQ_PART_V_RECENT = 5
} kvq_part;

/* Create a cache for cfg and allocate its full capacity on the current device: the packed store
   of codebook indices plus scales that the NQKV review describes ("What carries the argument"),
   filled append-only ("Assumptions", third item), with one plan per layer and KV head as in
   "RoPE-Aware Bit Allocation for KV-Cache Quantization", abstract (allocation per layer and KV
   head).  Every device buffer any later call needs is allocated here; no other call allocates
   device memory except kvq_alloc_bits, which grows its energy scratch to the largest
   calibration seen.
   Validates cfg before touching the GPU (KVQ_EINVAL).  *out is set only on KVQ_OK; the caller
   owns the cache and frees it with kvq_cache_destroy.
   Environment: KVQ_MERGE_POLL_LIMIT (integer, 0 .. 4194304, read here) bounds how long a decode
   split merger waits for the partials of the other splits; a test hook (see kvq_cache_status). */
kvq_status kvq_cache_create(const kvq_config* cfg, kvq_cache** out);

/* Free everything the cache owns; NULL is ignored.  Synchronizes the device. */
void kvq_cache_destroy(kvq_cache* cache);

/* Per-(layer, KV head) bit allocation (Block-GTQ; RoPE-aware bit allocation
   page, abstract: each RoPE block gets an energy score computed from keys
   alone, then integer widths are handed out one step at a time to the block
   whose marginal gain is largest).
   keys:   [n_tok][n_kv_heads][128] post-RoPE calibration keys (dtype), n_tok >= 1,
           16-byte aligned; with per_sequence_plans, [batch][n_tok][n_kv_heads][128]
           (n_tok keys of every sequence, each sequence's plans from its own keys).
           May be NULL for the UNIFORM and NF16 codecs, whose plans are fixed.
   block_weight: NULL, or a device fp64 array [n_kv_heads][64] ([batch][n_kv_heads][64]
           with per_sequence_plans) of per-block weights multiplying the energy score
           before the greedy.
   Computes m_j = sum over tokens of the block's squared norm / (2 n_tok) in fp64
   (terms summed in token order inside 256-token chunks, then chunk totals in
   order), widths b_j in [b_min, b_max] with sum_j 2 b_j = 128 k_bits by
   repeatedly raising the block with the largest s_j * delta(b_j) (ties to the
   smallest j), and per-block gains sqrt(m_j / mean m).  Writes the layer's plan.
   Errors: KVQ_EINVAL (null cache/keys, bad layer, n_tok < 1, bad dtype),
           KVQ_ESTATE (the layer already holds appended tokens). */
kvq_status kvq_alloc_bits(kvq_cache* cache, int32_t layer, const void* keys, int32_t dtype,
                          int64_t n_tok, const double* block_weight, kvq_stream stream);

/* Copy one layer's plan to host memory: the integer widths the greedy allocation handed to each
   RoPE block and the per-block gains ("RoPE-Aware Bit Allocation for KV-Cache Quantization",
   abstract: widths per layer and KV head under the bit budget).  Synchronizes the device.
   bits:  host int8 [n_kv_heads][64] per-block widths (required); with
          per_sequence_plans [batch][n_kv_heads][64].
   gains: host fp32, same shape as bits: per-block gains g_j (nullable).
   Errors: KVQ_EINVAL, KVQ_ESTATE (no plan yet), KVQ_EHIP. */
kvq_status kvq_get_plan(const kvq_cache* cache, int32_t layer, int8_t* bits, float* gains);

/* Quantize and append n_new tokens to every sequence of one layer
   (per-token scale, codebook lookup and bit-packing; append-only).  The quantizer is the
   TQ-MSE-style scalar codebook quantizer at the layer's per-block widths ("RoPE-Aware Bit
   Allocation for KV-Cache Quantization", abstract: built on TQ-MSE, matched K/V budgets), or the
   NQKV review's 16-level Gaussian-quantile codebook with one absmax scale per 256 values ("What
   carries the argument"); tokens are encoded once, when appended ("Assumptions", third item).
   k, v:  [batch][n_new][n_kv_heads][128] post-RoPE keys and values (dtype),
          16-byte aligned.
   n_new = 0 is a no-op.  Row quantizer, in IEEE fp32/fp64 with no fused ops:
   y = x * ig_j; s = fp16(fp32(sqrt(sum y^2 / 128))); u = y * fp32(1/s);
   code = number of codebook boundaries below u (the sum of squares in dim order).
   NF16: s = fp16(absmax) per 256 values, u = x * fp32(1/s).  Rotating codecs
   quantize the rotated rows (see kvq_codec); KIVI quantizes whole 128-position
   key tiles (see kvq_codec) and keeps the positions after the last whole tile in
   fp16.
   With a recent window R > 0, positions stay in fp16 (rounded once if given in
   fp32) while they are among the last R of the sequence; a position is
   quantized, from its fp16 copy, when it leaves the window, so the packed
   storage always covers positions 0 .. len-R-1 (KIVI: rounded down to a
   multiple of 128).
   Errors: KVQ_EINVAL, KVQ_ESTATE (no plan for the layer, or no rotation signs for a
   rotating codec), KVQ_ECAPACITY. */
kvq_status kvq_quantize_append(kvq_cache* cache, int32_t layer, const void* k, const void* v,
                               int32_t dtype, int64_t n_new, kvq_stream stream);

/* Grouped-query decode attention of one query per sequence against the packed
   cache of one layer ("RoPE-Aware Bit Allocation for KV-Cache Quantization", abstract: decoding
   reads the packed K3V3 cache directly at 128K context): logits sigma * <q_h, x_hat^K> over every
   appended token, softmax, weighted sum of x_hat^V; KV head of query head h is h / group.
   q:     [batch][n_q_heads][128] (dtype), 4-byte aligned.
   softmax_scale: sigma; <= 0 selects 1/sqrt(128).
   out:   [batch][n_q_heads][128] fp32 device buffer, 16-byte aligned.
   With a recent window, the last min(len, R) tokens are read in fp16 from the
   window (x_hat = the fp16 values) and the others from the packed storage.
   The context is split into chunks processed in parallel, each producing a
   partial (max, sum, weighted sum); the last chunks of each (sequence, KV head)
   to finish combine them in fixed order (with as many (sequence, KV head) units as
   the device has compute units, a second kernel on the same stream combines them).
   A combining workgroup waits a bounded time for the other chunks; if it gives up it
   writes NaN over its outputs and sets the cache's device error word, reported by
   kvq_cache_status.  Decode calls on one cache must not overlap in time (they share the
   partial buffers).
   Errors: KVQ_EINVAL (also a misaligned q or out), KVQ_ESTATE (layer empty or
   without plan). */
kvq_status kvq_decode_attn(kvq_cache* cache, int32_t layer, const void* q, int32_t dtype,
                           float softmax_scale, float* out, kvq_stream stream);

/* As kvq_decode_attn with an explicit number of context splits per (sequence,
   KV head); n_splits <= 0 lets the library choose.  The result does not depend
   on n_splits beyond fp32 rounding. */
kvq_status kvq_decode_attn_splits(kvq_cache* cache, int32_t layer, const void* q, int32_t dtype,
                                  float softmax_scale, float* out, int32_t n_splits,
                                  kvq_stream stream);

/* One decode step of a layer: appends one new position to every sequence and then attends
   with q over all positions, the new one included ("RoPE-Aware Bit Allocation for KV-Cache
   Quantization", abstract: decoding reads the packed cache directly; Pith review of NQKV,
   "Assumptions & free parameters", third item: the cache is encoded append-only, so a new
   position is quantized once, on arrival).
   k_new, v_new: [batch][n_kv_heads][128] (dtype), 16-byte aligned; q and out as for
   kvq_decode_attn; one dtype for all three inputs.
   Codes, scales and output are those of kvq_quantize_append(..., n_new = 1) followed by
   kvq_decode_attn.  For the Block-GTQ and uniform codecs without a recent window this is one
   launch: the workgroup that reads the new position's tile quantizes it, stores it, and
   uses it from its own copy; other codecs and recent windows run the two calls.
   Errors: those of the two calls (KVQ_EINVAL, KVQ_ESTATE, KVQ_ECAPACITY), all checked before
   anything is enqueued, so a rejected call appends nothing; KVQ_EHIP if a launch fails. */
kvq_status kvq_decode_step(kvq_cache* cache, int32_t layer, const void* k_new, const void* v_new,
                           const void* q, int32_t dtype, float softmax_scale, float* out,
                           kvq_stream stream);

/* As kvq_decode_attn (automatic split count), for callers that cannot allocate: code under
   HIP graph or stream capture, tight serving loops, harnesses that forbid allocation.  It makes
   no allocation of any kind: the split partials, maxima words and tag bases live in a fixed
   8 MiB device array of the library (one per device, held until the process ends; its address is
   looked up once per device on the first call there), not in the cache's buffers.  Each call
   first clears the words it merges on (a small kernel, no memset), so nothing of an earlier call
   is ever read.  Results are those of kvq_decode_attn on the same cache.  The cache's device
   error word reports a merge that gave up, as for kvq_decode_attn (see kvq_cache_status).
   Every call on a device shares that device's array: calls that overlap in time on one device
   race, whatever their caches.
   Errors: as kvq_decode_attn; KVQ_EINVAL also when the call needs more than 8 MiB of split
   scratch (batch * n_kv_heads * splits * group * 524 bytes; kvq_last_error has the figure). */
kvq_status kvq_decode_attn_noalloc(kvq_cache* cache, int32_t layer, const void* q, int32_t dtype,
                                   float softmax_scale, float* out, kvq_stream stream);

/* Key-cache fidelity diagnostics of `layer`: how well the stored keys preserve the
   attention logits, after "RoPE-Aware Bit Allocation for KV-Cache Quantization",
   abstract (per-layer query-key logit mean absolute error, keys only) and
   "KV Cache Quantization on WikiText-2 prompt 2048-token (train)", evaluation
   results (softmax KL divergence).  For sequence b and query head h (KV head
   h / G), over the len(layer) cached positions t, in fp64:
     a_t  = sigma * <q_h, k_t>     (k: the keys as given),
     a^_t = sigma * <q_h, k^_t>    (k^: the stored keys, dequantized as decode
                                    reads them; fp16 copies inside a recent window),
     mae[b][h] = mean_t |a_t - a^_t|,  kl[b][h] = KL(softmax(a) || softmax(a^)),
   with sigma = softmax_scale, or 1/sqrt(head_dim) when softmax_scale <= 0.
   q:    [batch][n_q_heads][head_dim] of `dtype`, device;
   keys: [batch][len(layer)][n_kv_heads][head_dim] of `dtype`, device, 16-byte
         aligned: the keys appended to this layer, in order (post-RoPE);
   mae, kl: [batch][n_q_heads] fp64, device, caller-owned.
   Uses a statistics buffer of the cache: calls on one cache must not overlap in
   time.  Errors: KVQ_EINVAL (null or misaligned pointer, bad dtype or scale),
   KVQ_ESTATE (layer empty or without plan). */
kvq_status kvq_key_fidelity(kvq_cache* cache, int32_t layer, const void* q, const void* keys,
                            int32_t dtype, float softmax_scale, double* mae, double* kl,
                            kvq_stream stream);

/* Random signs of the key rotation of one layer (codecs KVQ_CODEC_UNIFORM_ROT and
   KVQ_CODEC_BGTQ_ROT), after RoPE-Aware Bit Allocation for KV-Cache Quantization,
   abstract: the quantizer sits on top of TQ-MSE, whose quantizer rotates the whole vector
   at random before scalar quantization.  UNIFORM_ROT stores y = fp32(H (s * k) / sqrt(128))
   (the fast Walsh-Hadamard transform in fp64); BGTQ_ROT rotates the gain-normalised key
   fp32(k * ig) chunk by chunk inside its equal-width groups (see the codec).  Decode and the
   fidelity diagnostics rotate the query instead of the keys.  signs: host int8
   [n_kv_heads][128] indexed by dim, each +1 or -1; the caller draws them.  Must precede the
   layer's first append.  Synchronizes the device.
   Errors: KVQ_EINVAL (other codec, null or a value other than +-1), KVQ_ESTATE (the layer
   already holds tokens). */
kvq_status kvq_set_rotation(kvq_cache* cache, int32_t layer, const int8_t* signs);

/* Device-side status of the cache.  Synchronizes the device, then returns KVQ_EHIP (with the
   text in kvq_last_error) if a decode split merge gave up waiting since the last call of this
   function, else KVQ_OK.  After such a give-up every merged decode output is NaN until this call,
   which also clears the word and the merge bookkeeping (the cache's data are unaffected).
   Errors: KVQ_EINVAL (null cache), KVQ_EHIP (also a runtime error of the synchronization). */
kvq_status kvq_cache_status(kvq_cache* cache);

/* Read-only device view of one layer's packed storage and plans, for callers that read the
   packed cache in place (indices plus scales, as the NQKV review's cache holds them: "What
   carries the argument"; decode reads the packed cache directly: "RoPE-Aware Bit Allocation
   for KV-Cache Quantization", abstract).  No copy and no synchronization: the pointers address
   the cache's own memory, stay valid until kvq_cache_destroy, and see later appends of the
   layer (len and packed_len are those at the time of the call).  The caller must not write
   through them.  Layouts are those of kvq_layer_info; strides are in elements of each part:
     k_codes   uint32 [batch][n_kv][capacity][k_row_words]; strides (sequence, head, token)
     v_codes   uint32 [batch][n_kv][capacity/128][512][v_bits]; strides (sequence, head, tile)
     k_scales, v_scales  fp16 bit patterns; strides (sequence, head, token) for BGTQ, UNIFORM and
               the rotating codecs, (sequence, token, 256-value block) for NF16_B256, (sequence,
               head, 128-position tile: 256 halves) for KIVI
     k_recent, v_recent  fp16 rings of the recent window (NULL without one)
     plans     n_plans records of plan_bytes bytes, [n_kv] or [batch][n_kv] with per-sequence
               plans; at byte KVQ_PLAN_OFF_GAIN 128 fp32 gains by dim, KVQ_PLAN_OFF_FIELD_DIM 128
               uint8 dims in plan (field) order, KVQ_PLAN_OFF_FIELD_WIDTH their uint8 widths,
               KVQ_PLAN_OFF_BLOCK_WIDTH 64 int8 block widths, KVQ_PLAN_OFF_N_FIELDS the int32
               count of stored fields.
   Errors: KVQ_EINVAL (null cache or view, bad layer). */
#define KVQ_PLAN_BYTES 2256
#define KVQ_PLAN_OFF_GAIN 0
#define KVQ_PLAN_OFF_FIELD_DIM 1280
#define KVQ_PLAN_OFF_FIELD_WIDTH 1408
#define KVQ_PLAN_OFF_BLOCK_WIDTH 1664
#define KVQ_PLAN_OFF_N_FIELDS 2240
typedef struct {
  const uint32_t* k_codes;
  int64_t k_codes_strides[3];
  const uint32_t* v_codes;
  int64_t v_codes_strides[3];
  const uint16_t* k_scales;
  const uint16_t* v_scales;
  int64_t scale_strides[3];
  const uint16_t* k_recent;
  const uint16_t* v_recent;
  const void* plans;
  int32_t n_plans;
  int32_t plan_bytes;
  int64_t capacity;
  int64_t len;
  int64_t packed_len;
} kvq_view;
kvq_status kvq_cache_view(const kvq_cache* cache, int32_t layer, kvq_view* view);

/* Tokens appended so far to `layer` (host bookkeeping; does not synchronize). */
kvq_status kvq_seq_len(const kvq_cache* cache, int32_t layer, int64_t* len);

/* Layout facts of one layer (host bookkeeping; does not synchronize). */
kvq_status kvq_layer_info_get(const kvq_cache* cache, int32_t layer, kvq_layer_info* info);

/* Copy nbytes of one layer's packed storage, starting at byte `offset` of the
   part, to host memory dst.  Synchronizes the device.  Used by parity tests.
   Errors: KVQ_EINVAL (bad part, range outside the part), KVQ_EHIP. */
kvq_status kvq_read_cache(const kvq_cache* cache, int32_t layer, int32_t part, int64_t offset,
                          int64_t nbytes, void* dst);

/* Measurement aid, not a step of the method: one launch that reads nbytes of device memory
   once (16-byte loads, n_blocks workgroups of 256 threads, grid-stride) and writes nothing but,
   in practice never, one word of `sink` per workgroup.  Timing it over buffers of one decode
   launch's size gives the per-launch HBM read ceiling the decode kernel's effective rate is
   set against (the decode is bound by reading the packed cache: RoPE-Aware Bit Allocation for
   KV-Cache Quantization, abstract, serving from the packed cache).
   src: device, 16-byte aligned; nbytes a positive multiple of 16; sink: device uint32
   [n_blocks], caller-owned.  Errors: KVQ_EINVAL (bad pointer, size or n_blocks outside
   [1, 65536]), KVQ_EHIP. */
kvq_status kvq_probe_stream_read(const void* src, int64_t nbytes, int32_t n_blocks, uint32_t* sink,
                                 kvq_stream stream);

/* Host copies of the library's own constant tables (no GPU needed).
   kvq_codebook: bits in [1, 8]; centroids: 2^bits fp16 bit patterns;
                 boundaries: 2^bits - 1 fp32 values (either pointer nullable).
   kvq_delta:    8 fp32 greedy gains delta(b) = c(b) - c(b+1), b = 0..7.
   kvq_nf16_codebook: 16 fp16 levels and 15 fp32 boundaries. */
kvq_status kvq_codebook(int32_t bits, uint16_t* centroids, float* boundaries);
kvq_status kvq_delta(float* delta);
kvq_status kvq_nf16_codebook(uint16_t* levels, float* boundaries);

/* Human-readable name of a status; never NULL. */
const char* kvq_status_str(kvq_status status);

/* Text of the last HIP error recorded by this thread ("" if none); never NULL. */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
