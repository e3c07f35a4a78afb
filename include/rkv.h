/*
 * rkv.h -- C ABI of the write-time FP8 ring KV cache for MI355X (gfx950).
 *
 * The operations follow "Runway Characters: Serving a 57B Video Diffusion
 * Transformer for Real-Time Conversation" (arXiv:2611.05642):
 *
 *   ring cache with a device-side write position ....... §4.1
 *   RoPE at write and a delta rotation at reset ........ §4.2, Appendix G
 *   FP8 (e4m3) storage, only new tokens quantized ...... §4.3
 *   fused pre-attention (RoPE + quantize + ring write) . §4.4
 *   attention over the whole cache per call ........... §2 "The step budget",
 *                                                        Appendix G
 *   stacked allocation with per-layer views ........... §4.1
 *   one configuration object with switches ............ §8 "Keep the plain path"
 *
 * Conventions shared by every call:
 *
 * - Memory.  The caller owns every device buffer: the cache buffer handed to
 *   ring_cache_create and all inputs and outputs.  The library never
 *   allocates device memory, never synchronizes a stream and never reads
 *   device state on the host, so every call can be captured in a HIP graph
 *   (no memset nodes are recorded; clears are done by kernels).
 * - Streams.  Every call enqueues work on the given stream and returns.
 *   Calls that touch the same cache must be ordered by the caller (same
 *   stream, or events).  The attention workspace lives in the cache buffer
 *   and is shared by all layers: two cache_attend calls on one cache must
 *   not run concurrently.
 * - Tensors.  bf16 tensors are contiguous [n][n_heads][head_dim] (row-major,
 *   token-major), 16-byte aligned.  Positions are int32 device arrays.
 * - Errors.  Misuse that the host can see (null pointer, layer or size out
 *   of range, misaligned pointer, unsupported head_dim, buffer too small)
 *   returns RKV_EINVAL and enqueues nothing; a failed kernel launch returns
 *   RKV_EHIP.  rkv_last_error() gives a message for the calling thread.
 *   Device-state conditions are defined, not errors: attention over an empty
 *   cache writes zeros.
 */
#ifndef RKV_H
#define RKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  RKV_OK = 0,
  RKV_EINVAL = -1, /* bad argument; nothing was enqueued */
  RKV_EHIP = -2,   /* a HIP call or kernel launch failed */
};

/* Attention precision (the config switch keeps the plain path, §8 "Keep the
 * plain path behind every switch").
 *   RKV_PRECISE: Q enters the FP8 products as three power-of-two-scaled e4m3
 *                terms and the probabilities as two e4m3 terms (hi + lo/16).
 *   RKV_FAST:    one term each (plain FP8 attention as in §4.3). */
enum { RKV_PRECISE = 0, RKV_FAST = 1 };

/* Cache configuration, fixed at create time. */
typedef struct {
  int32_t n_layers;    /* independent layer caches in one allocation (>= 1) */
  int32_t n_slots;     /* ring slots per layer N (1 .. 1<<20) */
  int32_t n_heads;     /* heads H (1 .. 256) */
  int32_t head_dim;    /* D: 64 or 128 */
  int32_t max_queries; /* largest n_q of one cache_attend call (1 .. 1<<16;
                          also (ceil(max_queries / 128) x n_heads + the
                          attention workgroups, 4,096 when attn_workgroups is
                          0) x 128 x head_dim x 2 bytes of split partials
                          <= 1 GiB) */
  int32_t precision;   /* RKV_PRECISE or RKV_FAST */
  float rope_base;     /* RoPE base, omega_j = base^(-2j/D); 10000 */
  float scale_margin;  /* scale s = margin * amax / 448; 1.0 */
  int32_t attn_workgroups; /* persistent workgroups of one attention call
                              (1 .. 4096); 0 = two per compute unit */
  int32_t attn_merge_wait_us; /* longest wait of a workgroup for the last
                              arrival on a split unit before it leaves its
                              share of the merge to that arrival (0 .. 10000
                              microseconds; -1 = the default, 50).  0 leaves
                              every merge whose partials are not complete on
                              arrival to the last arrival; results do not
                              depend on this value */
  int32_t n_global;    /* global (sink) slots per layer beside the ring
                          (0 .. 1<<20; 0 = none): written once per session
                          with cache_write_global, read by every attention,
                          never rotated (§2 "The step budget": 1,246 global
                          slots beside a six-latent window) */
  int32_t rope_bands[3]; /* 3-D RoPE: pairs of the head's D/2 interleaved
                          pairs turned by the temporal position t, then by
                          y, then by x (contiguous bands; sum D/2); each band
                          is a RoPE of its own, omega = base^(-j / n_band)
                          for its j-th pair; positions are then int32
                          [n][3] = (t, y, x) per token and a reset turns
                          only the temporal band (§4.2, Appendix G).  All 0:
                          1-D RoPE over all pairs, omega_j = base^(-2j/D),
                          positions int32 [n]. */
} rkv_params;

/* Byte offsets into the cache buffer for one layer.  Layout (N_pad = N
 * rounded up to 64, plus n_global rounded up to 64: the ring's slots
 * [0, N), then the global slots [global_first_slot, + n_global) with
 * global_first_slot = N rounded up to 64; pad slots are zero and never
 * valid):
 *   codes_k  u8  [H][N_pad][D]        e4m3fn key codes, slot-major rows
 *   codes_v  u8  [H][N_pad/16][D][16] e4m3fn value codes, transposed per
 *                                      16-slot group (byte w of row d =
 *                                      slot 16*group + w)
 *   scale_k  f32 [H][N_pad]           per-(slot, head) key scale
 *   scale_v  f32 [H][N_pad]           per-(slot, head) value scale
 *   slot_pos i32 [N_pad]              position (3-D RoPE: temporal
 *                                      position t) each slot was written with
 *   slot_yx  i32 [2][N_pad]           3-D RoPE: spatial coordinates y, then x
 *   state    i32 [576]                {head, n_valid, ., g_valid}: the next
 *                                      write slot, the number of valid ring
 *                                      slots (the cyclic range [head-n_valid,
 *                                      head)) and of global slots read (1 +
 *                                      the highest global index written);
 *                                      the rest are ticket counters internal
 *                                      to the write kernel (a top counter at
 *                                      [2], 8 sub-counters at [64 (1 + j)]),
 *                                      zero between calls.
 *   normw    bf16 [2][D]              RMS-norm weights of the queries, then
 *                                      of the keys (ring_cache_set_qk_norm)
 *   static   f32 [2][H], i32          static scales of the keys, then of the
 *                                      values, and a flag (nonzero once
 *                                      calibrated: ring_cache_calibrate_static)
 *   vmax     f32 [H][8]               per head, the largest value scale
 *                                      written since the last reset (an upper
 *                                      bound of every cached value scale) is
 *                                      the max of the head's 8 entries. */
typedef struct {
  size_t codes_k, codes_v, scale_k, scale_v, slot_pos, state, vmax;
  size_t layer_bytes; /* distance between consecutive layers */
  int32_t n_slots_padded;
  size_t slot_yx;
  int32_t n_global, global_first_slot;
} rkv_layout;

typedef struct rkv_cache rkv_cache; /* opaque host-side handle */

/* Size in bytes of the cache buffer for these parameters (all layers, their
 * state, and the attention workspace), or 0 if the parameters are invalid
 * (including n_heads x max_queries so large that the attention's split-unit
 * partials, (n_heads * ceil(max_queries / 128) + workgroups) * 256 * head_dim
 * bytes, would reach 1 GiB). */
size_t ring_cache_bytes(const rkv_params* p);

/* Create a handle over a caller-owned device buffer of at least
 * ring_cache_bytes(p) bytes, 256-byte aligned.  Enqueues a kernel that
 * zeroes the whole buffer on `stream` (an empty cache).  *out receives the
 * handle.  The buffer must outlive the handle. */
int ring_cache_create(const rkv_params* p, void* dev_buf, size_t bytes, hipStream_t stream,
                      rkv_cache** out);

/* Free the host handle (not the device buffer).  Null is accepted. */
int ring_cache_destroy(rkv_cache* c);

/* Session reset (§6 "Session start" clears the dynamic cache): set head,
 * n_valid, vmax and every slot position of one layer (or all layers when
 * layer == -1) to zero, and return the layer to per-(token, head) scales
 * (static scales are calibrated once per session: Appendix G).  Codes and
 * per-slot scales are left as they are; slots outside the valid range are
 * never read.  The fused Q/K norm setting (model weights) is kept. */
int ring_cache_reset(rkv_cache* c, int32_t layer, hipStream_t stream);

/* Fill *out with the byte offsets of `layer` inside the cache buffer. */
int ring_cache_layout(const rkv_cache* c, int32_t layer, rkv_layout* out);

/* Ring write with RoPE and FP8 quantization fused (§4.1, §4.2, §4.3, §4.4).
 * k_bf16, v_bf16: [n][H][D] bf16 device tensors of the n new tokens.
 * pos: [n] int32 device positions ([n][3] = (t, y, x) with 3-D RoPE, each
 * pair turned by its band's coordinate).  Token i goes to slot
 * (head + i) mod N; its key is rotated at pos[i] (interleaved pairs
 * (2j, 2j+1), angle pos[i] * base^(-2j/D) computed in double precision),
 * then key and value rows are quantized per (token, head):
 * s = fp32(margin * amax / 448), code = e4m3(y / s) rounded to nearest even,
 * saturating at +-448.  slot_pos[slot] = pos[i].  Afterwards, on the device,
 * head <- (head + n) mod N and n_valid <- min(n_valid + n, N).
 * Requires 1 <= n <= N. */
int cache_write_rope_fp8(rkv_cache* c, int32_t layer, const void* k_bf16, const void* v_bf16,
                         const int32_t* pos, int32_t n, hipStream_t stream);

/* Global (sink) slot write (§2 "The step budget": global slots written once
 * per session, read by every attention, never rotated): tokens i = 0 .. n-1
 * go to global slots first + i, with the ring write's RoPE, quantization
 * (and static scales, RMS norm) and the same tensor layouts; the slots keep
 * their positions.  Afterwards g_valid = max(g_valid, first + n): every
 * global slot below g_valid is read by the attention, so the caller writes
 * them all (ring_cache_reset sets g_valid to 0).  Requires n >= 1 and
 * 0 <= first, first + n <= n_global. */
int cache_write_global(rkv_cache* c, int32_t layer, int32_t first, const void* k_bf16, const void* v_bf16,
                       const int32_t* pos, int32_t n, hipStream_t stream);

/* Delta rotation at a position reset (§4.2, Appendix G): for every valid
 * ring slot of `layer` (all layers when layer == -1) and every head,
 * dequantize the key, rotate pair j by delta * omega_j in fp32 (cos and sin
 * taken in double precision; with 3-D RoPE only the temporal pairs turn,
 * the spatial ones keep their values), take a new scale from the rotated
 * key's amax and requantize in place; slot_pos += delta.  Values and global
 * slots are not touched. */
int cache_delta_rotate(rkv_cache* c, int32_t layer, int32_t delta, hipStream_t stream);

/* Attention of n_q new queries over every valid slot of `layer`, the ring's
 * and the global slots below g_valid (§2, §4.3, Appendix G).  q_bf16:
 * [n_q][H][D] bf16 device tensor; q_pos: [n_q] (3-D RoPE: [n_q][3]) int32
 * device positions (RoPE is applied to Q here, at q_pos).  out_bf16:
 * [n_q][H][D] bf16 device tensor receiving softmax(q k^T / sqrt(D)) v over
 * the dequantized cache, computed with FP8 matrix instructions in the
 * configured precision, rounded to nearest even.  Non-causal.  An empty
 * cache gives zeros.  Requires 1 <= n_q <= max_queries. */
int cache_attend(rkv_cache* c, int32_t layer, const void* q_bf16, const int32_t* q_pos,
                 int32_t n_q, void* out_bf16, hipStream_t stream);

/* cache_attend for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same attention, same arguments, results (bit for bit), requirements and
 * errors, but the attention workspace (split-unit partials, arrival words,
 * prepared queries) lives in a fixed 32 MiB scratch array inside the library
 * (one per device, held from the library's load to process exit) instead of
 * the cache buffer.  It calls no allocating routine.  The workspace of a call
 * is (U + W) * (256 * D + 2048) + U * 128 * (3 * D + 13) bytes, U = H *
 * ceil(n_q / 128) units and W the persistent workgroups (each area rounded
 * up to 256 bytes); a call that would need more than 32 MiB returns
 * RKV_EINVAL and enqueues nothing (12 heads x 757 queries at D = 128 with 512
 * workgroups need about 23 MiB).  Every
 * cache_attend_noalloc call on a device shares that device's scratch: calls
 * that overlap on one device, from any cache or stream, race and must be
 * ordered by the caller.  The scratch keeps the last call's contents; each
 * call clears what must start at zero itself. */
int cache_attend_noalloc(rkv_cache* c, int32_t layer, const void* q_bf16, const int32_t* q_pos,
                         int32_t n_q, void* out_bf16, hipStream_t stream);

/* One call of the per-chunk sequence (§2 "The step budget", Appendix G: each
 * call writes its new chunk, then attends over the whole cache):
 * cache_write_rope_fp8(k, v, pos, n) followed by cache_attend(q, q_pos,
 * n_q, out), with the same arguments, results, requirements and errors
 * (checked before anything is enqueued).  For head_dim 128 the queries are
 * prepared in the write's launch, one launch fewer than the two calls.
 * Reads of q may not overlap the cache's own writes of this call: q, k, v
 * and out are distinct tensors. */
int cache_write_attend(rkv_cache* c, int32_t layer, const void* k_bf16, const void* v_bf16,
                       const int32_t* pos, int32_t n, const void* q_bf16, const int32_t* q_pos,
                       int32_t n_q, void* out_bf16, hipStream_t stream);

/* Fused pre-attention RMS norm (§4.4 "Fused pre-attention", Appendix G:
 * each block RMS-normalizes Q and K, then applies RoPE, then quantizes and
 * writes).  Once set for a layer, every write of that layer
 * (cache_write_rope_fp8, cache_write_attend) normalizes each (token, head)
 * key row, and every attention call (cache_attend, cache_write_attend) each
 * query row, before RoPE:
 *   y_d = x_d * w_d / sqrt(mean over d of x_d^2 + eps)
 * in fp32 (squares summed in fp32; the factor is the hardware reciprocal
 * square root).  Values are not normalized.
 * wq_bf16, wk_bf16: device bf16 [head_dim] weight vectors, each shared by all
 * heads, copied into the cache buffer on `stream` (device to device; the
 * caller may reuse them once the stream has passed the copy).  Both null:
 * the norm is off for the layer(s), the default.  layer -1: every layer.
 * eps: finite and > 0.  The setting is host state of the handle, read when
 * each later call is enqueued (calls already enqueued or captured keep the
 * setting they were made with).
 * Errors: RKV_EINVAL for a null cache, a layer out of range, exactly one
 * null weight pointer, a pointer not 2-byte aligned, or eps not finite and
 * > 0; RKV_EHIP if a copy cannot be enqueued. */
int ring_cache_set_qk_norm(rkv_cache* c, int32_t layer, const void* wq_bf16, const void* wk_bf16, float eps,
                           hipStream_t stream);

/* The pages' own scale mode (§4.3 "FP8 at write", Appendix G: scales per
 * (layer, head), calibrated once per session from the amax of the cache the
 * first steps filled, times a margin; values beyond them saturate; a reset
 * rotation keeps them and clamps).  For each layer (-1: all) this enqueues a
 * kernel that takes, per head, the largest magnitude of the dequantized keys
 * and of the values over the valid slots, sets the static scales
 * s = fp32(margin * amax / 448) (amax and the product in double precision)
 * and requantizes the head's valid keys and values to them
 * (code' = e4m3(code * s_slot / s), product and quotient in double
 * precision, saturating at +-448, which only a margin below 1 reaches).
 * From then on, every write of the layer quantizes with these scales
 * (e4m3 of the correctly rounded y / s, saturating) and stores them as the
 * slots' scales, every delta rotation requantizes each valid key with its
 * head's static key scale and clamps, and the attention applies the head's
 * two scales once (the key scale folded into the queries, the value scale
 * on the output) instead of reading per-slot scales.  A head whose amax is
 * 0 (nothing valid, or all zero) gets scale 0 and keeps the per-(token,
 * head) rule for its keys (values); a head with either scale 0 is attended
 * with its per-slot scales.  ring_cache_reset returns the layer to
 * per-(token, head) scales.  The mode is device state (graph-capturable).
 * margin in (0, 64] (the pages use 1.5).  Errors: RKV_EINVAL for a null
 * cache, a layer out of range or a bad margin; RKV_EHIP if the launch fails. */
int ring_cache_calibrate_static(rkv_cache* c, int32_t layer, float margin, hipStream_t stream);

/* Message for the last error on the calling thread ("" if none). */
const char* rkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RKV_H */
