// Host-side launchers of the gfx950 kernels (one per kernel family).  Each
// returns the hipError_t of its launch; argument validation happens in the
// C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>

#include "rkv_device.h"

namespace rkv {

// Attention workspace inside the cache buffer (shared by all layers).
constexpr int kSyncStride = 16;  // 64-bit words between units' arrival words

struct AttnWs {
  void* part_o;    // [units + grid][4 query slices][D/16 chunks][64 lanes] 16-byte chunks of fp16 c_h O / l
  float* part_ml;  // [units + grid][4 query slices][64 lanes] fp32 pairs (running max, sum)
  // [units][kSyncStride] per split unit, in the first word of its own 128-byte
  // line: tiles arrived (low half) | output blocks committed to a merge
  // (high half); zeroed for the call's units by q_prep_kernel
  unsigned long long* sync;
  // e4m3 codes of the RoPE'd queries, 3 terms x H x nq_pad rows x D, in
  // matrix-operand order: per term, head and block of 32 rows, per k-block
  // ks of 64 dims, 64 lanes x 32 bytes -- lane li + 32 gq holds dims
  // [64 ks + 32 gq, +32) of the block's row li
  uint8_t* qcodes;
  int32_t* qexp;   // [3 terms][H][nq_pad] E8M0 code (127 + e) of the 2^e scale of each query row and term
  int32_t nq_pad;  // max_queries rounded up to 128
  int32_t grid;    // persistent workgroups
  int32_t terms;   // 2 = precise (3 query terms, 2 probability terms), 1 = fast (one each)
  int32_t wait_ticks;  // bound on a merge wait, in ticks of the 100 MHz real-time clock
};

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_init_consts(const Geom& g, const double* turns, int n, hipStream_t s);
hipError_t launch_reset(const Geom& g, int layer_lo, int layer_hi, hipStream_t s);
// Static per-head scales from the valid cache of each layer in [layer_lo, layer_hi).
hipError_t launch_calibrate(const Geom& g, int layer_lo, int layer_hi, float margin, hipStream_t s);
// wk (and wq below): the layer's RMS-norm weights (bf16 [D]) of the fused
// pre-attention norm, null when it is off; eps its epsilon.
hipError_t launch_write(const Geom& g, int layer, const void* k, const void* v, const int32_t* pos,
                        int n, const uint16_t* wk, float eps, hipStream_t s);
// Global (sink) slots first .. first + n - 1 of the layer, written like the ring.
hipError_t launch_write_global(const Geom& g, int layer, int first, const void* k, const void* v, const int32_t* pos,
                               int n, const uint16_t* wk, float eps, hipStream_t s);
hipError_t launch_rotate(const Geom& g, int layer_lo, int layer_hi, int32_t delta,
                         const float* cosv, const float* sinv, hipStream_t s);
hipError_t launch_attend(const Geom& g, const AttnWs& ws, int layer, const void* q,
                         const int32_t* q_pos, int n_q, void* out, const uint16_t* wq, float eps,
                         hipStream_t s);
// The attention workspace of one call of n_q queries placed in the library's
// fixed device scratch (the entry point that allocates nothing): *need
// receives its size in bytes; when it fits in kScratchBytes, *out is `base`
// with its pointers moved into this device's scratch (the address found once
// per device with hipGetSymbolAddress).  Returns the error of that lookup.
constexpr size_t kScratchBytes = size_t(32) << 20;
hipError_t fixed_attn_ws(const Geom& g, const AttnWs& base, int n_q, AttnWs* out, size_t* need);
// Looks the scratch address up for the current device if not done yet (at
// cache creation, so that a first cache_attend_noalloc under graph capture
// finds it ready).
hipError_t scratch_init();
// Write, then attention, with the query preparation in the write's launch.
hipError_t launch_write_attend(const Geom& g, const AttnWs& ws, int layer, const void* k, const void* v,
                               const int32_t* pos, int n, const void* q, const int32_t* q_pos, int n_q,
                               void* out, const uint16_t* wq, const uint16_t* wk, float eps, hipStream_t s);

// Work of the write: `groups` 16-slot groups (a run of n slots meets at most
// n/16 + 2 of them) times n_heads / hg head groups of hg heads, the items.
// A write is bound by each wave's arithmetic latency: one head per item while
// the items fit in one resident grid (the 757-token, 12-head write: 612
// workgroups; beside the query preparation its chain ended 1.5 us sooner
// than with two heads), two heads per item for larger writes (one head per
// item slowed them by 30-50%: twice the items over a grid that is already
// full; four heads per workgroup ran 0.5 us slower still).  *wgs workgroups
// take them: one item each up to kWriteMaxWgs, several each beyond (a
// persistent grid whose workgroups load their next item while they process
// the current one).
#ifndef RKV_WRITE_MAX_WGS
#define RKV_WRITE_MAX_WGS 1024
#endif
constexpr int kWriteMaxWgs = RKV_WRITE_MAX_WGS;
inline void write_grid(const Geom& g, int n, int* groups, int* hg, int* items, int* wgs) {
  const int NG = (g.n_slots + 15) / 16;
  *groups = (n + 15) / 16 + 2;
  if (*groups > NG) *groups = NG;
  const int H = g.n_heads;
  *hg = H % 2 == 0 && *groups * H > kWriteMaxWgs ? 2 : 1;
  *items = *groups * (H / *hg);
  *wgs = *items < kWriteMaxWgs ? *items : kWriteMaxWgs;
}

}  // namespace rkv
