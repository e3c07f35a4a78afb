// Host-side launchers of the gfx950 kernels (one per kernel family).  Each
// returns the hipError_t of its launch; argument validation happens in the
// C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>

#include "rkv_device.h"

namespace rkv {

// Attention workspace inside the cache buffer (shared by all layers).
struct AttnWs {
  uint8_t* qcodes;   // [terms][H][nq_pad][D] e4m3 query codes
  uint8_t* qscale;   // [terms][H][nq_pad] E8M0 scale bytes (127 + exponent)
  float* head_c;     // [H] probability scale c_h = 448 * 2^-headroom / max s_v
  float* part_o;     // [units][32][D] fp32 partial outputs (split-KV)
  float* part_ml;    // [units][32][2] fp32 partial (max, sum)
  int32_t nq_pad;    // query rows allocated per head (multiple of 32)
  int32_t splits;    // KV splits per (head, 32-query block)
  int32_t terms;     // 2 = precise, 1 = fast
};

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_init_consts(const Geom& g, const double* turns, int n, hipStream_t s);
hipError_t launch_reset(const Geom& g, int layer_lo, int layer_hi, hipStream_t s);
hipError_t launch_write(const Geom& g, int layer, const void* k, const void* v, const int32_t* pos,
                        int n, hipStream_t s);
hipError_t launch_rotate(const Geom& g, int layer_lo, int layer_hi, int32_t delta,
                         const float* cosv, const float* sinv, hipStream_t s);
hipError_t launch_attend(const Geom& g, const AttnWs& ws, int layer, const void* q,
                         const int32_t* q_pos, int n_q, void* out, hipStream_t s);

}  // namespace rkv
