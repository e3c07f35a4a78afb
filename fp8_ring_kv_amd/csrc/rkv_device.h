// Device-side helpers and the cache geometry shared by the kernels and the
// host launcher.  gfx950 (CDNA4) only: OCP e4m3fn conversions, scaled FP8
// matrix instructions, 64-wide wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rkv {

constexpr float kE4M3Max = 448.0f;
constexpr int kTile = 64;        // slots per attention tile and per V transpose tile
constexpr int kMaxHalfDim = 64;  // D/2 for the largest supported head_dim (128)
// Per-head value-scale maxima are spread over kSub slots so that no single
// address takes more than a fraction of one launch's atomics.
constexpr int kSub = 8;
constexpr int kStateInts = 4;  // head, n_valid, top ticket counter of the write, g_valid
// A large write counts its tickets on kTicketSub sub-counters, each on its
// own 256-byte line kTicketStride ints past the previous one (sub-counter j
// at state[kTicketStride * (1 + j)]): atomics on one address serialize, so
// one counter for every workgroup of a large write cost ~15 ns per workgroup.
constexpr int kTicketSub = 8;
constexpr int kTicketStride = 64;
constexpr int kTicketSplitMin = 512;  // workgroups above which the tickets use the sub-counters
constexpr int kStateRegionInts = kTicketStride * (1 + kTicketSub);

// Byte offsets of one layer's arrays (relative to the layer's start) and the
// sizes every kernel needs.  Passed by value as a kernel argument.
// A layer's slot arrays hold the ring, slots [0, n_slots), padded to
// n_ring_pad = a multiple of 64, then the global (sink) slots [g0, g0 +
// n_global) with g0 = n_ring_pad, padded again: n_pad slots, n_tiles 64-slot
// tiles, of which the first n_ring_tiles are the ring's.
struct Geom {
  uint8_t* base;        // cache buffer
  size_t consts;        // offset of the constants block (double omega/(2 pi) table)
  size_t layer0;        // offset of layer 0
  size_t layer_bytes;   // stride between layers
  size_t off_codes_k, off_codes_v, off_scale_k, off_scale_v, off_slot_pos, off_slot_yx, off_state, off_vmax,
      off_normw, off_static;
  int32_t n_layers, n_slots, n_pad, n_tiles, n_heads, head_dim;
  int32_t n_ring_pad, n_ring_tiles, n_global;  // g0 = n_ring_pad
  // RoPE pair bands: pairs [0, band_t) turn with the temporal position,
  // [band_t, band_ty) with y, [band_ty, D/2) with x; pos_stride 1 (1-D
  // positions, band_t = D/2) or 3 ((t, y, x) per token)
  int32_t band_t, band_ty, pos_stride;
  float margin;
};

struct LayerPtrs {
  uint8_t* codes_k;
  uint8_t* codes_v;
  float* scale_k;
  float* scale_v;
  int32_t* slot_pos;
  int32_t* slot_yx;  // [2][n_pad] spatial coordinates (y, then x) of each slot (3-D RoPE)
  int32_t* state;  // {head, n_valid, top ticket counter, g_valid}, sub-counters at kTicketStride * (1 + j)
  uint32_t* vmax;  // [H][kSub] largest value scale written since the reset (fp32
                   // bits); the head's bound is the max over its kSub entries
  uint16_t* normw; // bf16 [2][D]: RMS-norm weights of the queries, then of the keys
  float* stat;     // [2][H] static per-head scales (keys, then values), then an int
                   // flag at [2H]: nonzero once calibrated (the pages' scale mode)
};

__host__ __device__ inline LayerPtrs layer_ptrs(const Geom& g, int layer) {
  uint8_t* b = g.base + g.layer0 + (size_t)layer * g.layer_bytes;
  LayerPtrs p;
  p.codes_k = b + g.off_codes_k;
  p.codes_v = b + g.off_codes_v;
  p.scale_k = reinterpret_cast<float*>(b + g.off_scale_k);
  p.scale_v = reinterpret_cast<float*>(b + g.off_scale_v);
  p.slot_pos = reinterpret_cast<int32_t*>(b + g.off_slot_pos);
  p.slot_yx = reinterpret_cast<int32_t*>(b + g.off_slot_yx);
  p.state = reinterpret_cast<int32_t*>(b + g.off_state);
  p.vmax = reinterpret_cast<uint32_t*>(b + g.off_vmax);
  p.normw = reinterpret_cast<uint16_t*>(b + g.off_normw);
  p.stat = reinterpret_cast<float*>(b + g.off_static);
  return p;
}

// True when head h of a layer is in the pages' static-scale mode with
// nonzero key and value scales: the calibration has requantized its valid
// cache, so every valid slot carries the head's scales (a head calibrated at
// amax 0 keeps the per-(token, head) rule).
__device__ inline bool static_head(const LayerPtrs& L, int n_heads, int h) {
  return reinterpret_cast<const int*>(L.stat)[2 * n_heads] != 0 && L.stat[h] > 0.f && L.stat[n_heads + h] > 0.f;
}

// Whether a slot is read by the attention: a ring slot of the valid cyclic
// range [head - n_valid, head), or a global slot below g_valid.  a = the
// oldest valid ring slot, (head - n_valid) mod N.
__device__ inline bool slot_valid(const Geom& g, int slot, int a, int nv, int gv) {
  if (slot >= g.n_ring_pad) return slot - g.n_ring_pad < gv;
  int rel = slot - a;
  if (rel < 0) rel += g.n_slots;
  return slot < g.n_slots && rel < nv;
}

// The position coordinate that turns RoPE pair j: t, y or x of a token whose
// positions start at p (pos_stride ints per token).
__device__ inline int32_t pair_coord(const Geom& g, const int32_t* p, int j) {
  if (g.pos_stride == 1) return p[0];
  return p[j < g.band_t ? 0 : (j < g.band_ty ? 1 : 2)];
}

__device__ inline const double* omega_turns(const Geom& g) {
  return reinterpret_cast<const double*>(g.base + g.consts);
}

// ---- scalar conversions -------------------------------------------------

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ inline uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp32(x / 448), correctly rounded, for x >= 0: the product with the
// rounded reciprocal, corrected once by its exact residual.  An exhaustive
// comparison with the division over every normal fp32 x gives identical
// results wherever the quotient is a normal number; below that (x < 2^-117)
// the division itself is taken, on a branch that is skipped unless a lane
// needs it.
__device__ inline float div448(float x) {
  constexpr float c = 1.f / kE4M3Max;
  const float q0 = x * c;
  float q = fmaf(fmaf(-q0, kE4M3Max, x), c, q0);
  if (__builtin_expect(x < 0x1p-117f, 0)) q = x / kE4M3Max;
  return q;
}

// 1/s for a scale s (0 for s = 0: an all-zero row quantizes to zero codes).
// One hardware reciprocal (within 1 ulp).  Scales below the fp32 normal
// range (amax * margin < 448 * 2^-126, about 5e-36) are outside the
// supported input range and quantize to zero codes.
__device__ inline float recip_scale(float s) { return s >= 0x1p-126f ? __builtin_amdgcn_rcpf(s) : 0.f; }

// Per-row constants of the exact quotient code e4m3(y / s) for bf16 values y
// with s = fp32(am / 448), am = fp32(amax * margin) holding a bf16 amax times
// a margin whose product is exact (1.0, 1.5).
//   y / s = R / (1 + delta), with R = 448 y / am and s = (am / 448)(1 + delta).
//   With 8-bit significands in y and amax, R is either an e4m3 midpoint
//   exactly or at least 1/(mantissa(am) * 31) >= 1.2e-4 (relative) from every
//   midpoint (midpoints have at most 5 significant bits).  So the code of
//   y / s is the code of R unless R is a midpoint, and then the sign of delta,
//   one value per row, decides: delta > 0 puts y / s below the midpoint in
//   magnitude, delta < 0 above, delta = 0 (s exact) leaves an exact tie that
//   goes to the even code.
//   Per element: q = y / s rounded to fp32 within about an ulp (the product
//   with 1/s plus one Newton correction, exact when y / s is representable),
//   then scaled by f = 1 -/+ 2^-20 when delta is positive/negative: far more
//   than q's error or |delta| (<= 2^-24), far less than the 1.2e-4 gap, so
//   every near-midpoint quotient lands on the side delta says and no other
//   code changes.  The hardware RNE conversion of the clamped result is the
//   code.  Checked on the host against an exact reference for every bf16
//   amax of one binade and every bf16 y with |y| <= amax, margins 1 and 1.5,
//   with the reciprocal exact or one ulp off either way.
struct VQuot {
  float s, r, f;
};
__device__ inline VQuot vquot_row(float am, float s) {
  VQuot c;
  c.s = s;
  c.r = recip_scale(s);
  const float e = fmaf(s, kE4M3Max, -am);  // the sign of delta, exactly
  c.f = e > 0.f ? 1.f - 0x1p-20f : (e < 0.f ? 1.f + 0x1p-20f : 1.f);
  return c;
}
__device__ inline float quant_v(float y, const VQuot& c) {
  const float q0 = y * c.r;
  return __builtin_amdgcn_fmed3f(fmaf(fmaf(-q0, c.s, y), c.r, q0) * c.f, -kE4M3Max, kE4M3Max);
}

// Two fp32 values -> two e4m3fn codes (round to nearest even) placed in the
// low (HI=false) or high 16 bits of `old`.  Inputs must already lie in
// [-448, 448]: the conversion is never asked to saturate.
template <bool HI>
__device__ inline uint32_t pack2_fp8(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// As pack2_fp8, of a / s and b / s (the conversion divides by its scale
// operand; for a power of two s the quotient is exact).
template <bool HI>
__device__ inline uint32_t pack2_fp8_div(float a, float b, uint32_t old, float s) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, old), a, b, s, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// Four e4m3fn codes of one dword -> four floats.
__device__ inline void unpack4_fp8(uint32_t w, float& a, float& b, float& c, float& d) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  a = lo[0];
  b = lo[1];
  c = hi[0];
  d = hi[1];
}

// RoPE angle of pair j at integer position p: theta = p * omega_j.  The
// angle reaches 3e4 rad at the pages' positions, where an fp32 product would
// be off by ~1e-3 rad, so it is formed and reduced in double precision as
// turns (t = p * omega_j / 2 pi, minus the nearest integer); the hardware
// sine and cosine take the reduced turns directly (max abs error ~1.2e-7 on
// [-0.5, 0.5], measured against double precision).
__device__ inline void rope_cs(int32_t p, double turns, float& c, float& s) {
  double t = (double)p * turns;
  t -= rint(t);
  const float r = (float)t;
  s = __builtin_amdgcn_sinf(r);
  c = __builtin_amdgcn_cosf(r);
}

// e4m3 input for a value already computed in fp32 arithmetic (RoPE'd or
// rotated keys): y * (1/s), clamped to the e4m3 range in one instruction.
__device__ inline float quant_mul(float y, float r) {
  return __builtin_amdgcn_fmed3f(y * r, -kE4M3Max, kE4M3Max);
}

// DPP move of a float (every lane reads a lane of its own 16-lane row).
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Max over each aligned group of W lanes (W = 2 .. 64), with DPP steps inside
// 16-lane rows (rotate by 8, mirror within 8, swap within 4 and 2) and lane
// swaps across rows (permlane16/32 swap): no LDS round trips.
// Sum over each aligned group of W lanes (W = 2 .. 16), with the same DPP
// steps as group_max; every lane of the group gets the total.
template <int W>
__device__ inline float group_sum(float v) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16, "group width");
  if constexpr (W >= 16) v += dpp_f<0x128>(v);  // row_ror:8
  if constexpr (W >= 8) v += dpp_f<0x141>(v);   // row_half_mirror
  if constexpr (W >= 4) v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0xB1>(v);                          // quad_perm [1,0,3,2]
  return v;
}

// RMS normalization of one row held by a group of lanes (the fused
// pre-attention norm): x * w / sqrt(mean(x^2) + eps), squares summed in fp32.
// ss is this lane's sum of squares; the group's total is over the D
// elements of the row.  The factor is the hardware reciprocal square root
// (within about 1 ulp).
template <int W>
__device__ inline float rms_factor(float ss, float inv_d, float eps) {
  return __builtin_amdgcn_rsqf(group_sum<W>(ss) * inv_d + eps);
}

template <int W>
__device__ inline float group_max(float v) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "group width");
  if constexpr (W >= 16) v = fmaxf(v, dpp_f<0x128>(v));  // row_ror:8
  if constexpr (W >= 8) v = fmaxf(v, dpp_f<0x141>(v));   // row_half_mirror
  if constexpr (W >= 4) v = fmaxf(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0xB1>(v));                          // quad_perm [1,0,3,2]
  if constexpr (W >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    v = fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
  }
  if constexpr (W >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    v = fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
  }
  return v;
}

}  // namespace rkv
