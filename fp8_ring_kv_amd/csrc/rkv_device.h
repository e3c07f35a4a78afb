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
constexpr int kStateInts = 4;  // head, n_valid, write ticket counter, 0

// Byte offsets of one layer's arrays (relative to the layer's start) and the
// sizes every kernel needs.  Passed by value as a kernel argument.
struct Geom {
  uint8_t* base;        // cache buffer
  size_t consts;        // offset of the constants block (double omega/(2 pi) table)
  size_t layer0;        // offset of layer 0
  size_t layer_bytes;   // stride between layers
  size_t off_codes_k, off_codes_v, off_scale_k, off_scale_v, off_slot_pos, off_state, off_vmax;
  int32_t n_layers, n_slots, n_pad, n_tiles, n_heads, head_dim;
  float margin;
};

struct LayerPtrs {
  uint8_t* codes_k;
  uint8_t* codes_v;
  float* scale_k;
  float* scale_v;
  int32_t* slot_pos;
  int32_t* state;  // {head, n_valid, write ticket counter, 0}
  uint32_t* vmax;  // [H][kSub] largest value scale written since the reset (fp32
                   // bits); the head's bound is the max over its kSub entries
};

__host__ __device__ inline LayerPtrs layer_ptrs(const Geom& g, int layer) {
  uint8_t* b = g.base + g.layer0 + (size_t)layer * g.layer_bytes;
  LayerPtrs p;
  p.codes_k = b + g.off_codes_k;
  p.codes_v = b + g.off_codes_v;
  p.scale_k = reinterpret_cast<float*>(b + g.off_scale_k);
  p.scale_v = reinterpret_cast<float*>(b + g.off_scale_v);
  p.slot_pos = reinterpret_cast<int32_t*>(b + g.off_slot_pos);
  p.state = reinterpret_cast<int32_t*>(b + g.off_state);
  p.vmax = reinterpret_cast<uint32_t*>(b + g.off_vmax);
  return p;
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

__device__ inline float clamp448(float x) { return fminf(fmaxf(x, -kE4M3Max), kE4M3Max); }

// e4m3(y / s) exactly as rounding the true quotient would give it, returned
// as an fp32 value the hardware RNE conversion maps to the right code.
// q = RN(y / s) (y * r with one Newton correction, r = 1/s).  The e4m3 grid
// and its midpoints are fp32 values, so RNE(q) equals RNE(y / s) unless q sits
// exactly on a midpoint while y / s does not (y / s within half an fp32 ulp of
// it -- frequent with bf16 inputs, whose quotients by the rounded scale land
// next to midpoints).  Then the sign of the exact residual y - q s (one fma)
// says which side y / s is on, and q moves one fp32 ulp that way.
__device__ inline float quant_div(float y, float s, float r) {
  float q = y * r;
  q = fmaf(fmaf(-q, s, y), r, q);
  const float res = fmaf(-q, s, y);
  const uint32_t b = __float_as_uint(q);
  const uint32_t a = b & 0x7FFFFFFFu;
  // midpoint test: normal e4m3 range (|q| >= 2^-6): the 20 fp32 mantissa bits
  // below the 3 e4m3 ones are 1000...0; subnormal range: 1024 |q| is odd.
  // Evaluated without short-circuits so that it compiles to selects.
  const float t = __uint_as_float(a) * 1024.f;
  const bool normal = a >= 0x3C800000u;
  const bool mid_n = (a & 0xFFFFFu) == 0x80000u;
  const bool mid_s = (t == rintf(t)) & ((((int)t) & 1) != 0);
  const bool adj = (normal ? mid_n : mid_s) & (res != 0.f);
  const uint32_t step = ((res > 0.f) == (q > 0.f)) ? 1u : 0xFFFFFFFFu;
  q = __uint_as_float(b + (adj ? step : 0u));
  return clamp448(q);
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
