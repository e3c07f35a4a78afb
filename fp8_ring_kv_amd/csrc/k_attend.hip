// FP8 attention over the ring cache for gfx950, one launch per call.
//
// Runway Characters paper: every call attends its new queries over all
// slots of its cache, after the chunk was written (§2 "The step budget",
// Appendix G); queries get RoPE at their own positions and cached keys are
// used as stored (§4.2); the cache is e4m3 with per-head descales and only
// the queries are quantized per call (§4.3).
//
// Work: unit u = (head h, block qb of 32 queries), u = h * nqb + qb; each
// unit needs `count` 64-slot tiles (the tiles holding valid slots, in cyclic
// order from the tile of the oldest valid slot).  A persistent grid of G
// workgroups (one per compute unit) cuts the unit-major list of all
// units * count (unit, tile) pairs into G equal contiguous ranges, so every
// workgroup gets the same matrix work to within one tile.  Workgroups are
// dealt to the 8 XCDs round-robin; ranges are assigned so that each XCD
// takes a contiguous block of them (a few heads), keeping their K/V in its L2.
//
// A workgroup handles each unit its range meets as one segment:
//   1. RoPE on the unit's 32 queries (angles in double precision) and their
//      split into one or two e4m3 terms with power-of-two scales (applied
//      exactly by the E8M0 scale operand of the matrix instruction), staged
//      in LDS;
//   2. its 4 waves take interleaved tiles of the segment.  Per tile a wave
//      computes S^T = K Q^T with v_mfma_scale_f32_32x32x64_f8f6f4 (rows =
//      slots, columns = queries: one lane owns one query, so the row max and
//      sum are in-lane plus one swap with lane ^ 32), applies the per-slot
//      key scale, updates an online softmax in fp32 (exp2 domain), turns
//      P * s_v * c_h into one or two e4m3 terms and accumulates
//      O^T += V^T P^T with the same instruction.  The loop is software
//      pipelined: the next tile's Q K^T products are issued before this
//      tile's softmax, so the matrix cores and the vector ALUs overlap;
//   3. the 4 waves merge in LDS;
//   4. a whole unit writes its bf16 output; a unit split between
//      workgroups writes a partial (O, max, sum) and the last workgroup to
//      finish its part merges the partials and writes the output.
//
// Probability scale: c_h = 448 / (4 vmax_h), vmax_h being the largest value
// scale written to head h since the reset (kept by the write kernel).  The
// running row maximum is raised only when a tile exceeds it by more than 2
// (log2 units), so P <= 4 and P * s_v * c_h <= 448 always fits e4m3.
#include "rkv_launch.h"

namespace rkv {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 2.f;  // log2 headroom of the running maximum

struct AttnArgs {
  Geom g;
  AttnWs ws;
  int layer;
  int n_q;
  int nqb;  // 32-query blocks
  const uint4* q;
  const int32_t* q_pos;
  uint16_t* out;
  float kscale;  // log2(e) / sqrt(D)
};

// Smallest e with amax <= 448 * 2^e (amax > 0): amax = f * 2^ex, f in [0.5, 1),
// and 448 = 0.875 * 2^9.
__device__ inline int pow2_exponent(float amax) {
  int ex;
  const float f = frexpf(amax, &ex);
  const int e = ex - 9 + (f > 0.875f ? 1 : 0);
  return e < -127 ? -127 : e;  // E8M0 holds 2^-127 .. 2^127
}

// row_newbcast:r -- every lane of a 16-lane row receives lane r of that row.
// r is a compile-time constant after unrolling; the switch folds away.
__device__ inline float bcast16(float v, int r) {
  int x = __float_as_int(v);
  switch (r) {
    case 0: x = __builtin_amdgcn_update_dpp(0, x, 0x150, 0xF, 0xF, false); break;
    case 1: x = __builtin_amdgcn_update_dpp(0, x, 0x151, 0xF, 0xF, false); break;
    case 2: x = __builtin_amdgcn_update_dpp(0, x, 0x152, 0xF, 0xF, false); break;
    case 3: x = __builtin_amdgcn_update_dpp(0, x, 0x153, 0xF, 0xF, false); break;
    case 4: x = __builtin_amdgcn_update_dpp(0, x, 0x154, 0xF, 0xF, false); break;
    case 5: x = __builtin_amdgcn_update_dpp(0, x, 0x155, 0xF, 0xF, false); break;
    case 6: x = __builtin_amdgcn_update_dpp(0, x, 0x156, 0xF, 0xF, false); break;
    case 7: x = __builtin_amdgcn_update_dpp(0, x, 0x157, 0xF, 0xF, false); break;
    case 8: x = __builtin_amdgcn_update_dpp(0, x, 0x158, 0xF, 0xF, false); break;
    case 9: x = __builtin_amdgcn_update_dpp(0, x, 0x159, 0xF, 0xF, false); break;
    case 10: x = __builtin_amdgcn_update_dpp(0, x, 0x15A, 0xF, 0xF, false); break;
    case 11: x = __builtin_amdgcn_update_dpp(0, x, 0x15B, 0xF, 0xF, false); break;
    case 12: x = __builtin_amdgcn_update_dpp(0, x, 0x15C, 0xF, 0xF, false); break;
    case 13: x = __builtin_amdgcn_update_dpp(0, x, 0x15D, 0xF, 0xF, false); break;
    case 14: x = __builtin_amdgcn_update_dpp(0, x, 0x15E, 0xF, 0xF, false); break;
    case 15: x = __builtin_amdgcn_update_dpp(0, x, 0x15F, 0xF, 0xF, false); break;
  }
  return __int_as_float(x);
}

__device__ inline v8i load32(const uint8_t* p0, const uint8_t* p1) {
  const uint4 a = *reinterpret_cast<const uint4*>(p0);
  const uint4 b = *reinterpret_cast<const uint4*>(p1);
  v8i r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
  return r;
}

__device__ inline v16f mfma_fp8(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// max / sum over the two halves of the wave (lane l and lane l ^ 32)
__device__ inline float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ inline float half_swap_add(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// Per-wave tile operands (lane = li + 32 gq).
//   K operand of S^T = K Q^T: lane li holds slot 32 sub + krow(li), bytes
//   [64 ks + 32 gq, +32).  krow permutes the slots so that accumulator
//   register r of lane group gq is slot 16 gq + r of the 32-slot half.
//   Scales: lane holds slot 32 sub + 16 gq + lane % 16 (broadcast per register
//   with row_newbcast).  V operand of O^T += V^T P^T: lane holds row
//   d = 32 b + li of the transposed V tile, bytes [16 gq, +16) and
//   [32 + 16 gq, +16) -- the slots of P^T's lane group gq.
template <int D>
struct KOp {
  v8i k[2][D / 64];
};
template <int D>
struct VOp {
  v8i v[D / 32];
  float sk[2], sv[2];
};

struct TileSrc {
  const uint8_t* kbase;  // codes_k of the head
  const uint8_t* vbase;  // codes_v of the head
  const float* skb;      // scale_k of the head
  const float* svb;      // scale_v of the head
};

template <int D>
__device__ inline void load_k(KOp<D>& f, const TileSrc& src, int T, int lane) {
  const int li = lane & 31, gq = lane >> 5;
  const int krow = 16 * ((li >> 2) & 1) + 4 * (li >> 3) + (li & 3);
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const uint8_t* kp = src.kbase + (size_t)(T * kTile + 32 * sub + krow) * D + 32 * gq;
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) f.k[sub][ks] = load32(kp + 64 * ks, kp + 64 * ks + 16);
  }
}

template <int D>
__device__ inline void load_v(VOp<D>& f, const TileSrc& src, int T, int lane) {
  const int li = lane & 31, gq = lane >> 5;
  const uint8_t* vt = src.vbase + (size_t)T * D * kTile;
#pragma unroll
  for (int b = 0; b < D / 32; ++b) {
    const uint8_t* vp = vt + (size_t)(32 * b + li) * kTile + 16 * gq;
    f.v[b] = load32(vp, vp + 32);
  }
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int cs = T * kTile + 32 * sub + 16 * gq + (lane & 15);
    f.sk[sub] = src.skb[cs];
    f.sv[sub] = src.svb[cs];
  }
}

template <int D, int TERMS>
__device__ inline void qk(v16f (&acc)[2], const KOp<D>& f, const v8i (&qf)[TERMS][D / 64],
                          const int (&qs)[TERMS]) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    acc[sub] = v16f{};
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
      for (int t = 0; t < TERMS; ++t) acc[sub] = mfma_fp8(f.k[sub][ks], qf[t][ks], acc[sub], 127, qs[t]);
  }
}

template <int D>
struct WaveState {
  float m, l;  // running max (log2 units), running sum of this lane's slots
  v16f O[D / 32];
};

// Softmax of one tile's S^T (in registers) and its P V product.
template <int D, int TERMS>
__device__ inline void softmax_pv(v16f (&acc)[2], const VOp<D>& vf, WaveState<D>& st,
                                  unsigned long long mask, float kscale, float ch, int lane) {
  constexpr int DB = D / 32;
  const int gq = lane >> 5;
  const float tk0 = vf.sk[0] * kscale, tk1 = vf.sk[1] * kscale;
  const float sv0 = vf.sv[0] * ch, sv1 = vf.sv[1] * ch;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    acc[0][r] *= bcast16(tk0, r);
    acc[1][r] *= bcast16(tk1, r);
  }
  if (mask != ~0ull) {  // partially valid tile (ring edge, partial fill, padding)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (!((mask >> (32 * sub + 16 * gq + r)) & 1ull)) acc[sub][r] = -INFINITY;
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, fmaxf(acc[0][r], acc[1][r]));
  tmax = half_swap_max(tmax);
  if (__ballot(tmax > st.m + kLazy) != 0ull) {
    const float mnew = fmaxf(st.m, tmax);
    const float alpha = __builtin_amdgcn_exp2f(st.m - mnew);
    st.l *= alpha;
#pragma unroll
    for (int b = 0; b < DB; ++b) st.O[b] *= alpha;
    st.m = mnew;
  }
  // P <= 4 and s_v c_h <= 112, so the conversions below never overflow
  // (fp32 rounding a hair above 448 still rounds to 448 in e4m3).
  v8i ph, pl;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int sub = w >> 2, r0 = 4 * (w & 3);
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = __builtin_amdgcn_exp2f(acc[sub][r0 + e] - st.m);
      st.l += p;
      x[e] = p * bcast16(sub ? sv1 : sv0, r0 + e);
    }
    uint32_t hw = pack2_fp8<false>(x[0], x[1], 0u);
    hw = pack2_fp8<true>(x[2], x[3], hw);
    ph[w] = (int)hw;
    if (TERMS == 2) {  // second term: 16 (x - e4m3(x)), descaled by 2^-4
      float d0, d1, d2, d3;
      unpack4_fp8(hw, d0, d1, d2, d3);
      uint32_t lw = pack2_fp8<false>((x[0] - d0) * 16.f, (x[1] - d1) * 16.f, 0u);
      lw = pack2_fp8<true>((x[2] - d2) * 16.f, (x[3] - d3) * 16.f, lw);
      pl[w] = (int)lw;
    }
  }
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    st.O[b] = mfma_fp8(vf.v[b], ph, st.O[b], 127, 127);
    if (TERMS == 2) st.O[b] = mfma_fp8(vf.v[b], pl, st.O[b], 127, 127 - 4);
  }
}

template <int D>
struct __attribute__((aligned(16))) AttnSmem {
  uint8_t q[2][32 * (D + 16)];  // staged query codes per term, rows padded by 16 bytes
  int qexp[2][32];
  float merge[4][32 * D + 64];  // per wave: O^T as [d][32 queries], then m[32], l[32]
  int flag;
};

// bf16 output row piece: n = D / 8 columns of one query row
template <int CPT>
__device__ inline void store_out(uint16_t* dst, const float (&o)[CPT], float inv) {
  uint32_t pk[CPT / 2];
#pragma unroll
  for (int c = 0; c < CPT / 2; ++c)
    pk[c] = f32_to_bf16_rne(o[2 * c] * inv) | (f32_to_bf16_rne(o[2 * c + 1] * inv) << 16);
#pragma unroll
  for (int c = 0; c < CPT / 8; ++c)
    reinterpret_cast<uint4*>(dst)[c] = make_uint4(pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]);
}

// ---------------------------------------------------------------------------
template <int D, int TERMS>
__global__ __launch_bounds__(256, 1) void attend_kernel(AttnArgs A) {
  constexpr int KS = D / 64, DB = D / 32;
  constexpr int EPT = D / 8;  // query elements per thread in the Q prep
  constexpr int CPT = D / 8;  // output columns per thread in the merges
  __shared__ AttnSmem<D> sm;

  const Geom& g = A.g;
  const int H = g.n_heads, N = g.n_slots, NP = g.n_pad, NT = g.n_tiles;
  const int G = (int)gridDim.x;
  const int b = (int)blockIdx.x;
  const int gi = G % 8 == 0 ? (b & 7) * (G / 8) + (b >> 3) : b;  // this workgroup's range
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 31, gq = lane >> 5;
  const int qrow = threadIdx.x >> 3, qpart = threadIdx.x & 7;  // Q prep: 8 threads per row
  const int row = threadIdx.x & 31, part = threadIdx.x >> 5;   // merges: 8 column blocks

  const LayerPtrs L = layer_ptrs(g, A.layer);
  const int head = L.state[0], nv = L.state[1];
  int a = head - nv;
  if (a < 0) a += N;
  const int T0 = a / kTile;  // tile of the oldest valid slot
  int count = 0;             // tiles holding valid slots, in cyclic order from T0
  if (nv > 0) {
    const int e = a + nv - 1;
    count = e < N ? e / kTile - T0 + 1 : (NT - T0) + (e - N) / kTile + 1;
    if (count > NT) count = NT;
  }
  const int U = A.nqb * H;

  if (count == 0) {  // empty cache: every output row is zero
    for (int u = gi; u < U; u += G) {
      const int h = u / A.nqb, qi = 32 * (u % A.nqb) + row;
      if (qi < A.n_q) {
        uint4* dst = reinterpret_cast<uint4*>(A.out + ((size_t)qi * H + h) * D + part * CPT);
#pragma unroll
        for (int c = 0; c < CPT / 8; ++c) dst[c] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    return;
  }

  const long long W = (long long)U * count;
  const long long r_lo = (long long)gi * W / G, r_hi = (long long)(gi + 1) * W / G;
  auto tile_of = [&](int kk) { const int T = T0 + kk; return T >= NT ? T - NT : T; };
  auto tile_mask = [&](int T) {
    const int sl = T * kTile + lane;
    int rel = sl - a;
    if (rel < 0) rel += N;
    return __ballot(sl < N && rel < nv);
  };

  for (long long x = r_lo; x < r_hi;) {
    const int u = (int)(x / count);
    const int t_lo = (int)(x - (long long)u * count);
    const long long rem = r_hi - x;
    const int t_hi = rem < count - t_lo ? t_lo + (int)rem : count;
    x += t_hi - t_lo;
    const int h = u / A.nqb, qb = u % A.nqb;
    const float vmaxh = __uint_as_float(L.vmax[h]);
    const float ch = vmaxh > 0.f ? kE4M3Max / (4.f * vmaxh) : 1.f;
    TileSrc src;
    src.kbase = L.codes_k + (size_t)h * NP * D;
    src.vbase = L.codes_v + (size_t)h * NT * D * kTile;
    src.skb = L.scale_k + (size_t)h * NP;
    src.svb = L.scale_v + (size_t)h * NP;

    // ---- 1. queries: RoPE and one or two e4m3 terms, staged in LDS ----
    {
      const int iq = 32 * qb + qrow;
      float y[EPT];
      float am = 0.f;
      if (iq < A.n_q) {
        const uint4* qp = A.q + (((size_t)iq * H + h) * D + qpart * EPT) / 8;
        const int32_t p = A.q_pos[iq];
        const double* turns = omega_turns(g);
#pragma unroll
        for (int c = 0; c < EPT / 8; ++c) {
          const uint4 w = qp[c];
          const float xv[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                               bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            float cs, sn;
            rope_cs(p, turns[qpart * EPT / 2 + 4 * c + m], cs, sn);
            y[8 * c + 2 * m] = xv[2 * m] * cs - xv[2 * m + 1] * sn;
            y[8 * c + 2 * m + 1] = xv[2 * m] * sn + xv[2 * m + 1] * cs;
          }
        }
#pragma unroll
        for (int e = 0; e < EPT; ++e) am = fmaxf(am, fabsf(y[e]));
      } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) y[e] = 0.f;
      }
#pragma unroll
      for (int t = 0; t < TERMS; ++t) {
        am = group_max<8>(am);
        const int e = am > 0.f ? pow2_exponent(am) : 0;
        uint32_t wd[EPT / 4];
#pragma unroll
        for (int c = 0; c < EPT / 4; ++c) {
          const uint32_t w = pack2_fp8<false>(clamp448(ldexpf(y[4 * c], -e)), clamp448(ldexpf(y[4 * c + 1], -e)), 0u);
          wd[c] = pack2_fp8<true>(clamp448(ldexpf(y[4 * c + 2], -e)), clamp448(ldexpf(y[4 * c + 3], -e)), w);
        }
        uint8_t* dst = sm.q[t] + qrow * (D + 16) + qpart * EPT;
        if constexpr (EPT == 16) {
          *reinterpret_cast<uint4*>(dst) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        } else {
          *reinterpret_cast<uint2*>(dst) = make_uint2(wd[0], wd[1]);
        }
        if (qpart == 0) sm.qexp[t][qrow] = e;
        // residual for the next term
        am = 0.f;
#pragma unroll
        for (int c = 0; c < EPT / 4; ++c) {
          float d0, d1, d2, d3;
          unpack4_fp8(wd[c], d0, d1, d2, d3);
          y[4 * c] -= ldexpf(d0, e);
          y[4 * c + 1] -= ldexpf(d1, e);
          y[4 * c + 2] -= ldexpf(d2, e);
          y[4 * c + 3] -= ldexpf(d3, e);
        }
#pragma unroll
        for (int k = 0; k < EPT; ++k) am = fmaxf(am, fabsf(y[k]));
      }
    }
    __syncthreads();
    v8i qf[TERMS][KS];
    int qs[TERMS];
#pragma unroll
    for (int t = 0; t < TERMS; ++t) {
      const uint8_t* qp = sm.q[t] + li * (D + 16) + 32 * gq;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[t][ks] = load32(qp + 64 * ks, qp + 64 * ks + 16);
      qs[t] = 127 + sm.qexp[t][li];
    }

    // ---- 2. this wave's tiles t_lo + wave, +4, ...: software pipelined ----
    WaveState<D> st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int bb = 0; bb < DB; ++bb) st.O[bb] = v16f{};
    const int first = t_lo + wave;
    const int nw = first < t_hi ? (t_hi - first + 3) / 4 : 0;
    if (nw > 0) {
      KOp<D> kf;
      VOp<D> v0, v1;
      v16f s0[2], s1[2];
      load_k<D>(kf, src, tile_of(first), lane);
      load_v<D>(v0, src, tile_of(first), lane);
      qk<D, TERMS>(s0, kf, qf, qs);
      if (nw > 1) load_k<D>(kf, src, tile_of(first + 4), lane);
      for (int j = 0; j < nw; j += 2) {
        // tile j: S in s0, V in v0; K of tile j + 1 in kf
        if (j + 1 < nw) {
          qk<D, TERMS>(s1, kf, qf, qs);
          if (j + 2 < nw) load_k<D>(kf, src, tile_of(first + 4 * (j + 2)), lane);
          load_v<D>(v1, src, tile_of(first + 4 * (j + 1)), lane);
        }
        softmax_pv<D, TERMS>(s0, v0, st, tile_mask(tile_of(first + 4 * j)), A.kscale, ch, lane);
        if (j + 1 >= nw) break;
        // tile j + 1: S in s1, V in v1; K of tile j + 2 in kf
        if (j + 2 < nw) {
          qk<D, TERMS>(s0, kf, qf, qs);
          if (j + 3 < nw) load_k<D>(kf, src, tile_of(first + 4 * (j + 3)), lane);
          load_v<D>(v0, src, tile_of(first + 4 * (j + 2)), lane);
        }
        softmax_pv<D, TERMS>(s1, v1, st, tile_mask(tile_of(first + 4 * (j + 1))), A.kscale, ch, lane);
      }
    }

    // ---- 3. merge the 4 waves in LDS ----
    {
      const float l = half_swap_add(st.l);
      float* sO = sm.merge[wave];
#pragma unroll
      for (int bb = 0; bb < DB; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sO[(32 * bb + 8 * (r >> 2) + 4 * gq + (r & 3)) * 32 + li] = st.O[bb][r];
      if (gq == 0) {
        sO[32 * D + li] = st.m;
        sO[32 * D + 32 + li] = l;
      }
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm.merge[w][32 * D + row]);
    float wt[4], Ls = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wt[w] = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm.merge[w][32 * D + row] - M);
      Ls += wt[w] * sm.merge[w][32 * D + 32 + row];
    }
    float o[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int d = part * CPT + c;
      o[c] = wt[0] * sm.merge[0][d * 32 + row] + wt[1] * sm.merge[1][d * 32 + row] +
             wt[2] * sm.merge[2][d * 32 + row] + wt[3] * sm.merge[3][d * 32 + row];
    }
    const int qi = 32 * qb + row;
    uint16_t* orow = A.out + ((size_t)qi * H + h) * D + part * CPT;

    // ---- 4. whole unit: output; split unit: partial, the last to finish merges ----
    if (t_lo == 0 && t_hi == count) {
      if (qi < A.n_q) store_out<CPT>(orow, o, Ls > 0.f ? 1.f / (ch * Ls) : 0.f);
    } else {
      // Partial id gi + u is distinct for every (workgroup, unit) pair: ranges
      // are ordered, so a later workgroup never meets an earlier unit.
      const size_t seg = (size_t)gi + u;
      float4* po = reinterpret_cast<float4*>(A.ws.part_o + (seg * 32 + row) * D + part * CPT);
#pragma unroll
      for (int c = 0; c < CPT / 4; ++c) po[c] = make_float4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
      if (part == 0) {
        A.ws.part_ml[(seg * 32 + row) * 2] = M;
        A.ws.part_ml[(seg * 32 + row) * 2 + 1] = Ls;
      }
      // release this partial device-wide, then add this segment's tiles to
      // the unit's counter; whoever completes the count merges
      __threadfence();
      __syncthreads();
      if (threadIdx.x == 0) {
        const int prev = atomicAdd(&A.ws.count[u], t_hi - t_lo);
        sm.flag = prev + (t_hi - t_lo) == count;
      }
      __syncthreads();
      if (sm.flag) {
        __threadfence();  // acquire the other segments' partials
        const long long ulo = (long long)u * count, uhi = ulo + count;
        // segments of unit u, in order: the workgroup range holding tile-unit
        // y is floor(((y + 1) G - 1) / W); the next segment starts at its end
        float Mu = -INFINITY;
        for (long long y = ulo; y < uhi;) {
          const long long w = ((y + 1) * G - 1) / W;
          Mu = fmaxf(Mu, A.ws.part_ml[(((size_t)w + u) * 32 + row) * 2]);
          y = (w + 1) * W / G;
        }
        float acc[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
        float Lu = 0.f;
        for (long long y = ulo; y < uhi;) {
          const long long w = ((y + 1) * G - 1) / W;
          const size_t id = ((size_t)w + u) * 32 + row;
          const float sc = __builtin_amdgcn_exp2f(A.ws.part_ml[id * 2] - Mu);
          Lu += sc * A.ws.part_ml[id * 2 + 1];
          const float4* p4 = reinterpret_cast<const float4*>(A.ws.part_o + id * D + part * CPT);
#pragma unroll
          for (int c = 0; c < CPT / 4; ++c) {
            const float4 v4 = p4[c];
            acc[4 * c] += sc * v4.x;
            acc[4 * c + 1] += sc * v4.y;
            acc[4 * c + 2] += sc * v4.z;
            acc[4 * c + 3] += sc * v4.w;
          }
          y = (w + 1) * W / G;
        }
        if (qi < A.n_q) store_out<CPT>(orow, acc, Lu > 0.f ? 1.f / (ch * Lu) : 0.f);
        if (threadIdx.x == 0) A.ws.count[u] = 0;  // ready for the next call
      }
    }
    __syncthreads();  // LDS is reused by the next segment
  }
}

hipError_t launch_attend(const Geom& g, const AttnWs& ws, int layer, const void* q,
                         const int32_t* q_pos, int n_q, void* out, hipStream_t s) {
  const int D = g.head_dim;
  AttnArgs A;
  A.g = g;
  A.ws = ws;
  A.layer = layer;
  A.n_q = n_q;
  A.nqb = (n_q + 31) / 32;
  A.q = (const uint4*)q;
  A.q_pos = q_pos;
  A.out = (uint16_t*)out;
  A.kscale = kLog2e / sqrtf((float)D);
  const dim3 grid(ws.grid);
  if (D == 128) {
    if (ws.terms == 2) hipLaunchKernelGGL((attend_kernel<128, 2>), grid, dim3(256), 0, s, A);
    else hipLaunchKernelGGL((attend_kernel<128, 1>), grid, dim3(256), 0, s, A);
  } else {
    if (ws.terms == 2) hipLaunchKernelGGL((attend_kernel<64, 2>), grid, dim3(256), 0, s, A);
    else hipLaunchKernelGGL((attend_kernel<64, 1>), grid, dim3(256), 0, s, A);
  }
  return hipGetLastError();
}

}  // namespace rkv
