// FP8 attention over the ring cache for gfx950.
//
// Runway Characters paper: every call attends its new queries over all
// slots of its cache, after the chunk was written (§2 "The step budget",
// Appendix G); queries get RoPE at their own positions and cached keys are
// used as stored (§4.2); the cache is e4m3 with per-head descales and only
// the queries are quantized per call (§4.3).
//
// Three launches per call:
//   q_prep  -- RoPE on Q at q_pos (double-precision angles), Q split into
//              one or two e4m3 terms with power-of-two scales (the scale
//              goes into the matrix instruction's E8M0 operand, exactly);
//              one extra workgroup per head computes the probability scale
//              c_h = 448 / max s_v over the valid slots.
//   attend  -- split-KV flash attention.  Work unit = (head, 32-query block,
//              KV split); its 4 waves take interleaved 64-slot tiles.  Per
//              tile a wave computes S^T = K Q^T with
//              v_mfma_scale_f32_32x32x64_f8f6f4 (rows = slots, columns =
//              queries, so one lane owns one query row and the row max/sum
//              are in-lane plus one swap with lane+32), applies the per-slot
//              key scale, updates an online softmax in fp32 (exp2 domain),
//              turns P * s_v * c_h into one or two e4m3 terms and
//              accumulates O^T += V^T P^T with the same instruction.  The 4
//              waves merge in LDS.
//   combine -- merges the KV splits and writes bf16 (skipped when 1 split).
//
// Ring addressing: the valid slots are the cyclic range [head - n_valid,
// head).  Tiles are visited in cyclic order from the tile holding the
// oldest valid slot; a tile's slot mask comes from one ballot, fully valid
// tiles skip masking.
#include "rkv_launch.h"

namespace rkv {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Q prep: 16 query rows x one head per workgroup; thread (tau, lane) owns 8
// elements of row tau.  The extra workgroup column (blockIdx.x == nblk)
// computes c_h for head blockIdx.y.

// Smallest e with amax <= 448 * 2^e (amax > 0): amax = f * 2^ex, f in [0.5, 1),
// and 448 = 0.875 * 2^9.
__device__ inline int pow2_exponent(float amax) {
  int ex;
  const float f = frexpf(amax, &ex);
  const int e = ex - 9 + (f > 0.875f ? 1 : 0);
  return e < -127 ? -127 : e;  // E8M0 holds 2^-127 .. 2^127
}

template <int D>
__global__ __launch_bounds__(16 * (D / 8)) void q_prep_kernel(Geom g, AttnWs ws, int layer,
                                                             const uint4* __restrict__ q,
                                                             const int32_t* __restrict__ q_pos,
                                                             int n_q, int nblk) {
  constexpr int LPR = D / 8;
  const int h = blockIdx.y;
  const int H = g.n_heads;
  if ((int)blockIdx.x == nblk) {
    // probability scale for this head: c_h = 448 / max over valid slots of s_v
    const LayerPtrs L = layer_ptrs(g, layer);
    const int N = g.n_slots;
    const int head = L.state[0], nv = L.state[1];
    int a = head - nv;
    if (a < 0) a += N;
    float mx = 0.f;
    for (int k = threadIdx.x; k < nv; k += blockDim.x) {
      int sl = a + k;
      if (sl >= N) sl -= N;
      mx = fmaxf(mx, L.scale_v[(size_t)h * g.n_pad + sl]);
    }
    __shared__ float red[256];
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int o = blockDim.x / 2; o > 0; o >>= 1) {
      if ((int)threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
      __syncthreads();
    }
    if (threadIdx.x == 0) ws.head_c[h] = red[0] > 0.f ? kE4M3Max / red[0] : 1.f;
    return;
  }

  const int tau = threadIdx.x / LPR, lane = threadIdx.x % LPR;
  const int iq = 16 * blockIdx.x + tau;
  const bool active = iq < n_q;
  uint4 w = make_uint4(0u, 0u, 0u, 0u);
  int32_t p = 0;
  if (active) {
    w = q[((size_t)iq * H + h) * LPR + lane];
    p = q_pos[iq];
  }
  const float x[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                      bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
  const double* turns = omega_turns(g);
  float y[8];
  float am = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float c = 1.f, s = 0.f;
    if (active) rope_cs(p, turns[4 * lane + m], c, s);
    y[2 * m] = x[2 * m] * c - x[2 * m + 1] * s;
    y[2 * m + 1] = x[2 * m] * s + x[2 * m + 1] * c;
    am = fmaxf(am, fmaxf(fabsf(y[2 * m]), fabsf(y[2 * m + 1])));
  }
  const size_t row = (size_t)h * ws.nq_pad + iq;
  const size_t term_codes = (size_t)H * ws.nq_pad * D;
  const size_t term_scales = (size_t)H * ws.nq_pad;
  for (int t = 0; t < ws.terms; ++t) {
    am = group_max<LPR>(am);
    const int e = am > 0.f ? pow2_exponent(am) : 0;
    uint2 c;
    c.x = pack2_fp8<false>(clamp448(ldexpf(y[0], -e)), clamp448(ldexpf(y[1], -e)), 0u);
    c.x = pack2_fp8<true>(clamp448(ldexpf(y[2], -e)), clamp448(ldexpf(y[3], -e)), c.x);
    c.y = pack2_fp8<false>(clamp448(ldexpf(y[4], -e)), clamp448(ldexpf(y[5], -e)), 0u);
    c.y = pack2_fp8<true>(clamp448(ldexpf(y[6], -e)), clamp448(ldexpf(y[7], -e)), c.y);
    *reinterpret_cast<uint2*>(ws.qcodes + t * term_codes + row * D + 8 * lane) = c;
    if (lane == 0) ws.qscale[t * term_scales + row] = (uint8_t)(127 + e);
    // residual for the next term (exact: each term is within a factor 2 of y)
    float d[8];
    unpack4_fp8(c.x, d[0], d[1], d[2], d[3]);
    unpack4_fp8(c.y, d[4], d[5], d[6], d[7]);
    am = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      y[k] -= ldexpf(d[k], e);
      am = fmaxf(am, fabsf(y[k]));
    }
  }
}

// ---------------------------------------------------------------------------
// Attention main kernel.

struct AttnArgs {
  Geom g;
  AttnWs ws;
  int layer;
  int n_q;
  int nqb;  // 32-query blocks
  uint16_t* out;
  float kscale;  // log2(e) / sqrt(D)
};

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

template <int D, int TERMS>
__global__ __launch_bounds__(256, 2) void attend_kernel(AttnArgs A) {
  constexpr int KS = D / 64;  // 64-wide steps along head_dim
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  __shared__ float sO[4][32][D + 1];
  __shared__ float sM[4][32], sL[4][32];

  const Geom& g = A.g;
  const int H = g.n_heads, N = g.n_slots, NP = g.n_pad, NT = g.n_tiles;
  const int unit = blockIdx.x;
  const int qb = unit % A.nqb;
  const int hs = unit / A.nqb;
  const int h = hs % H;
  const int split = hs / H;
  const int S = A.ws.splits;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 31, gq = lane >> 5;

  const LayerPtrs L = layer_ptrs(g, A.layer);
  const int head = L.state[0], nv = L.state[1];
  int a = head - nv;
  if (a < 0) a += N;
  const int T0 = a / kTile;  // tile of the oldest valid slot
  int count = 0;               // tiles holding valid slots, in cyclic order from T0
  if (nv > 0) {
    const int e = a + nv - 1;
    count = e < N ? e / kTile - T0 + 1 : (NT - T0) + (e - N) / kTile + 1;
    if (count > NT) count = NT;
  }
  const int k_lo = (int)((long long)split * count / S);
  const int k_hi = (int)((long long)(split + 1) * count / S);

  // Q^T fragments (B operand): lane (li, gq) holds bytes [64 ks + 32 gq, +32) of query row li.
  const int iq = 32 * qb + li;
  const size_t qrow = (size_t)h * A.ws.nq_pad + iq;
  const size_t term_codes = (size_t)H * A.ws.nq_pad * D;
  const size_t term_scales = (size_t)H * A.ws.nq_pad;
  v8i qf[TERMS][KS];
  int qs[TERMS];
#pragma unroll
  for (int t = 0; t < TERMS; ++t) {
    const uint8_t* qp = A.ws.qcodes + t * term_codes + qrow * D + 32 * gq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[t][ks] = load32(qp + 64 * ks, qp + 64 * ks + 16);
    qs[t] = A.ws.qscale[t * term_scales + qrow];
  }
  const float ch = A.ws.head_c[h];

  // K row held by A-operand lane li: slot pi(li) of each 32-slot half, so that
  // accumulator register r of lane group gq is slot 16 gq + r.
  const int krow = 16 * ((li >> 2) & 1) + 4 * (li >> 3) + (li & 3);

  float m = -INFINITY, l = 0.f;
  v16f O[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) O[b] = v16f{};

  const uint8_t* kbase = L.codes_k + (size_t)h * NP * D;
  const uint8_t* vbase = L.codes_v + (size_t)h * NT * D * kTile;
  const float* skb = L.scale_k + (size_t)h * NP;
  const float* svb = L.scale_v + (size_t)h * NP;

  for (int kk = k_lo + wave; kk < k_hi; kk += 4) {
    int T = T0 + kk;
    if (T >= NT) T -= NT;
    const int s0 = T * kTile;
    // slot validity (lane = slot within the tile)
    const int sl = s0 + lane;
    int rel = sl - a;
    if (rel < 0) rel += N;
    const unsigned long long mask = __ballot(sl < N && rel < nv);
    if (mask == 0ull) continue;

    // S^T = K Q^T for the two 32-slot halves
    v16f acc[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const uint8_t* kp = kbase + (size_t)(s0 + 32 * sub + krow) * D + 32 * gq;
      acc[sub] = v16f{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const v8i kf = load32(kp + 64 * ks, kp + 64 * ks + 16);
#pragma unroll
        for (int t = 0; t < TERMS; ++t) acc[sub] = mfma_fp8(kf, qf[t][ks], acc[sub], 127, qs[t]);
      }
    }
    // per-slot constants: lane holds slot 16*(lane/32) + lane%16 of each half
    float tk[2], sv[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int cs = s0 + 32 * sub + 16 * gq + (lane & 15);
      tk[sub] = skb[cs] * A.kscale;
      sv[sub] = svb[cs] * ch;
    }
    float y[2][16];
    const bool full = mask == ~0ull;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = acc[sub][r] * bcast16(tk[sub], r);
        if (!full && !((mask >> (32 * sub + 16 * gq + r)) & 1ull)) v = -INFINITY;
        y[sub][r] = v;
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, y[sub][r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mnew = fmaxf(m, tmax);
    if (__ballot(mnew > m) != 0ull) {
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      l *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) O[b] *= alpha;
      m = mnew;
    }
    // probabilities -> one or two e4m3 terms, B operand of O^T += V^T P^T
    v8i ph, pl;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int sub = w >> 2, r0 = 4 * (w & 3);
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = __builtin_amdgcn_exp2f(y[sub][r0 + e] - m);
        l += p;
        x[e] = fminf(p * bcast16(sv[sub], r0 + e), kE4M3Max);
      }
      uint32_t hw = pack2_fp8<false>(x[0], x[1], 0u);
      hw = pack2_fp8<true>(x[2], x[3], hw);
      ph[w] = (int)hw;
      if (TERMS == 2) {
        float d0, d1, d2, d3;
        unpack4_fp8(hw, d0, d1, d2, d3);
        uint32_t lw = pack2_fp8<false>((x[0] - d0) * 16.f, (x[1] - d1) * 16.f, 0u);
        lw = pack2_fp8<true>((x[2] - d2) * 16.f, (x[3] - d3) * 16.f, lw);
        pl[w] = (int)lw;
      }
    }
    // O^T += V^T P^T: lane (li, gq) holds row d = 32 b + li of the V tile,
    // bytes [16 gq, +16) and [32 + 16 gq, +16) -- the slots of P^T's lane group gq.
    const uint8_t* vt = vbase + (size_t)T * D * kTile;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const uint8_t* vp = vt + (size_t)(32 * b + li) * kTile + 16 * gq;
      const v8i vf = load32(vp, vp + 32);
      O[b] = mfma_fp8(vf, ph, O[b], 127, 127);
      if (TERMS == 2) O[b] = mfma_fp8(vf, pl, O[b], 127, 127 - 4);
    }
  }

  // merge the 4 waves
  l += __shfl_xor(l, 32);
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) sO[wave][li][32 * b + 8 * (r >> 2) + 4 * gq + (r & 3)] = O[b][r];
  if (gq == 0) {
    sM[wave][li] = m;
    sL[wave][li] = l;
  }
  __syncthreads();

  const int row = threadIdx.x >> 3, part = threadIdx.x & 7;
  constexpr int CPT = D / 8;  // contiguous columns per thread
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, sM[w][row]);
  float wt[4];
  float Ls = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wt[w] = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sM[w][row] - M);
    Ls += wt[w] * sL[w][row];
  }
  float o[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int d = part * CPT + c;
    o[c] = wt[0] * sO[0][row][d] + wt[1] * sO[1][row][d] + wt[2] * sO[2][row][d] + wt[3] * sO[3][row][d];
  }
  const int qi = 32 * qb + row;
  if (S == 1) {
    if (qi < A.n_q) {
      const float inv = Ls > 0.f ? 1.f / (ch * Ls) : 0.f;
      uint32_t pk[CPT / 2];
#pragma unroll
      for (int c = 0; c < CPT / 2; ++c)
        pk[c] = f32_to_bf16_rne(o[2 * c] * inv) | (f32_to_bf16_rne(o[2 * c + 1] * inv) << 16);
      uint4* dst = reinterpret_cast<uint4*>(A.out + ((size_t)qi * H + h) * D + part * CPT);
#pragma unroll
      for (int c = 0; c < CPT / 8; ++c) dst[c] = make_uint4(pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]);
    }
  } else {
    float4* dst = reinterpret_cast<float4*>(A.ws.part_o + ((size_t)unit * 32 + row) * D + part * CPT);
#pragma unroll
    for (int c = 0; c < CPT / 4; ++c) dst[c] = make_float4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
    if (part == 0) {
      A.ws.part_ml[((size_t)unit * 32 + row) * 2] = M;
      A.ws.part_ml[((size_t)unit * 32 + row) * 2 + 1] = Ls;
    }
  }
}

// ---------------------------------------------------------------------------
// Split combine: one workgroup per (head, 32-query block), 8 threads per row.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs A) {
  const int H = A.g.n_heads;
  const int qb = blockIdx.x % A.nqb, h = blockIdx.x / A.nqb;
  const int S = A.ws.splits;
  const int row = threadIdx.x >> 3, part = threadIdx.x & 7;
  constexpr int CPT = D / 8;
  const int qi = 32 * qb + row;
  if (qi >= A.n_q) return;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) {
    const size_t u = ((size_t)s * H + h) * A.nqb + qb;
    M = fmaxf(M, A.ws.part_ml[(u * 32 + row) * 2]);
  }
  float o[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) o[c] = 0.f;
  float Ls = 0.f;
  for (int s = 0; s < S; ++s) {
    const size_t u = ((size_t)s * H + h) * A.nqb + qb;
    const float ms = A.ws.part_ml[(u * 32 + row) * 2];
    const float w = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    Ls += w * A.ws.part_ml[(u * 32 + row) * 2 + 1];
    const float4* src = reinterpret_cast<const float4*>(A.ws.part_o + (u * 32 + row) * D + part * CPT);
#pragma unroll
    for (int c = 0; c < CPT / 4; ++c) {
      const float4 v = src[c];
      o[4 * c] += w * v.x;
      o[4 * c + 1] += w * v.y;
      o[4 * c + 2] += w * v.z;
      o[4 * c + 3] += w * v.w;
    }
  }
  const float inv = Ls > 0.f ? 1.f / (A.ws.head_c[h] * Ls) : 0.f;
  uint32_t pk[CPT / 2];
#pragma unroll
  for (int c = 0; c < CPT / 2; ++c)
    pk[c] = f32_to_bf16_rne(o[2 * c] * inv) | (f32_to_bf16_rne(o[2 * c + 1] * inv) << 16);
  uint4* dst = reinterpret_cast<uint4*>(A.out + ((size_t)qi * H + h) * D + part * CPT);
#pragma unroll
  for (int c = 0; c < CPT / 8; ++c) dst[c] = make_uint4(pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]);
}

hipError_t launch_attend(const Geom& g, const AttnWs& ws, int layer, const void* q,
                         const int32_t* q_pos, int n_q, void* out, hipStream_t s) {
  const int D = g.head_dim;
  const int nqb = (n_q + 31) / 32;
  const int nblk = 2 * nqb;  // 16-row q_prep blocks covering 32 * nqb rows
  dim3 pgrid(nblk + 1, g.n_heads);
  if (D == 128)
    hipLaunchKernelGGL(q_prep_kernel<128>, pgrid, dim3(256), 0, s, g, ws, layer, (const uint4*)q, q_pos, n_q, nblk);
  else
    hipLaunchKernelGGL(q_prep_kernel<64>, pgrid, dim3(128), 0, s, g, ws, layer, (const uint4*)q, q_pos, n_q, nblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  AttnArgs A;
  A.g = g;
  A.ws = ws;
  A.layer = layer;
  A.n_q = n_q;
  A.nqb = nqb;
  A.out = (uint16_t*)out;
  A.kscale = kLog2e / sqrtf((float)D);
  dim3 agrid(nqb * g.n_heads * ws.splits);
  if (D == 128) {
    if (ws.terms == 2) hipLaunchKernelGGL((attend_kernel<128, 2>), agrid, dim3(256), 0, s, A);
    else hipLaunchKernelGGL((attend_kernel<128, 1>), agrid, dim3(256), 0, s, A);
  } else {
    if (ws.terms == 2) hipLaunchKernelGGL((attend_kernel<64, 2>), agrid, dim3(256), 0, s, A);
    else hipLaunchKernelGGL((attend_kernel<64, 1>), agrid, dim3(256), 0, s, A);
  }
  e = hipGetLastError();
  if (e != hipSuccess || ws.splits == 1) return e;
  dim3 cgrid(nqb * g.n_heads);
  if (D == 128) hipLaunchKernelGGL(combine_kernel<128>, cgrid, dim3(256), 0, s, A);
  else hipLaunchKernelGGL(combine_kernel<64>, cgrid, dim3(256), 0, s, A);
  return hipGetLastError();
}

}  // namespace rkv
