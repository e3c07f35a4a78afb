// Ring-cache kernels for gfx950: buffer clear, session reset, the fused
// RoPE + FP8 write, and the in-place delta rotation.
//
// Runway Characters paper: §4.1 (ring slots, device-side write position,
// each slot keeps its written position), §4.2 and Appendix G (RoPE once at
// write; at a reset every cached key is dequantized, rotated by the position
// change and requantized; values untouched), §4.3 (K and V stored in e4m3,
// only new tokens quantized), §4.4 (the pre-attention chain fused into one
// pass per token).
//
// Both hot kernels are HBM-bound sweeps: every lane moves 16-byte vectors,
// consecutive lanes cover consecutive bytes of a row, and the per-row amax
// is a reduction across the lanes of that row (no LDS round trip except for
// the V transpose).
#include "rkv_launch.h"
#include "write_body.h"

namespace rkv {

// ---------------------------------------------------------------------------
// Buffer clear (create) -- a kernel, not a memset node, so it can sit in a graph.
__global__ void fill_zero_kernel(uint4* p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint4*)p, n16);
  return hipGetLastError();
}

struct TurnsTable {
  double t[kMaxHalfDim];
};

__global__ void init_consts_kernel(Geom g, TurnsTable tab, int n) {
  double* dst = reinterpret_cast<double*>(g.base + g.consts);
  if ((int)threadIdx.x < n) dst[threadIdx.x] = tab.t[threadIdx.x];
}

hipError_t launch_init_consts(const Geom& g, const double* turns, int n, hipStream_t s) {
  TurnsTable tab{};
  for (int j = 0; j < n && j < kMaxHalfDim; ++j) tab.t[j] = turns[j];
  hipLaunchKernelGGL(init_consts_kernel, dim3(1), dim3(64), 0, s, g, tab, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Session reset: head = n_valid = g_valid = 0 and every slot position = 0.
__global__ void reset_kernel(Geom g, int layer_lo) {
  const LayerPtrs L = layer_ptrs(g, layer_lo + (int)blockIdx.y);
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < g.n_pad) {
    L.slot_pos[i] = 0;
    L.slot_yx[i] = 0;
    L.slot_yx[g.n_pad + i] = 0;
  }
  if (blockIdx.x == 0)
    for (int j = (int)threadIdx.x; j < kStateRegionInts; j += (int)blockDim.x) L.state[j] = 0;
  if (blockIdx.x == 0)
    for (int j = (int)threadIdx.x; j < g.n_heads * kSub; j += (int)blockDim.x) L.vmax[j] = 0u;
  // back to per-(token, head) scales until the next calibration
  if (blockIdx.x == 0)
    for (int j = (int)threadIdx.x; j <= 2 * g.n_heads; j += (int)blockDim.x) L.stat[j] = 0.f;
}

hipError_t launch_reset(const Geom& g, int layer_lo, int layer_hi, hipStream_t s) {
  dim3 grid((g.n_pad + 255) / 256, layer_hi - layer_lo);
  hipLaunchKernelGGL(reset_kernel, grid, dim3(256), 0, s, g, layer_lo);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Static-scale calibration, the pages' own scale mode (Appendix G; §4.3 "FP8
// at write"): per (layer, head), amax = the largest magnitude of the
// dequantized keys (values) over the valid slots, s = fp32(margin amax / 448);
// then the head's valid cache is requantized with these scales, the layer's
// flag is set, and later writes quantize with these scales and reset
// rotations requantize each head's keys with its key scale (a head at amax
// 0 gets scale 0, which the write, the rotation and the attention read as
// "keep the per-(token, head) rule").  One workgroup per (head, layer) scans the
// head's codes 16 bytes per thread.  The products code * scale are exact in
// double precision and the scale is formed as margin * amax / 448 in double,
// rounded once to float.
__device__ inline double max16_scaled(uint4 w, const float* sc, bool per_elem, double m) {
  float x[16];
  unpack4_fp8(w.x, x[0], x[1], x[2], x[3]);
  unpack4_fp8(w.y, x[4], x[5], x[6], x[7]);
  unpack4_fp8(w.z, x[8], x[9], x[10], x[11]);
  unpack4_fp8(w.w, x[12], x[13], x[14], x[15]);
#pragma unroll
  for (int e = 0; e < 16; ++e) m = fmax(m, fabs((double)x[e]) * (double)sc[per_elem ? e : 0]);
  return m;
}

__global__ __launch_bounds__(256) void calibrate_kernel(Geom g, int layer_lo, float margin) {
  __shared__ double red[2][256];
  const LayerPtrs L = layer_ptrs(g, layer_lo + (int)blockIdx.y);
  const int h = (int)blockIdx.x, H = g.n_heads, D = g.head_dim, N = g.n_slots, NP = g.n_pad;
  const int head = L.state[0], nv = L.state[1], gv = L.state[3];
  int a = head - nv;
  if (a < 0) a += N;
  auto valid = [&](int slot) { return slot_valid(g, slot, a, nv, gv); };  // ring and global slots
  const int CH = D / 16;  // 16-byte chunks per key row
  double mk = 0.0, mv = 0.0;
  for (int idx = (int)threadIdx.x; idx < NP * CH; idx += 256) {  // keys: slot-major rows
    const int slot = idx / CH, c = idx % CH;
    if (!valid(slot)) continue;
    const uint4 w = *reinterpret_cast<const uint4*>(L.codes_k + ((size_t)h * NP + slot) * D + 16 * c);
    mk = max16_scaled(w, L.scale_k + (size_t)h * NP + slot, false, mk);
  }
  for (int idx = (int)threadIdx.x; idx < g.n_tiles * D * 4; idx += 256) {  // values: [16-slot group][d][16 slots]
    const int tile = idx / (D * 4), d = (idx / 4) % D, qtr = idx % 4;
    const int s0 = kTile * tile + 16 * qtr;
    const uint4 w = *reinterpret_cast<const uint4*>(L.codes_v + (((size_t)h * 4 * g.n_tiles + 4 * tile + qtr) * D + d) * 16);
    float sc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = valid(s0 + e) ? L.scale_v[(size_t)h * NP + s0 + e] : 0.f;
    mv = max16_scaled(w, sc, true, mv);
  }
  red[0][threadIdx.x] = mk;
  red[1][threadIdx.x] = mv;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      red[0][threadIdx.x] = fmax(red[0][threadIdx.x], red[0][threadIdx.x + w]);
      red[1][threadIdx.x] = fmax(red[1][threadIdx.x], red[1][threadIdx.x + w]);
    }
    __syncthreads();
  }
  const float sk = (float)((double)margin * red[0][0] / (double)kE4M3Max);
  const float sv = (float)((double)margin * red[1][0] / (double)kE4M3Max);
  if (threadIdx.x == 0) {
    L.stat[h] = sk;
    L.stat[H + h] = sv;
    if (h == 0) reinterpret_cast<int*>(L.stat)[2 * H] = 1;
  }
  // Requantize the head's valid cache with the new scales (the pages' cache
  // is bf16 until the calibration and FP8 with the head's scales from then
  // on): code' = e4m3(code * s_slot / s) with the product and quotient in
  // double precision, so that every valid slot carries the head's scales
  // and the attention can apply them per head.  Every element is at most
  // amax = 448 s / margin, so only a margin below 1 saturates (at +-448,
  // the clamp below).  Only this workgroup touches
  // the head's slots, and every one of its reads above came before the
  // reduction's barriers.
  auto requant16 = [](uint4 w, const float* sc, bool per_elem, float s) {
    float x[16];
    unpack4_fp8(w.x, x[0], x[1], x[2], x[3]);
    unpack4_fp8(w.y, x[4], x[5], x[6], x[7]);
    unpack4_fp8(w.z, x[8], x[9], x[10], x[11]);
    unpack4_fp8(w.w, x[12], x[13], x[14], x[15]);
    float q[16];
#pragma unroll
    for (int e = 0; e < 16; ++e)
      q[e] = __builtin_amdgcn_fmed3f((float)((double)x[e] * (double)sc[per_elem ? e : 0] / (double)s), -kE4M3Max,
                                     kE4M3Max);
    uint4 o;
    uint32_t* ow = &o.x;
#pragma unroll
    for (int c = 0; c < 4; ++c) ow[c] = pack2_fp8<true>(q[4 * c + 2], q[4 * c + 3], pack2_fp8<false>(q[4 * c], q[4 * c + 1], 0u));
    return o;
  };
  if (sk > 0.f) {
    for (int idx = (int)threadIdx.x; idx < NP * CH; idx += 256) {
      const int slot = idx / CH, c = idx % CH;
      if (!valid(slot)) continue;
      uint4* p = reinterpret_cast<uint4*>(L.codes_k + ((size_t)h * NP + slot) * D + 16 * c);
      *p = requant16(*p, L.scale_k + (size_t)h * NP + slot, false, sk);
    }
  }
  if (sv > 0.f) {
    for (int idx = (int)threadIdx.x; idx < g.n_tiles * D * 4; idx += 256) {
      const int tile = idx / (D * 4), d = (idx / 4) % D, qtr = idx % 4;
      const int s0 = kTile * tile + 16 * qtr;
      bool any = false;
      float sc[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool ok = valid(s0 + e);
        any |= ok;
        sc[e] = ok ? L.scale_v[(size_t)h * NP + s0 + e] : 0.f;
      }
      if (!any) continue;
      uint4* p = reinterpret_cast<uint4*>(L.codes_v + (((size_t)h * 4 * g.n_tiles + 4 * tile + qtr) * D + d) * 16);
      const uint4 old = *p;
      const uint4 nw = requant16(old, sc, true, sv);
      // slots outside the valid range keep their bytes
      uint4 o;
      const uint32_t* a = &old.x;
      const uint32_t* b = &nw.x;
      uint32_t* r = &o.x;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t m = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (valid(s0 + 4 * c + e)) m |= 0xFFu << (8 * e);
        r[c] = (b[c] & m) | (a[c] & ~m);
      }
      *p = o;
    }
  }
  __syncthreads();  // every thread's scale reads above are done before the scales change
  for (int slot = (int)threadIdx.x; slot < NP; slot += 256) {
    if (!valid(slot)) continue;
    if (sk > 0.f) L.scale_k[(size_t)h * NP + slot] = sk;
    if (sv > 0.f) L.scale_v[(size_t)h * NP + slot] = sv;
  }
  // every valid value scale of the head is now s: the head's bound
  if (sv > 0.f && (int)threadIdx.x < kSub) L.vmax[h * kSub + threadIdx.x] = __float_as_uint(sv);
}

hipError_t launch_calibrate(const Geom& g, int layer_lo, int layer_hi, float margin, hipStream_t s) {
  hipLaunchKernelGGL(calibrate_kernel, dim3(g.n_heads, layer_hi - layer_lo), dim3(256), 0, s, g, layer_lo, margin);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused write (the body is in write_body.h).
template <int D, int HG, bool GL = false>
__global__ __launch_bounds__(16 * (D / 8)) void write_rope_fp8_kernel(
    Geom g, int layer, const uint4* __restrict__ k, const uint4* __restrict__ v,
    const int32_t* __restrict__ pos, int n, const uint16_t* wk, float eps, int groups, int items, int gfirst) {
  const int b = (int)blockIdx.x, nw = (int)gridDim.x;
  write_rope_fp8_body<D, HG, GL>(g, layer, k, v, pos, n, wk, eps, b, nw, groups, items, b, nw, gfirst);
}

template <int D, int HG, bool GL = false>
static void launch_write_t(const Geom& g, int layer, const void* k, const void* v, const int32_t* pos,
                           int n, const uint16_t* wk, float eps, int groups, int items, int wgs, hipStream_t s,
                           int gfirst = 0) {
  hipLaunchKernelGGL((write_rope_fp8_kernel<D, HG, GL>), dim3(wgs), dim3(16 * (D / 8)), 0, s, g, layer,
                     (const uint4*)k, (const uint4*)v, pos, n, wk, eps, groups, items, gfirst);
}

hipError_t launch_write_global(const Geom& g, int layer, int first, const void* k, const void* v, const int32_t* pos,
                               int n, const uint16_t* wk, float eps, hipStream_t s) {
  // 16-slot groups met by the n slots from g0 + first
  const int b0 = g.n_ring_pad + first;
  const int groups = (b0 + n + 15) / 16 - b0 / 16;
  const int hg = g.n_heads % 2 == 0 ? 2 : 1;
  const int items = groups * (g.n_heads / hg);
  const int wgs = items < kWriteMaxWgs ? items : kWriteMaxWgs;
  if (g.head_dim == 128) {
    if (hg == 2) launch_write_t<128, 2, true>(g, layer, k, v, pos, n, wk, eps, groups, items, wgs, s, first);
    else launch_write_t<128, 1, true>(g, layer, k, v, pos, n, wk, eps, groups, items, wgs, s, first);
  } else {
    if (hg == 2) launch_write_t<64, 2, true>(g, layer, k, v, pos, n, wk, eps, groups, items, wgs, s, first);
    else launch_write_t<64, 1, true>(g, layer, k, v, pos, n, wk, eps, groups, items, wgs, s, first);
  }
  return hipGetLastError();
}

hipError_t launch_write(const Geom& g, int layer, const void* k, const void* v, const int32_t* pos,
                        int n, const uint16_t* wk, float eps, hipStream_t s) {
  int groups, hg, items, wgs;
  write_grid(g, n, &groups, &hg, &items, &wgs);
  if (g.head_dim == 128) {
    if (hg == 2) launch_write_t<128, 2>(g, layer, k, v, pos, n, wk, eps, groups, items, wgs, s);
    else launch_write_t<128, 1>(g, layer, k, v, pos, n, wk, eps, groups, items, wgs, s);
  } else {
    if (hg == 2) launch_write_t<64, 2>(g, layer, k, v, pos, n, wk, eps, groups, items, wgs, s);
    else launch_write_t<64, 1>(g, layer, k, v, pos, n, wk, eps, groups, items, wgs, s);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Delta rotation.  One (slot, head) key row per D/16 lanes (16 codes each);
// rows are visited in memory order (head-major, slot-minor) so each
// workgroup streams a contiguous block of codes_k.  Only slots of the valid
// cyclic range [head - n_valid, head) are touched.  Each thread takes kRPT
// rows, 256 / (D/16) rows apart, and issues all their loads before any
// arithmetic: more bytes in flight than one row per thread, which a
// streaming pass over HBM needs to cover the memory latency.  The code rows
// are read and written with the nontemporal hint (a one-pass stream).
struct RotTable {
  float c[kMaxHalfDim];
  float s[kMaxHalfDim];
};
constexpr int kRPT = 4;  // rows per thread
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) void rotate_kernel(Geom g, int layer_lo, int32_t delta,
                                                    RotTable tab) {
  constexpr int LPR = D / 16;
  constexpr int RPW = 256 / LPR;  // rows per workgroup and pass
  __shared__ float cs[D / 2], sn[D / 2];
  if (threadIdx.x < D / 2) {
    cs[threadIdx.x] = tab.c[threadIdx.x];
    sn[threadIdx.x] = tab.s[threadIdx.x];
  }
  __syncthreads();

  const LayerPtrs L = layer_ptrs(g, layer_lo + (int)blockIdx.y);
  const int N = g.n_slots, NP = g.n_pad;
  const int head = L.state[0], nv = L.state[1];
  // the pages' static-scale mode: every key of a head is requantized with the
  // head's scale, values beyond it saturate (a head calibrated at amax 0 has
  // scale 0 and keeps the per-(token, head) rule)
  const bool smode = reinterpret_cast<const int*>(L.stat)[2 * g.n_heads] != 0;
  int a = head - nv;
  if (a < 0) a += N;
  const int lane = threadIdx.x % LPR;

  uint4 w[kRPT];
  float sc[kRPT], st[kRPT];
  size_t r[kRPT];
  int slot[kRPT];
  bool valid[kRPT];
#pragma unroll
  for (int k = 0; k < kRPT; ++k) {
    const int row = (blockIdx.x * kRPT + k) * RPW + threadIdx.x / LPR;  // ring rows only: globals never move
    const int h = row / g.n_ring_pad;
    slot[k] = row % g.n_ring_pad;
    int rel = slot[k] - a;
    if (rel < 0) rel += N;
    valid[k] = h < g.n_heads && slot[k] < N && rel < nv;
    r[k] = (size_t)h * NP + slot[k];
    w[k] = make_uint4(0u, 0u, 0u, 0u);
    sc[k] = st[k] = 0.f;
    if (valid[k]) {
      const u4v t = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(L.codes_k + r[k] * D + 16 * lane));
      w[k] = make_uint4(t[0], t[1], t[2], t[3]);
      sc[k] = L.scale_k[r[k]];
      if (smode) st[k] = L.stat[h];
    }
  }
#pragma unroll
  for (int k = 0; k < kRPT; ++k) {
    float x[16];
    unpack4_fp8(w[k].x, x[0], x[1], x[2], x[3]);
    unpack4_fp8(w[k].y, x[4], x[5], x[6], x[7]);
    unpack4_fp8(w[k].z, x[8], x[9], x[10], x[11]);
    unpack4_fp8(w[k].w, x[12], x[13], x[14], x[15]);
    float y[16];
    float am = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float c = cs[8 * lane + m], s = sn[8 * lane + m];
      const float x0 = x[2 * m] * sc[k], x1 = x[2 * m + 1] * sc[k];
      y[2 * m] = x0 * c - x1 * s;
      y[2 * m + 1] = x0 * s + x1 * c;
      am = fmaxf(am, fmaxf(fabsf(y[2 * m]), fabsf(y[2 * m + 1])));
    }
    am = group_max<LPR>(am);
    const float sn2 = st[k] > 0.f ? st[k] : am * g.margin / kE4M3Max;
    const float rn = sn2 > 0.f ? 1.f / sn2 : 0.f;
    uint4 o;
    uint32_t* ow = &o.x;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t t = pack2_fp8<false>(quant_mul(y[4 * q], rn), quant_mul(y[4 * q + 1], rn), 0u);
      ow[q] = pack2_fp8<true>(quant_mul(y[4 * q + 2], rn), quant_mul(y[4 * q + 3], rn), t);
    }
    if (valid[k]) {
      __builtin_nontemporal_store(u4v{o.x, o.y, o.z, o.w}, reinterpret_cast<u4v*>(L.codes_k + r[k] * D + 16 * lane));
      if (lane == 0) {
        L.scale_k[r[k]] = sn2;
        if (r[k] < (size_t)NP) L.slot_pos[slot[k]] += delta;  // head 0 rows
      }
    }
  }
}

hipError_t launch_rotate(const Geom& g, int layer_lo, int layer_hi, int32_t delta,
                         const float* cosv, const float* sinv, hipStream_t s) {
  RotTable tab{};
  const int half = g.head_dim / 2;
  for (int j = 0; j < half; ++j) {
    tab.c[j] = cosv[j];
    tab.s[j] = sinv[j];
  }
  const int lpr = g.head_dim / 16;
  const long long rows_per_wg = (long long)(256 / lpr) * kRPT;
  const long long rows = (long long)g.n_heads * g.n_ring_pad;
  dim3 grid((unsigned)((rows + rows_per_wg - 1) / rows_per_wg), layer_hi - layer_lo);
  if (g.head_dim == 128)
    hipLaunchKernelGGL(rotate_kernel<128>, grid, dim3(256), 0, s, g, layer_lo, delta, tab);
  else
    hipLaunchKernelGGL(rotate_kernel<64>, grid, dim3(256), 0, s, g, layer_lo, delta, tab);
  return hipGetLastError();
}

}  // namespace rkv
