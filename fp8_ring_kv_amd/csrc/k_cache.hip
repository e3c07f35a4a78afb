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
// Session reset: head = n_valid = 0 and every slot position = 0.
__global__ void reset_kernel(Geom g, int layer_lo) {
  const LayerPtrs L = layer_ptrs(g, layer_lo + (int)blockIdx.y);
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < g.n_pad) L.slot_pos[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x < kStateInts) L.state[threadIdx.x] = 0;
  if (blockIdx.x == 0)
    for (int j = (int)threadIdx.x; j < g.n_heads * kSub; j += (int)blockDim.x) L.vmax[j] = 0u;
}

hipError_t launch_reset(const Geom& g, int layer_lo, int layer_hi, hipStream_t s) {
  dim3 grid((g.n_pad + 255) / 256, layer_hi - layer_lo);
  hipLaunchKernelGGL(reset_kernel, grid, dim3(256), 0, s, g, layer_lo);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused write.  One workgroup per (16-slot group of the ring, HG heads).  The
// groups touched by a write of n tokens are consecutive (mod the group count
// ceil(N/16), pad slots excluded) starting at the group holding `head`; a
// contiguous run of n slots meets at most n/16 + 2 of them (one partial group
// at each end, plus the short last group when it wraps).  The grid covers
// that many and each thread works out from the device-side head whether its
// slot is written and by which token: token i = (slot - head) mod N, written
// iff i < n.  Thread (tau, lane) owns 8 elements of token row tau in each of
// the HG heads: its loads for all heads are in flight together and its RoPE
// cos/sin serve all of them.
template <int D, int HG>
__global__ __launch_bounds__(16 * (D / 8)) void write_rope_fp8_kernel(
    Geom g, int layer, const uint4* __restrict__ k, const uint4* __restrict__ v,
    const int32_t* __restrict__ pos, int n) {
  constexpr int LPR = D / 8;  // lanes per token row
  __shared__ uint2 vcodes[HG][16][LPR];
  __shared__ float vmx[HG][16];

  const LayerPtrs L = layer_ptrs(g, layer);
  const int N = g.n_slots, NP = g.n_pad, H = g.n_heads;
  const int head = L.state[0];
  const int nvalid = L.state[1];
  const int h0 = blockIdx.y * HG;
  const int NG = (N + 15) / 16;  // 16-slot groups of the ring (the last may be short)
  const int G = (head / 16 + (int)blockIdx.x) % NG;
  const int tau = threadIdx.x / LPR;
  const int lane = threadIdx.x % LPR;
  const int slot = 16 * G + tau;
  int i = slot - head;
  if (i < 0) i += N;
  const bool active = slot < N && i < n;

  uint4 kw[HG], vw[HG];
  int32_t p = 0;
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) kw[hh] = vw[hh] = make_uint4(0u, 0u, 0u, 0u);
  if (active) {
    const size_t row = ((size_t)i * H + h0) * LPR + lane;
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      kw[hh] = k[row + hh * LPR];
      vw[hh] = v[row + hh * LPR];
    }
    p = pos[i];
  }
  // Tickets for the device-side write position, taken once head and n_valid
  // are read (and after the row loads are issued: a returning atomic holds
  // up every later load's wait): whoever takes the last ticket knows every
  // workgroup has read them and may advance them.  Workgroup w takes a ticket on
  // sub-counter w % kSub; the last arrival of each sub-group takes one on the
  // top counter, so no counter sees more than ceil(total / kSub) atomics.
  // The increment depends on the loaded head (it is always 1), so it cannot
  // be issued before the load returns.  No workgroup reads what another one
  // writes, so relaxed device-scope atomics suffice; the next kernel on the
  // stream sees the new state.
  // (The returned ticket is looked at only at the end of the kernel.)
  const int wg = (int)(blockIdx.y * gridDim.x + blockIdx.x);
  int t1 = 0;
  if (threadIdx.x == 0)
    t1 = __hip_atomic_fetch_add(&L.state[4 + wg % kSub], head < 0x7FFFFFFF ? 1 : 2, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
  // angles for every lane (the table index is always in range; inactive
  // lanes rotate zeros), so the four table loads issue together
  float cs[4], sn[4];
  const double* turns = omega_turns(g);
#pragma unroll
  for (int m = 0; m < 4; ++m) rope_cs(p, turns[4 * lane + m], cs[m], sn[m]);

#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    const float x[8] = {bf16_lo(kw[hh].x), bf16_hi(kw[hh].x), bf16_lo(kw[hh].y), bf16_hi(kw[hh].y),
                        bf16_lo(kw[hh].z), bf16_hi(kw[hh].z), bf16_lo(kw[hh].w), bf16_hi(kw[hh].w)};
    const float u[8] = {bf16_lo(vw[hh].x), bf16_hi(vw[hh].x), bf16_lo(vw[hh].y), bf16_hi(vw[hh].y),
                        bf16_lo(vw[hh].z), bf16_hi(vw[hh].z), bf16_lo(vw[hh].w), bf16_hi(vw[hh].w)};
    float y[8];
    float ak = 0.f, av = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      y[2 * m] = x[2 * m] * cs[m] - x[2 * m + 1] * sn[m];
      y[2 * m + 1] = x[2 * m] * sn[m] + x[2 * m + 1] * cs[m];
      ak = fmaxf(ak, fmaxf(fabsf(y[2 * m]), fabsf(y[2 * m + 1])));
      av = fmaxf(av, fmaxf(fabsf(u[2 * m]), fabsf(u[2 * m + 1])));
    }
    ak = group_max<LPR>(ak);
    av = group_max<LPR>(av);
    // scale s = fp32(margin * amax / 448); codes = e4m3(y / s)
    const float sk = ak * g.margin / kE4M3Max, sv = av * g.margin / kE4M3Max;
    const float rk = sk > 0.f ? 1.f / sk : 0.f;
    const float rv = sv > 0.f ? 1.f / sv : 0.f;
    // keys are fp32 RoPE results (a rounding away from the exact rotation
    // already), values are raw bf16 whose quotients often sit on e4m3 midpoints
    uint2 ck, cv;
    ck.x = pack2_fp8<false>(quant_mul(y[0], rk), quant_mul(y[1], rk), 0u);
    ck.x = pack2_fp8<true>(quant_mul(y[2], rk), quant_mul(y[3], rk), ck.x);
    ck.y = pack2_fp8<false>(quant_mul(y[4], rk), quant_mul(y[5], rk), 0u);
    ck.y = pack2_fp8<true>(quant_mul(y[6], rk), quant_mul(y[7], rk), ck.y);
    cv.x = pack2_fp8<false>(quant_div(u[0], sv, rv), quant_div(u[1], sv, rv), 0u);
    cv.x = pack2_fp8<true>(quant_div(u[2], sv, rv), quant_div(u[3], sv, rv), cv.x);
    cv.y = pack2_fp8<false>(quant_div(u[4], sv, rv), quant_div(u[5], sv, rv), 0u);
    cv.y = pack2_fp8<true>(quant_div(u[6], sv, rv), quant_div(u[7], sv, rv), cv.y);
    if (active) {
      const size_t r = (size_t)(h0 + hh) * NP + slot;
      *reinterpret_cast<uint2*>(L.codes_k + r * D + 8 * lane) = ck;
      if (lane == 0) {
        L.scale_k[r] = sk;
        L.scale_v[r] = sv;
      }
    }
    vcodes[hh][tau][lane] = cv;
    if (lane == 0) vmx[hh][tau] = active ? sv : 0.f;
  }
  if (active && lane == 0 && h0 == 0) L.slot_pos[slot] = p;
  // LDS-only barrier: the transpose below needs the LDS writes above, not
  // the global stores (a __syncthreads fence would wait for those too)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // V: transposed 64-slot tiles, row d holds the tile's slots in order.  The
  // group's 16 slots are 16 consecutive bytes of each row; thread t writes
  // 8 of them (tokens 8*half .. 8*half+7) of row d, for each head.
  {
    const int t = threadIdx.x;
    const int d = t >> 1, half = t & 1;
    bool act[8];
    int nact = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sl = 16 * G + 8 * half + e;
      int ii = sl - head;
      if (ii < 0) ii += N;
      act[e] = sl < N && ii < n;
      nact += act[e];
    }
    const int T = (16 * G) / kTile, w0 = (16 * G) % kTile;
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      const uint8_t* vb = reinterpret_cast<const uint8_t*>(vcodes[hh]);
      uint32_t b[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = vb[(8 * half + e) * D + d];
      uint8_t* dst = L.codes_v + (((size_t)(h0 + hh) * g.n_tiles + T) * D + d) * kTile + w0 + 8 * half;
      if (nact == 8) {
        uint2 w;
        w.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
        w.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
        *reinterpret_cast<uint2*>(dst) = w;
      } else if (nact > 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (act[e]) dst[e] = (uint8_t)b[e];
      }
    }
  }

  // Running per-head maximum of the value scales (non-negative floats order
  // like their bit patterns); nothing waits for these atomics.
  if ((int)threadIdx.x < HG) {
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, vmx[threadIdx.x][e]);
    if (mx > 0.f) atomicMax(&L.vmax[(h0 + threadIdx.x) * kSub + blockIdx.x % kSub], __float_as_uint(mx));
  }
  // The last arrival of each sub-group takes a ticket on the top counter;
  // the last of those advances the write position.
  if (threadIdx.x == 0) {
    const int total = (int)(gridDim.x * gridDim.y);
    const int k = wg % kSub;
    const int ksize = (total - k + kSub - 1) / kSub;  // workgroups with wg % kSub == k
    const int nsub = total < kSub ? total : kSub;
    if (t1 == ksize - 1) {
      __hip_atomic_store(&L.state[4 + k], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int t2 = __hip_atomic_fetch_add(&L.state[2], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (t2 == nsub - 1) {
        __hip_atomic_store(&L.state[2], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        L.state[0] = (int)(((long long)head + n) % N);
        L.state[1] = nvalid + n < N ? nvalid + n : N;
      }
    }
  }
}

template <int D, int HG>
static void launch_write_t(const Geom& g, int layer, const void* k, const void* v, const int32_t* pos,
                           int n, int groups, hipStream_t s) {
  dim3 grid(groups, g.n_heads / HG);
  hipLaunchKernelGGL((write_rope_fp8_kernel<D, HG>), grid, dim3(16 * (D / 8)), 0, s, g, layer,
                     (const uint4*)k, (const uint4*)v, pos, n);
}

hipError_t launch_write(const Geom& g, int layer, const void* k, const void* v, const int32_t* pos,
                        int n, hipStream_t s) {
  const int NG = (g.n_slots + 15) / 16;
  int groups = (n + 15) / 16 + 2;
  if (groups > NG) groups = NG;
  const int H = g.n_heads;
  const int hg = H % 4 == 0 ? 4 : (H % 2 == 0 ? 2 : 1);
  if (g.head_dim == 128) {
    if (hg == 4) launch_write_t<128, 4>(g, layer, k, v, pos, n, groups, s);
    else if (hg == 2) launch_write_t<128, 2>(g, layer, k, v, pos, n, groups, s);
    else launch_write_t<128, 1>(g, layer, k, v, pos, n, groups, s);
  } else {
    if (hg == 4) launch_write_t<64, 4>(g, layer, k, v, pos, n, groups, s);
    else if (hg == 2) launch_write_t<64, 2>(g, layer, k, v, pos, n, groups, s);
    else launch_write_t<64, 1>(g, layer, k, v, pos, n, groups, s);
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
  int a = head - nv;
  if (a < 0) a += N;
  const int lane = threadIdx.x % LPR;

  uint4 w[kRPT];
  float sc[kRPT];
  size_t r[kRPT];
  int slot[kRPT];
  bool valid[kRPT];
#pragma unroll
  for (int k = 0; k < kRPT; ++k) {
    const int row = (blockIdx.x * kRPT + k) * RPW + threadIdx.x / LPR;
    const int h = row / NP;
    slot[k] = row % NP;
    int rel = slot[k] - a;
    if (rel < 0) rel += N;
    valid[k] = h < g.n_heads && slot[k] < N && rel < nv;
    r[k] = (size_t)h * NP + slot[k];
    w[k] = make_uint4(0u, 0u, 0u, 0u);
    sc[k] = 0.f;
    if (valid[k]) {
      const u4v t = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(L.codes_k + r[k] * D + 16 * lane));
      w[k] = make_uint4(t[0], t[1], t[2], t[3]);
      sc[k] = L.scale_k[r[k]];
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
    const float sn2 = am * g.margin / kE4M3Max;
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
  const long long rows = (long long)g.n_heads * g.n_pad;
  dim3 grid((unsigned)((rows + rows_per_wg - 1) / rows_per_wg), layer_hi - layer_lo);
  if (g.head_dim == 128)
    hipLaunchKernelGGL(rotate_kernel<128>, grid, dim3(256), 0, s, g, layer_lo, delta, tab);
  else
    hipLaunchKernelGGL(rotate_kernel<64>, grid, dim3(256), 0, s, g, layer_lo, delta, tab);
  return hipGetLastError();
}

}  // namespace rkv
