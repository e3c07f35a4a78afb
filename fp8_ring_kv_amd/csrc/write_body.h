// Fused RoPE + FP8 ring write, as a device function of the workgroup's
// coordinates: write_rope_fp8_kernel runs it on every workgroup of its grid;
// the write-and-prepare launch runs it on the first workgroups of its grid,
// beside the query preparation.
//
// Runway Characters paper: §4.1 (ring slots, device-side write position,
// each slot keeps its written position), §4.2 (RoPE once at write), §4.3
// (K and V stored in e4m3, only new tokens quantized), §4.4 (the
// pre-attention chain fused into one pass per token).
#pragma once

#include "rkv_launch.h"

namespace rkv {

// Fused write.  The work items are (16-slot group of the ring, HG heads).
// The groups touched by a write of n tokens are consecutive (mod the group
// count ceil(N/16), pad slots excluded) starting at the group holding `head`;
// a contiguous run of n slots meets at most n/16 + 2 of them (one partial
// group at each end, plus the short last group when it wraps).  Each thread
// works out from the device-side head whether its slot is written and by
// which token: token i = (slot - head) mod N, written iff i < n.  Thread
// (tau, lane) owns 8 elements of token row tau in each of the HG heads: its
// loads for all heads are in flight together and its RoPE cos/sin serve all
// of them.
// A workgroup takes items item0, item0 + istride, ... below n_items (item =
// by * groups + bx: group offset bx from the start group, head group by):
// one item each for writes of up to a grid's worth, several for large ones,
// where the next item's rows load while the current one is quantized and
// stored (all workgroups loading, then all computing, then all storing left
// each phase to run on its own).
// wgi, nwg: this workgroup's index and the number of workgroups taking
// tickets.  wk: the layer's key RMS-norm weights (bf16 [D], shared by the
// heads) when the fused pre-attention norm is on, else null; eps its epsilon.
// GL: the tokens go to the global (sink) slots gfirst .. gfirst + n - 1 (the
// array slots g0 + gfirst + i, no wrap, no ticket); g_valid is raised to
// gfirst + n.  The ring write (GL false) ignores gfirst.
template <int HG>
struct WriteRows {  // one thread's share of one work item
  uint4 kw[HG], vw[HG];
  int32_t pc[4];       // the coordinate that turns each of this lane's 4 pairs
  int32_t pt, py, px;  // the token's position
  float sk[HG], sv[HG];  // the heads' static scales (read whether or not they are in use)
};

template <int D, int HG, bool GL = false>
__device__ inline void write_rope_fp8_body(const Geom& g, int layer, const uint4* __restrict__ k,
                                           const uint4* __restrict__ v, const int32_t* __restrict__ pos,
                                           int n, const uint16_t* __restrict__ wk, float eps, int item0,
                                           int istride, int groups, int n_items, int wgi, int nwg,
                                           int gfirst = 0) {
  constexpr int LPR = D / 8;  // lanes per token row
  __shared__ uint2 vcodes[HG][16][LPR];
  __shared__ float vmx[HG][16];

  const LayerPtrs L = layer_ptrs(g, layer);
  const int N = g.n_slots, NP = g.n_pad, H = g.n_heads;
  const int head = GL ? 0 : L.state[0];
  const int nvalid = GL ? 0 : L.state[1];
  // the pages' static per-(layer, head) scales, once calibrated
  const bool smode = reinterpret_cast<const int*>(L.stat)[2 * H] != 0;
  const int NG = (N + 15) / 16;  // 16-slot groups of the ring (the last may be short)
  const int b0 = g.n_ring_pad + gfirst;  // first array slot of a global write
  const int tau = threadIdx.x / LPR;
  const int lane = threadIdx.x % LPR;
  // token written to array slot sl, or -1 (ring: (sl - head) mod N)
  auto token_of = [&](int sl) {
    if constexpr (GL) {
      const int t = sl - b0;
      return t >= 0 && t < n ? t : -1;
    } else {
      int t = sl - head;
      if (t < 0) t += N;
      return sl < N && t < n ? t : -1;
    }
  };
  auto group_of = [&](int item) {
    const int bx = item % groups;
    return GL ? b0 / 16 + bx : (head / 16 + bx) % NG;
  };
  auto load = [&](int item, WriteRows<HG>& w) {
    const int h0 = (item / groups) * HG;
    const int i = token_of(16 * group_of(item) + tau);
    // loaded beside the rows, with no test of the mode first: a load issued
    // among the arithmetic would wait for every store before it
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      w.sk[hh] = L.stat[h0 + hh];
      w.sv[hh] = L.stat[H + h0 + hh];
    }
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) w.kw[hh] = w.vw[hh] = make_uint4(0u, 0u, 0u, 0u);
    w.pc[0] = w.pc[1] = w.pc[2] = w.pc[3] = 0;
    w.pt = w.py = w.px = 0;
    if (i >= 0) {
      const size_t row = ((size_t)i * H + h0) * LPR + lane;
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        w.kw[hh] = k[row + hh * LPR];
        w.vw[hh] = v[row + hh * LPR];
      }
      const int32_t* pp = pos + (size_t)i * g.pos_stride;
#pragma unroll
      for (int m = 0; m < 4; ++m) w.pc[m] = pair_coord(g, pp, 4 * lane + m);
      w.pt = pp[0];
      if (g.pos_stride == 3) {
        w.py = pp[1];
        w.px = pp[2];
      }
    }
  };

  WriteRows<HG> cur;
  load(item0, cur);
  // Ticket for the device-side write position, taken once head and n_valid
  // are read (the increment depends on the loaded head; it is always 1).
  // Whoever takes the last ticket knows that every workgroup has read the
  // position and may advance it.  Up to kTicketSplitMin workgroups count on
  // the top counter alone.  Larger grids count workgroup w on sub-counter
  // w mod kTicketSub and the last of each sub-group on the top counter:
  // atomics on one address serialize (~15 ns each), which cost a
  // 2,184-workgroup write 13 us, while the second level adds one atomic
  // round trip at the end (0.4 us on a 294-workgroup write).  No workgroup
  // reads what another writes: relaxed device-scope atomics suffice; the
  // next kernel on the stream sees the new state.
  // The ticket goes out once every load of the first item has returned (the
  // frequency table included): vector memory operations complete in order, so
  // a wait for a load issued after the ticket, or one the compiler cannot
  // place relative to it, would wait for its round trip too.  Issued here, it
  // returns while the arithmetic below runs.
  double tw[4];
  const double* turns = omega_turns(g);
#pragma unroll
  for (int m = 0; m < 4; ++m) tw[m] = turns[4 * lane + m];
  // the norm weights of this lane's 8 elements (the same for every head)
  uint4 wkv = make_uint4(0u, 0u, 0u, 0u);
  if (wk != nullptr) wkv = reinterpret_cast<const uint4*>(wk)[lane];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh)
    asm volatile("" ::"v"(cur.kw[hh].x), "v"(cur.kw[hh].y), "v"(cur.kw[hh].z), "v"(cur.kw[hh].w),
                 "v"(cur.vw[hh].x), "v"(cur.vw[hh].y), "v"(cur.vw[hh].z), "v"(cur.vw[hh].w));
  asm volatile("" ::"v"(cur.pc[0]), "v"(cur.pc[1]), "v"(cur.pc[2]), "v"(cur.pc[3]), "v"(tw[0]), "v"(tw[1]),
               "v"(tw[2]), "v"(tw[3]), "v"(wkv.x), "v"(wkv.y), "v"(wkv.z), "v"(wkv.w) : "memory");
  const bool two_level = nwg > kTicketSplitMin;
  const int sub = wgi % kTicketSub;
  int* const counter = two_level ? L.state + kTicketStride * (1 + sub) : L.state + 2;
  int ticket = -1;
  if (!GL && threadIdx.x == 0)
    ticket = __hip_atomic_fetch_add(counter, head < 0x7FFFFFFF ? 1 : 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  for (int item = item0; item < n_items; item += istride) {
    // the next item's rows load while this one is processed
    WriteRows<HG> nxt;
    const bool more = item + istride < n_items;
    if (more) load(item + istride, nxt);
    const int h0 = (item / groups) * HG;
    const int G = group_of(item);
    const int slot = 16 * G + tau;
    const bool active = token_of(slot) >= 0;
    // angles for every lane (the table index is always in range; inactive
    // lanes rotate zeros)
    float cs[4], sn[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) rope_cs(cur.pc[m], tw[m], cs[m], sn[m]);

#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      const uint4 kq = cur.kw[hh], vq = cur.vw[hh];
      float x[8] = {bf16_lo(kq.x), bf16_hi(kq.x), bf16_lo(kq.y), bf16_hi(kq.y),
                    bf16_lo(kq.z), bf16_hi(kq.z), bf16_lo(kq.w), bf16_hi(kq.w)};
      if (wk != nullptr) {  // fused RMS norm of the key row, before RoPE
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
        const float r = rms_factor<LPR>(ss, 1.f / D, eps);
        const float w[8] = {bf16_lo(wkv.x), bf16_hi(wkv.x), bf16_lo(wkv.y), bf16_hi(wkv.y),
                            bf16_lo(wkv.z), bf16_hi(wkv.z), bf16_lo(wkv.w), bf16_hi(wkv.w)};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = x[e] * r * w[e];
      }
      const float u[8] = {bf16_lo(vq.x), bf16_hi(vq.x), bf16_lo(vq.y), bf16_hi(vq.y),
                          bf16_lo(vq.z), bf16_hi(vq.z), bf16_lo(vq.w), bf16_hi(vq.w)};
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
      // scale s = fp32(margin * amax / 448); codes = e4m3(y / s).  Keys are
      // fp32 RoPE results (a rounding away from the exact rotation already):
      // y * (1/s).  Values are raw bf16, whose quotients often sit next to
      // e4m3 midpoints: the exact quotient code (vquot_row).
      // Static scales (once calibrated): correctly rounded quotients,
      // saturating at +-448.  A head calibrated at amax 0 has a zero static
      // scale and keeps the per-(token, head) rule, keys and values separately.
      const float stk = smode ? cur.sk[hh] : 0.f;
      const float stv = smode ? cur.sv[hh] : 0.f;
      float sk, sv, rk;
      VQuot qv;
      if (stk > 0.f) {
        sk = stk;
      } else {
        sk = div448(ak * g.margin);
      }
      rk = recip_scale(sk);
      if (stv > 0.f) {
        sv = stv;
        qv.s = sv;
        qv.r = recip_scale(sv);
        qv.f = 1.f;
      } else {
        const float amv = av * g.margin;
        sv = div448(amv);
        qv = vquot_row(amv, sv);
      }
      uint2 ck, cv;
      ck.x = pack2_fp8<false>(quant_mul(y[0], rk), quant_mul(y[1], rk), 0u);
      ck.x = pack2_fp8<true>(quant_mul(y[2], rk), quant_mul(y[3], rk), ck.x);
      ck.y = pack2_fp8<false>(quant_mul(y[4], rk), quant_mul(y[5], rk), 0u);
      ck.y = pack2_fp8<true>(quant_mul(y[6], rk), quant_mul(y[7], rk), ck.y);
      cv.x = pack2_fp8<false>(quant_v(u[0], qv), quant_v(u[1], qv), 0u);
      cv.x = pack2_fp8<true>(quant_v(u[2], qv), quant_v(u[3], qv), cv.x);
      cv.y = pack2_fp8<false>(quant_v(u[4], qv), quant_v(u[5], qv), 0u);
      cv.y = pack2_fp8<true>(quant_v(u[6], qv), quant_v(u[7], qv), cv.y);
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
    if (active && lane == 0 && h0 == 0) {
      L.slot_pos[slot] = cur.pt;
      if (g.pos_stride == 3) {
        L.slot_yx[slot] = cur.py;
        L.slot_yx[NP + slot] = cur.px;
      }
    }
    // LDS-only barrier: the transpose below needs the LDS writes above, not
    // the global stores (a __syncthreads fence would wait for those too)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // V: transposed 16-slot groups, [group][d][16 slots]: the group's bytes
    // of one head are D * 16 contiguous bytes (whole cache lines, written by
    // this workgroup alone); thread t writes 8 of row d's 16 (tokens 8*half ..
    // 8*half+7), for each head.
    {
      const int t = threadIdx.x;
      const int d = t >> 1, half = t & 1;
      bool act[8];
      int nact = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        act[e] = token_of(16 * G + 8 * half + e) >= 0;
        nact += act[e];
      }
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const uint8_t* vb = reinterpret_cast<const uint8_t*>(vcodes[hh]);
        uint32_t b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = vb[(8 * half + e) * D + d];
        uint8_t* dst = L.codes_v + (((size_t)(h0 + hh) * 4 * g.n_tiles + G) * D + d) * 16 + 8 * half;
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

    // Running per-head maximum of the value scales (non-negative floats
    // order like their bit patterns); nothing waits for these atomics.
    if ((int)threadIdx.x < HG) {
      float mx = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, vmx[threadIdx.x][e]);
      if (mx > 0.f) atomicMax(&L.vmax[(h0 + threadIdx.x) * kSub + (item % groups) % kSub], __float_as_uint(mx));
    }
    // every thread is done with this item's LDS before the next item writes it
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (more) cur = nxt;
  }

  if constexpr (GL) {  // global slots: no ring position to advance
    if (threadIdx.x == 0 && wgi == 0) atomicMax(&L.state[3], gfirst + n);
    return;
  }
  // Two levels: the last workgroup of a sub-group clears its sub-counter and
  // takes a top ticket.  The one that takes the last top ticket clears the
  // top counter and advances the device-side write position (every
  // workgroup had read it before taking its ticket).
  if (threadIdx.x == 0) {
    bool last = false;
    if (!two_level) {
      last = ticket == nwg - 1;
    } else if (ticket == (nwg - sub + kTicketSub - 1) / kTicketSub - 1) {
      __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = __hip_atomic_fetch_add(&L.state[2], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == kTicketSub - 1;
    }
    if (last) {
      __hip_atomic_store(&L.state[2], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      L.state[0] = (int)(((long long)head + n) % N);
      L.state[1] = nvalid + n < N ? nvalid + n : N;
    }
  }
}

}  // namespace rkv
