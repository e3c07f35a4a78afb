// FP8 attention over the ring cache for gfx950.
//
// Runway Characters paper: every call attends its new queries over all
// slots of its cache, after the chunk was written (§2 "The step budget",
// Appendix G); queries get RoPE at their own positions and cached keys are
// used as stored (§4.2); the cache is e4m3 with per-head descales and only
// the queries are quantized per call (§4.3).
//
// Two launches per call.  q_prep_kernel applies RoPE to the queries at their
// positions (angles in double precision) and splits each (query, head) row
// into three e4m3 terms (one in fast mode) with power-of-two scales, applied
// exactly by the E8M0 scale operand of the matrix instruction.  attend_kernel then does the
// attention proper:
//
// Work: unit u = (head h, group qg of 128 queries), u = h * nqg + qg; each
// unit needs `count` 64-slot tiles (the ring tiles holding valid slots, in
// cyclic order from the tile of the oldest valid slot, then the tiles of the
// valid global slots).  A persistent grid of G
// 4-wave workgroups, two per compute unit, cuts the unit-major list of all
// units * count (unit, tile) pairs into G equal contiguous ranges; when the
// units are fewer than the workgroup slots, G is a multiple of the unit
// count, so every range lies inside one unit.  Workgroups are dealt to the 8
// XCDs round-robin; ranges are assigned so that each XCD takes a contiguous
// block of them (whole heads where possible), keeping their K/V in its L2.
//
// A workgroup handles each unit its range meets as one segment:
//   1. wave w loads the prepared terms of queries 32 w .. 32 w + 31;
//   2. the tiles stream through a ring of LDS buffers: the K tile, the
//      transposed V tile and the 128 slot scales of a tile are copied from
//      global memory straight into LDS (global_load_lds_dwordx4) two
//      tiles ahead.  Every wave reads every tile.  Per tile a wave computes
//      S^T = K Q^T with v_mfma_scale_f32_32x32x64_f8f6f4 (rows = slots,
//      columns = queries: one lane owns one query, so the row max and sum
//      are in-lane plus one swap with lane ^ 32), applies the per-slot key
//      scale, updates an online softmax in fp32 (exp2 domain), turns
//      P * s_v * c_h into one or two e4m3 terms and accumulates
//      O^T += V^T P^T with the same instruction.  Each wave interleaves its
//      own matrix and vector work: the softmax of tile j runs between the
//      P V products of tile j - 1 and the Q K^T products of tile j + 1;
//   3. a whole unit writes its bf16 output; a unit split between
//      workgroups writes a partial (O, max, sum) per wave, and the unit's
//      16 output blocks are merged by the workgroups whose ranges end in it
//      (each its share, after a bounded wait for the unit's last tile) or by
//      the last to arrive.
//
// Probability scale: c_h = 448 / (64 vmax_h), vmax_h being the largest value
// scale written to head h since the reset (kept by the write kernel).  The
// running row maximum is raised only when a tile exceeds it by more than 6
// (log2 units), and then by a whole number of log2 units, so P <= 64 and
// P * s_v * c_h <= 448 always fits e4m3.  (With
// a headroom of 2 the raise, a wave-wide branch over 32 queries, ran on 54%
// of the tiles of the 757 x 5,788 workload; with 6 on 14%.  The smaller c_h
// moves only probabilities below about 1/100 of the row maximum into the
// e4m3 subnormal range, where the second term still carries them.)
#include <cmath>
#include <mutex>
#include <type_traits>

#include "rkv_launch.h"
#include "write_body.h"

namespace rkv {

// Fixed attention workspace of cache_attend_noalloc, for callers that cannot
// allocate (graph capture, serving loops): one copy per device, held from
// module load to process exit, shared by every such call on that device.
// Host code never passes this name to a kernel (on the host it is only a
// stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device.
__device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t scratch_init() {
  void* p = nullptr;
  return scratch_ptr(&p);
}

hipError_t fixed_attn_ws(const Geom& g, const AttnWs& base, int n_q, AttnWs* out, size_t* need) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t H = g.n_heads, D = g.head_dim;
  const size_t nq_pad = (size_t)(n_q + 127) / 128 * 128;
  const size_t units = nq_pad / 128 * H;
  const size_t segs = units + (size_t)base.grid;
  const size_t o_part = 0;
  const size_t o_ml = up(o_part + segs * 128 * D * 2);
  const size_t o_sync = up(o_ml + segs * 4 * 64 * 2 * 4);
  const size_t o_q = up(o_sync + units * kSyncStride * 8);
  const size_t o_qe = up(o_q + 3 * H * nq_pad * D);
  *need = up(o_qe + 3 * H * nq_pad * 4);
  if (*need > kScratchBytes) return hipSuccess;
  void* p = nullptr;
  const hipError_t e = scratch_ptr(&p);
  if (e != hipSuccess) return e;
  uint8_t* b = static_cast<uint8_t*>(p);
  *out = base;
  out->part_o = b + o_part;
  out->part_ml = reinterpret_cast<float*>(b + o_ml);
  out->sync = reinterpret_cast<unsigned long long*>(b + o_sync);
  out->qcodes = b + o_q;
  out->qexp = reinterpret_cast<int32_t*>(b + o_qe);
  out->nq_pad = (int32_t)nq_pad;
  return hipSuccess;
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;  // LDS byte, addressed without a generic pointer

constexpr double kLog2e = 1.4426950408889634;  // log2(e)
constexpr float kLazy = 6.f;             // log2 headroom of the running maximum
constexpr float kHeadroom = 64.f;        // 2^kLazy: c_h = 448 / (kHeadroom vmax_h)
constexpr float kLog2Seven = 2.8073549f; // log2(448 / kHeadroom): static scales feed P' = 7 P
constexpr int kQG = 128;      // queries per unit: 4 waves x 32

// Terms of the two precisions (TERMS = 2: precise, 1: fast).  Precise mode
// splits each query into three e4m3 terms (q known to about 2^-12 relative:
// with two, about 2^-8, a query whose outlier channels meet a key's moved
// single outputs by up to 2.9e-2 of the value scale) and each probability
// into two (hi + lo / 16); fast mode takes one of each.
template <int TERMS>
constexpr int q_terms() { return TERMS == 2 ? 3 : 1; }

struct AttnArgs {
  Geom g;
  AttnWs ws;
  int layer;
  int n_q;
  int nqg;  // 128-query groups
  const uint4* q;
  const int32_t* q_pos;
  uint16_t* out;
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
    case 0: x = __builtin_amdgcn_mov_dpp(x, 0x150, 0xF, 0xF, true); break;
    case 1: x = __builtin_amdgcn_mov_dpp(x, 0x151, 0xF, 0xF, true); break;
    case 2: x = __builtin_amdgcn_mov_dpp(x, 0x152, 0xF, 0xF, true); break;
    case 3: x = __builtin_amdgcn_mov_dpp(x, 0x153, 0xF, 0xF, true); break;
    case 4: x = __builtin_amdgcn_mov_dpp(x, 0x154, 0xF, 0xF, true); break;
    case 5: x = __builtin_amdgcn_mov_dpp(x, 0x155, 0xF, 0xF, true); break;
    case 6: x = __builtin_amdgcn_mov_dpp(x, 0x156, 0xF, 0xF, true); break;
    case 7: x = __builtin_amdgcn_mov_dpp(x, 0x157, 0xF, 0xF, true); break;
    case 8: x = __builtin_amdgcn_mov_dpp(x, 0x158, 0xF, 0xF, true); break;
    case 9: x = __builtin_amdgcn_mov_dpp(x, 0x159, 0xF, 0xF, true); break;
    case 10: x = __builtin_amdgcn_mov_dpp(x, 0x15A, 0xF, 0xF, true); break;
    case 11: x = __builtin_amdgcn_mov_dpp(x, 0x15B, 0xF, 0xF, true); break;
    case 12: x = __builtin_amdgcn_mov_dpp(x, 0x15C, 0xF, 0xF, true); break;
    case 13: x = __builtin_amdgcn_mov_dpp(x, 0x15D, 0xF, 0xF, true); break;
    case 14: x = __builtin_amdgcn_mov_dpp(x, 0x15E, 0xF, 0xF, true); break;
    case 15: x = __builtin_amdgcn_mov_dpp(x, 0x15F, 0xF, 0xF, true); break;
  }
  return __int_as_float(x);
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
// One tile in LDS, filled by wave-wide copies of 16 bytes per lane (1 KiB
// chunks): D/16 chunks of K, D/16 chunks of transposed V, then the scales.
//   K: 16-byte piece c of slot row r sits at piece r * (D/16) + (c ^ ksw(r)).
//      A wave reads its K operand as lane li -> row krow(li) (below); the
//      swizzle puts the 8 rows read by every 8 consecutive lanes on 8
//      different 16-byte bank groups.
//   V^T: piece c (0..3) of row d at piece 4 d + (c ^ ((d >> 1) & 3)); 8
//      consecutive lanes read 8 consecutive rows, again on distinct groups.
//   scales: s_k[64] at byte 0, s_v[64] at byte 256 of the scale area.
template <int D>
struct TileLds {
  static constexpr int KC = D / 16;  // K chunks (= V chunks)
  static constexpr int V_OFF = KC * 1024;
  static constexpr int S_OFF = 2 * KC * 1024;
  static constexpr int BYTES = 2 * KC * 1024 + 512;
  static constexpr int COPIES = KC / 2 + 1;  // copy instructions per wave and tile
};

constexpr int kWaves = 4;          // waves per workgroup, one per SIMD
constexpr int kBufs = 4;           // LDS ring of tile buffers

template <int D>
__device__ inline int ksw(int r) {
  return D == 128 ? ((r & 3) | (((r >> 4) & 1) << 2)) : (((r >> 1) & 1) | (((r >> 4) & 1) << 1));
}
__device__ inline int vsw(int d) { return (d >> 1) & 3; }

struct TileSrc {
  const uint8_t* kbase;  // codes_k of the head
  const uint8_t* vbase;  // codes_v of the head
  const float* skb;      // scale_k of the head
  const float* svb;      // scale_v of the head
};

// Per-lane source offsets of one wave's copies.  Wave w copies K chunks
// w, w + 4, .. (chunk c holds pieces P = 64 c + lane: row r = P / (D/16),
// stored piece P % (D/16)), the V chunks with the same numbers, and a quarter
// of the scales.  With the swizzle, the source column of a K piece depends on
// the lane and on one bit of c (bit 1 for D = 128, bit 0 for D = 64) that is
// the same for all of a wave's chunks, so one offset (relative to the chunk's
// first row) serves them all; V likewise.
template <int D>
struct CopyOffsets {
  uint32_t k, v;
  __device__ CopyOffsets(int wave, int lane) {
    constexpr int PR = D / 16;  // pieces per K row
    const int P = wave * 64 + lane, r = P / PR, lc = (P % PR) ^ ksw<D>(r);
    k = (uint32_t)((r - wave * (64 / PR)) * D + 16 * lc);
    const int d = lane >> 2;  // row within a V chunk (16 rows of 64 bytes)
    // source: 16-slot sub-tile p = (lane & 3) ^ vsw(d) of the tile, row d of
    // the chunk's 16 (the cache stores V^T as [16-slot group][D][16])
    v = (uint32_t)(16 * D * ((lane & 3) ^ vsw(d)) + 16 * d);
  }
};

__device__ inline void copy16(const void* gp, lds_u8* lp) {
  __builtin_amdgcn_global_load_lds((global_void*)gp, (lds_void*)lp, 16, 0, 0);
}

// Copy tile T of the head into an LDS buffer (this wave's share: the same
// number of copy instructions in every wave).  With static scales (ST) the
// per-slot scales are not needed and not copied.
template <int D, bool ST = false>
__device__ inline void copy_tile(lds_u8* lbuf, const TileSrc& src, int T, const CopyOffsets<D>& co,
                                 int wave, int lane) {
  constexpr int KC = TileLds<D>::KC;
  const uint8_t* kt = src.kbase + (size_t)T * kTile * D;
  const uint8_t* vt = src.vbase + (size_t)T * kTile * D;
#pragma unroll
  for (int j = 0; j < KC / 4; ++j) {
    const int c = wave + 4 * j;
    copy16(kt + c * 1024 + co.k, lbuf + c * 1024);
    copy16(vt + c * 256 + co.v, lbuf + TileLds<D>::V_OFF + c * 1024);
  }
  // scales: waves 0, 1 copy s_k[32 w, +32), waves 2, 3 s_v[32 (w - 2), +32),
  // 4 per lane on lanes 0..7
  if constexpr (!ST) {
    const float* sb = (wave < 2 ? src.skb : src.svb) + T * kTile + 32 * (wave & 1);
    if (lane < 8) copy16(sb + 4 * lane, lbuf + TileLds<D>::S_OFF + 128 * wave);
  }
}

// Wait until at most N of this wave's vector memory operations are in flight
// (the copies of the tiles after the one needed), then meet the other waves:
// after the barrier every wave's copies of that tile have landed.  One asm
// block, so no LDS access moves across it.
template <int N>
__device__ inline void wait_copies_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
// The same with at most n tiles' copies (CW instructions each) in flight,
// n = 0 .. 3.
template <int CW>
__device__ inline void wait_tiles_and_barrier(int n) {
  switch (n) {
    case 0: wait_copies_and_barrier<0>(); break;
    case 1: wait_copies_and_barrier<CW>(); break;
    case 2: wait_copies_and_barrier<2 * CW>(); break;
    default: wait_copies_and_barrier<3 * CW>(); break;
  }
}

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
};

__device__ inline v8i lds32(const lds_u8* p0, const lds_u8* p1) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) const u32x4 lds_u4;
  const u32x4 a = *reinterpret_cast<lds_u4*>(p0);
  const u32x4 b = *reinterpret_cast<lds_u4*>(p1);
  v8i r;
  r[0] = (int)a[0]; r[1] = (int)a[1]; r[2] = (int)a[2]; r[3] = (int)a[3];
  r[4] = (int)b[0]; r[5] = (int)b[1]; r[6] = (int)b[2]; r[7] = (int)b[3];
  return r;
}

// Per-lane byte offsets of the operand pieces inside a tile buffer.  With
// the swizzles the lane-dependent part of every K piece is one of 2 KS values
// (the half h and block ks enter by XOR) and the slot half sub by a constant;
// V pieces by XOR of the half h and a constant per 32-row block.
template <int D>
struct TileOffsets {
  uint32_t k[D / 64][2];
  uint32_t v[2];
  uint32_t sk4;  // key scales of slots 16 gq .. 16 gq + 15 (every lane of the half reads them)
  uint32_t sv4;  // value scales of the same slots
  __device__ TileOffsets(int lane) {
    const int li = lane & 31, gq = lane >> 5;
    const int krow = 16 * ((li >> 2) & 1) + 4 * (li >> 3) + (li & 3);
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
      for (int h = 0; h < 2; ++h) k[ks][h] = (uint32_t)(krow * D + 16 * ((4 * ks + 2 * gq + h) ^ ksw<D>(krow)));
#pragma unroll
    for (int h = 0; h < 2; ++h) v[h] = (uint32_t)(TileLds<D>::V_OFF + 64 * li + 16 * ((gq + 2 * h) ^ vsw(li)));
    sk4 = (uint32_t)(TileLds<D>::S_OFF + 64 * gq);
    sv4 = (uint32_t)(TileLds<D>::S_OFF + 256 + 64 * gq);
  }
};

template <int D>
__device__ inline void read_k(KOp<D>& f, const lds_u8* lb, const TileOffsets<D>& o) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)  // slot half sub: rows + 32, a constant offset (ksw ignores bit 5)
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks)
      f.k[sub][ks] = lds32(lb + 32 * D * sub + o.k[ks][0], lb + 32 * D * sub + o.k[ks][1]);
}

template <int D>
__device__ inline void read_v(VOp<D>& f, const lds_u8* lb, const TileOffsets<D>& o) {
#pragma unroll
  for (int b = 0; b < D / 32; ++b)  // row block b: rows + 32 b, a constant offset (vsw ignores bit 5)
    f.v[b] = lds32(lb + 2048 * b + o.v[0], lb + 2048 * b + o.v[1]);
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

// Softmax of one tile's S^T (in registers), in two parts.
// The queries carry the softmax scale log2(e)/sqrt(D), so S is in log2
// units once multiplied by the key scale s_k.  Scores are kept relative to
// mc = m - log2 c_h (m the running max): y - mc = fma(S, s_k, -mc), one
// instruction per score, with the old mc; a tile that raises the max shifts
// its scores by the change.  P' = exp2(y - mc) = P c_h, x = P' s_v, and the
// running sum l accumulates P' (so the output is O / l).  The key and value
// scales of the 16 slots of a lane's half arrive as 16-byte LDS reads that
// every lane of the half shares, one value per accumulator register.
// The running max m starts at the first tile's max and moves only in whole
// steps (log2 units): when a tile's max exceeds it by more than the headroom
// kLazy, m rises by the ceiling of the excess, so the factor 2^(m_old -
// m_new) that rescales O, l and the P V products of the tile before (issued
// after the raise, with the factor in their scale operand) is an exact
// power of two.
// ST (the pages' static per-head scales, every valid slot of the head
// carrying them): s_k is already in the queries, so y - mc = S - mc, and
// l2c = log2 7, so P' = 7 P is fed as x directly (7 = 448 / 64, the
// headroom); s_v is applied once to the output.  No per-slot scale is read.
//
// Part A: scores relative to mc, the mask, the tile max and the lazy raise.
// Returns the (integer, <= 0) exponent of the rescale factor, 0 without a
// raise.
template <int D, bool ST>
__device__ inline int softmax_a(v16f (&acc)[2], WaveState<D>& st, unsigned long long mask, float l2c, int lane,
                                const lds_u8* sp) {
  constexpr int DB = D / 32;
  typedef float v4f __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) const v4f lds_v4f;
  const int gq = lane >> 5;
  // before the first tile there is no max: scores relative to 0, and the
  // first tile always raises the max
  const float mcu = st.m == -INFINITY ? 0.f : st.m - l2c;
  if constexpr (ST) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[0][r] -= mcu;
      acc[1][r] -= mcu;
    }
  } else {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {  // the scales of a slot half, four reads issued before their use
      v4f sk[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) sk[w] = *reinterpret_cast<lds_v4f*>(sp + 128 * sub + 16 * w);
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[sub][4 * w + e] = __builtin_fmaf(acc[sub][4 * w + e], sk[w][e], -mcu);
    }
  }
  if (mask != ~0ull) {  // partially valid tile (ring edge, partial fill, padding)
    const uint32_t m0 = (uint32_t)(mask >> (16 * gq)) & 0xFFFFu;  // slots 16 gq + r
    const uint32_t m1 = (uint32_t)(mask >> (32 + 16 * gq)) & 0xFFFFu;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (!((m0 >> r) & 1u)) acc[0][r] = -INFINITY;
      if (!((m1 >> r) & 1u)) acc[1][r] = -INFINITY;
    }
  }
  float tmax = fmaxf(acc[0][0], acc[1][0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) tmax = fmaxf(fmaxf(tmax, acc[0][r]), acc[1][r]);  // max3 chain
  tmax = half_swap_max(tmax) + mcu;  // the tile's max of y
  int dm = 0;
  if (__ballot(tmax > st.m + kLazy) != 0ull) {
    // The first raise sets the tile's max (there is nothing to rescale: O
    // and l are zero); a later one moves m up by a whole number, at least
    // to the tile's max.
    const bool first = st.m == -INFINITY;
    const float d = first ? -256.f : -ceilf(fmaxf(tmax - st.m, 0.f));
    const float mnew = first ? tmax : st.m - d;
    const float alpha = __builtin_amdgcn_exp2f(d);
    st.l *= alpha;
#pragma unroll
    for (int b = 0; b < DB; ++b) st.O[b] *= alpha;
    st.m = mnew;
    const float shift = (mnew - l2c) - mcu;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[0][r] -= shift;
      acc[1][r] -= shift;
    }
    dm = (int)d;
  }
  return dm;
}

// Part B: P' = exp2 of the shifted scores, the running sum, and the P terms
// of the tile (high, and with two terms the low term 16 (x - e4m3(x))),
// interleaved with the wave's matrix work of the iteration: the P V products
// of the tile before (values in LDS at vb, its P terms ph0/pl0, e = their
// rescale exponent) and the Q K^T products of the tile after (keys at kb ->
// snext).  A wave that issues matrix instructions back to back stalls the
// vector ALU of its SIMD while it waits for the matrix unit; between vector
// instructions of its own, each one issues as the previous one finishes.
// Matrix operands and value scales are read from LDS one step before their
// use, so that few registers hold them.  QK_ON false: no tile after (snext
// stays zero).
template <int D, int TERMS, bool ST, int QT, bool QK_ON = true>
__device__ inline void softmax_b_mfma(v16f (&acc)[2], WaveState<D>& st, const lds_u8* sp, v8i& ph, v8i& pl,
                                      const lds_u8* vb, const v8i& ph0, const v8i& pl0, int e, const lds_u8* kb,
                                      const TileOffsets<D>& off, const v8i (&qf)[QT][D / 64], const int (&qs)[QT],
                                      v16f (&snext)[2]) {
  // x = P' s_v is formed once and reused; contracting x - e4m3(x) into
  // fma(P', s_v, -e4m3(x)) would recompute the product
#pragma clang fp contract(off)
  constexpr int DB = D / 32, KS = D / 64;
  typedef float v4f __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) const v4f lds_v4f;
  // the P V products of the tile before, rescaled by 2^e through the scale
  // operand (e >= -127: a smaller factor leaves nothing of them in fp32)
  const int eh = 127 + (e < -127 ? -127 : e);
  const int el = eh - 4 < 0 ? 0 : eh - 4;
  // Matrix instruction k: first the P V products (block b, term t), then the
  // next tile's Q K^T products (slot half sub and block ks, query term t).
  // Operand n (of NOP) is the values of block b, then the keys of (sub, ks).
  constexpr int NPV = DB * TERMS, NM = NPV + 2 * KS * QT;
  constexpr int SPG = (NM + 7) / 8;  // matrix instructions per group of 4 scores
  auto op_of = [](int k) { return k < NPV ? k / TERMS : DB + (k - NPV) / QT; };
  auto load_op = [&](int n) {
    if (n < DB) return lds32(vb + 2048 * n + off.v[0], vb + 2048 * n + off.v[1]);
    const int sub = (n - DB) / KS, ks = (n - DB) % KS;
    return lds32(kb + 32 * D * sub + off.k[ks][0], kb + 32 * D * sub + off.k[ks][1]);
  };
  v8i opr[2];  // operand double buffer: operand n in opr[n % 2]
  auto mm = [&](int k) {
    if (k >= NM) return;
    const v8i& a = opr[op_of(k) % 2];
    if (k < NPV) {
      const int b = k / TERMS, t = k % TERMS;
      st.O[b] = mfma_fp8(a, t == 0 ? ph0 : pl0, st.O[b], 127, t == 0 ? eh : el);
    } else {
      const int k2 = k - NPV, sub = (k2 / QT) / KS, ks = (k2 / QT) % KS, t = k2 % QT;
      if constexpr (QK_ON) snext[sub] = mfma_fp8(a, qf[t][ks], snext[sub], 127, qs[t]);
    }
    // the next instruction's operand, if it needs a new one
    if (k + 1 < NM && op_of(k + 1) != op_of(k)) opr[op_of(k + 1) % 2] = load_op(op_of(k + 1));
  };
  auto read_sv = [&](int w) { return *reinterpret_cast<lds_v4f*>(sp + 256 + 128 * (w >> 2) + 16 * (w & 3)); };
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) snext[sub] = v16f{};
  opr[0] = load_op(0);
  v4f sv[2];  // value scales of group w in sv[w % 2], read one group ahead
  if constexpr (!ST) sv[0] = read_sv(0);
  // P' <= 64 c_h and s_v c_h <= 7, so the conversions below never
  // overflow (fp32 rounding a hair above 448 still rounds to 448 in e4m3).
  // The vector work of each group of 4 scores comes in up to three pieces,
  // each after one matrix instruction; scheduling barriers keep that order.
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int sub = w >> 2, r0 = 4 * (w & 3);
    mm(w * SPG);
    if constexpr (!ST) {
      if (w + 1 < 8) sv[(w + 1) % 2] = read_sv(w + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    float x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float p = __builtin_amdgcn_exp2f(acc[sub][r0 + k]);
      st.l += p;
      x[k] = p;
    }
    __builtin_amdgcn_sched_barrier(0);
    if (SPG > 1) {
      mm(w * SPG + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!ST) {
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = x[k] * sv[w % 2][k];
    }
    // (the low-half conversion keeps the high half of its third operand,
    // which the high-half conversion overwrites: any value will do)
    uint32_t blank;  // an opaque value (the asm defines it), so no copy is needed
    asm volatile("" : "=v"(blank));
    uint32_t hw = pack2_fp8<false>(x[0], x[1], blank);
    hw = pack2_fp8<true>(x[2], x[3], hw);
    ph[w] = (int)hw;
    if (TERMS == 2) {  // second term: 16 (x - e4m3(x)), descaled by 2^-4
      float d0, d1, d2, d3;
      unpack4_fp8(hw, d0, d1, d2, d3);
      __builtin_amdgcn_sched_barrier(0);
      if (SPG > 2) {
        mm(w * SPG + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
      const float l0 = x[0] - d0;
      uint32_t lw = pack2_fp8_div<false>(l0, x[1] - d1, __float_as_uint(l0), 0.0625f);
      lw = pack2_fp8_div<true>(x[2] - d2, x[3] - d3, lw, 0.0625f);
      pl[w] = (int)lw;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int k = 8 * SPG; k < NM; ++k) mm(k);
}

template <int D>
struct __attribute__((aligned(16))) AttnSmem {
  uint8_t kv[kBufs][TileLds<D>::BYTES];  // ring of tile buffers
  int flag;
};

// ---------------------------------------------------------------------------
// Query preparation, one launch before the attention: RoPE at q_pos (angles
// in double precision) and the split of each (query, head) row into QT
// e4m3 terms with power-of-two scales: term t holds e4m3(y_t / 2^e_t) with
// e_t the smallest exponent that fits the row (448 * 2^e_t >= amax), y_0 = y
// and y_{t+1} the residual; the E8M0 operand 127 + e_t of the matrix
// instruction applies 2^e_t exactly.  Rows n_q .. nq_rows - 1 are zero.
// 8 threads per row, each with D/16 RoPE pairs.
struct QPrepArgs {
  Geom g;
  AttnWs ws;
  int n_q;
  int nq_rows;  // 128-query groups of this call x 128
  const uint4* q;  // bf16 [n_q][H][D]
  const int32_t* q_pos;
  float qscale;  // softmax scale in log2 units, log2(e) / sqrt(D), rounded once to float
  const uint16_t* wq;  // query RMS-norm weights (bf16 [D]) of the fused pre-attention norm, null when off
  float eps;           // its epsilon
  int layer;           // the cache layer (its static scales, when calibrated)
};

// Body of one 256-thread workgroup number `block` of the preparation.
template <int D, int QT>
__device__ inline void q_prep_body(const QPrepArgs& A, int block) {
  constexpr int TPR = 8;          // threads per row
  constexpr int EPT = D / TPR;    // elements per thread: 16 or 8
  const int H = A.g.n_heads;
  const int r = (int)((block * 256 + threadIdx.x) / TPR);  // h * nq_rows + qi
  const int part = (int)(threadIdx.x % TPR);
  {  // the arrival words of this call's units start at zero
    const int gt = (int)(block * 256 + threadIdx.x);
    if (gt < H * (A.nq_rows / 128)) A.ws.sync[(size_t)gt * kSyncStride] = 0ull;
  }
  if (r >= H * A.nq_rows) return;  // whole rows only: the reductions stay inside live lanes
  const int h = r / A.nq_rows, qi = r % A.nq_rows;
  // rows past n_q read row n_q - 1 (every load in range, no branch around
  // the loads) and are zeroed
  const bool active = qi < A.n_q;
  const int qr = active ? qi : A.n_q - 1;
  const uint4* qp = A.q + ((size_t)qr * H + h) * (D / 8) + part * (EPT / 8);
  const int32_t* pq = A.q_pos + (size_t)qr * A.g.pos_stride;  // (t) or (t, y, x)
  const int j0 = part * (EPT / 2);                             // this thread's first RoPE pair
  const double* turns = omega_turns(A.g) + j0;
  float xs[EPT];
#pragma unroll
  for (int c = 0; c < EPT / 8; ++c) {
    const uint4 w = qp[c];
    const float xv[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                         bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
    for (int e = 0; e < 8; ++e) xs[8 * c + e] = active ? xv[e] : 0.f;
  }
  if (A.wq != nullptr) {  // fused RMS norm of the query row, before RoPE
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) ss = fmaf(xs[e], xs[e], ss);
    const float rn = rms_factor<TPR>(ss, 1.f / D, A.eps);
    const uint4* wp = reinterpret_cast<const uint4*>(A.wq) + part * (EPT / 8);
#pragma unroll
    for (int c = 0; c < EPT / 8; ++c) {
      const uint4 w = wp[c];
      const float wv[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                           bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[8 * c + e] = xs[8 * c + e] * rn * wv[e];
    }
  }
  // With the pages' static scales the head's key scale is folded into the
  // query, so the products with the key codes come out in log2 units.
  float qsc = A.qscale;
  {
    const LayerPtrs L = layer_ptrs(A.g, A.layer);
    if (static_head(L, H, h)) qsc = A.qscale * L.stat[h];
  }
  float y[EPT];
  float am = 0.f;
#pragma unroll
  for (int c = 0; c < EPT / 8; ++c) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float cs, sn;
      rope_cs(pair_coord(A.g, pq, j0 + 4 * c + m), turns[4 * c + m], cs, sn);
      const float x0 = xs[8 * c + 2 * m], x1 = xs[8 * c + 2 * m + 1];
      y[8 * c + 2 * m] = (x0 * cs - x1 * sn) * qsc;
      y[8 * c + 2 * m + 1] = (x0 * sn + x1 * cs) * qsc;
      am = fmaxf(am, fmaxf(fabsf(y[8 * c + 2 * m]), fabsf(y[8 * c + 2 * m + 1])));
    }
  }
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    am = group_max<TPR>(am);
    const int e = am > 0.f ? pow2_exponent(am) : 0;
    uint32_t wd[EPT / 4];
    float nm = 0.f;
#pragma unroll
    for (int c = 0; c < EPT / 4; ++c) {
      float* yy = &y[4 * c];
      // |y| <= 448 * 2^e by the choice of e: no clamping needed
      const float z0 = ldexpf(yy[0], -e);
      const uint32_t cw = pack2_fp8<false>(z0, ldexpf(yy[1], -e), __float_as_uint(z0));
      wd[c] = pack2_fp8<true>(ldexpf(yy[2], -e), ldexpf(yy[3], -e), cw);
      if (t + 1 < QT) {
        float d0, d1, d2, d3;
        unpack4_fp8(wd[c], d0, d1, d2, d3);
        yy[0] -= ldexpf(d0, e);
        yy[1] -= ldexpf(d1, e);
        yy[2] -= ldexpf(d2, e);
        yy[3] -= ldexpf(d3, e);
        nm = fmaxf(nm, fmaxf(fmaxf(fabsf(yy[0]), fabsf(yy[1])), fmaxf(fabsf(yy[2]), fabsf(yy[3]))));
      }
    }
    const size_t row = ((size_t)t * H + h) * A.ws.nq_pad + qi;
    // codes in the order the attention's lanes read them as matrix operands
    // (qcodes in rkv_launch.h): dims [d0, d0 + EPT) lie in 32-byte chunk
    // d0 / 32 of the row, block ks = d0 / 64, lane half gq = chunk % 2
    const int d0 = part * EPT;
    const size_t opnd = ((row / 32) * (D / 64) + d0 / 64) * 64 + (qi % 32) + 32 * ((d0 / 32) % 2);
    uint8_t* dst = A.ws.qcodes + opnd * 32 + d0 % 32;
    if constexpr (EPT == 16) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    } else {
      *reinterpret_cast<uint2*>(dst) = make_uint2(wd[0], wd[1]);
    }
    if (part == 0) A.ws.qexp[row] = 127 + e;  // E8M0 code of 2^e
    am = nm;
  }
}

template <int D, int TERMS>
__global__ __launch_bounds__(256) void q_prep_kernel(QPrepArgs A) {
  q_prep_body<D, q_terms<TERMS>()>(A, (int)blockIdx.x);
}

// Write and query preparation in one launch (D = 128: both use 256-thread
// workgroups): the first wgs workgroups write the new tokens, the rest
// prepare the queries.  The two touch disjoint memory.
struct WritePrepArgs {
  QPrepArgs P;
  int layer;
  const uint4* k;
  const uint4* v;
  const int32_t* pos;
  int n;
  int groups, items, wgs;  // the write's work items and workgroups (write_grid)
  const uint16_t* wk;  // key RMS-norm weights, null when off (epsilon in P.eps)
};

template <int HG, int TERMS>
__global__ __launch_bounds__(256) void write_prep_kernel(WritePrepArgs W) {
  const int b = (int)blockIdx.x, nw = W.wgs;
  if (b < nw)
    write_rope_fp8_body<128, HG>(W.P.g, W.layer, W.k, W.v, W.pos, W.n, W.wk, W.P.eps, b, nw, W.groups, W.items, b,
                                 nw);
  else
    q_prep_body<128, q_terms<TERMS>()>(W.P, b - nw);
}

__device__ inline v8i gload32(const uint8_t* p) {
  const uint4 a = reinterpret_cast<const uint4*>(p)[0];
  const uint4 b = reinterpret_cast<const uint4*>(p)[1];
  v8i r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
  return r;
}

// Output of one query row held by a lane, NB 32-dim blocks from orow:
// O^T[d][query] for d = 32 b + 8 (r / 4) + 4 gq + r % 4, scaled by inv, as bf16.
template <int NB>
__device__ inline void store_rows(uint16_t* orow, const v16f (&O)[NB], float inv, int gq) {
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const uint32_t lo = f32_to_bf16_rne(O[b][4 * g4] * inv) | (f32_to_bf16_rne(O[b][4 * g4 + 1] * inv) << 16);
      const uint32_t hi = f32_to_bf16_rne(O[b][4 * g4 + 2] * inv) | (f32_to_bf16_rne(O[b][4 * g4 + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + 32 * b + 8 * g4 + 4 * gq) = make_uint2(lo, hi);
    }
}

// ---------------------------------------------------------------------------
// Split-unit partials.  part_o: per segment and wave, the wave's 32 queries x
// D dims of O / l as fp16, in D/16 chunks of 16 bytes per lane (chunk 2 b + c
// holds register values 8 c .. 8 c + 7 of block b), chunk-major so that every
// store and load covers 1 KiB contiguously.  part_ml: per segment, wave and
// lane, the row's (max, sum).
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
constexpr int kSc1 = 16;                 // buffer cache-policy operand: sc1
constexpr int kRsrcWord3 = 0x00020000;   // raw byte-addressed buffer, 32-bit dwords

struct PartRsrc {
  __amdgpu_buffer_rsrc_t o, ml;
  template <int D>
  __device__ static PartRsrc make(const AttnWs& ws, int segs) {
    PartRsrc r;
    r.o = __builtin_amdgcn_make_buffer_rsrc(ws.part_o, 0, segs * 128 * D * 2, kRsrcWord3);
    r.ml = __builtin_amdgcn_make_buffer_rsrc(ws.part_ml, 0, segs * kWaves * 64 * 8, kRsrcWord3);
    return r;
  }
};

__device__ inline int pack_h2(float a, float b) {
  const h2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(int, v);
}

// chunk0: index of the lane's first 16-byte chunk (chunk c at chunk0 + 64 c)
template <int D>
__device__ inline void store_partial(const PartRsrc& pr, int chunk0, const v16f (&O)[D / 32], float inv) {
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      v4i d;
#pragma unroll
      for (int k = 0; k < 4; ++k) d[k] = pack_h2(O[b][8 * c + 2 * k] * inv, O[b][8 * c + 2 * k + 1] * inv);
      __builtin_amdgcn_raw_buffer_store_b128(d, pr.o, (chunk0 + 64 * (2 * b + c)) * 16, 0, kSc1);
    }
}

__device__ inline void store_ml(const PartRsrc& pr, int idx, float m, float l) {
  const v2i d = {__float_as_int(m), __float_as_int(l)};
  __builtin_amdgcn_raw_buffer_store_b64(d, pr.ml, idx * 8, 0, kSc1);
}

// Merge of one output block of split unit u: query slice qs (32 queries) x
// dim block b (32 dims), over all the unit's segments in segment order, by
// one wave (the same arithmetic whichever wave and workgroup does it).  With
// an even split (ek > 0 ranges per unit, none empty) the unit's ranges are
// u ek .. u ek + ek - 1.  Otherwise the segment of the workgroup range
// holding (unit, tile) pair y is floor(((y + 1) G - 1) / W), and the next
// starts at that range's end.  Segments are taken kMB at a time, their loads
// issued together; a short batch points its spare loads past the end of the
// buffer, which returns zeros without a memory access.
template <int D>
__device__ __attribute__((always_inline)) inline void merge_block(const PartRsrc& pr, int u, int count, long long W,
                                                                  int G, int ek, int qs, int b, int lane,
                                                                  uint16_t* orow, bool store, float ch, int gq) {
  constexpr int CH = D / 16, kMB = 8;
  constexpr int kPast = 0x40000000;  // a byte offset beyond any partial buffer
  const long long uhi = (long long)(u + 1) * count;
  long long y = (long long)u * count;
  int j0 = 0;  // even split: the batch's first range of the unit
  float Mu = -INFINITY, Lu = 0.f;
  v16f acc = v16f{};
  while (ek > 0 ? j0 < ek : y < uhi) {
    int sg[kMB];
    bool ok[kMB];
#pragma unroll
    for (int k = 0; k < kMB; ++k) {
      if (ek > 0) {
        ok[k] = j0 + k < ek;
        sg[k] = u * ek + j0 + k + u;
      } else {
        const long long w = y < uhi ? ((y + 1) * G - 1) / W : -1;
        ok[k] = w >= 0;
        sg[k] = (int)w + u;
        if (ok[k]) y = (w + 1) * W / G;
      }
    }
    j0 += kMB;
    v2i ml[kMB];
    v4i o[kMB][2];
#pragma unroll
    for (int k = 0; k < kMB; ++k) {
      const int base = sg[k] * kWaves + qs;
      ml[k] = __builtin_amdgcn_raw_buffer_load_b64(pr.ml, ok[k] ? (base * 64 + lane) * 8 : kPast, 0, kSc1);
#pragma unroll
      for (int c = 0; c < 2; ++c)
        o[k][c] = __builtin_amdgcn_raw_buffer_load_b128(pr.o, ok[k] ? ((base * CH + 2 * b + c) * 64 + lane) * 16 : kPast,
                                                        0, kSc1);
    }
    float Mb = Mu;
#pragma unroll
    for (int k = 0; k < kMB; ++k)
      if (ok[k]) Mb = fmaxf(Mb, __int_as_float(ml[k][0]));
    const float sc = __builtin_amdgcn_exp2f(Mu - Mb);  // 0 on the first batch
    Lu *= sc;
    acc *= sc;
#pragma unroll
    for (int k = 0; k < kMB; ++k) {
      const float wk = ok[k] ? __builtin_amdgcn_exp2f(__int_as_float(ml[k][0]) - Mb) * __int_as_float(ml[k][1]) : 0.f;
      Lu += wk;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // (the element goes through a scalar first: a bit_cast of a vector
          // element directly reads element 0)
          const int wd = o[k][c][e];
          const h2 v = __builtin_bit_cast(h2, wd);
          acc[8 * c + 2 * e] += wk * (float)v[0];
          acc[8 * c + 2 * e + 1] += wk * (float)v[1];
        }
    }
    Mu = Mb;
  }
  const v16f a1[1] = {acc};
  if (store) store_rows<1>(orow + 32 * b, a1, Lu > 0.f ? 1.f / (ch * Lu) : 0.f, gq);
}

constexpr int kLastArrival = 1 << 30;                  // flag beside a block mask
template <int D>
constexpr uint32_t kAllBlocks = (1u << (4 * (D / 32))) - 1u;  // 4 query slices x D/32 dim blocks

// Share of split unit u's output blocks that the workgroup with range gi
// merges when the unit is where its range ends: block j goes to the
// workgroup ranges spanning the unit round-robin, j = (gi - first) mod
// their number.  (Ranges that are empty when W < G take no part: their
// blocks fall to the last arrival.)
template <int D>
__device__ inline uint32_t merge_share(int u, int count, long long W, int G, int ek, int gi) {
  const long long w_first = ek > 0 ? (long long)u * ek : (((long long)u * count + 1) * G - 1) / W;
  const long long w_last = ek > 0 ? w_first + ek - 1 : (((long long)(u + 1) * count) * G - 1) / W;
  const int nseg = (int)(w_last - w_first + 1), sidx = gi - (int)w_first;
  uint32_t m = 0u;
  for (int j = sidx; j < 4 * (D / 32); j += nseg) m |= 1u << j;
  return m;
}

// Issue priority from progress: the two waves a SIMD holds come from two
// workgroups; the SIMD favours the older one, so without this the first
// workgroup of every compute unit finishes well before the second, which
// then runs alone.  A wave that is behind in its segment takes precedence.
__device__ inline void set_progress_priority(int j, int nk) {
  switch ((4 * j) / nk) {
    case 0: __builtin_amdgcn_s_setprio(3); break;
    case 1: __builtin_amdgcn_s_setprio(2); break;
    case 2: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

// ---------------------------------------------------------------------------
// Two workgroups of 4 waves per compute unit, one wave of each per SIMD.
// Each wave overlaps its own matrix and vector work: while it computes the
// softmax of tile j, its P V products of tile j - 1 and Q K^T products of
// tile j + 1 run on the matrix unit, one instruction issued between
// stretches of vector instructions.
template <int D, int TERMS>
__global__ __launch_bounds__(64 * kWaves, 2) void attend_kernel(AttnArgs A) {
  constexpr int KS = D / 64, DB = D / 32;
  __shared__ AttnSmem<D> sm;

  const Geom& g = A.g;
  const int H = g.n_heads, N = g.n_slots, NP = g.n_pad, NT = g.n_tiles;
  const int G = (int)gridDim.x;
  const int bid = (int)blockIdx.x;
  const int gi = G % 8 == 0 ? (bid & 7) * (G / 8) + (bid >> 3) : bid;  // this workgroup's range
  // wave w serves queries 32 w .. 32 w + 31 of the unit.  The wave index is
  // uniform per wave; readfirstlane lets the compiler keep what derives from
  // it in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int li = lane & 31, gq = lane >> 5;

  const LayerPtrs L = layer_ptrs(g, A.layer);
  const int U = A.nqg * H;
  // This wave's 32 prepared queries of unit u (B operand of S^T = K Q^T).
  constexpr int QT = q_terms<TERMS>();
  v8i qf[QT][KS];
  int qs[QT];
  auto load_q = [&](int u) {
    const int h = u / A.nqg, qi = kQG * (u % A.nqg) + 32 * wave + li;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const size_t row = ((size_t)t * H + h) * A.ws.nq_pad + qi;
      // lane l's 32 bytes of block ks are at operand index ((32-row block) KS + ks) 64 + l:
      // each wave's loads are contiguous 2 KiB
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[t][ks] = gload32(A.ws.qcodes + (((row / 32) * KS + ks) * 64 + lane) * 32);
      qs[t] = A.ws.qexp[row];
    }
  };
  // The ring state first: vector loads complete in issue order, so a state
  // read issued after the queries' loads would wait for all of them.
  const int head = L.state[0], nv = L.state[1], gv = L.state[3];
  // With a grid that is a multiple of the unit count, every range lies in
  // unit gi / (G / U) whatever the ring holds: its queries load while the
  // ring state is read.
  const int u_pre = G % U == 0 ? gi / (G / U) : -1;
  // The head's value bound and static-scale mode: read for that unit here,
  // before this kernel stores anything, they are scalar loads that no wait
  // for the queries' vector loads holds up (read in the loop they would
  // delay the first tile copies by the queries' round trip).
  auto head_consts = [&](int h, uint32_t& vm, bool& sh, float& svh) {
    vm = 0u;  // the head's bound: max over its kSub slots (bit order = value order)
#pragma unroll
    for (int k2 = 0; k2 < kSub; ++k2) vm = max(vm, L.vmax[h * kSub + k2]);
    // the pages' static per-head scales (every valid slot of the head
    // carries them): P' = 7 P with no per-slot factor, s_v on the output
    // (static_head, with the three words read together rather than one
    // after another)
    const int on = reinterpret_cast<const int*>(L.stat)[2 * H];
    const float skh = L.stat[h], svv = L.stat[H + h];
    sh = (on != 0) & (skh > 0.f) & (svv > 0.f);
    svh = sh ? svv : 1.f;
  };
  uint32_t vm_pre = 0u;
  bool sh_pre = false;
  float svh_pre = 1.f;
  if (u_pre >= 0) {
    load_q(u_pre);
    head_consts(u_pre / A.nqg, vm_pre, sh_pre, svh_pre);
  }
  int a = head - nv;
  if (a < 0) a += N;
  const int NTR = g.n_ring_tiles;
  const int T0 = a / kTile;  // tile of the oldest valid slot
  int count_r = 0;           // ring tiles holding valid slots, in cyclic order from T0
  if (nv > 0) {
    const int e = a + nv - 1;
    count_r = e < N ? e / kTile - T0 + 1 : (NTR - T0) + (e - N) / kTile + 1;
    if (count_r > NTR) count_r = NTR;
  }
  // then the tiles of the global slots below g_valid
  const int count = count_r + (gv + kTile - 1) / kTile;

  if (count == 0) {  // empty cache: every output row is zero
    for (int u = gi; u < U; u += G) {
      const int h = u / A.nqg, qi = kQG * (u % A.nqg) + 32 * wave + li;
      if (qi < A.n_q) {
        uint4* dst = reinterpret_cast<uint4*>(A.out + ((size_t)qi * H + h) * D + (D / 2) * gq);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) dst[c] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    return;
  }

  const TileOffsets<D> off(lane);
  const CopyOffsets<D> coff(wave, lane);
  lds_u8* const kv0 = (lds_u8*)&sm.kv[0][0];  // the tile buffers, as LDS addresses
  constexpr int KVB = TileLds<D>::BYTES;
  constexpr int C = TileLds<D>::COPIES;
  const long long W = (long long)U * count;
  // Range gi is pairs [gi W / G, (gi + 1) W / G) of the unit-major list.  An
  // even split -- ek = G / U ranges per unit, each holding at least one tile
  // -- puts range gi in unit gi / ek, as tiles [j count / ek, (j + 1) count /
  // ek) with j = gi mod ek: the same bounds in 32-bit arithmetic.  The
  // general case's 64-bit divisions are scalar routines of ~170 instructions
  // each, and the merges after the loop would need 2 per segment.
  const int ek = G % U == 0 && count >= G / U && (long long)G * count < (1ll << 31) ? G / U : 0;
  long long r_lo, r_hi;
  int u_first;  // unit of the range's first pair
  if (ek > 0) {
    u_first = gi / ek;
    const int j = gi - u_first * ek;
    r_lo = (long long)u_first * count + j * count / ek;
    r_hi = (long long)u_first * count + (j + 1) * count / ek;
  } else {
    r_lo = (long long)gi * W / G;
    r_hi = (long long)(gi + 1) * W / G;
    u_first = (int)(r_lo / count);
  }
  auto tile_of = [&](int kk) {
    if (kk >= count_r) return NTR + (kk - count_r);  // global tiles follow the ring's
    const int T = T0 + kk;
    return T >= NTR ? T - NTR : T;
  };
  int fin[2], nfin = 0;  // split units with output blocks for this workgroup to merge,
  int fin_blocks[2];     // ... those blocks, with kLastArrival if it was their last arrival

  // a segment that is not the range's last ends at its unit's end: the next
  // one starts at tile 0 of the next unit
  int u = u_first;
  for (long long x = r_lo; x < r_hi; ++u) {
    const int t_lo = (int)(x - (long long)u * count);
    const long long rem = r_hi - x;
    const int t_hi = rem < count - t_lo ? t_lo + (int)rem : count;
    x += t_hi - t_lo;
    const int nk = t_hi - t_lo;
    const int h = u / A.nqg, qg = u % A.nqg;
    uint32_t vm = vm_pre;
    bool sh = sh_pre;
    float svh = svh_pre;
    if (u != u_pre) head_consts(h, vm, sh, svh);
    const float vmaxh = __uint_as_float(vm);
    const float ch = vmaxh > 0.f ? kE4M3Max / (kHeadroom * vmaxh) : 1.f;
    const float l2c = sh ? kLog2Seven : __log2f(ch);
    TileSrc src;
    src.kbase = L.codes_k + (size_t)h * NP * D;
    src.vbase = L.codes_v + (size_t)h * NT * D * kTile;
    src.skb = L.scale_k + (size_t)h * NP;
    src.svb = L.scale_v + (size_t)h * NP;
    auto buf = [&](int tj) { return kv0 + (tj % kBufs) * KVB; };

    // ---- 1. the unit's queries (unless already loaded), then the copies of
    //         the first two tiles ----
    const int qi = kQG * qg + 32 * wave + li;
    if (u != u_pre) load_q(u);

    // ---- 2. the segment's tiles, copied two ahead into the ring of 4
    //         buffers (tile t in buffer t % 4), one barrier per tile.
    //         Iteration j computes the softmax of tile j between the P V
    //         products of tile j - 1 and the Q K^T products of tile j + 1 ----
    WaveState<D> st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b) st.O[b] = v16f{};
    auto run_tiles = [&](auto static_tag) {
      constexpr bool ST = decltype(static_tag)::value;
      // copy instructions per wave and tile (no scales with static scales)
      constexpr int CW = ST ? TileLds<D>::COPIES - 1 : TileLds<D>::COPIES;
      constexpr int AHEAD = kBufs - 2;  // tiles copied ahead of the one being read
      for (int tj = 0; tj < AHEAD && tj < nk; ++tj)
        copy_tile<D, ST>(buf(tj), src, tile_of(t_lo + tj), coff, wave, lane);
      // tile 0 has landed once at most the copies of tiles 1 .. AHEAD - 1 are in flight
      wait_tiles_and_barrier<CW>(nk - 1 < AHEAD - 1 ? nk - 1 : AHEAD - 1);
      v16f sacc[2];
      {
        KOp<D> kf;
        read_k<D>(kf, buf(0), off);
        qk<D, QT>(sacc, kf, qf, qs);
      }
      v8i ph0 = v8i{}, pl0 = v8i{};  // P terms of the tile before (none before tile 0)
      // Iteration j; QK: the Q K^T products of tile j + 1 (every iteration
      // but the last, which is peeled off the loop: a runtime test around
      // those products, or a second copy inside the loop, spilled registers)
      auto iter = [&](int j, auto qk_tag) {
        constexpr bool QK = decltype(qk_tag)::value;
        // Tile j + 1 (whose keys this iteration reads) has landed once at
        // most the copies of tiles j + 2, j + 3 are in flight; after the
        // barrier every wave is done with tile j - 2, whose buffer takes
        // tile j + AHEAD.
        const int last = nk - 1 < j + AHEAD - 1 ? nk - 1 : j + AHEAD - 1;  // last tile copied so far
        const int ahead = last - (j + 1);
        wait_tiles_and_barrier<CW>(ahead < 0 ? 0 : ahead);
        set_progress_priority(j, nk);
        if (j + AHEAD < nk) copy_tile<D, ST>(buf(j + AHEAD), src, tile_of(t_lo + j + AHEAD), coff, wave, lane);
        const lds_u8* lb = buf(j);
        // Only the first and last tiles of the ring's valid range, the
        // ring's last tile (pad slots) and the last global tile can hold
        // invalid slots: the others skip the mask.
        const int kk = t_lo + j;
        const int T = tile_of(kk);
        unsigned long long mask = ~0ull;
        if (kk == 0 || kk == count_r - 1 || kk == count - 1 || T == NTR - 1)
          mask = __ballot(slot_valid(g, T * kTile + lane, a, nv, gv));
        const int e = softmax_a<D, ST>(sacc, st, mask, l2c, lane, lb + off.sk4);
        // operands of the iteration's matrix work: the keys of tile j + 1
        // (none in the last iteration) and the values of tile j - 1 (before
        // tile 0, tile 0's: its products with the zero P terms add nothing,
        // and no code is a NaN)
        v16f snext[2];
        v8i ph, pl;
        softmax_b_mfma<D, TERMS, ST, QT, QK>(sacc, st, lb + off.sk4, ph, pl, buf(j > 0 ? j - 1 : 0), ph0, pl0, e,
                                             buf(QK ? j + 1 : j), off, qf, qs, snext);
        sacc[0] = snext[0];
        sacc[1] = snext[1];
        ph0 = ph;
        pl0 = pl;
      };
      for (int j = 0; j + 1 < nk; ++j) iter(j, std::true_type{});
      iter(nk - 1, std::false_type{});
      // the last tile's P V products
      VOp<D> vf;
      read_v<D>(vf, buf(nk - 1), off);
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        st.O[b] = mfma_fp8(vf.v[b], ph0, st.O[b], 127, 127);
        if (TERMS == 2) st.O[b] = mfma_fp8(vf.v[b], pl0, st.O[b], 127, 127 - 4);
      }
    };
    if (sh) run_tiles(std::true_type{});
    else run_tiles(std::false_type{});
    __builtin_amdgcn_s_setprio(0);

    // ---- 3. whole unit: output; split unit: partial, the last to finish merges ----
    const float Lw = half_swap_add(st.l);
    uint16_t* orow = A.out + ((size_t)qi * H + h) * D;
    if (t_lo == 0 && t_hi == count) {
      if (qi < A.n_q) store_rows<DB>(orow, st.O, Lw > 0.f ? svh / Lw : 0.f, gq);
    } else {
      // Partial id gi + u is distinct for every (workgroup, unit) pair: ranges
      // are ordered, so a later workgroup never meets an earlier unit.  The
      // partial is c_h O / l in fp16 (|c_h O / l| <= 448 * 7: the largest
      // e4m3 value code times s_v c_h) plus the row's max and sum in fp32.
      // Partials travel with sc1 (device-coherent) buffer accesses, the cache
      // policy of agent-scope relaxed atomics: stores write through and loads
      // bypass the per-XCD L2s, so no fence has to write back or invalidate a
      // whole L2.  Each thread's stores complete (vmcnt 0) before the barrier,
      // and the barrier before the counter update; the finisher reads only
      // after the counter says every segment has stored.
      const int seg = gi + u;
      const PartRsrc pr = PartRsrc::make<D>(A.ws, G + U);
      // (static scales: O / l is 7 P-weighted codes, and c_h s_v / l makes the
      // merge's final 1 / (c_h l) give s_v O / l)
      store_partial<D>(pr, (seg * kWaves + wave) * (D / 16) * 64 + lane, st.O, Lw > 0.f ? ch * svh / Lw : 0.f);
      store_ml(pr, (seg * kWaves + wave) * 64 + lane, st.m, Lw);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      // Arrival: one atomic add of (tiles | committed blocks << 32) on the
      // unit's word.  A workgroup whose range ends in this unit commits to
      // merge its share of the unit's output blocks after the loop; the
      // arrival that completes the tile count takes every block not
      // committed by another workgroup.
      const bool waits = x >= r_hi;
      if (threadIdx.x == 0) {
        const uint32_t commit = waits ? merge_share<D>(u, count, W, G, ek, gi) : 0u;
        const unsigned long long old = __hip_atomic_fetch_add(
            &A.ws.sync[(size_t)u * kSyncStride], (unsigned long long)nk | ((unsigned long long)commit << 32),
            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = (int)(uint32_t)old + nk == count;
        sm.flag = last ? kLastArrival | (int)(kAllBlocks<D> & ~(uint32_t)(old >> 32)) : (int)commit;
      }
      __syncthreads();
      if (sm.flag != 0) {  // blocks of this unit to merge after the loop
        fin[nfin] = u;
        fin_blocks[nfin++] = sm.flag;
      }
    }
    __syncthreads();  // LDS is reused by the next segment
  }

  // ---- 4. merges of split units.  The last arrival merges its blocks at
  //         once.  A committed workgroup waits (bounded) for the unit's tile
  //         count to complete, then merges its committed blocks; if its wait
  //         runs out it withdraws the commitment with a second atomic add,
  //         and merges them all the same if that add shows the count
  //         complete (the last arrival then excluded them), else leaves them
  //         to the last arrival.  Each block is merged exactly once, with the
  //         same arithmetic whoever merges it. ----
  for (int f = 0; f < nfin; ++f) {
    const int u = fin[f];
    int blocks = fin_blocks[f];
    if (!(blocks & kLastArrival)) {
      if (threadIdx.x == 0) {
        unsigned long long* const word = &A.ws.sync[(size_t)u * kSyncStride];
        bool ready = false;
        const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
        for (int it = 0; it < (1 << 16); ++it) {
          ready = (int)(uint32_t)__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == count;
          if (ready || __builtin_amdgcn_s_memrealtime() - t0 >= (unsigned long long)A.ws.wait_ticks) break;
          __builtin_amdgcn_s_sleep(2);
        }
        if (!ready) {
          const unsigned long long old = __hip_atomic_fetch_sub(word, (unsigned long long)(uint32_t)blocks << 32,
                                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((int)(uint32_t)old != count) blocks = 0;
        }
        sm.flag = blocks;
      }
      __syncthreads();
      blocks = sm.flag;
      __syncthreads();  // sm.flag is rewritten for the next unit
    }
    const int h = u / A.nqg, qg = u % A.nqg;
    uint32_t vm = 0u;
#pragma unroll
    for (int k2 = 0; k2 < kSub; ++k2) vm = max(vm, L.vmax[h * kSub + k2]);
    const float vmaxh = __uint_as_float(vm);
    const float ch = vmaxh > 0.f ? kE4M3Max / (kHeadroom * vmaxh) : 1.f;
    const PartRsrc pr = PartRsrc::make<D>(A.ws, G + U);
    uint32_t bits = (uint32_t)blocks & kAllBlocks<D>;
    for (int n = 0; bits; ++n) {  // the n-th block goes to wave n % 4
      const int j = __builtin_ctz(bits);
      bits &= bits - 1;
      if (n % kWaves == wave) {
        const int qs = j / DB, b = j % DB, qi = kQG * qg + 32 * qs + li;
        merge_block<D>(pr, u, count, W, G, ek, qs, b, lane, A.out + ((size_t)qi * H + h) * D, qi < A.n_q, ch, gq);
      }
    }
  }
}

static QPrepArgs make_prep_args(const Geom& g, const AttnWs& ws, int layer, const void* q, const int32_t* q_pos,
                                int n_q, const uint16_t* wq, float eps) {
  QPrepArgs P;
  P.layer = layer;
  P.wq = wq;
  P.eps = eps;
  P.g = g;
  P.ws = ws;
  P.n_q = n_q;
  P.nq_rows = ((n_q + kQG - 1) / kQG) * kQG;
  P.q = (const uint4*)q;
  P.q_pos = q_pos;
  P.qscale = (float)(kLog2e / std::sqrt((double)g.head_dim));
  return P;
}

static int prep_blocks(const QPrepArgs& P) {
  const int rows = P.g.n_heads * P.nq_rows, rows_per_block = 256 / 8;
  return (rows + rows_per_block - 1) / rows_per_block;
}

// The attention kernel alone (its queries prepared by an earlier launch on
// the stream).
static hipError_t launch_attend_main(const Geom& g, const AttnWs& ws, int layer, const void* q,
                                     const int32_t* q_pos, int n_q, void* out, hipStream_t s) {
  const int D = g.head_dim;
  const int nqg = (n_q + kQG - 1) / kQG;
  AttnArgs A;
  A.g = g;
  A.ws = ws;
  A.layer = layer;
  A.n_q = n_q;
  A.nqg = nqg;
  A.q = (const uint4*)q;
  A.q_pos = q_pos;
  A.out = (uint16_t*)out;
  // With at least one workgroup slot per unit, the grid is a multiple of the
  // unit count (preferably also of the 8 XCDs) that fills at least 7/8 of the
  // slots, so that every workgroup's range lies inside one unit: one segment
  // per workgroup, equal splits.  Without such a multiple (e.g. 288 units for
  // 512 slots) the full grid is used and ranges cross units.
  int G = ws.grid;
  const int U = nqg * g.n_heads;
  if (U <= ws.grid) {
    int best = 0;
    for (int kk = ws.grid / U; kk >= 1 && U * kk * 8 >= ws.grid * 7; --kk) {
      if (best == 0) best = U * kk;
      if (U * kk % 8 == 0) { best = U * kk; break; }
    }
    if (best > 0) G = best;
  }
  const dim3 grid(G);
  if (D == 128) {
    if (ws.terms == 2) hipLaunchKernelGGL((attend_kernel<128, 2>), grid, dim3(64 * kWaves), 0, s, A);
    else hipLaunchKernelGGL((attend_kernel<128, 1>), grid, dim3(64 * kWaves), 0, s, A);
  } else {
    if (ws.terms == 2) hipLaunchKernelGGL((attend_kernel<64, 2>), grid, dim3(64 * kWaves), 0, s, A);
    else hipLaunchKernelGGL((attend_kernel<64, 1>), grid, dim3(64 * kWaves), 0, s, A);
  }
  return hipGetLastError();
}

hipError_t launch_attend(const Geom& g, const AttnWs& ws, int layer, const void* q,
                         const int32_t* q_pos, int n_q, void* out, const uint16_t* wq, float eps,
                         hipStream_t s) {
  const QPrepArgs P = make_prep_args(g, ws, layer, q, q_pos, n_q, wq, eps);
  const dim3 pgrid(prep_blocks(P));
  if (g.head_dim == 128) {
    if (ws.terms == 2) hipLaunchKernelGGL((q_prep_kernel<128, 2>), pgrid, dim3(256), 0, s, P);
    else hipLaunchKernelGGL((q_prep_kernel<128, 1>), pgrid, dim3(256), 0, s, P);
  } else {
    if (ws.terms == 2) hipLaunchKernelGGL((q_prep_kernel<64, 2>), pgrid, dim3(256), 0, s, P);
    else hipLaunchKernelGGL((q_prep_kernel<64, 1>), pgrid, dim3(256), 0, s, P);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attend_main(g, ws, layer, q, q_pos, n_q, out, s);
}

template <int HG>
static void launch_write_prep_t(const WritePrepArgs& W, int blocks, int terms, hipStream_t s) {
  if (terms == 2) hipLaunchKernelGGL((write_prep_kernel<HG, 2>), dim3(blocks), dim3(256), 0, s, W);
  else hipLaunchKernelGGL((write_prep_kernel<HG, 1>), dim3(blocks), dim3(256), 0, s, W);
}

hipError_t launch_write_attend(const Geom& g, const AttnWs& ws, int layer, const void* k, const void* v,
                               const int32_t* pos, int n, const void* q, const int32_t* q_pos, int n_q,
                               void* out, const uint16_t* wq, const uint16_t* wk, float eps, hipStream_t s) {
  if (g.head_dim != 128) {  // 128-thread write workgroups: two launches, then the attention
    hipError_t e = launch_write(g, layer, k, v, pos, n, wk, eps, s);
    if (e != hipSuccess) return e;
    return launch_attend(g, ws, layer, q, q_pos, n_q, out, wq, eps, s);
  }
  WritePrepArgs W;
  W.P = make_prep_args(g, ws, layer, q, q_pos, n_q, wq, eps);
  W.wk = wk;
  W.layer = layer;
  W.k = (const uint4*)k;
  W.v = (const uint4*)v;
  W.pos = pos;
  W.n = n;
  int hg;
  write_grid(g, n, &W.groups, &hg, &W.items, &W.wgs);
  const int blocks = W.wgs + prep_blocks(W.P);
  if (hg == 2) launch_write_prep_t<2>(W, blocks, ws.terms, s);
  else launch_write_prep_t<1>(W, blocks, ws.terms, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attend_main(g, ws, layer, q, q_pos, n_q, out, s);
}

}  // namespace rkv
