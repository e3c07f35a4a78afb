// C ABI of the ring KV cache: argument validation, buffer layout and kernel
// launches.  No device allocation, no stream synchronization, no host read
// of device state (see include/rkv.h).
#include "rkv.h"

#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "rkv_launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return RKV_EHIP;
}

constexpr size_t kAlign = 256;
constexpr size_t kConstsBytes = 4096;
constexpr int kMaxWorkgroups = 4096;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Compute units of the current device (the persistent attention grid has two
// workgroups per unit); 256 on MI355X.
int compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
    return n;
  return 256;
}

struct Plan {
  rkv::Geom g;
  rkv::AttnWs ws;  // pointers filled relative to base 0 (offsets) until create
  size_t ws_parto, ws_partml, ws_sync, ws_qcodes, ws_qexp;
  size_t part_bytes;  // fp16 split-unit partials: (units + workgroups) x 128 queries x D x 2 bytes
  size_t total;
};

// The attention kernel addresses the split-unit partials through 32-bit
// buffer offsets and uses 2^30 as an offset past the end of the buffer, so
// that buffer must stay below 1 GiB: (units + workgroups) * 256 * D < 2^30,
// e.g. 256 heads x 14,000 queries at D = 128.
constexpr size_t kMaxPartBytes = size_t(1) << 30;

bool params_ok(const rkv_params* p, std::string* why) {
  if (!p) return *why = "params is null", false;
  if (p->n_layers < 1 || p->n_layers > 4096) return *why = "n_layers out of range [1, 4096]", false;
  if (p->n_slots < 1 || p->n_slots > (1 << 20)) return *why = "n_slots out of range [1, 2^20]", false;
  if (p->n_heads < 1 || p->n_heads > 256) return *why = "n_heads out of range [1, 256]", false;
  if (p->head_dim != 64 && p->head_dim != 128) return *why = "head_dim must be 64 or 128", false;
  if (p->max_queries < 1 || p->max_queries > (1 << 16))
    return *why = "max_queries out of range [1, 2^16]", false;
  if (p->precision != RKV_PRECISE && p->precision != RKV_FAST)
    return *why = "precision must be RKV_PRECISE or RKV_FAST", false;
  if (!(p->rope_base > 1.0f) || !std::isfinite(p->rope_base))
    return *why = "rope_base must be finite and > 1", false;
  if (!(p->scale_margin > 0.0f) || !(p->scale_margin <= 64.0f))
    return *why = "scale_margin must be in (0, 64]", false;
  if (p->attn_workgroups < 0 || p->attn_workgroups > kMaxWorkgroups)
    return *why = "attn_workgroups out of range [0, 4096]", false;
  if (p->attn_merge_wait_us < -1 || p->attn_merge_wait_us > 10000)
    return *why = "attn_merge_wait_us out of range [-1, 10000]", false;
  if (p->n_global < 0 || p->n_global > (1 << 20)) return *why = "n_global out of range [0, 2^20]", false;
  // The attention's split partials (one per unit and per workgroup, 128
  // queries x head_dim fp16) are addressed with 32-bit buffer offsets, and a
  // 1 GiB offset stands for "past the end" in the merge's spare loads: the
  // partial buffer must stay within 1 GiB (for head_dim 128 and the default
  // grid: units = ceil(max_queries / 128) x n_heads up to 28,672).
  {
    const long long units = ((long long)p->max_queries + 127) / 128 * p->n_heads;
    const long long grid = p->attn_workgroups > 0 ? p->attn_workgroups : kMaxWorkgroups;
    if ((units + grid) * 128 * p->head_dim * 2 > (1ll << 30))
      return *why = "ceil(max_queries / 128) x n_heads too large: the attention partials would exceed 1 GiB", false;
  }
  const int32_t* b = p->rope_bands;
  if (b[0] || b[1] || b[2]) {
    if (b[0] < 0 || b[1] < 0 || b[2] < 0 || b[0] + b[1] + b[2] != p->head_dim / 2)
      return *why = "rope_bands must be non-negative pair counts summing to head_dim / 2 (or all 0)", false;
  }
  return true;
}

Plan make_plan(const rkv_params* p) {
  Plan pl{};
  rkv::Geom& g = pl.g;
  const size_t H = p->n_heads, D = p->head_dim;
  // the ring, padded to whole tiles, then the global (sink) slots
  const size_t NR = align_up((size_t)p->n_slots, rkv::kTile);
  const size_t NP = NR + align_up((size_t)p->n_global, rkv::kTile);
  g.n_layers = p->n_layers;
  g.n_slots = p->n_slots;
  g.n_pad = (int32_t)NP;
  g.n_tiles = (int32_t)(NP / rkv::kTile);
  g.n_ring_pad = (int32_t)NR;
  g.n_ring_tiles = (int32_t)(NR / rkv::kTile);
  g.n_global = p->n_global;
  const int32_t* bands = p->rope_bands;
  if (bands[0] || bands[1] || bands[2]) {
    g.band_t = bands[0];
    g.band_ty = bands[0] + bands[1];
    g.pos_stride = 3;
  } else {
    g.band_t = g.band_ty = p->head_dim / 2;
    g.pos_stride = 1;
  }
  g.n_heads = p->n_heads;
  g.head_dim = p->head_dim;
  g.margin = p->scale_margin;
  g.consts = 0;
  g.layer0 = kConstsBytes;
  size_t o = 0;
  g.off_codes_k = o;
  o = align_up(o + H * NP * D, kAlign);
  g.off_codes_v = o;
  o = align_up(o + H * NP * D, kAlign);
  g.off_scale_k = o;
  o = align_up(o + H * NP * 4, kAlign);
  g.off_scale_v = o;
  o = align_up(o + H * NP * 4, kAlign);
  g.off_slot_pos = o;
  o = align_up(o + NP * 4, kAlign);
  g.off_slot_yx = o;
  o = align_up(o + 2 * NP * 4, kAlign);
  g.off_state = o;
  o = align_up(o + rkv::kStateRegionInts * 4, kAlign);
  g.off_vmax = o;
  o = align_up(o + H * rkv::kSub * 4, kAlign);
  g.off_normw = o;
  o = align_up(o + 2 * D * 2, kAlign);
  g.off_static = o;
  o = align_up(o + (2 * H + 1) * 4, kAlign);
  g.layer_bytes = o;

  size_t w = g.layer0 + (size_t)p->n_layers * g.layer_bytes;
  // Attention workspace: one partial result per segment of the persistent
  // grid -- at most units + workgroups of them, each 128 query rows x D fp16
  // plus (max, sum) per row and half-wave -- and per unit (head x 128-query
  // group) an arrival word on a line of its own.
  const size_t nqg = align_up((size_t)p->max_queries, 128) / 128;
  const size_t units = nqg * H;
  const int grid = p->attn_workgroups > 0 ? p->attn_workgroups : 2 * compute_units();
  const size_t segs = units + (size_t)grid;
  pl.ws.grid = grid;
  pl.ws.terms = p->precision == RKV_PRECISE ? 2 : 1;
  // the device real-time clock counts at 100 MHz
  pl.ws.wait_ticks = 100 * (p->attn_merge_wait_us < 0 ? 50 : p->attn_merge_wait_us);
  pl.ws_parto = w;
  pl.part_bytes = segs * 128 * D * 2;
  w = align_up(w + pl.part_bytes, kAlign);
  pl.ws_partml = w;
  w = align_up(w + segs * 4 * 64 * 2 * 4, kAlign);
  pl.ws_sync = w;
  w = align_up(w + units * rkv::kSyncStride * 8, kAlign);
  // prepared queries: up to three e4m3 terms per element and an exponent per row and term
  pl.ws.nq_pad = (int32_t)(nqg * 128);
  pl.ws_qcodes = w;
  w = align_up(w + 3 * (size_t)H * pl.ws.nq_pad * D, kAlign);
  pl.ws_qexp = w;
  w = align_up(w + 3 * (size_t)H * pl.ws.nq_pad * 4, kAlign);
  pl.total = w;
  return pl;
}

}  // namespace

struct rkv_cache {
  rkv_params p;
  rkv::Geom g;
  rkv::AttnWs ws;
  size_t bytes;
  double half_turns[rkv::kMaxHalfDim];  // omega_j / (2 pi)
  double omega[rkv::kMaxHalfDim];
  std::vector<float> norm_eps;  // per layer: eps of the fused Q/K RMS norm, < 0 when off
  // the layer's query and key norm weights (bf16 [D] each), null when off
  const uint16_t* norm_q(int layer) const {
    return norm_eps[layer] >= 0.f ? rkv::layer_ptrs(g, layer).normw : nullptr;
  }
  const uint16_t* norm_k(int layer) const {
    return norm_eps[layer] >= 0.f ? rkv::layer_ptrs(g, layer).normw + g.head_dim : nullptr;
  }
};

extern "C" {

const char* rkv_last_error(void) { return g_err.c_str(); }

size_t ring_cache_bytes(const rkv_params* p) {
  std::string why;
  if (!params_ok(p, &why)) {
    g_err = why;
    return 0;
  }
  const Plan pl = make_plan(p);
  if (pl.part_bytes >= kMaxPartBytes) {
    g_err = "n_heads x max_queries too large for the attention workspace (partials must stay below 1 GiB)";
    return 0;
  }
  return pl.total;
}

int ring_cache_create(const rkv_params* p, void* dev_buf, size_t bytes, hipStream_t stream,
                      rkv_cache** out) {
  std::string why;
  if (!out) return fail(RKV_EINVAL, "out is null");
  *out = nullptr;
  if (!params_ok(p, &why)) return fail(RKV_EINVAL, why);
  if (!dev_buf) return fail(RKV_EINVAL, "dev_buf is null");
  if (reinterpret_cast<uintptr_t>(dev_buf) % kAlign)
    return fail(RKV_EINVAL, "dev_buf must be 256-byte aligned");
  const Plan pl = make_plan(p);
  if (pl.part_bytes >= kMaxPartBytes)
    return fail(RKV_EINVAL, "n_heads x max_queries too large for the attention workspace (partials must stay below 1 GiB)");
  if (bytes < pl.total)
    return fail(RKV_EINVAL, "buffer too small: need " + std::to_string(pl.total) + " bytes");

  rkv_cache* c = new (std::nothrow) rkv_cache();
  if (!c) return fail(RKV_EINVAL, "out of host memory");
  c->p = *p;
  c->g = pl.g;
  c->g.base = static_cast<uint8_t*>(dev_buf);
  c->ws = pl.ws;
  c->ws.part_o = c->g.base + pl.ws_parto;
  c->ws.part_ml = reinterpret_cast<float*>(c->g.base + pl.ws_partml);
  c->ws.sync = reinterpret_cast<unsigned long long*>(c->g.base + pl.ws_sync);
  c->ws.qcodes = c->g.base + pl.ws_qcodes;
  c->ws.qexp = reinterpret_cast<int32_t*>(c->g.base + pl.ws_qexp);
  c->bytes = pl.total;
  c->norm_eps.assign(p->n_layers, -1.f);
  // RoPE frequencies: one band of D/2 pairs, omega_j = base^(-2j/D), or three
  // bands (t, y, x) of n_b pairs each, omega = base^(-j/n_b) within a band
  const int half = p->head_dim / 2;
  for (int j = 0; j < half; ++j) {
    int lo = 0, nb = half;
    if (c->g.pos_stride == 3) {
      if (j < c->g.band_t) {
        lo = 0, nb = c->g.band_t;
      } else if (j < c->g.band_ty) {
        lo = c->g.band_t, nb = c->g.band_ty - c->g.band_t;
      } else {
        lo = c->g.band_ty, nb = half - c->g.band_ty;
      }
    }
    c->omega[j] = std::pow((double)p->rope_base, -(double)(j - lo) / nb);
    c->half_turns[j] = c->omega[j] / (2.0 * M_PI);
  }
  hipError_t e = rkv::launch_fill_zero(dev_buf, pl.total, stream);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "fill kernel launch");
  }
  // the fixed scratch of cache_attend_noalloc, looked up now on this device
  // (a failure here is reported by that call, which tries again)
  (void)rkv::scratch_init();
  e = rkv::launch_init_consts(c->g, c->half_turns, half, stream);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "init kernel launch");
  }
  *out = c;
  g_err.clear();
  return RKV_OK;
}

int ring_cache_destroy(rkv_cache* c) {
  delete c;
  return RKV_OK;
}

static int layer_range(const rkv_cache* c, int32_t layer, bool allow_all, int* lo, int* hi) {
  if (layer == -1 && allow_all) {
    *lo = 0;
    *hi = c->p.n_layers;
    return RKV_OK;
  }
  if (layer < 0 || layer >= c->p.n_layers)
    return fail(RKV_EINVAL, "layer " + std::to_string(layer) + " out of range");
  *lo = layer;
  *hi = layer + 1;
  return RKV_OK;
}

int ring_cache_reset(rkv_cache* c, int32_t layer, hipStream_t stream) {
  if (!c) return fail(RKV_EINVAL, "cache is null");
  int lo, hi;
  if (int r = layer_range(c, layer, true, &lo, &hi)) return r;
  hipError_t e = rkv::launch_reset(c->g, lo, hi, stream);
  if (e != hipSuccess) return hip_fail(e, "reset kernel launch");
  return RKV_OK;
}

int ring_cache_layout(const rkv_cache* c, int32_t layer, rkv_layout* out) {
  if (!c) return fail(RKV_EINVAL, "cache is null");
  if (!out) return fail(RKV_EINVAL, "out is null");
  int lo, hi;
  if (int r = layer_range(c, layer, false, &lo, &hi)) return r;
  const size_t b = c->g.layer0 + (size_t)layer * c->g.layer_bytes;
  out->codes_k = b + c->g.off_codes_k;
  out->codes_v = b + c->g.off_codes_v;
  out->scale_k = b + c->g.off_scale_k;
  out->scale_v = b + c->g.off_scale_v;
  out->slot_pos = b + c->g.off_slot_pos;
  out->state = b + c->g.off_state;
  out->vmax = b + c->g.off_vmax;
  out->layer_bytes = c->g.layer_bytes;
  out->n_slots_padded = c->g.n_pad;
  out->slot_yx = b + c->g.off_slot_yx;
  out->n_global = c->g.n_global;
  out->global_first_slot = c->g.n_ring_pad;
  return RKV_OK;
}

static bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

int cache_write_rope_fp8(rkv_cache* c, int32_t layer, const void* k_bf16, const void* v_bf16,
                         const int32_t* pos, int32_t n, hipStream_t stream) {
  if (!c) return fail(RKV_EINVAL, "cache is null");
  int lo, hi;
  if (int r = layer_range(c, layer, false, &lo, &hi)) return r;
  if (!k_bf16 || !v_bf16 || !pos) return fail(RKV_EINVAL, "null tensor pointer");
  if (!aligned(k_bf16, 16) || !aligned(v_bf16, 16)) return fail(RKV_EINVAL, "k/v must be 16-byte aligned");
  if (!aligned(pos, 4)) return fail(RKV_EINVAL, "pos must be 4-byte aligned");
  if (n < 1 || n > c->p.n_slots)
    return fail(RKV_EINVAL, "n = " + std::to_string(n) + " outside [1, n_slots]");
  hipError_t e = rkv::launch_write(c->g, layer, k_bf16, v_bf16, pos, n, c->norm_k(layer), c->norm_eps[layer], stream);
  if (e != hipSuccess) return hip_fail(e, "write kernel launch");
  return RKV_OK;
}

int cache_write_global(rkv_cache* c, int32_t layer, int32_t first, const void* k_bf16, const void* v_bf16,
                       const int32_t* pos, int32_t n, hipStream_t stream) {
  if (!c) return fail(RKV_EINVAL, "cache is null");
  int lo, hi;
  if (int r = layer_range(c, layer, false, &lo, &hi)) return r;
  if (!k_bf16 || !v_bf16 || !pos) return fail(RKV_EINVAL, "null tensor pointer");
  if (!aligned(k_bf16, 16) || !aligned(v_bf16, 16)) return fail(RKV_EINVAL, "k/v must be 16-byte aligned");
  if (!aligned(pos, 4)) return fail(RKV_EINVAL, "pos must be 4-byte aligned");
  if (n < 1 || first < 0 || (long long)first + n > c->p.n_global)
    return fail(RKV_EINVAL, "global slots [" + std::to_string(first) + ", " + std::to_string((long long)first + n) +
                                ") outside [0, n_global = " + std::to_string(c->p.n_global) + ")");
  hipError_t e = rkv::launch_write_global(c->g, layer, first, k_bf16, v_bf16, pos, n, c->norm_k(layer),
                                          c->norm_eps[layer], stream);
  if (e != hipSuccess) return hip_fail(e, "global write kernel launch");
  return RKV_OK;
}

int cache_delta_rotate(rkv_cache* c, int32_t layer, int32_t delta, hipStream_t stream) {
  if (!c) return fail(RKV_EINVAL, "cache is null");
  int lo, hi;
  if (int r = layer_range(c, layer, true, &lo, &hi)) return r;
  // only the temporal pairs turn; spatial pairs (3-D RoPE) keep their values
  float cs[rkv::kMaxHalfDim], sn[rkv::kMaxHalfDim];
  const int half = c->p.head_dim / 2;
  for (int j = 0; j < half; ++j) {
    const double phi = j < c->g.band_t ? (double)delta * c->omega[j] : 0.0;
    cs[j] = (float)std::cos(phi);
    sn[j] = (float)std::sin(phi);
  }
  hipError_t e = rkv::launch_rotate(c->g, lo, hi, delta, cs, sn, stream);
  if (e != hipSuccess) return hip_fail(e, "rotate kernel launch");
  return RKV_OK;
}

int cache_attend(rkv_cache* c, int32_t layer, const void* q_bf16, const int32_t* q_pos,
                 int32_t n_q, void* out_bf16, hipStream_t stream) {
  if (!c) return fail(RKV_EINVAL, "cache is null");
  int lo, hi;
  if (int r = layer_range(c, layer, false, &lo, &hi)) return r;
  if (!q_bf16 || !q_pos || !out_bf16) return fail(RKV_EINVAL, "null tensor pointer");
  if (!aligned(q_bf16, 16) || !aligned(out_bf16, 16))
    return fail(RKV_EINVAL, "q/out must be 16-byte aligned");
  if (!aligned(q_pos, 4)) return fail(RKV_EINVAL, "q_pos must be 4-byte aligned");
  if (n_q < 1 || n_q > c->p.max_queries)
    return fail(RKV_EINVAL, "n_q = " + std::to_string(n_q) + " outside [1, max_queries]");
  hipError_t e = rkv::launch_attend(c->g, c->ws, layer, q_bf16, q_pos, n_q, out_bf16, c->norm_q(layer),
                                     c->norm_eps[layer], stream);
  if (e != hipSuccess) return hip_fail(e, "attend kernel launch");
  return RKV_OK;
}

int cache_attend_noalloc(rkv_cache* c, int32_t layer, const void* q_bf16, const int32_t* q_pos,
                         int32_t n_q, void* out_bf16, hipStream_t stream) {
  if (!c) return fail(RKV_EINVAL, "cache is null");
  int lo, hi;
  if (int r = layer_range(c, layer, false, &lo, &hi)) return r;
  if (!q_bf16 || !q_pos || !out_bf16) return fail(RKV_EINVAL, "null tensor pointer");
  if (!aligned(q_bf16, 16) || !aligned(out_bf16, 16))
    return fail(RKV_EINVAL, "q/out must be 16-byte aligned");
  if (!aligned(q_pos, 4)) return fail(RKV_EINVAL, "q_pos must be 4-byte aligned");
  if (n_q < 1 || n_q > c->p.max_queries)
    return fail(RKV_EINVAL, "n_q = " + std::to_string(n_q) + " outside [1, max_queries]");
  rkv::AttnWs ws;
  size_t need = 0;
  hipError_t e = rkv::fixed_attn_ws(c->g, c->ws, n_q, &ws, &need);
  if (e != hipSuccess) return hip_fail(e, "scratch symbol lookup");
  if (need > rkv::kScratchBytes)
    return fail(RKV_EINVAL, "n_q x n_heads needs " + std::to_string(need) + " bytes of attention scratch, more than the " +
                                std::to_string(rkv::kScratchBytes) + " bytes of the fixed scratch");
  e = rkv::launch_attend(c->g, ws, layer, q_bf16, q_pos, n_q, out_bf16, c->norm_q(layer), c->norm_eps[layer], stream);
  if (e != hipSuccess) return hip_fail(e, "attend kernel launch");
  return RKV_OK;
}

int cache_write_attend(rkv_cache* c, int32_t layer, const void* k_bf16, const void* v_bf16,
                       const int32_t* pos, int32_t n, const void* q_bf16, const int32_t* q_pos,
                       int32_t n_q, void* out_bf16, hipStream_t stream) {
  if (!c) return fail(RKV_EINVAL, "cache is null");
  int lo, hi;
  if (int r = layer_range(c, layer, false, &lo, &hi)) return r;
  if (!k_bf16 || !v_bf16 || !pos || !q_bf16 || !q_pos || !out_bf16) return fail(RKV_EINVAL, "null tensor pointer");
  if (!aligned(k_bf16, 16) || !aligned(v_bf16, 16)) return fail(RKV_EINVAL, "k/v must be 16-byte aligned");
  if (!aligned(q_bf16, 16) || !aligned(out_bf16, 16))
    return fail(RKV_EINVAL, "q/out must be 16-byte aligned");
  if (!aligned(pos, 4) || !aligned(q_pos, 4)) return fail(RKV_EINVAL, "pos/q_pos must be 4-byte aligned");
  if (n < 1 || n > c->p.n_slots)
    return fail(RKV_EINVAL, "n = " + std::to_string(n) + " outside [1, n_slots]");
  if (n_q < 1 || n_q > c->p.max_queries)
    return fail(RKV_EINVAL, "n_q = " + std::to_string(n_q) + " outside [1, max_queries]");
  hipError_t e = rkv::launch_write_attend(c->g, c->ws, layer, k_bf16, v_bf16, pos, n, q_bf16, q_pos, n_q,
                                          out_bf16, c->norm_q(layer), c->norm_k(layer), c->norm_eps[layer],
                                          stream);
  if (e != hipSuccess) return hip_fail(e, "write/attend kernel launch");
  return RKV_OK;
}

int ring_cache_set_qk_norm(rkv_cache* c, int32_t layer, const void* wq_bf16, const void* wk_bf16, float eps,
                           hipStream_t stream) {
  if (!c) return fail(RKV_EINVAL, "cache is null");
  int lo, hi;
  if (int r = layer_range(c, layer, true, &lo, &hi)) return r;
  if (!wq_bf16 && !wk_bf16) {
    for (int l = lo; l < hi; ++l) c->norm_eps[l] = -1.f;
    g_err.clear();
    return RKV_OK;
  }
  if (!wq_bf16 || !wk_bf16) return fail(RKV_EINVAL, "wq and wk must both be set or both be null");
  if (!aligned(wq_bf16, 2) || !aligned(wk_bf16, 2)) return fail(RKV_EINVAL, "weights must be 2-byte aligned");
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(RKV_EINVAL, "eps must be finite and > 0");
  const size_t bytes = (size_t)c->p.head_dim * 2;
  for (int l = lo; l < hi; ++l) {
    uint16_t* dst = rkv::layer_ptrs(c->g, l).normw;
    hipError_t e = hipMemcpyAsync(dst, wq_bf16, bytes, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(dst + c->p.head_dim, wk_bf16, bytes, hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "norm weight copy");
    c->norm_eps[l] = eps;
  }
  g_err.clear();
  return RKV_OK;
}

int ring_cache_calibrate_static(rkv_cache* c, int32_t layer, float margin, hipStream_t stream) {
  if (!c) return fail(RKV_EINVAL, "cache is null");
  int lo, hi;
  if (int r = layer_range(c, layer, true, &lo, &hi)) return r;
  if (!(margin > 0.f) || !(margin <= 64.f)) return fail(RKV_EINVAL, "margin must be in (0, 64]");
  hipError_t e = rkv::launch_calibrate(c->g, lo, hi, margin, stream);
  if (e != hipSuccess) return hip_fail(e, "calibrate kernel launch");
  g_err.clear();
  return RKV_OK;
}

}  // extern "C"
