// api.hip -- the C ABI (include/peagle.h): argument validation, weight
// tiling, workspace planning and the launch sequence of the draft forward.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/peagle.h"
#include "pe_internal.hpp"

using namespace pe;

namespace {

thread_local std::string g_err;

pe_status fail(pe_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

}  // namespace

namespace pe {
pe_status set_error(pe_status st, const char *msg) { return fail(st, "%s", msg); }
}  // namespace pe

namespace {

pe_status hip_fail(hipError_t e, const char *what) {
  return fail(PE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kPipe = 8;  // tile loads in flight per GEMM wave (kernel constant)

struct Tiled {
  u32x4 *ptr = nullptr;
  int N = 0, K = 0, NT = 0, KT = 0;
};

struct LayerT {
  Tiled qkv, o, gateup, down;
  float *attn_norm = nullptr, *mlp_norm = nullptr;
  // transposed tiles for the backward's data gradients (pe_model_prepare_backward)
  Tiled qkvT, oT, guT, downT;
};

// Tile counts of an [N, K] weight in the fragment-tile layout.
struct TileDims {
  int NT, KT;
};
TileDims tile_dims(int N, int K, int ktile) { return {(N + 15) / 16, (K + ktile - 1) / ktile}; }

// Everything the decode planners need, derived from the configuration and
// the device's compute-unit count alone (no device memory).
struct DecodeShape {
  pe_config cfg;
  int cus, ktile;
  size_t esz;
  TileDims fc, lm, qkv, o, gateup, down;
};

DecodeShape decode_shape(const pe_config &c, int cus) {
  DecodeShape d;
  d.cfg = c;
  d.cus = cus;
  d.ktile = c.dtype == PE_BF16 ? 32 : 16;
  d.esz = c.dtype == PE_BF16 ? 2 : 4;
  const int H = c.hidden, I = c.intermediate, hd = c.head_dim;
  d.fc = tile_dims(H, 3 * H, d.ktile);
  d.lm = tile_dims(c.vocab, H, d.ktile);
  d.qkv = tile_dims((c.n_q_heads + 2 * c.n_kv_heads) * hd, H, d.ktile);
  d.o = tile_dims(H, c.n_q_heads * hd, d.ktile);
  d.gateup = tile_dims(2 * I, H, d.ktile);
  d.down = tile_dims(H, I, d.ktile);
  return d;
}

}  // namespace

struct pe_model {
  pe_config cfg;
  int ktile = 32;      // contraction elements per tile
  size_t esz = 2;      // bytes per dtype element
  int num_cus = 256;
  size_t lds_budget = 159 * 1024;  // dynamic LDS per GEMM workgroup
  DecodeShape shape;   // tile counts and device size the decode planners use
  Tiled fc, lm;
  Tiled fcT, lmT;      // transposed tiles (backward)
  bool has_bwd = false;
  std::vector<LayerT> layers;
  float *final_norm = nullptr;
  double *inv_freq = nullptr;
  const void *embed = nullptr;
  std::vector<void *> allocs;
  // optional LM-head timing
  mutable bool prof = false;
  mutable std::vector<hipEvent_t> ev0, ev1;
  mutable int nrec = 0;
};

struct pe_mask {
  int n_max = 0, K = 0;
  int2 *table = nullptr;  // [n_max*K] (anchor, depth) of every grid cell
};

namespace {

// Work split of one GEMM: 8-wave workgroups; each wave keeps nkw weight
// tiles per strip in flight and the matching activation fragments in
// registers, so nkw is capped by the register budget (more activation rows,
// fewer slots).  Larger K is split over KS workgroup columns.  KS == 0 marks
// a contraction no split up to kMaxSplits can serve.
struct GemmPlan {
  GemmLaunch L;
  int KS, kc, nkw, Mv, nf;
};

constexpr int kMaxSplits = 64;

// Share of the LM head's strips handed out at run time instead of by XCD
// range (per cent): the XCDs' streaming rates differ from call to call, so
// their static ranges end up to 20-30 us apart.  Measured in alternating
// runs: 6% takes the GPT-OSS-shaped forward from 490.4 to 485.5 us (16K
// context 528.8 -> 524.5, Qwen3-Coder shape 407.6 -> 406.3); 8-10% gain the
// same or less.
constexpr int kLmPoolPercent = 6;

// Modelled cost of a K split in tile-times per CU: the in-kernel
// completion's tail (fc, QKV and residual epilogues), a finalize kernel
// (other epilogues), or, for the LM head, a cost that keeps it whole unless
// nothing else fits (its argmax is folded only when it is not split).
constexpr int kSplitCostInKernel = 90;
constexpr int kSplitCostKernel = 100;
constexpr int kSplitCostLmHead = 1000;

bool finishes_in_kernel(int epi) { return epi == EPI_FC || epi == EPI_RESID || epi == EPI_QKV; }

GemmPlan plan_gemm(int cus, int NT, int KT, int Mv, int nf, int epi) {
  GemmPlan g{};
  g.Mv = Mv;
  g.nf = nf;
  const int W = kGemmWaves;
  const int max_slots = nf == 1 ? 18 : nf == 2 ? 8 : nf == 3 ? 4 : 2;  // as the kernel's buckets
  // One workgroup per CU (8 waves at up to 256 VGPRs).  The modelled
  // makespan of a plan is what the busiest workgroup streams: its strip
  // rounds x tiles per chunk, plus the activation slice it loads before its
  // first strip (nf x tiles per chunk: every workgroup loads its own, and
  // these bytes set the ramp of the short projections), plus the split's
  // cost.  Splits that leave a wave fewer than 4 tile slots keep too few
  // loads in flight; they are only planned when nothing else fits, and
  // splits beyond 16 only when no split up to 16 fits.  Fitted to A/B runs
  // on the MI355X: QKV split 3 ways at 16 rows and 2 ways at 32 rows, O 4
  // ways at 32 rows, down unchanged.
  const int split_cost = epi == EPI_ARGMAX ? kSplitCostLmHead
                         : finishes_in_kernel(epi) ? kSplitCostInKernel : kSplitCostKernel;
  const int floor_slots = max_slots < 4 ? max_slots : 4;
  long best = -1;
  for (int pass = 0; pass < 2 && best < 0; ++pass) {
    for (int KS = 1; KS <= kMaxSplits && KS <= KT && (KS <= 16 || best < 0); ++KS) {
      const int kc = (KT + KS - 1) / KS;
      const int nkw = (kc + W - 1) / W;
      if (nkw > max_slots) continue;
      const int ks = (KT + kc - 1) / kc;  // no empty chunk
      if (pass == 0 && ks > 1 && nkw < floor_slots) continue;
      int G = cus / ks;
      if (G < 1) G = 1;
      if (G > NT) G = NT;
      const long rounds = (NT + G - 1) / G;
      const long cost = rounds * kc + (long)nf * kc + (ks > 1 ? split_cost : 0);
      if (best < 0 || cost < best) {
        best = cost;
        g.KS = ks; g.kc = kc; g.nkw = nkw; g.L.grid = G;
      }
    }
  }
  // Measured exceptions to the model (forward A/B on the MI355X) for
  // in-kernel-finished projections, keyed by 16-row groups, strips and k
  // tiles: the model's split and its neighbours were timed in one process.
  struct SplitOverride {
    int epi, nf, NT, KT_lo, KT_hi, KS;  // epi -1: any in-kernel-finished epilogue
  };
  static constexpr SplitOverride kOverrides[] = {
      // GPT-OSS-20B shape, 16 rows: fc (model 11 ways) and down (model 7);
      // 4.4 us less per forward over the five launches, 4 ways lose 2.4 us
      // per launch, 6 ways 0.5 us
      {-1, 1, 180, 256, 270, 5},
      // Qwen3-Coder-30B shape, 32 rows: down (model 7 ways); 2.3 us less
      // per forward, 5 ways lose 1 us per launch
      {EPI_RESID, 2, 128, 192, 192, 4},
      // Qwen3-Coder-30B shape: fc of the 4 + 1 fused rows (model 7 ways);
      // 0.9-1.9 us less per forward
      {EPI_FC, 1, 128, 192, 192, 4},
  };
  if (finishes_in_kernel(epi))
    for (const SplitOverride &o : kOverrides)
      if ((o.epi < 0 || o.epi == epi) && nf == o.nf && NT == o.NT && KT >= o.KT_lo && KT <= o.KT_hi) {
        const int kc = (KT + o.KS - 1) / o.KS;
        g.KS = (KT + kc - 1) / kc; g.kc = kc; g.nkw = (kc + W - 1) / W;
        g.L.grid = std::min(NT, std::max(1, cus / g.KS));
      }
  g.L.waves = W;
  g.L.lds = (size_t)W * nf * 1024 + 256;
  g.L.maxkw = g.nkw <= 2 ? 2 : g.nkw <= 4 ? 4 : g.nkw <= 8 ? 8 : g.nkw <= 12 ? 12 : 18;
  return g;
}

struct AttnPlan {
  int L, S;
};

// Split-KV plan: splits of a whole number of 64-key tiles.  Each split ends
// in a partial the combine kernel reads, so fewer, longer splits win until
// the grid no longer covers the chip: measured on the MI355X (kernel plus
// combine), 5 tiles per split at the 4K context and 9 at 16K (head_dim 64,
// register-ring kernel), 4 tiles at head_dim 128 (LDS-ring kernel, two
// workgroups per CU).
AttnPlan plan_attn(const DecodeShape &m, int B, int K, long C) {
  const int G = m.cfg.n_q_heads / m.cfg.n_kv_heads;
  const int qparts = ((K * G + 15) / 16 * 16 + 63) / 64;
  const long units = (long)B * m.cfg.n_kv_heads * qparts;
  const long keys = C + K;
  const long tiles = (keys + 63) / 64;
  const bool lds_ring = m.cfg.dtype == PE_BF16 && m.cfg.head_dim == 128;
  const long min_tp = lds_ring ? 4 : 5;
  const long wg_target = (long)m.cus * (lds_ring ? 4 : 2);
  long per = (units * tiles + wg_target - 1) / wg_target;
  if (per < min_tp) per = min_tp;
  if (per > tiles) per = tiles;
  AttnPlan a;
  a.L = (int)(per * 64);
  a.S = (int)((keys + a.L - 1) / a.L);
  if (a.S < 1) a.S = 1;
  return a;
}

struct WsLayout {
  size_t xres, xg, ssq, q, kb, vb, attn_out, mlp_h, gpart, apart, blk, cnt, keys, total;
  int RP;
  AttnPlan ap;
  const char *unsupported;  // non-NULL: why this shape cannot run
};

// The attention kernel addresses one (sequence, kv head) cache slice of
// ctx_stride * head_dim elements through a buffer resource whose
// out-of-range offset must lie beyond the slice.
constexpr long kCacheSliceBytesMax = 0x7FFF0000L;

// B sequences of block K within the build limits; B is bounded before the
// product is formed, so no argument overflows it.
bool decode_rows_ok(int B, int K) {
  return B >= 1 && B <= PE_DECODE_ROWS_MAX - 1 && K >= 1 && K <= PE_K_MAX && B * K <= PE_DECODE_ROWS_MAX;
}

WsLayout layout(const DecodeShape &m, int B, int K, long C) {
  const pe_config &c = m.cfg;
  WsLayout w{};
  // Compared by division, so that no ctx_stride overflows the product.
  if (C > kCacheSliceBytesMax / ((long)c.head_dim * (long)m.esz)) {
    w.unsupported = "ctx_stride * head_dim * element size exceeds the 2 GiB cache slice limit";
    return w;
  }
  const int G = c.n_q_heads / c.n_kv_heads;
  const int R = K * G;
  const int M = B * K, nf = (M + 15) / 16, nf_fc = (B + 1 + 15) / 16;
  w.RP = (R + 15) / 16 * 16;
  w.ap = plan_attn(m, B, K, C);
  size_t part = 0, blk = 0;
  auto upd = [&](const TileDims &t, int Mv, int nfr, int epi) {
    const bool lm = epi == EPI_ARGMAX;
    const GemmPlan g = plan_gemm(m.cus, t.NT, t.KT, Mv, nfr, epi);
    if (g.KS == 0) {
      w.unsupported = "a projection's contraction is too long for the activation rows held in registers";
      return;
    }
    if (g.KS > 1) part = std::max(part, (size_t)g.KS * t.NT * nfr * 1024);
    if (lm) {
      const size_t nb = g.KS > 1 ? (size_t)(t.NT + 3) / 4 : (size_t)g.L.grid;
      blk = std::max(blk, nb * kMaxRows * 8);
    }
  };
  upd(m.fc, B + 1, nf_fc, EPI_FC);
  upd(m.fc, M, nf, EPI_FC);  // cache extension: one fc row per block row
  if (c.n_layers > 0) {
    upd(m.qkv, M, nf, EPI_QKV); upd(m.o, M, nf, EPI_RESID); upd(m.gateup, M, nf, EPI_SWIGLU);
    upd(m.down, M, nf, EPI_RESID);
  }
  upd(m.lm, M, nf, EPI_ARGMAX);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  const size_t H = c.hidden, esz = m.esz;
  w.xres = take((size_t)kMaxRows * H * 4);
  w.xg = take((size_t)kMaxRows * H * esz);
  w.ssq = take((size_t)(H / 16) * kMaxRows * 4);
  w.q = take((size_t)B * c.n_kv_heads * w.RP * c.head_dim * esz);
  w.kb = take((size_t)B * c.n_kv_heads * K * c.head_dim * esz);
  w.vb = take((size_t)B * c.n_kv_heads * K * c.head_dim * esz);
  w.attn_out = take((size_t)kMaxRows * c.n_q_heads * c.head_dim * esz);
  w.mlp_h = take((size_t)kMaxRows * c.intermediate * esz);
  if (part > (size_t)kCacheSliceBytesMax)
    w.unsupported = "the split-K partial strips exceed 2 GiB";
  w.gpart = take(std::max(part, (size_t)256));
  const size_t qparts = (size_t)(w.RP + 63) / 64;
  w.apart = take((size_t)B * c.n_kv_heads * qparts * w.ap.S * (64 * (size_t)c.head_dim + 128) * 4);
  w.blk = take(std::max(blk, (size_t)256));
  // Arrival counters (one per weight strip of the split projections; the LM
  // head uses the first) and the LM head's row keys: zero from
  // pe_workspace_init on, and every launch leaves them at zero.
  const int nt_max = std::max({m.fc.NT, m.qkv.NT, m.o.NT, m.gateup.NT, m.down.NT, 1});
  w.cnt = take((size_t)nt_max * 4);
  w.keys = take((size_t)kMaxRows * 8);
  w.total = off;
  return w;
}

pe_status tile_matrix(pe_model *m, Tiled &t, const void *const *srcs, const int *rows, int nsrc,
                      int N, int K, int map, hipStream_t s) {
  t.N = N;
  t.K = K;
  t.NT = (N + 15) / 16;
  t.KT = (K + m->ktile - 1) / m->ktile;
  const size_t bytes = (size_t)t.NT * t.KT * 1024;
  if (bytes > 0x7FFFF000ull)
    return fail(PE_ERR_UNSUPPORTED, "a %d x %d weight exceeds 2 GiB of tiles", N, K);
  hipError_t e = hipMalloc(&t.ptr, bytes);
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(weight tiles)");
  m->allocs.push_back(t.ptr);
  RepackParams rp{};
  for (int i = 0; i < 3; ++i) {
    rp.src[i] = i < nsrc ? srcs[i] : nullptr;
    rp.src_rows[i] = i < nsrc ? rows[i] : 0x7FFFFFFF;
  }
  rp.N = N; rp.K = K; rp.NT = t.NT; rp.KT = t.KT; rp.map = map;
  rp.hd = m->cfg.head_dim; rp.nq = m->cfg.n_q_heads; rp.nkv = m->cfg.n_kv_heads;
  rp.I = m->cfg.intermediate; rp.dst = t.ptr;
  e = launch_repack(m->cfg.dtype, rp, s);
  if (e != hipSuccess) return hip_fail(e, "weight tiling launch");
  return PE_OK;
}

pe_status gain_copy(pe_model *m, const void *src, float *&dst, hipStream_t s) {
  hipError_t e = hipMalloc(&dst, (size_t)m->cfg.hidden * 4);
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(gain)");
  m->allocs.push_back(dst);
  e = launch_gain_to_f32(m->cfg.dtype, src, dst, m->cfg.hidden, s);
  if (e != hipSuccess) return hip_fail(e, "gain conversion launch");
  return PE_OK;
}

void destroy(pe_model *m) {
  if (!m) return;
  for (void *p : m->allocs) (void)hipFree(p);
  for (hipEvent_t ev : m->ev0) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : m->ev1) (void)hipEventDestroy(ev);
  delete m;
}

pe_status check_cfg(const pe_config *c) {
  if (c->dtype != PE_F32 && c->dtype != PE_BF16)
    return fail(PE_ERR_INVALID_ARGUMENT, "dtype %d is neither PE_F32 nor PE_BF16", c->dtype);
  const int ktile = c->dtype == PE_BF16 ? 32 : 16;
  const int kmin = kPipe * ktile;  // each contraction spans at least kPipe tiles
  if (c->hidden <= 0 || c->n_layers < 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
      c->head_dim <= 0 || c->intermediate <= 0 || c->vocab <= 0)
    return fail(PE_ERR_INVALID_ARGUMENT, "config sizes must be positive (n_layers >= 0)");
  if (c->n_q_heads % c->n_kv_heads)
    return fail(PE_ERR_INVALID_ARGUMENT, "n_q_heads %d is not a multiple of n_kv_heads %d",
                c->n_q_heads, c->n_kv_heads);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PE_ERR_UNSUPPORTED, "head_dim %d: supported 64, 128", c->head_dim);
  if (c->dtype == PE_F32 && c->head_dim != 64)
    return fail(PE_ERR_UNSUPPORTED, "fp32 models support head_dim 64 only");
  if (c->hidden % 16 || c->vocab % 16 || c->intermediate % 8)
    return fail(PE_ERR_UNSUPPORTED, "hidden and vocab must be multiples of 16, intermediate of 8");
  if (c->hidden < kmin || c->intermediate < kmin || c->n_q_heads * c->head_dim < kmin)
    return fail(PE_ERR_UNSUPPORTED, "hidden, intermediate and n_q_heads*head_dim must be >= %d",
                kmin);
  if (c->n_q_heads / c->n_kv_heads * PE_K_MAX > 256)
    return fail(PE_ERR_UNSUPPORTED, "query heads per kv head must be <= 16");
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f))
    return fail(PE_ERR_INVALID_ARGUMENT, "rope_theta must be > 0 and rms_eps >= 0");
  return PE_OK;
}

// Workspace of the training-shape forward.
struct TrainLayout {
  size_t anc, dep, inv, rope, yfc, xres, u, q, kall, vall, k0, v0, attn, h, keys, total;
};

TrainLayout train_layout(const pe_model *m, long n, int K, long L) {
  const pe_config &c = m->cfg;
  TrainLayout t{};
  const size_t H = c.hidden, esz = m->esz, hd = c.head_dim;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + std::max(bytes, (size_t)1), 256); return o; };
  t.anc = take((size_t)L * 4);
  t.dep = take((size_t)L * 4);
  t.inv = take((size_t)n * K * 4);
  t.rope = take(c.n_layers > 0 ? (size_t)n * (hd / 2) * 8 : 0);
  t.yfc = take((size_t)(n + 1) * H * 4);
  t.xres = take((size_t)L * H * 4);
  const size_t Lp = (size_t)(L + 15) / 16 * 16;  // tiled activations hold whole 16-row groups
  t.u = take(Lp * H * esz);
  const bool layers = c.n_layers > 0;
  t.q = take(layers ? (size_t)L * c.n_q_heads * hd * esz : 0);
  t.kall = take(layers ? (size_t)L * c.n_kv_heads * hd * esz : 0);
  t.vall = take(layers ? (size_t)L * c.n_kv_heads * hd * esz : 0);
  t.k0 = take(layers ? (size_t)n * c.n_kv_heads * hd * esz : 0);
  t.v0 = take(layers ? (size_t)n * c.n_kv_heads * hd * esz : 0);
  t.attn = take(layers ? Lp * c.n_q_heads * hd * esz : 0);
  t.h = take(layers ? Lp * c.intermediate * esz : 0);
  t.keys = take((size_t)L * 8);
  t.total = off;
  return t;
}

constexpr long kTrainRowsMax = 1L << 22;  // 128-row blocks stay well within the grid's y limit

pe_status check_train_shape(const pe_model *m, const pe_mask *mask, int32_t n, int32_t K, int32_t L) {
  if (!m || !mask) return fail(PE_ERR_INVALID_ARGUMENT, "model and mask must be non-NULL");
  if (m->cfg.hidden % m->ktile || m->cfg.intermediate % m->ktile)
    return fail(PE_ERR_UNSUPPORTED, "the training forward needs hidden and intermediate multiples of %d",
                m->ktile);
  if (K != mask->K) return fail(PE_ERR_INVALID_ARGUMENT, "K=%d differs from the mask's K=%d", K, mask->K);
  if (n < 1 || n > mask->n_max)
    return fail(PE_ERR_INVALID_ARGUMENT, "n=%d outside [1, n_max=%d]", n, mask->n_max);
  if (L < 1 || (long)L > (long)n * K || L > kTrainRowsMax)
    return fail(PE_ERR_INVALID_ARGUMENT, "L=%d outside [1, min(n*K=%ld, %ld)]", L, (long)n * K,
                kTrainRowsMax);
  return PE_OK;
}

// The layered forward of a block of K rows per sequence: input fusion (the
// parallel drafter's NTP + MTP rows, or cache-extension rows with their own
// inputs), N decoder layers, final norm, LM head with argmax.
enum DraftMode : int { DRAFT_PARALLEL = 0, EXTEND_TARGET = 1, EXTEND_DRAFTER = 2 };

struct DraftCall {
  int N, B, K, mode;
  const void *in;            // [B,3H] (parallel), [B,K,3H] (extend, target), fp32 [B,K,H] (extend, drafter)
  const int32_t *tok;        // [B] (parallel) or [B,K]
  const void *mask_emb, *h_shared;
  const int32_t *ctx_lens;
  int64_t C;
  int pos_off;
  const void *const *kc, *const *vc;
  void *const *kc_out, *const *vc_out;  // extend: caches to append to (or NULL)
  int32_t *draft_out;
  float *logits_out, *z_out;
};

pe_status enqueue_draft(const pe_model *m, const WsLayout &W, const DraftCall &d, char *ws, hipStream_t s) {
  const pe_config &c = m->cfg;
  const int N = d.N, B = d.B, K = d.K;
  const int64_t ctx_stride = d.C;
  float *xres = reinterpret_cast<float *>(ws + W.xres);
  void *xg = ws + W.xg;
  float *ssq = reinterpret_cast<float *>(ws + W.ssq);
  const int M = B * K;
  const int nf = (M + 15) / 16;
  const int H = c.hidden, hd = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads;
  const int G = nq / nkv;

  GemmParams base{};
  base.part = reinterpret_cast<floatx4 *>(ws + W.gpart);
  base.H = H;
  base.Kb = K;
  base.B = B;
  base.eps = c.rms_eps;
  base.inv_width = 1.0f / (float)H;

  unsigned *cnt = reinterpret_cast<unsigned *>(ws + W.cnt);
  int lm_blocks = 0;
  bool tokens_written = false;  // the LM head wrote draft_out itself
  auto run = [&](const Tiled &t, int epi, int nfr, GemmParams p) -> pe_status {
    const int Mv = p.act_rows + (p.act_extra ? 1 : 0);
    const GemmPlan pl = plan_gemm(m->num_cus, t.NT, t.KT, Mv, nfr, epi);
    p.wt = t.ptr; p.wbytes = (unsigned)((size_t)t.NT * t.KT * 1024); p.NT = t.NT; p.KT = t.KT;
    p.N = t.N; p.K = t.K;
    p.epi = epi; p.KS = pl.KS; p.kc = pl.kc; p.nkw = pl.nkw; p.Mv = Mv;
    lm_blocks = pl.KS > 1 ? (t.NT + 3) / 4 : pl.L.grid;
    // Split FC and residual projections finish their strips in-kernel; an
    // unsplit LM head writes the tokens itself.
    if (pl.KS > 1 && finishes_in_kernel(epi)) p.cnt = cnt;
    if (epi == EPI_ARGMAX && pl.KS == 1 && d.draft_out) {
      p.cnt = cnt;
      p.keys = reinterpret_cast<unsigned long long *>(ws + W.keys);
      p.draft_out = d.draft_out;
      // Only where workgroups stream many strips: with a few strips each the
      // ranges barely drift apart, and the ticket round trip would be a cost.
      p.pool = t.NT >= 8 * pl.L.grid ? t.NT * kLmPoolPercent / 100 : 0;
      tokens_written = true;
    }
    hipError_t e = launch_gemm(c.dtype, nfr, p, pl.L, s);
    if (e != hipSuccess) return hip_fail(e, "GEMM launch");
    return PE_OK;
  };

  pe_status st;
  const float *g0 = N > 0 ? m->layers[0].attn_norm : m->final_norm;
  if (d.mode == DRAFT_PARALLEL) {
    // Input fusion: fc over the B hidden rows plus h_shared, then embeddings.
    GemmParams p = base;
    p.act = d.in; p.act_ld = 3L * H; p.act_rows = B; p.act_extra = d.h_shared;
    p.M = B + 1;
    p.xres = xres; p.xg = xg; p.ssq_out = ssq;
    p.gnext = g0;
    p.embed = m->embed; p.tok = d.tok; p.mask_emb = d.mask_emb; p.V = c.vocab;
    if ((st = run(m->fc, EPI_FC, (B + 1 + 15) / 16, p)) != PE_OK) return st;
  } else if (d.mode == EXTEND_TARGET) {
    // Every block row has its own token and target hidden state.
    GemmParams p = base;
    p.act = d.in; p.act_ld = 3L * H; p.act_rows = M;
    p.M = M; p.fc_direct = 1;
    p.xres = xres; p.xg = xg; p.ssq_out = ssq;
    p.gnext = g0;
    p.embed = m->embed; p.tok = d.tok; p.V = c.vocab;
    if ((st = run(m->fc, EPI_FC, nf, p)) != PE_OK) return st;
  } else {
    // Rows fed back from the drafter: x = E[token] + z.
    hipError_t e = launch_fuse_feedback(c.dtype, reinterpret_cast<const float *>(d.in), m->embed, d.tok, M, H,
                                        c.vocab, g0, xres, xg, ssq, s);
    if (e != hipSuccess) return hip_fail(e, "feedback fusion launch");
  }
  for (int l = 0; l < N; ++l) {
    const LayerT &L = m->layers[l];
    {
      GemmParams p = base;
      p.act = xg; p.act_ld = H; p.act_rows = M; p.M = M;
      p.ssq = ssq; p.ssq_strips = H / 16;
      p.q = ws + W.q; p.kb = ws + W.kb; p.vb = ws + W.vb;
      p.ctx_lens = d.ctx_lens; p.inv_freq = m->inv_freq;
      p.nq = nq; p.nkv = nkv; p.hd = hd; p.RP = W.RP;
      p.C = ctx_stride; p.pos_off = d.pos_off;
      if (d.kc_out) { p.kc_out = d.kc_out[l]; p.vc_out = d.vc_out[l]; }
      if ((st = run(L.qkv, EPI_QKV, nf, p)) != PE_OK) return st;
    }
    {
      AttnParams a{};
      a.q = ws + W.q; a.kb = ws + W.kb; a.vb = ws + W.vb;
      a.kc = d.kc[l]; a.vc = d.vc[l];
      a.ctx_lens = d.ctx_lens; a.C = ctx_stride; a.ctx_off = d.pos_off;
      a.B = B; a.Kb = K; a.nq = nq; a.nkv = nkv; a.hd = hd; a.G = G; a.R = K * G; a.RP = W.RP;
      a.L = W.ap.L; a.S = W.ap.S;
      a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
      a.out = ws + W.attn_out;
      a.part = reinterpret_cast<float *>(ws + W.apart);
      hipError_t e = launch_attention(c.dtype, a, s);
      if (e != hipSuccess) return hip_fail(e, "attention launch");
    }
    {
      GemmParams p = base;
      p.act = ws + W.attn_out; p.act_ld = (long)nq * hd; p.act_rows = M; p.M = M;
      p.xres = xres; p.xg = xg; p.ssq_out = ssq; p.gnext = L.mlp_norm;
      if ((st = run(L.o, EPI_RESID, nf, p)) != PE_OK) return st;
    }
    {
      GemmParams p = base;
      p.act = xg; p.act_ld = H; p.act_rows = M; p.M = M;
      p.ssq = ssq; p.ssq_strips = H / 16;
      p.hout = ws + W.mlp_h; p.I = c.intermediate;
      if ((st = run(L.gateup, EPI_SWIGLU, nf, p)) != PE_OK) return st;
    }
    {
      GemmParams p = base;
      p.act = ws + W.mlp_h; p.act_ld = c.intermediate; p.act_rows = M; p.M = M;
      p.xres = xres; p.xg = xg; p.ssq_out = ssq;
      p.gnext = (l + 1 < N) ? m->layers[l + 1].attn_norm : m->final_norm;
      if ((st = run(L.down, EPI_RESID, nf, p)) != PE_OK) return st;
    }
  }
  // LM head with fused argmax (skipped when neither tokens nor logits are wanted).
  if (d.draft_out || d.logits_out) {
    GemmParams p = base;
    p.act = xg; p.act_ld = H; p.act_rows = M; p.M = M;
    p.ssq = ssq; p.ssq_strips = H / 16;
    p.logits = d.logits_out;
    p.blk_best = reinterpret_cast<unsigned long long *>(ws + W.blk);
    p.V = c.vocab;
    const bool prof = m->prof && m->nrec < (int)m->ev0.size();
    if (prof) (void)hipEventRecord(m->ev0[m->nrec], s);
    if ((st = run(m->lm, EPI_ARGMAX, nf, p)) != PE_OK) return st;
    if (prof) {
      (void)hipEventRecord(m->ev1[m->nrec], s);
      ++m->nrec;
    }
    if (d.draft_out && !tokens_written) {
      hipError_t e = launch_argmax_final(p.blk_best, lm_blocks, M, d.draft_out, s);
      if (e != hipSuccess) return hip_fail(e, "argmax launch");
    }
  }
  if (d.z_out) {
    hipError_t e = launch_norm_rows(xres, m->final_norm, ssq, M, H, c.rms_eps, d.z_out, s);
    if (e != hipSuccess) return hip_fail(e, "final norm launch");
  }
  return PE_OK;
}

}  // namespace

extern "C" {

const char *pe_last_error(void) { return g_err.c_str(); }

const char *pe_version(void) {
  return "peagle-gfx950: LDS-staged MFMA weight-streaming GEMM, MFMA split-KV decode attention";
}

pe_status pe_model_create(const pe_config *cfg, const pe_weights *w, void *stream, pe_model **out) {
  if (!cfg || !w || !out) return fail(PE_ERR_INVALID_ARGUMENT, "cfg, w and out must be non-NULL");
  *out = nullptr;
  pe_status st = check_cfg(cfg);
  if (st != PE_OK) return st;
  if (!w->embed || !w->fc || !w->final_norm || !w->lm_head || (cfg->n_layers > 0 && !w->layers))
    return fail(PE_ERR_INVALID_ARGUMENT, "a required weight pointer is NULL");
  for (int l = 0; l < cfg->n_layers; ++l) {
    const pe_layer_weights &L = w->layers[l];
    if (!L.attn_norm || !L.wq || !L.wk || !L.wv || !L.wo || !L.mlp_norm || !L.w_gate || !L.w_up ||
        !L.w_down)
      return fail(PE_ERR_INVALID_ARGUMENT, "layer %d has a NULL weight pointer", l);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  pe_model *m = new pe_model();
  m->cfg = *cfg;
  m->ktile = cfg->dtype == PE_BF16 ? 32 : 16;
  m->esz = cfg->dtype == PE_BF16 ? 2 : 4;
  m->embed = w->embed;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { destroy(m); return hip_fail(e, "hipGetDevice"); }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) { destroy(m); return hip_fail(e, "hipDeviceGetAttribute"); }
  m->num_cus = cus > 0 ? cus : 256;
  m->shape = decode_shape(*cfg, m->num_cus);
  e = gemm_set_lds_limits();
  if (e == hipSuccess) e = attn_set_lds_limits();
  if (e != hipSuccess) { destroy(m); return hip_fail(e, "hipFuncSetAttribute(LDS)"); }

  const int H = cfg->hidden, hd = cfg->head_dim, nq = cfg->n_q_heads, nkv = cfg->n_kv_heads;
  const int I = cfg->intermediate;
  {
    const void *srcs[1] = {w->fc};
    const int rows[1] = {H};
    if ((st = tile_matrix(m, m->fc, srcs, rows, 1, H, 3 * H, MAP_IDENTITY, s)) != PE_OK) {
      destroy(m); return st;
    }
  }
  {
    const void *srcs[1] = {w->lm_head};
    const int rows[1] = {cfg->vocab};
    if ((st = tile_matrix(m, m->lm, srcs, rows, 1, cfg->vocab, H, MAP_IDENTITY, s)) != PE_OK) {
      destroy(m); return st;
    }
  }
  m->layers.resize(cfg->n_layers);
  for (int l = 0; l < cfg->n_layers; ++l) {
    const pe_layer_weights &L = w->layers[l];
    LayerT &T = m->layers[l];
    const void *qkv_src[3] = {L.wq, L.wk, L.wv};
    const int qkv_rows[3] = {nq * hd, nkv * hd, nkv * hd};
    const void *o_src[1] = {L.wo};
    const int o_rows[1] = {H};
    const void *gu_src[2] = {L.w_gate, L.w_up};
    const int gu_rows[2] = {I, I};
    const void *d_src[1] = {L.w_down};
    const int d_rows[1] = {H};
    if ((st = tile_matrix(m, T.qkv, qkv_src, qkv_rows, 3, (nq + 2 * nkv) * hd, H, MAP_QKV, s)) ||
        (st = tile_matrix(m, T.o, o_src, o_rows, 1, H, nq * hd, MAP_IDENTITY, s)) ||
        (st = tile_matrix(m, T.gateup, gu_src, gu_rows, 2, 2 * I, H, MAP_GATEUP, s)) ||
        (st = tile_matrix(m, T.down, d_src, d_rows, 1, H, I, MAP_IDENTITY, s)) ||
        (st = gain_copy(m, L.attn_norm, T.attn_norm, s)) ||
        (st = gain_copy(m, L.mlp_norm, T.mlp_norm, s))) {
      destroy(m);
      return st;
    }
  }
  if ((st = gain_copy(m, w->final_norm, m->final_norm, s)) != PE_OK) { destroy(m); return st; }
  {
    std::vector<double> f(hd / 2);
    for (int i = 0; i < hd / 2; ++i) f[i] = pow((double)cfg->rope_theta, -2.0 * i / hd);
    e = hipMalloc(&m->inv_freq, f.size() * sizeof(double));
    if (e != hipSuccess) { destroy(m); return hip_fail(e, "hipMalloc(inv_freq)"); }
    m->allocs.push_back(m->inv_freq);
    e = hipMemcpyAsync(m->inv_freq, f.data(), f.size() * sizeof(double), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) { destroy(m); return hip_fail(e, "hipMemcpyAsync(inv_freq)"); }
  }
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) { destroy(m); return hip_fail(e, "hipStreamSynchronize after weight tiling"); }
  *out = m;
  return PE_OK;
}

pe_status pe_model_destroy(pe_model *m) {
  if (!m) return fail(PE_ERR_INVALID_ARGUMENT, "model is NULL");
  destroy(m);
  return PE_OK;
}

pe_status pe_draft_workspace_size(const pe_model *m, int32_t B, int32_t K, int64_t ctx_stride,
                                  size_t *bytes) {
  if (!m || !bytes) return fail(PE_ERR_INVALID_ARGUMENT, "model and bytes must be non-NULL");
  if (!decode_rows_ok(B, K))
    return fail(PE_ERR_UNSUPPORTED, "B=%d K=%d outside 1<=K<=%d, B*K<=%d, B+1<=%d", B, K, PE_K_MAX,
                PE_DECODE_ROWS_MAX, PE_DECODE_ROWS_MAX);
  if (ctx_stride < 0) return fail(PE_ERR_INVALID_ARGUMENT, "ctx_stride must be >= 0");
  const WsLayout W = layout(m->shape, B, K, ctx_stride);
  if (W.unsupported) return fail(PE_ERR_UNSUPPORTED, "B=%d K=%d ctx_stride=%ld: %s", B, K, (long)ctx_stride,
                                 W.unsupported);
  *bytes = W.total;
  return PE_OK;
}

pe_status pe_draft_shape_check(const pe_config *cfg, int32_t B, int32_t K, int64_t ctx_stride,
                               int32_t num_cus) {
  if (!cfg) return fail(PE_ERR_INVALID_ARGUMENT, "cfg must be non-NULL");
  pe_status st = check_cfg(cfg);
  if (st != PE_OK) return st;
  if (num_cus < 1) return fail(PE_ERR_INVALID_ARGUMENT, "num_cus must be >= 1");
  if (!decode_rows_ok(B, K))
    return fail(PE_ERR_UNSUPPORTED, "B=%d K=%d outside 1<=K<=%d, B*K<=%d, B+1<=%d", B, K, PE_K_MAX,
                PE_DECODE_ROWS_MAX, PE_DECODE_ROWS_MAX);
  if (ctx_stride < 0) return fail(PE_ERR_INVALID_ARGUMENT, "ctx_stride must be >= 0");
  const WsLayout W = layout(decode_shape(*cfg, num_cus), B, K, ctx_stride);
  if (W.unsupported) return fail(PE_ERR_UNSUPPORTED, "B=%d K=%d ctx_stride=%ld: %s", B, K, (long)ctx_stride,
                                 W.unsupported);
  return PE_OK;
}

pe_status pe_workspace_init(void *workspace, size_t ws_bytes, void *stream) {
  if (!workspace) return fail(PE_ERR_INVALID_ARGUMENT, "workspace is NULL");
  hipError_t e = launch_zero(workspace, ws_bytes, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "workspace zero launch");
  return PE_OK;
}

}  // extern "C"

namespace {

// Argument checks of the parallel-drafting forward shared by both entry
// points (everything except the workspace).
pe_status check_forward(const pe_model *m, int32_t N, int32_t B, int32_t K, const void *hidden3,
                        const int32_t *token_ids, const void *mask_emb, const void *h_shared,
                        const int32_t *ctx_lens, int64_t ctx_stride, const void *const *k_cache,
                        const void *const *v_cache, int32_t *draft_out, float *logits_out) {
  if (!m) return fail(PE_ERR_INVALID_ARGUMENT, "model is NULL");
  const pe_config &c = m->cfg;
  if (N < 0 || N > c.n_layers)
    return fail(PE_ERR_INVALID_ARGUMENT, "N=%d outside [0, n_layers=%d]", N, c.n_layers);
  if (!decode_rows_ok(B, K))
    return fail(PE_ERR_UNSUPPORTED, "B=%d K=%d outside 1<=K<=%d, B*K<=%d, B+1<=%d", B, K, PE_K_MAX,
                PE_DECODE_ROWS_MAX, PE_DECODE_ROWS_MAX);
  if (!hidden3 || !token_ids || !mask_emb || !h_shared || !draft_out)
    return fail(PE_ERR_INVALID_ARGUMENT, "hidden3, token_ids, mask_emb, h_shared and draft_out "
                                         "must be non-NULL");
  if (ctx_stride < 0) return fail(PE_ERR_INVALID_ARGUMENT, "ctx_stride must be >= 0");
  if (N > 0) {
    if (!ctx_lens || !k_cache || !v_cache)
      return fail(PE_ERR_INVALID_ARGUMENT, "ctx_lens, k_cache and v_cache must be non-NULL when N > 0");
    for (int l = 0; l < N; ++l) {
      if (!k_cache[l] || !v_cache[l])
        return fail(PE_ERR_INVALID_ARGUMENT, "cache pointer of layer %d is NULL", l);
      if (misaligned(k_cache[l]) || misaligned(v_cache[l]))
        return fail(PE_ERR_INVALID_ARGUMENT, "cache pointer of layer %d is not 16-byte aligned", l);
    }
  }
  if (misaligned(hidden3) || misaligned(mask_emb) || misaligned(h_shared) ||
      (logits_out && misaligned(logits_out)))
    return fail(PE_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  return PE_OK;
}

DraftCall forward_call(int32_t N, int32_t B, int32_t K, const void *hidden3, const int32_t *token_ids,
                       const void *mask_emb, const void *h_shared, const int32_t *ctx_lens, int64_t ctx_stride,
                       const void *const *k_cache, const void *const *v_cache, int32_t *draft_out,
                       float *logits_out) {
  DraftCall d{};
  d.N = N; d.B = B; d.K = K; d.mode = DRAFT_PARALLEL;
  d.in = hidden3; d.tok = token_ids; d.mask_emb = mask_emb; d.h_shared = h_shared;
  d.ctx_lens = ctx_lens; d.C = ctx_stride; d.pos_off = 0;
  d.kc = k_cache; d.vc = v_cache;
  d.draft_out = draft_out; d.logits_out = logits_out;
  return d;
}

// Scratch of the allocation-free forward: one array per device, in the
// library's code object (allocated when the module loads, held until the
// process ends).  Host code never passes `scratch` itself to a kernel: the
// name is a host-side stand-in, and the device address comes from
// hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = PE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's scratch address; the first call on a device also
// zeroes it on `s` (a fill kernel, no allocation).
pe_status scratch_for_device(hipStream_t s, void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PE_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    e = launch_zero(ptr, kScratchBytes, s);
    if (e != hipSuccess) return hip_fail(e, "scratch zero launch");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PE_OK;
}

}  // namespace

extern "C" {

pe_status pe_draft_forward(const pe_model *m, int32_t N, int32_t B, int32_t K, const void *hidden3,
                           const int32_t *token_ids, const void *mask_emb, const void *h_shared,
                           const int32_t *ctx_lens, int64_t ctx_stride, const void *const *k_cache,
                           const void *const *v_cache, int32_t *draft_out, float *logits_out,
                           void *workspace, size_t ws_bytes, void *stream) {
  pe_status st = check_forward(m, N, B, K, hidden3, token_ids, mask_emb, h_shared, ctx_lens, ctx_stride, k_cache,
                               v_cache, draft_out, logits_out);
  if (st != PE_OK) return st;
  if (misaligned(workspace)) return fail(PE_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  if (!workspace) return fail(PE_ERR_WORKSPACE, "workspace is NULL");
  const WsLayout W = layout(m->shape, B, K, ctx_stride);
  if (W.unsupported) return fail(PE_ERR_UNSUPPORTED, "B=%d K=%d ctx_stride=%ld: %s", B, K, (long)ctx_stride,
                                 W.unsupported);
  if (ws_bytes < W.total)
    return fail(PE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, W.total);
  const DraftCall d = forward_call(N, B, K, hidden3, token_ids, mask_emb, h_shared, ctx_lens, ctx_stride, k_cache,
                                   v_cache, draft_out, logits_out);
  return enqueue_draft(m, W, d, reinterpret_cast<char *>(workspace), reinterpret_cast<hipStream_t>(stream));
}

pe_status pe_draft_forward_noalloc(const pe_model *m, int32_t N, int32_t B, int32_t K, const void *hidden3,
                                   const int32_t *token_ids, const void *mask_emb, const void *h_shared,
                                   const int32_t *ctx_lens, int64_t ctx_stride, const void *const *k_cache,
                                   const void *const *v_cache, int32_t *draft_out, float *logits_out,
                                   void *stream) {
  pe_status st = check_forward(m, N, B, K, hidden3, token_ids, mask_emb, h_shared, ctx_lens, ctx_stride, k_cache,
                               v_cache, draft_out, logits_out);
  if (st != PE_OK) return st;
  const WsLayout W = layout(m->shape, B, K, ctx_stride);
  if (W.unsupported) return fail(PE_ERR_UNSUPPORTED, "B=%d K=%d ctx_stride=%ld: %s", B, K, (long)ctx_stride,
                                 W.unsupported);
  if (W.total > kScratchBytes)
    return fail(PE_ERR_UNSUPPORTED, "B=%d K=%d ctx_stride=%ld needs %zu bytes of scratch; the allocation-free "
                "forward holds %zu (use pe_draft_forward with a workspace)", B, K, (long)ctx_stride, W.total,
                kScratchBytes);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void *ws = nullptr;
  if ((st = scratch_for_device(s, &ws)) != PE_OK) return st;
  const DraftCall d = forward_call(N, B, K, hidden3, token_ids, mask_emb, h_shared, ctx_lens, ctx_stride, k_cache,
                                   v_cache, draft_out, logits_out);
  return enqueue_draft(m, W, d, reinterpret_cast<char *>(ws), s);
}

pe_status pe_draft_extend(const pe_model *m, int32_t N, int32_t B, int32_t T, const void *inputs,
                          int32_t input_kind, const int32_t *token_ids, const int32_t *ctx_lens,
                          int32_t pos_offset, int64_t ctx_stride, void *const *k_cache, void *const *v_cache,
                          int32_t *draft_out, float *logits_out, float *z_out, void *workspace, size_t ws_bytes,
                          void *stream) {
  if (!m) return fail(PE_ERR_INVALID_ARGUMENT, "model is NULL");
  const pe_config &c = m->cfg;
  if (N < 0 || N > c.n_layers)
    return fail(PE_ERR_INVALID_ARGUMENT, "N=%d outside [0, n_layers=%d]", N, c.n_layers);
  if (B < 1 || B > PE_DECODE_ROWS_MAX || T < 1 || T > PE_K_MAX || B * T > PE_DECODE_ROWS_MAX)
    return fail(PE_ERR_UNSUPPORTED, "B=%d T=%d outside 1<=T<=%d, B*T<=%d", B, T, PE_K_MAX, PE_DECODE_ROWS_MAX);
  if (input_kind != PE_INPUT_TARGET && input_kind != PE_INPUT_DRAFTER)
    return fail(PE_ERR_INVALID_ARGUMENT, "input_kind %d is neither PE_INPUT_TARGET nor PE_INPUT_DRAFTER",
                input_kind);
  if (!inputs || !token_ids) return fail(PE_ERR_INVALID_ARGUMENT, "inputs and token_ids must be non-NULL");
  if (pos_offset < 0 || ctx_stride < 1)
    return fail(PE_ERR_INVALID_ARGUMENT, "pos_offset must be >= 0 and ctx_stride >= 1");
  if (N > 0) {
    if (!ctx_lens || !k_cache || !v_cache)
      return fail(PE_ERR_INVALID_ARGUMENT, "ctx_lens, k_cache and v_cache must be non-NULL when N > 0");
    for (int l = 0; l < N; ++l) {
      if (!k_cache[l] || !v_cache[l])
        return fail(PE_ERR_INVALID_ARGUMENT, "cache pointer of layer %d is NULL", l);
      if (misaligned(k_cache[l]) || misaligned(v_cache[l]))
        return fail(PE_ERR_INVALID_ARGUMENT, "cache pointer of layer %d is not 16-byte aligned", l);
    }
  }
  if (misaligned(inputs) || (logits_out && misaligned(logits_out)) || (z_out && misaligned(z_out)) ||
      misaligned(workspace))
    return fail(PE_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  if (!workspace) return fail(PE_ERR_WORKSPACE, "workspace is NULL");
  const WsLayout W = layout(m->shape, B, T, ctx_stride);
  if (W.unsupported) return fail(PE_ERR_UNSUPPORTED, "B=%d T=%d ctx_stride=%ld: %s", B, T, (long)ctx_stride,
                                 W.unsupported);
  if (ws_bytes < W.total)
    return fail(PE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, W.total);
  DraftCall d{};
  d.N = N; d.B = B; d.K = T; d.mode = input_kind == PE_INPUT_TARGET ? EXTEND_TARGET : EXTEND_DRAFTER;
  d.in = inputs; d.tok = token_ids;
  d.ctx_lens = ctx_lens; d.C = ctx_stride; d.pos_off = pos_offset;
  d.kc = reinterpret_cast<const void *const *>(k_cache);
  d.vc = reinterpret_cast<const void *const *>(v_cache);
  d.kc_out = k_cache; d.vc_out = v_cache;
  d.draft_out = draft_out; d.logits_out = logits_out; d.z_out = z_out;
  return enqueue_draft(m, W, d, reinterpret_cast<char *>(workspace), reinterpret_cast<hipStream_t>(stream));
}

pe_status pe_accept(int32_t B, int32_t K, const int32_t *draft, const int32_t *target,
                    int32_t *accept_len, int32_t *out_tokens, void *stream) {
  if (B < 0) return fail(PE_ERR_INVALID_ARGUMENT, "B=%d must be >= 0", B);
  if (K < 1 || K > PE_K_MAX) return fail(PE_ERR_INVALID_ARGUMENT, "K=%d outside [1, %d]", K, PE_K_MAX);
  if (B == 0) return PE_OK;
  if (!draft || !target || !accept_len)
    return fail(PE_ERR_INVALID_ARGUMENT, "draft, target and accept_len must be non-NULL");
  hipError_t e = launch_accept(B, K, draft, target, accept_len, out_tokens,
                               reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "accept launch");
  return PE_OK;
}

pe_status pe_mask_create(int32_t n_max, int32_t K, void *stream, pe_mask **out) {
  if (!out) return fail(PE_ERR_INVALID_ARGUMENT, "out must be non-NULL");
  *out = nullptr;
  if (K < 1 || K > PE_K_MAX) return fail(PE_ERR_INVALID_ARGUMENT, "K=%d outside [1, %d]", K, PE_K_MAX);
  if (n_max < 1 || (long)n_max * K > kTrainRowsMax)
    return fail(PE_ERR_INVALID_ARGUMENT, "n_max=%d: need 1 <= n_max and n_max*K <= %ld", n_max,
                kTrainRowsMax);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  pe_mask *mk = new pe_mask();
  mk->n_max = n_max;
  mk->K = K;
  hipError_t e = hipMalloc(&mk->table, (size_t)n_max * K * sizeof(int2));
  if (e != hipSuccess) { delete mk; return hip_fail(e, "hipMalloc(mask table)"); }
  e = launch_mask_table(n_max, K, mk->table, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipFree(mk->table);
    delete mk;
    return hip_fail(e, "mask table build");
  }
  *out = mk;
  return PE_OK;
}

pe_status pe_mask_destroy(pe_mask *mk) {
  if (!mk) return fail(PE_ERR_INVALID_ARGUMENT, "mask is NULL");
  (void)hipFree(mk->table);
  delete mk;
  return PE_OK;
}

pe_status pe_mask_materialize(const pe_mask *mk, int32_t n, const int32_t *rows, int32_t L, uint8_t *out,
                              void *stream) {
  if (!mk || !rows || !out) return fail(PE_ERR_INVALID_ARGUMENT, "mask, rows and out must be non-NULL");
  if (n < 1 || n > mk->n_max) return fail(PE_ERR_INVALID_ARGUMENT, "n=%d outside [1, %d]", n, mk->n_max);
  if (L < 1 || L > 65536 || (long)L > (long)n * mk->K)
    return fail(PE_ERR_INVALID_ARGUMENT, "L=%d outside [1, min(n*K, 65536)]", L);
  hipError_t e = launch_mask_materialize(mk->table, n * mk->K, rows, L, out,
                                         reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mask materialize launch");
  return PE_OK;
}

pe_status pe_train_workspace_size(const pe_model *m, int32_t n, int32_t K, int32_t L, size_t *bytes) {
  if (!m || !bytes) return fail(PE_ERR_INVALID_ARGUMENT, "model and bytes must be non-NULL");
  if (K < 1 || K > PE_K_MAX) return fail(PE_ERR_INVALID_ARGUMENT, "K=%d outside [1, %d]", K, PE_K_MAX);
  if (n < 1 || L < 1 || (long)L > (long)n * K || L > kTrainRowsMax)
    return fail(PE_ERR_INVALID_ARGUMENT, "need n >= 1 and 1 <= L <= min(n*K, %ld)", kTrainRowsMax);
  *bytes = train_layout(m, n, K, L).total;
  return PE_OK;
}

}  // extern "C"

namespace {

// Activations of one layer that the backward reads (per-layer buffers of a
// training step; the plain forward reuses one set for every layer).
struct StepLayer {
  float *x = nullptr, *xm = nullptr, *lse = nullptr;  // residual in, after attention; softmax lse
  void *u1 = nullptr, *q = nullptr, *kall = nullptr, *vall = nullptr, *k0 = nullptr, *v0 = nullptr;
  void *attn = nullptr, *u2 = nullptr, *gu = nullptr, *h = nullptr;
};
struct StepSaves {
  std::vector<StepLayer> layer;
  float *xN = nullptr;   // residual after the last layer
  void *z = nullptr;     // final-norm rows (fragment tiles)
  void *logits = nullptr;  // [L][V] dtype
};

pe_status check_train_args(const pe_model *m, const pe_mask *mask, int32_t N, int32_t n, int32_t K,
                           const void *hidden3, const int32_t *token_ids, const void *mask_emb,
                           const void *h_shared, const int32_t *rows, int32_t L, const void *logits_out,
                           const void *workspace) {
  pe_status st = check_train_shape(m, mask, n, K, L);
  if (st != PE_OK) return st;
  const pe_config &c = m->cfg;
  if (N < 0 || N > c.n_layers)
    return fail(PE_ERR_INVALID_ARGUMENT, "N=%d outside [0, n_layers=%d]", N, c.n_layers);
  if (!hidden3 || !token_ids || !mask_emb || !h_shared || !rows)
    return fail(PE_ERR_INVALID_ARGUMENT, "hidden3, token_ids, mask_emb, h_shared and rows must be non-NULL");
  if (misaligned(hidden3) || misaligned(mask_emb) || misaligned(h_shared) ||
      (logits_out && misaligned(logits_out)) || misaligned(workspace))
    return fail(PE_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  if (!workspace) return fail(PE_ERR_WORKSPACE, "workspace is NULL");
  return PE_OK;
}

// The training-shape forward over L cells.  The first n_lead cells produce
// no outputs; cell n_lead + i writes output row out_rows[i] (out_rows NULL:
// cell i writes row i; targets outside [0, L_out) are dropped).  The LM head
// starts at the 16-row group holding cell n_lead.  With sv, every layer
// writes its own activation buffers (kept for the backward), the gate/up
// pre-activations and softmax statistics are kept too, and the logits go to
// sv->logits (rows from the 16-row group of n_lead on).
pe_status enqueue_train(const pe_model *m, const pe_mask *mask, int32_t N, int32_t n, int32_t K,
                        const void *hidden3, const int32_t *token_ids, const void *mask_emb,
                        const void *h_shared, const int32_t *rows, int32_t L, int32_t n_lead,
                        const int32_t *out_rows, int32_t L_out, void *logits_out, int32_t *argmax_out,
                        const TrainLayout &W, char *ws, const StepSaves *sv, void *stream) {
  pe_status st;
  const pe_config &c = m->cfg;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int *anc = reinterpret_cast<int *>(ws + W.anc);
  int *dep = reinterpret_cast<int *>(ws + W.dep);
  int *inv = reinterpret_cast<int *>(ws + W.inv);
  float *yfc = reinterpret_cast<float *>(ws + W.yfc);
  float *xres = reinterpret_cast<float *>(ws + W.xres);
  void *u = ws + W.u;
  const int H = c.hidden, hd = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads;
  const int dt = c.dtype;

  auto gemm = [&](const Tiled &t, int epi, TileGemmParams p) -> pe_status {
    p.wt = t.ptr; p.NT = t.NT; p.KT = t.KT; p.N = t.N; p.K = t.K;
    hipError_t e = launch_gemm_tile(dt, epi, p, m->num_cus, s);
    return e == hipSuccess ? PE_OK : hip_fail(e, "GEMM launch");
  };
  hipError_t e = launch_gather_rows(mask->table, n * K, rows, L, anc, dep, inv, s);
  if (e != hipSuccess) return hip_fail(e, "row gather launch");
  // Input fusion: fc over the n hidden rows and h_shared, then E[x_p] or mask_emb.
  {
    TileGemmParams p{};
    p.A = hidden3; p.lda = 3L * H; p.M = n;
    p.C = yfc; p.ldc = H;
    if ((st = gemm(m->fc, BEPI_STORE, p)) != PE_OK) return st;
    e = launch_matvec_tiled(dt, m->fc.ptr, m->fc.NT, m->fc.KT, H, h_shared, 3 * H, yfc + (size_t)n * H, s);
    if (e != hipSuccess) return hip_fail(e, "shared-state projection launch");
    e = launch_train_fuse(dt, yfc, m->embed, token_ids, mask_emb, anc, dep, L, n, H, c.vocab,
                          sv ? sv->layer.empty() ? sv->xN : sv->layer[0].x : xres, s);
    if (e != hipSuccess) return hip_fail(e, "fusion launch");
  }
  float *rope = reinterpret_cast<float *>(ws + W.rope);
  if (N > 0 && (e = launch_rope_table(m->inv_freq, n, hd / 2, rope, s)) != hipSuccess)
    return hip_fail(e, "rotation table launch");
  for (int l = 0; l < N; ++l) {
    const LayerT &Lw = m->layers[l];
    StepLayer B;
    if (sv) {
      B = sv->layer[l];
    } else {
      B.x = B.xm = xres; B.u1 = B.u2 = u;
      B.q = ws + W.q; B.kall = ws + W.kall; B.vall = ws + W.vall; B.k0 = ws + W.k0; B.v0 = ws + W.v0;
      B.attn = ws + W.attn; B.h = ws + W.h;
    }
    float *xnext = sv ? (l + 1 < N ? sv->layer[l + 1].x : sv->xN) : xres;
    if ((e = launch_rmsnorm_tiled(dt, B.x, Lw.attn_norm, L, H, c.rms_eps, B.u1, s)) != hipSuccess)
      return hip_fail(e, "RMSNorm launch");
    {
      TileGemmParams p{};
      p.A = B.u1; p.lda = H; p.M = L; p.a_tiled = 1;
      p.q = B.q; p.kall = B.kall; p.vall = B.vall; p.k0 = B.k0; p.v0 = B.v0;
      p.anc = anc; p.dep = dep; p.rope = rope;
      p.n = n; p.nq = nq; p.nkv = nkv; p.hd = hd;
      if ((st = gemm(Lw.qkv, BEPI_QKV, p)) != PE_OK) return st;
    }
    {
      TrainAttnParams a{};
      a.q = B.q; a.k0 = B.k0; a.v0 = B.v0; a.kall = B.kall; a.vall = B.vall;
      a.anc = anc; a.dep = dep; a.inv = inv;
      a.L = L; a.n = n; a.K = K; a.nq = nq; a.nkv = nkv; a.hd = hd; a.G = nq / nkv;
      a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
      a.out = B.attn;
      a.lse = B.lse;
      if ((e = launch_attn_train(dt, a, s)) != hipSuccess) return hip_fail(e, "attention launch");
    }
    {
      TileGemmParams p{};
      p.A = B.attn; p.lda = (long)nq * hd; p.M = L; p.a_tiled = 1;
      p.C = B.xm; p.Cin = B.x; p.ldc = H;  // xm = x + attn W_o (in place when they coincide)
      if ((st = gemm(Lw.o, BEPI_ACCUM, p)) != PE_OK) return st;
    }
    if ((e = launch_rmsnorm_tiled(dt, B.xm, Lw.mlp_norm, L, H, c.rms_eps, B.u2, s)) != hipSuccess)
      return hip_fail(e, "RMSNorm launch");
    {
      TileGemmParams p{};
      p.A = B.u2; p.lda = H; p.M = L; p.a_tiled = 1;
      p.h = B.h; p.I = c.intermediate; p.gu = B.gu;
      if ((st = gemm(Lw.gateup, B.gu ? BEPI_SWIGLU_SAVE : BEPI_SWIGLU, p)) != PE_OK) return st;
    }
    {
      TileGemmParams p{};
      p.A = B.h; p.lda = c.intermediate; p.M = L; p.a_tiled = 1;
      p.C = xnext; p.Cin = B.xm; p.ldc = H;  // x' = xm + h W_down
      if ((st = gemm(Lw.down, BEPI_ACCUM, p)) != PE_OK) return st;
    }
  }
  void *zrows = sv ? sv->z : u;
  if ((e = launch_rmsnorm_tiled(dt, sv ? sv->xN : xres, m->final_norm, L, H, c.rms_eps, zrows, s)) != hipSuccess)
    return hip_fail(e, "RMSNorm launch");
  if (sv) {
    logits_out = sv->logits;
    argmax_out = nullptr;
    out_rows = nullptr;
  }
  if (n_lead < L && (logits_out || argmax_out)) {
    // Rows before the 16-row group of cell n_lead are skipped; the group's
    // earlier rows are computed but not written.
    const int r0 = n_lead & ~15;
    TileGemmParams p{};
    p.A = reinterpret_cast<const char *>(zrows) + (size_t)(r0 >> 4) * m->lm.KT * 1024;
    p.lda = H; p.M = L - r0; p.a_tiled = 1;
    p.logits = sv ? reinterpret_cast<char *>(logits_out) + (size_t)r0 * c.vocab * m->esz : logits_out;
    p.ldc = c.vocab;
    p.out_rows = out_rows; p.row_skip = n_lead - r0; p.out_M = L_out;
    if (argmax_out) {  // the training step keeps only the logits
      p.keys = reinterpret_cast<unsigned long long *>(ws + W.keys);
      if ((e = launch_zero(p.keys, (size_t)p.M * 8, s)) != hipSuccess) return hip_fail(e, "key reset launch");
    }
    const bool prof = m->prof && m->nrec < (int)m->ev0.size();
    if (prof) (void)hipEventRecord(m->ev0[m->nrec], s);
    if ((st = gemm(m->lm, out_rows ? BEPI_LMHEAD_MAP : BEPI_LMHEAD, p)) != PE_OK) return st;
    if (prof) {
      (void)hipEventRecord(m->ev1[m->nrec], s);
      ++m->nrec;
    }
    if (argmax_out) {
      e = launch_argmax_rows(p.keys, p.M, argmax_out, out_rows, p.row_skip, L_out, s);
      if (e != hipSuccess) return hip_fail(e, "argmax launch");
    }
  }
  return PE_OK;
}

// Workspace of a training step: the forward's row bookkeeping, every
// layer's saved activations, the logits, and the backward's scratch.
struct StepLayout {
  TrainLayout tl{};
  std::vector<StepLayer> off;  // byte offsets stored in the pointer fields
  size_t xN = 0, z = 0, logits = 0, dlA = 0, row_loss = 0;
  size_t dx = 0, dx2 = 0, dxt = 0, gbuf = 0, dgu = 0, doutt = 0, D = 0, dq = 0, dk = 0, dv = 0, dqkv = 0;
  size_t packA = 0, packB = 0, part = 0, dntp = 0, dshared = 0, pk = 0, pv = 0, qt = 0, kpart = 0, kpart_bytes = 0;
  int qsplit = 1;
  size_t total = 0;
};

size_t tiles_bytes(long rows, long k, int ktile) {
  return (size_t)((rows + 15) / 16) * (size_t)((k + ktile - 1) / ktile) * 1024;
}

StepLayout step_layout(const pe_model *m, int N, long n, int K, long L) {
  const pe_config &c = m->cfg;
  StepLayout t{};
  const size_t H = c.hidden, esz = m->esz, hd = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads;
  const size_t I = c.intermediate, V = c.vocab;
  const size_t Lp = (size_t)(L + 15) / 16 * 16;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + std::max(bytes, (size_t)1), 256); return o; };
  t.tl.anc = take((size_t)L * 4);
  t.tl.dep = take((size_t)L * 4);
  t.tl.inv = take((size_t)n * K * 4);
  t.tl.rope = take(N > 0 ? (size_t)n * (hd / 2) * 8 : 0);
  t.tl.yfc = take((size_t)(n + 1) * H * 4);
  t.tl.keys = take((size_t)L * 8);
  t.off.resize(N);
  auto at = [](size_t o) { return reinterpret_cast<void *>(o); };
  for (int l = 0; l < N; ++l) {
    StepLayer &B = t.off[l];
    B.x = reinterpret_cast<float *>(at(take(L * H * 4)));
    B.xm = reinterpret_cast<float *>(at(take(L * H * 4)));
    B.lse = reinterpret_cast<float *>(at(take(L * nq * 4)));
    B.u1 = at(take(Lp * H * esz));
    B.q = at(take(L * nq * hd * esz));
    B.kall = at(take(L * nkv * hd * esz));
    B.vall = at(take(L * nkv * hd * esz));
    B.k0 = at(take(n * nkv * hd * esz));
    B.v0 = at(take(n * nkv * hd * esz));
    B.attn = at(take(Lp * nq * hd * esz));
    B.u2 = at(take(Lp * H * esz));
    B.gu = at(take(L * 2 * I * esz));
    B.h = at(take(Lp * I * esz));
  }
  t.xN = take(L * H * 4);
  t.z = take(Lp * H * esz);
  t.logits = take(L * V * esz);
  t.dlA = take(tiles_bytes(L, (long)V, m->ktile));
  t.row_loss = take(L * 4 * 3);  // row losses, then the cross-entropy's 2L scratch floats
  const size_t wide = std::max(std::max(H, I), nq * hd);
  t.dx = take(L * H * 4);
  t.dx2 = take(L * H * 4);
  t.dxt = take(L * H * esz);
  t.gbuf = take(L * wide * 4);
  t.dgu = take(L * 2 * I * esz);
  t.doutt = take(L * nq * hd * esz);
  t.D = take(L * nq * 4);
  t.dq = take(L * nq * hd * 4);
  t.dk = take(L * nkv * hd * 4);
  t.dv = take(L * nkv * hd * 4);
  t.dqkv = take(L * (nq + 2 * nkv) * hd * esz);
  const int kt = m->ktile;
  size_t a = tiles_bytes((long)V, L, kt);
  a = std::max(a, tiles_bytes((long)(2 * I), L, kt));
  a = std::max(a, tiles_bytes((long)((nq + 2 * nkv) * hd), L, kt));
  a = std::max(a, tiles_bytes((long)H, std::max(L, n), kt));
  t.packA = take(a);
  size_t b = tiles_bytes((long)std::max(std::max(H, I), nq * hd), L, kt);
  b = std::max(b, tiles_bytes((long)(3 * H), n, kt));
  t.packB = take(b);
  t.part = take((size_t)((L + 63) / 64) * H * 4);
  t.dntp = take(n * H * esz);
  t.dshared = take(H * 4);
  // Query shares per depth-0 key tile in the attention backward: about 256
  // rows each, at most 16.
  t.qsplit = (int)std::min<long>(16, std::max<long>(1, L / 256));
  t.pk = take((size_t)t.qsplit * n * nkv * hd * 4);
  t.pv = take((size_t)t.qsplit * n * nkv * hd * 4);
  t.qt = take(attn_bwd_tile_bytes((int)L, (int)nkv, (int)(nq / nkv), (int)hd, c.dtype));
  // K-split partials of the backward's GEMMs, the largest that any of them
  // plans: data gradients C [L][Nw] = dY W (the transposed weight [Nw][Kw])
  // and weight gradients C [rows][cols] += A^T B over Kr rows
  size_t kp = 0;
  auto ksplit_need = [&](size_t M, size_t Nw, size_t Kw) {
    const TileDims d = tile_dims((int)Nw, (int)Kw, kt);
    const int ks = tile_gemm_ksplit((long)M, d.NT, d.KT, m->num_cus);
    kp = std::max(kp, (size_t)(ks - 1) * M * Nw * 4);
  };
  ksplit_need(L, H, V);
  ksplit_need(V, H, L);
  ksplit_need(H, 3 * H, n);
  if (N > 0) {
    ksplit_need(L, I, H);
    ksplit_need(L, H, 2 * I);
    ksplit_need(L, nq * hd, H);
    ksplit_need(L, H, (nq + 2 * nkv) * hd);
    ksplit_need(H, I, L);
    ksplit_need(I, H, L);
    ksplit_need(H, nq * hd, L);
    ksplit_need(nq * hd, H, L);
    ksplit_need(nkv * hd, H, L);
  }
  t.kpart = take(kp);
  t.kpart_bytes = kp;
  t.total = off;
  return t;
}

// Backward of the training step enqueued after the forward with saves:
// cross-entropy -> LM head -> final norm -> layers in reverse -> input
// fusion.  Data gradients: C = dY W with W's transposed tiles; weight
// gradients: C += dY^T X with both operands packed transposed (k = rows).
pe_status enqueue_backward(const pe_model *m, int32_t N, int32_t n, int32_t K, const void *hidden3,
                           const void *h_shared, int32_t L, int32_t n_lead, const int32_t *labels,
                           float loss_scale, float *loss_out, const pe_grads *gr, const StepLayout &SL,
                           const StepSaves &sv, char *ws, hipStream_t s) {
  const pe_config &c = m->cfg;
  const int dt = c.dtype, H = c.hidden, I = c.intermediate, V = c.vocab;
  const int hd = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads, kt = m->ktile;
  const int QKV = (nq + 2 * nkv) * hd;
  const int KTL = (L + kt - 1) / kt;
  int *anc = reinterpret_cast<int *>(ws + SL.tl.anc);
  int *dep = reinterpret_cast<int *>(ws + SL.tl.dep);
  int *inv = reinterpret_cast<int *>(ws + SL.tl.inv);
  auto F = [&](size_t o) { return reinterpret_cast<float *>(ws + o); };
  float *dx = F(SL.dx), *dx2 = F(SL.dx2), *gbuf = F(SL.gbuf), *part = F(SL.part);
  void *dxt = ws + SL.dxt, *packA = ws + SL.packA, *packB = ws + SL.packB;
  const int nblk = (L + 63) / 64;
  hipError_t e;
  pe_status st;
  auto chk = [&](hipError_t err, const char *what) { return err == hipSuccess ? PE_OK : hip_fail(err, what); };
  auto gemm = [&](const void *A, int a_tiled, long lda, int M, const u32x4 *Bt, int NT, int KT, int Nn, int Kk,
                  int epi, float *C, long ldc) -> pe_status {
    TileGemmParams p{};
    p.A = A; p.a_tiled = a_tiled; p.lda = lda; p.M = M;
    p.wt = Bt; p.NT = NT; p.KT = KT; p.N = Nn; p.K = Kk;
    p.C = C; p.ldc = ldc;
    if (epi == BEPI_STORE || epi == BEPI_ACCUM) {
      // split over K when the tiles alone leave CUs idle (partials summed after)
      const int ks = tile_gemm_ksplit(M, NT, KT, m->num_cus);
      if (ks > 1 && (size_t)(ks - 1) * M * ldc * 4 <= SL.kpart_bytes) {
        p.ksplit = ks;
        p.kpart = F(SL.kpart);
        p.kpart_stride = (long)M * ldc;
      }
    }
    pe_status r = chk(launch_gemm_tile(dt, epi, p, m->num_cus, s), "backward GEMM launch");
    if (r == PE_OK && p.ksplit > 1)
      r = chk(launch_ksum(C, ldc, M, Nn, p.kpart, p.kpart_stride, p.ksplit, s), "K-split sum launch");
    return r;
  };
  auto dgrad = [&](const void *dY, long ld, const Tiled &WT, float *out) {  // out [L][WT.N] = dY W
    return gemm(dY, 0, ld, L, WT.ptr, WT.NT, WT.KT, WT.N, WT.K, BEPI_STORE, out, WT.N);
  };
  // grad[rows][cols] += A^T B over the L cells, with A [L][rows] (packed into
  // packA) and B [L][cols] (packed into packB) already transposed.
  auto wgrad = [&](int rows, int cols, int a_row0, float *grad, int Kk) {
    const int KTk = (Kk + kt - 1) / kt;
    const char *A = reinterpret_cast<const char *>(packA) + (size_t)(a_row0 / 16) * KTk * 1024;
    return gemm(A, 1, 0, rows, reinterpret_cast<const u32x4 *>(packB), (cols + 15) / 16, KTk, cols, Kk, BEPI_ACCUM,
                grad, cols);
  };
  auto packT = [&](int kind, const void *src, long ld, int R, int C, void *dst) {
    return chk(launch_pack_t(dt, kind, src, ld, R, C, dst, (R + kt - 1) / kt, 0, s), "pack launch");
  };

  // ---- loss and LM head: dlogits as tiles of [L][V] and of [V][L] (packA)
  void *dlA = ws + SL.dlA;
  if ((st = chk(launch_ce_tiles(dt, sv.logits, L, V, anc, dep, labels, n, n_lead, loss_scale, F(SL.row_loss),
                                F(SL.row_loss) + L, dlA,
                                packA, s), "cross-entropy launch")) != PE_OK) return st;
  if (loss_out && (st = chk(launch_sum_acc(F(SL.row_loss), L, loss_out, s), "loss sum launch")) != PE_OK) return st;
  if ((st = gemm(dlA, 1, V, L, m->lmT.ptr, m->lmT.NT, m->lmT.KT, m->lmT.N, m->lmT.K, BEPI_STORE, gbuf, H)) != PE_OK)
    return st;                                                                      // dz [L][H]
  if (gr->lm_head) {
    if ((st = packT(PACK_TILED, sv.z, 0, L, H, packB)) != PE_OK) return st;          // z^T
    if ((st = wgrad(V, H, 0, gr->lm_head, L)) != PE_OK) return st;
  }
  if ((st = chk(launch_rms_bwd(dt, sv.xN, m->final_norm, gbuf, nullptr, L, H, c.rms_eps, dx, dxt, part, s),
                "RMSNorm backward launch")) != PE_OK) return st;
  if (gr->final_norm && (st = chk(launch_colsum_acc(part, nblk, H, gr->final_norm, s), "gain sum")) != PE_OK)
    return st;

  for (int l = N - 1; l >= 0; --l) {
    const LayerT &Lw = m->layers[l];
    const StepLayer &B = sv.layer[l];
    const pe_layer_grads *g = gr->layers ? &gr->layers[l] : nullptr;
    // MLP: x_out = xm + (silu(gate) up) W_down^T; dx holds dL/dx_out.
    if ((st = dgrad(dxt, H, Lw.downT, gbuf)) != PE_OK) return st;                    // dh [L][I]
    if (g && g->w_down) {
      if ((st = packT(PACK_ROW, dxt, H, L, H, packA)) != PE_OK) return st;
      if ((st = packT(PACK_TILED, B.h, 0, L, I, packB)) != PE_OK) return st;
      if ((st = wgrad(H, I, 0, g->w_down, L)) != PE_OK) return st;
    }
    if ((st = chk(launch_swiglu_bwd(dt, gbuf, B.gu, L, I, ws + SL.dgu, s), "SwiGLU backward launch")) != PE_OK)
      return st;
    if ((st = dgrad(ws + SL.dgu, 2L * I, Lw.guT, gbuf)) != PE_OK) return st;         // du2 [L][H]
    if (g && (g->w_gate || g->w_up)) {
      if ((st = packT(PACK_ROW, ws + SL.dgu, 2L * I, L, 2 * I, packA)) != PE_OK) return st;
      if ((st = packT(PACK_TILED, B.u2, 0, L, H, packB)) != PE_OK) return st;
      if (g->w_gate && (st = wgrad(I, H, 0, g->w_gate, L)) != PE_OK) return st;
      if (g->w_up && (st = wgrad(I, H, I, g->w_up, L)) != PE_OK) return st;
    }
    // mlp norm: dxm = dx + RMSNorm'(xm) du2
    if ((st = chk(launch_rms_bwd(dt, B.xm, Lw.mlp_norm, gbuf, dx, L, H, c.rms_eps, dx2, dxt, part, s),
                  "RMSNorm backward launch")) != PE_OK) return st;
    if (g && g->mlp_norm && (st = chk(launch_colsum_acc(part, nblk, H, g->mlp_norm, s), "gain sum")) != PE_OK)
      return st;
    // O projection: xm = x + attn W_o^T
    if ((st = dgrad(dxt, H, Lw.oT, gbuf)) != PE_OK) return st;                       // d attn [L][nq hd]
    if (g && g->wo) {
      if ((st = packT(PACK_ROW, dxt, H, L, H, packA)) != PE_OK) return st;
      if ((st = packT(PACK_TILED, B.attn, 0, L, nq * hd, packB)) != PE_OK) return st;
      if ((st = wgrad(H, nq * hd, 0, g->wo, L)) != PE_OK) return st;
    }
    // attention
    if ((st = chk(launch_attn_bwd_pre(dt, gbuf, B.attn, L, nq, hd, ws + SL.doutt, F(SL.D), s),
                  "attention backward launch")) != PE_OK) return st;
    {
      AttnBwdParams a{};
      a.q = B.q; a.k0 = B.k0; a.v0 = B.v0; a.kall = B.kall; a.vall = B.vall;
      a.dout = ws + SL.doutt; a.lse = B.lse; a.D = F(SL.D);
      a.anc = anc; a.dep = dep; a.inv = inv;
      a.L = L; a.n = n; a.K = K; a.nq = nq; a.nkv = nkv; a.hd = hd; a.G = nq / nkv;
      a.scale = (float)(1.0 / sqrt((double)hd));
      a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
      a.dq = F(SL.dq); a.dk = F(SL.dk); a.dv = F(SL.dv);
      a.qsplit = SL.qsplit; a.pk = F(SL.pk); a.pv = F(SL.pv);
      {
        const int G = nq / nkv, QC = 64 / G, Tq = (L + QC - 1) / QC, NC = hd / kt, NKC = dt == 1 ? 2 : 4;
        a.qt = reinterpret_cast<u32x4 *>(ws + SL.qt);
        a.qinfo = reinterpret_cast<float4 *>(ws + SL.qt + (size_t)nkv * Tq * (8 * NC + 2 * (hd / 16) * NKC) * 1024);
      }
      if ((st = chk(launch_attn_bwd(dt, a, s), "attention backward launch")) != PE_OK) return st;
    }
    if ((st = chk(launch_rope_bwd(dt, F(SL.dq), F(SL.dk), F(SL.dv), anc, dep, m->inv_freq, L, nq, nkv, hd,
                                  ws + SL.dqkv, s), "RoPE backward launch")) != PE_OK) return st;
    if ((st = dgrad(ws + SL.dqkv, QKV, Lw.qkvT, gbuf)) != PE_OK) return st;          // du1 [L][H]
    if (g && (g->wq || g->wk || g->wv)) {
      if ((st = packT(PACK_ROW, ws + SL.dqkv, QKV, L, QKV, packA)) != PE_OK) return st;
      if ((st = packT(PACK_TILED, B.u1, 0, L, H, packB)) != PE_OK) return st;
      if (g->wq && (st = wgrad(nq * hd, H, 0, g->wq, L)) != PE_OK) return st;
      if (g->wk && (st = wgrad(nkv * hd, H, nq * hd, g->wk, L)) != PE_OK) return st;
      if (g->wv && (st = wgrad(nkv * hd, H, (nq + nkv) * hd, g->wv, L)) != PE_OK) return st;
    }
    // attn norm: dx = dxm + RMSNorm'(x) du1
    if ((st = chk(launch_rms_bwd(dt, B.x, Lw.attn_norm, gbuf, dx2, L, H, c.rms_eps, dx, dxt, part, s),
                  "RMSNorm backward launch")) != PE_OK) return st;
    if (g && g->attn_norm && (st = chk(launch_colsum_acc(part, nblk, H, g->attn_norm, s), "gain sum")) != PE_OK)
      return st;
  }

  // ---- input fusion: depth-0 cells E[x_p] + fc(h_p), deeper cells mask_emb + fc(h_shared)
  void *dntp = ws + SL.dntp;
  float *dsh = F(SL.dshared);
  if ((st = chk(launch_zero(dntp, (size_t)n * H * m->esz, s), "zero launch")) != PE_OK) return st;
  if ((st = chk(launch_zero(dsh, (size_t)H * 4, s), "zero launch")) != PE_OK) return st;
  if ((st = chk(launch_fuse_bwd(dt, dx, anc, dep, L, n, H, dntp, gr->embed_rows, part, s), "fusion backward")) !=
      PE_OK) return st;
  if ((st = chk(launch_colsum_acc(part, nblk, H, dsh, s), "column sum")) != PE_OK) return st;
  if (gr->mask_emb && (st = chk(launch_colsum_acc(part, nblk, H, gr->mask_emb, s), "column sum")) != PE_OK)
    return st;
  if (gr->h_shared &&
      (st = chk(launch_matvec_acc(dt, m->fcT.ptr, m->fcT.NT, m->fcT.KT, 3 * H, dsh, H, gr->h_shared, s),
                "shared-state gradient")) != PE_OK) return st;
  if (gr->fc) {
    if ((st = packT(PACK_ROW, dntp, H, n, H, packA)) != PE_OK) return st;
    if ((st = packT(PACK_ROW, hidden3, 3L * H, n, 3 * H, packB)) != PE_OK) return st;
    if ((st = wgrad(H, 3 * H, 0, gr->fc, n)) != PE_OK) return st;
    if ((st = chk(launch_outer_acc(dt, dsh, h_shared, H, 3 * H, gr->fc, s), "outer product")) != PE_OK) return st;
  }
  (void)KTL;
  (void)e;
  return PE_OK;
}

}  // namespace

extern "C" {

pe_status pe_train_forward(const pe_model *m, const pe_mask *mask, int32_t N, int32_t n, int32_t K,
                           const void *hidden3, const int32_t *token_ids, const void *mask_emb,
                           const void *h_shared, const int32_t *rows, int32_t L, void *logits_out,
                           int32_t *argmax_out, void *workspace, size_t ws_bytes, void *stream) {
  pe_status st = check_train_args(m, mask, N, n, K, hidden3, token_ids, mask_emb, h_shared, rows, L, logits_out,
                                  workspace);
  if (st != PE_OK) return st;
  const TrainLayout W = train_layout(m, n, K, L);
  if (ws_bytes < W.total) return fail(PE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, W.total);
  return enqueue_train(m, mask, N, n, K, hidden3, token_ids, mask_emb, h_shared, rows, L, 0, nullptr, L,
                       logits_out, argmax_out, W, reinterpret_cast<char *>(workspace), nullptr, stream);
}

pe_status pe_train_forward_chunk(const pe_model *m, const pe_mask *mask, int32_t N, int32_t n, int32_t K,
                                 const void *hidden3, const int32_t *token_ids, const void *mask_emb,
                                 const void *h_shared, const int32_t *cells, int32_t L, int32_t n_lead,
                                 const int32_t *out_rows, int32_t L_out, void *logits_out, int32_t *argmax_out,
                                 void *workspace, size_t ws_bytes, void *stream) {
  if (n_lead < 0 || n_lead > L)
    return fail(PE_ERR_INVALID_ARGUMENT, "n_lead=%d outside [0, L=%d]", n_lead, L);
  if (L_out < 1) return fail(PE_ERR_INVALID_ARGUMENT, "L_out=%d must be >= 1", L_out);
  if (n_lead < L && (logits_out || argmax_out) && !out_rows)
    return fail(PE_ERR_INVALID_ARGUMENT, "out_rows must be non-NULL when cells past n_lead write outputs");
  pe_status st = check_train_args(m, mask, N, n, K, hidden3, token_ids, mask_emb, h_shared, cells, L, logits_out,
                                  workspace);
  if (st != PE_OK) return st;
  const TrainLayout W = train_layout(m, n, K, L);
  if (ws_bytes < W.total) return fail(PE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, W.total);
  return enqueue_train(m, mask, N, n, K, hidden3, token_ids, mask_emb, h_shared, cells, L, n_lead, out_rows,
                       L_out, logits_out, argmax_out, W, reinterpret_cast<char *>(workspace), nullptr, stream);
}

pe_status pe_model_prepare_backward(pe_model *m, const pe_weights *w, void *stream) {
  if (!m || !w) return fail(PE_ERR_INVALID_ARGUMENT, "model and weights must be non-NULL");
  const pe_config &c = m->cfg;
  if (!w->fc || !w->lm_head || (c.n_layers > 0 && !w->layers))
    return fail(PE_ERR_INVALID_ARGUMENT, "a required weight pointer is NULL");
  if (c.hidden % m->ktile || c.intermediate % m->ktile)
    return fail(PE_ERR_UNSUPPORTED, "the backward needs hidden and intermediate multiples of %d", m->ktile);
  if (m->has_bwd) return PE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int H = c.hidden, I = c.intermediate, hd = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads;
  const int kt = m->ktile;
  // Tiles of the transpose of row-major sources stacked along the
  // transpose's k axis (source i holds rows[i] rows of cols columns).
  auto build = [&](Tiled &t, const void *const *src, const int *rows, int nsrc, int cols) -> pe_status {
    int K = 0;
    for (int i = 0; i < nsrc; ++i) K += rows[i];
    t.N = cols; t.K = K; t.NT = (cols + 15) / 16; t.KT = (K + kt - 1) / kt;
    const size_t bytes = (size_t)t.NT * t.KT * 1024;
    if (bytes > 0x7FFFF000ull) return fail(PE_ERR_UNSUPPORTED, "transposed weight tiles exceed 2 GiB");
    hipError_t e = hipMalloc(&t.ptr, bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(transposed weight tiles)");
    m->allocs.push_back(t.ptr);
    int kt0 = 0;
    for (int i = 0; i < nsrc; ++i) {
      if (i + 1 < nsrc && rows[i] % kt) return fail(PE_ERR_UNSUPPORTED, "stacked weight rows not a multiple of %d", kt);
      e = launch_pack_t(c.dtype, PACK_ROW, src[i], cols, rows[i], cols, t.ptr, t.KT, kt0, s);
      if (e != hipSuccess) return hip_fail(e, "transposed tiling launch");
      kt0 += rows[i] / kt;
    }
    return PE_OK;
  };
  pe_status st;
  {
    const void *src[1] = {w->lm_head};
    const int rows[1] = {c.vocab};
    if ((st = build(m->lmT, src, rows, 1, H)) != PE_OK) return st;
  }
  {
    const void *src[1] = {w->fc};
    const int rows[1] = {H};
    if ((st = build(m->fcT, src, rows, 1, 3 * H)) != PE_OK) return st;
  }
  for (int l = 0; l < c.n_layers; ++l) {
    const pe_layer_weights &Lw = w->layers[l];
    if (!Lw.wq || !Lw.wk || !Lw.wv || !Lw.wo || !Lw.w_gate || !Lw.w_up || !Lw.w_down)
      return fail(PE_ERR_INVALID_ARGUMENT, "layer %d has a NULL weight pointer", l);
    LayerT &T = m->layers[l];
    const void *qkv[3] = {Lw.wq, Lw.wk, Lw.wv};
    const int qkv_rows[3] = {nq * hd, nkv * hd, nkv * hd};
    const void *o[1] = {Lw.wo};
    const int o_rows[1] = {H};
    const void *gu[2] = {Lw.w_gate, Lw.w_up};
    const int gu_rows[2] = {I, I};
    const void *dn[1] = {Lw.w_down};
    const int dn_rows[1] = {H};
    if ((st = build(T.qkvT, qkv, qkv_rows, 3, H)) || (st = build(T.oT, o, o_rows, 1, nq * hd)) ||
        (st = build(T.guT, gu, gu_rows, 2, H)) || (st = build(T.downT, dn, dn_rows, 1, I)))
      return st;
  }
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize after transposed tiling");
  m->has_bwd = true;
  return PE_OK;
}

pe_status pe_train_step_workspace_size(const pe_model *m, int32_t N, int32_t n, int32_t K, int32_t L,
                                       size_t *bytes) {
  if (!m || !bytes) return fail(PE_ERR_INVALID_ARGUMENT, "model and bytes must be non-NULL");
  if (N < 0 || N > m->cfg.n_layers)
    return fail(PE_ERR_INVALID_ARGUMENT, "N=%d outside [0, n_layers=%d]", N, m->cfg.n_layers);
  if (n < 1 || K < 1 || L < 1 || (long)L > (long)n * K || L > kTrainRowsMax)
    return fail(PE_ERR_INVALID_ARGUMENT, "need n >= 1 and 1 <= L <= min(n*K, %ld)", kTrainRowsMax);
  *bytes = step_layout(m, N, n, K, L).total;
  return PE_OK;
}

pe_status pe_train_step(const pe_model *m, const pe_mask *mask, int32_t N, int32_t n, int32_t K,
                        const void *hidden3, const int32_t *token_ids, const void *mask_emb, const void *h_shared,
                        const int32_t *cells, int32_t L, int32_t n_lead, const int32_t *labels, float loss_scale,
                        float *loss_out, const pe_grads *grads, void *workspace, size_t ws_bytes, void *stream) {
  pe_status st = check_train_args(m, mask, N, n, K, hidden3, token_ids, mask_emb, h_shared, cells, L, nullptr,
                                  workspace);
  if (st != PE_OK) return st;
  const pe_config &c = m->cfg;
  if (!m->has_bwd) return fail(PE_ERR_INVALID_ARGUMENT, "call pe_model_prepare_backward before pe_train_step");
  if (!labels || !grads) return fail(PE_ERR_INVALID_ARGUMENT, "labels and grads must be non-NULL");
  if (N > 0 && !grads->layers) return fail(PE_ERR_INVALID_ARGUMENT, "grads->layers must be non-NULL when N > 0");
  if (n_lead < 0 || n_lead > L) return fail(PE_ERR_INVALID_ARGUMENT, "n_lead=%d outside [0, L=%d]", n_lead, L);
  if (c.head_dim != 64 && !(c.dtype == PE_BF16 && c.head_dim == 128))
    return fail(PE_ERR_UNSUPPORTED, "the attention backward supports head_dim 64 (and 128 for bf16)");
  if (c.n_q_heads / c.n_kv_heads > 64) return fail(PE_ERR_UNSUPPORTED, "GQA groups above 64 heads");
  if (c.hidden > 4096) return fail(PE_ERR_UNSUPPORTED, "hidden above 4096");
  const StepLayout SL = step_layout(m, N, n, K, L);
  if (ws_bytes < SL.total) return fail(PE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, SL.total);
  char *ws = reinterpret_cast<char *>(workspace);
  StepSaves sv;
  sv.layer.resize(N);
  auto P = [&](const void *off) -> void * { return ws + reinterpret_cast<size_t>(off); };
  for (int l = 0; l < N; ++l) {
    const StepLayer &O = SL.off[l];
    StepLayer &B = sv.layer[l];
    B.x = reinterpret_cast<float *>(P(O.x)); B.xm = reinterpret_cast<float *>(P(O.xm));
    B.lse = reinterpret_cast<float *>(P(O.lse));
    B.u1 = P(O.u1); B.q = P(O.q); B.kall = P(O.kall); B.vall = P(O.vall); B.k0 = P(O.k0); B.v0 = P(O.v0);
    B.attn = P(O.attn); B.u2 = P(O.u2); B.gu = P(O.gu); B.h = P(O.h);
  }
  sv.xN = reinterpret_cast<float *>(ws + SL.xN);
  sv.z = ws + SL.z;
  sv.logits = ws + SL.logits;
  if ((st = enqueue_train(m, mask, N, n, K, hidden3, token_ids, mask_emb, h_shared, cells, L, n_lead, nullptr, L,
                          nullptr, nullptr, SL.tl, ws, &sv, stream)) != PE_OK)
    return st;
  return enqueue_backward(m, N, n, K, hidden3, h_shared, L, n_lead, labels, loss_scale, loss_out, grads, SL, sv, ws,
                          reinterpret_cast<hipStream_t>(stream));
}

pe_status pe_profile_enable(pe_model *m, int32_t enable) {
  if (!m) return fail(PE_ERR_INVALID_ARGUMENT, "model is NULL");
  if (enable && m->ev0.empty()) {
    const int n = 4096;
    m->ev0.resize(n);
    m->ev1.resize(n);
    for (int i = 0; i < n; ++i) {
      hipError_t e = hipEventCreate(&m->ev0[i]);
      if (e == hipSuccess) e = hipEventCreate(&m->ev1[i]);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
  }
  m->prof = enable != 0;
  m->nrec = 0;
  return PE_OK;
}

pe_status pe_profile_read(pe_model *m, int32_t *count, double *mean_ms) {
  if (!m || !count || !mean_ms) return fail(PE_ERR_INVALID_ARGUMENT, "NULL argument");
  *count = m->nrec;
  *mean_ms = 0.0;
  if (m->nrec == 0) return PE_OK;
  hipError_t e = hipEventSynchronize(m->ev1[m->nrec - 1]);
  if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  double sum = 0.0;
  for (int i = 0; i < m->nrec; ++i) {
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, m->ev0[i], m->ev1[i]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    sum += ms;
  }
  *mean_ms = sum / m->nrec;
  m->nrec = 0;
  return PE_OK;
}

}  // extern "C"
