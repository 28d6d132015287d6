// libdllm host runtime: argument validation, workspace planning, the launch sequences of
// prefill / refresh / block step, the generation loop and the C ABI (include/dllm.h).
#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "../../include/dllm.h"
#include "../../include/dllm_synth.h"
#include "kernels.h"

using namespace dllm;

namespace {

thread_local std::string g_err;

dllm_status fail(dllm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIP_TRY(expr)                                                              \
  do {                                                                             \
    hipError_t _e = (expr);                                                        \
    if (_e != hipSuccess)                                                          \
      return fail(DLLM_E_HIP, "%s failed: %s", #expr, hipGetErrorString(_e));      \
  } while (0)

// ------------------------------------------------------------------ profiling
struct Prof {
  int cls = DLLM_K_NONE;
  int every = 1;               // time one launch in `every`
  long long seen = 0;          // launches of the class since selection
  std::vector<hipEvent_t> ev;  // pairs
  size_t used = 0;             // events recorded
};
Prof g_prof;

struct ProfScope {
  hipStream_t st;
  bool on;
  ProfScope(int cls, hipStream_t s) : st(s), on(cls == g_prof.cls) {
    if (!on) return;
    on = (g_prof.seen++ % g_prof.every) == 0;
    if (!on) return;
    if (g_prof.used + 2 > g_prof.ev.size()) {
      for (int i = 0; i < 256; ++i) {
        hipEvent_t e;
        // timing only: no system-scope fence (an L2 write-back and invalidate) at record
        if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
          on = false;
          return;
        }
        g_prof.ev.push_back(e);
      }
    }
    (void)hipEventRecord(g_prof.ev[g_prof.used], st);
  }
  ~ProfScope() {
    if (!on) return;
    (void)hipEventRecord(g_prof.ev[g_prof.used + 1], st);
    g_prof.used += 2;
  }
};

// Host-side roctx range around the enqueue of one stage (prefill, refresh, a step), so a
// profiler's marker trace shows which kernels each stage launched.
struct Range {
  explicit Range(const char* name) { roctxRangePushA(name); }
  ~Range() { roctxRangePop(); }
};

// ------------------------------------------------------------------ shapes
struct Dims {
  int L, d, Hq, Hkv, D, F, V, mask, dtype, esz;
  int B, P, G, K, S, Sp, mode, nblocks;
  float tau, eps, theta, lscale;
};

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

dllm_status check_model(const dllm_model_desc* m) {
  if (!m) return fail(DLLM_E_NULL, "model descriptor is NULL");
  if (m->dtype != DLLM_F32 && m->dtype != DLLM_BF16) return fail(DLLM_E_ARG, "bad dtype %d", m->dtype);
  if (m->n_layers < 1 || m->d_model < 1 || m->n_heads < 1 || m->n_kv_heads < 1 ||
      m->head_dim < 2 || m->d_ffn < 1 || m->vocab < 2)
    return fail(DLLM_E_SHAPE, "model sizes must be positive (vocab >= 2, head_dim >= 2)");
  if (m->n_heads % m->n_kv_heads) return fail(DLLM_E_SHAPE, "n_heads %% n_kv_heads != 0");
  if (m->head_dim % 2 || 128 % m->head_dim)
    return fail(DLLM_E_UNSUPPORTED, "head_dim must be even and divide 128");
  if (m->d_model % 64 || m->d_ffn % 64 || (m->n_heads * m->head_dim) % 64)
    return fail(DLLM_E_UNSUPPORTED, "d_model, d_ffn and n_heads*head_dim must be multiples of 64");
  if (m->dtype == DLLM_BF16 &&
      (m->head_dim != 128 || m->d_model % 256 || m->d_ffn % 256 || (m->n_heads * 128) % 256 ||
       m->vocab % 8))
    return fail(DLLM_E_UNSUPPORTED,
                "bf16 models need head_dim 128, d_model, d_ffn, n_heads*128 multiples of 256 "
                "and vocab a multiple of 8");
  if (m->mask_id < 0 || m->mask_id >= m->vocab) return fail(DLLM_E_ARG, "mask_id outside [0, vocab)");
  if (!std::isfinite(m->rope_theta) || m->rope_theta <= 0.f) return fail(DLLM_E_ARG, "bad rope_theta");
  if (!std::isfinite(m->norm_eps) || m->norm_eps < 0.f) return fail(DLLM_E_ARG, "bad norm_eps");
  if (!std::isfinite(m->logit_scale)) return fail(DLLM_E_ARG, "bad logit_scale");
  if (!m->embed || !m->final_norm || !m->lm_head) return fail(DLLM_E_NULL, "embed/final_norm/lm_head is NULL");
  if (!m->attn_norm || !m->w_qkv || !m->w_o || !m->ffn_norm || !m->w_gate_up || !m->w_down)
    return fail(DLLM_E_NULL, "a per-layer weight array is NULL");
  for (int l = 0; l < m->n_layers; ++l)
    if (!m->attn_norm[l] || !m->w_qkv[l] || !m->w_o[l] || !m->ffn_norm[l] || !m->w_gate_up[l] ||
        !m->w_down[l])
      return fail(DLLM_E_NULL, "layer %d has a NULL weight", l);
  return DLLM_OK;
}

dllm_status dims_of(const dllm_model_desc* m, const dllm_seq_desc* s, Dims* o) {
  dllm_status st = check_model(m);
  if (st) return st;
  if (!s) return fail(DLLM_E_NULL, "sequence descriptor is NULL");
  if (s->batch < 1 || s->prompt_len < 0 || s->gen_len < 1 || s->block_len < 1)
    return fail(DLLM_E_SHAPE, "batch, gen_len, block_len must be >= 1 and prompt_len >= 0");
  if (s->gen_len % s->block_len) return fail(DLLM_E_SHAPE, "gen_len %% block_len != 0");
  if (s->block_len > 64) return fail(DLLM_E_UNSUPPORTED, "block_len > 64");
  if (s->cache_mode != DLLM_CACHE_NONE && s->cache_mode != DLLM_CACHE_PREFIX &&
      s->cache_mode != DLLM_CACHE_DUAL)
    return fail(DLLM_E_ARG, "bad cache_mode %d", s->cache_mode);
  if (std::isnan(s->threshold)) return fail(DLLM_E_ARG, "threshold is NaN");
  Dims& d = *o;
  d.L = m->n_layers; d.d = m->d_model; d.Hq = m->n_heads; d.Hkv = m->n_kv_heads;
  d.D = m->head_dim; d.F = m->d_ffn; d.V = m->vocab; d.mask = m->mask_id; d.dtype = m->dtype;
  d.esz = m->dtype == DLLM_F32 ? 4 : 2;
  d.B = s->batch; d.P = s->prompt_len; d.G = s->gen_len; d.K = s->block_len;
  d.S = d.P + d.G; d.Sp = (d.S + 63) / 64 * 64; d.mode = s->cache_mode;
  d.nblocks = d.G / d.K;
  d.tau = s->threshold; d.eps = m->norm_eps; d.theta = m->rope_theta; d.lscale = m->logit_scale;
  if ((double)d.B * d.S > 1e8 || (double)d.S > 1e6) return fail(DLLM_E_UNSUPPORTED, "sequence too long");
  if (d.dtype == DLLM_F32 && d.S > 12000)
    return fail(DLLM_E_UNSUPPORTED, "fp32 models support S <= 12000");
  // a no-cache step stages the block rows of x in the FFN activation buffer
  if (d.mode == DLLM_CACHE_NONE && (size_t)d.S * d.F * d.esz < (size_t)d.K * d.d * sizeof(float))
    return fail(DLLM_E_UNSUPPORTED, "no-cache mode needs S * d_ffn * esize >= 4 * block_len * d_model");
  return DLLM_OK;
}

// Rows per sequence recomputed by a step of block b.
int step_rows(const Dims& d, int b) {
  int s0 = d.P + b * d.K;
  return d.mode == DLLM_CACHE_PREFIX ? d.S - s0 : d.K;
}

struct Ws {
  size_t x, h, q, o, a, logits, rcos, rsin, gpart, gcnt, apart, acnt, cpm, cps, cpi,
      conf, argmax, nun, rem, rss, total;
  size_t gpart_floats, apart_floats;
  int gcnt_n, acnt_n;
};

void plan_gemms(const Dims& d, int M, bool lm, size_t* pf, int* cn) {
  const int Nqkv = (d.Hq + 2 * d.Hkv) * d.D;
  GemmPlan ps[5] = {gemm_plan(d.dtype, M, Nqkv, d.d, EPI_QKV),
                    gemm_plan(d.dtype, M, d.d, d.Hq * d.D, EPI_RESID),
                    gemm_plan(d.dtype, M, 2 * d.F, d.d, EPI_SWIGLU),
                    gemm_plan(d.dtype, M, d.d, d.F, EPI_RESID),
                    gemm_plan(d.dtype, d.B * d.K, d.V, d.d, EPI_F32)};
  for (int i = 0; i < (lm ? 5 : 4); ++i) {
    if (ps[i].part_floats > *pf) *pf = ps[i].part_floats;
    if (ps[i].counters > *cn) *cn = ps[i].counters;
  }
}

Ws plan_ws(const Dims& d) {
  Ws w{};
  const size_t Mmax = (size_t)d.B * d.S;
  size_t gpf = 0, apf = 0;
  int gcn = 0, acn = 0;
  plan_gemms(d, (int)Mmax, false, &gpf, &gcn);
  {  // the refresh's attention (all S rows; short sequences take the split-KV kernel)
    AttnPlan ap = attn_plan(d.dtype, d.B, d.Hq, d.Hkv, d.S, d.S, d.D);
    apf = ap.part_floats;
    acn = ap.counters;
  }
  for (int b = 0; b < d.nblocks; ++b) {
    int R = step_rows(d, b);
    plan_gemms(d, d.B * R, true, &gpf, &gcn);
    AttnPlan ap = attn_plan(d.dtype, d.B, d.Hq, d.Hkv, R, d.S, d.D);
    if (ap.part_floats > apf) apf = ap.part_floats;
    if (ap.counters > acn) acn = ap.counters;
    if (d.mode == DLLM_CACHE_DUAL) break;  // every block has the same row count
  }
  ConfPlan cp = conf_plan(d.B * d.K, d.V, d.B);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += up(bytes); return o; };
  w.x = take(Mmax * d.d * 4);
  w.h = take(Mmax * d.d * d.esz);
  w.q = take((size_t)d.B * d.Hq * d.S * d.D * d.esz);
  w.o = take(Mmax * d.Hq * d.D * d.esz);
  w.a = take(Mmax * d.F * d.esz);
  w.logits = take((size_t)d.B * d.K * d.V * 4);
  w.rcos = take((size_t)d.S * (d.D / 2) * 4);
  w.rsin = take((size_t)d.S * (d.D / 2) * 4);
  w.gpart = take(gpf * 4);
  w.apart = take(apf * 4);
  w.cpm = take(cp.part_elems * 4);
  w.cps = take(cp.part_elems * 4);
  w.cpi = take(cp.part_elems * 4);
  w.conf = take((size_t)d.B * d.K * 4);
  w.argmax = take((size_t)d.B * d.K * 4);
  w.nun = take((size_t)d.B * 4);
  w.rem = take((size_t)d.B * 4);
  // per-row segment sums of squares of a deferred-factor RMSNorm (rows <= kSkinnyRows)
  w.rss = take((size_t)kSkinnyRows * ((d.d + kFoldSeg - 1) / kFoldSeg) * 4);
  // counters last, contiguous, zeroed at prefill
  w.gcnt = take((size_t)gcn * 4);
  w.acnt = take((size_t)acn * 4);
  w.total = off;
  w.gpart_floats = gpf;
  w.apart_floats = apf;
  w.gcnt_n = gcn;
  w.acnt_n = acn;
  return w;
}

size_t cache_bytes(const Dims& d) {
  return (size_t)d.L * 2 * d.B * d.Hkv * d.Sp * d.D * d.esz;
}

dllm_status check_buffers(const Dims& d, const dllm_seq_desc* s, Ws* w) {
  if (!s->tokens) return fail(DLLM_E_NULL, "tokens is NULL");
  if (!s->kv_cache) return fail(DLLM_E_NULL, "kv_cache is NULL");
  if (!s->workspace) return fail(DLLM_E_NULL, "workspace is NULL");
  *w = plan_ws(d);
  if (s->kv_cache_bytes < cache_bytes(d))
    return fail(DLLM_E_WORKSPACE, "kv_cache_bytes %zu < %zu", s->kv_cache_bytes, cache_bytes(d));
  if (s->workspace_bytes < w->total)
    return fail(DLLM_E_WORKSPACE, "workspace_bytes %zu < %zu", s->workspace_bytes, w->total);
  return DLLM_OK;
}

// ------------------------------------------------------------------ execution
struct Pending {  // split-K partials of a residual GEMM not yet added into x
  int splits = 0;
  PartView view;
};

// The RMS factor of the last norm, left for the next GEMM's split-K reduction to apply.
struct RowScale {
  bool on = false;
  const float* rss = nullptr;
  int rseg = 0;
};

struct Ctx {
  const Dims& d;
  const dllm_model_desc* m;
  const dllm_seq_desc* s;
  Ws w;
  char* ws;
  hipStream_t st;
  mutable Pending pend;
  mutable RowScale rs;
  template <typename P> P* at(size_t off) const { return reinterpret_cast<P*>(ws + off); }
  void* cache_k(int l) const {
    return (char*)s->kv_cache + (size_t)l * 2 * d.B * d.Hkv * d.Sp * d.D * d.esz;
  }
  void* cache_vt(int l) const {
    return (char*)cache_k(l) + (size_t)d.B * d.Hkv * d.Sp * d.D * d.esz;
  }
};

// The split partials of a GEMM whose reduction the caller runs itself.
struct Deferred {
  bool on = false;
  PartView pv;
  EpiArgs e;
};

// One GEMM with its epilogue.  With `defer`, a weight-streaming GEMM (whose partials
// cover every output column) leaves its reduce_epilogue to the caller: the partials and
// the epilogue arguments (the deferred RMS factor attached) are returned in *defer.
dllm_status gemm(const Ctx& c, int cls, int epi, const void* X, int ldx, const void* W, int M,
                 int Nv, int K, const EpiArgs& e, Deferred* defer = nullptr) {
  GemmPlan p = gemm_plan(c.d.dtype, M, Nv, K, epi);
  if (p.part_floats > c.w.gpart_floats || p.counters > c.w.gcnt_n)
    return fail(DLLM_E_WORKSPACE, "internal: GEMM plan exceeds the workspace plan");
  if (c.pend.splits)
    return fail(DLLM_E_STATE, "internal: pending residual partials not consumed");
  EpiArgs er = e;
  if (c.rs.on) {  // the input rows still carry their RMS factor
    if (p.kind != GEMM_SKINNY || epi == EPI_RESID)
      return fail(DLLM_E_STATE, "internal: deferred RMS factor without a split-K reduction");
    er.rss = c.rs.rss;
    er.rseg = c.rs.rseg;
    er.rd = c.d.d;
    er.reps = c.d.eps;
    c.rs = RowScale{};
  }
  {
    ProfScope ps(cls, c.st);
    HIP_TRY(launch_gemm_only(c.d.dtype, epi, p, X, ldx, W, M, Nv, K, er, c.at<float>(c.w.gpart),
                             c.at<int>(c.w.gcnt), c.st));
  }
  if (p.reduce && defer && p.kind == GEMM_SKINNY) {  // partials cover every column
    defer->on = true;
    defer->pv = p.view(c.at<float>(c.w.gpart), M, Nv);
    defer->e = er;
  } else if (p.reduce) {
    ProfScope ps(DLLM_K_SPLIT_REDUCE, c.st);
    HIP_TRY(launch_reduce_epilogue(epi, p.view(c.at<float>(c.w.gpart), M, Nv), er, c.st));
  }
  if (p.deferred && epi == EPI_RESID) {
    c.pend.splits = p.splits;
    c.pend.view = p.view(c.at<float>(c.w.gpart), M, Nv);
  }
  return DLLM_OK;
}

// RMSNorm of `rows` rows of x into h (see launch_rmsnorm); adds pending residual partials.
// When the consumer is a skinny bf16 GEMM (rows <= kSkinnyRows) the per-row factor is
// deferred: h = x * g, spread over (row, 512-column segment) workgroups, and the GEMM's
// split-K reduction multiplies each row by 1 / rms (it distributes over the row's dot
// products), so no kernel needs a whole row on one CU.
dllm_status norm(const Ctx& c, int rows, int Rin, int Kout, const void* g) {
  ProfScope ps(DLLM_K_RMSNORM, c.st);
  PartView pv = c.pend.view;
  pv.splits = c.pend.splits;
  if (c.d.dtype == BF16 && rows <= kSkinnyRows) {
    HIP_TRY(launch_fold_scale(c.d.dtype, c.at<float>(c.w.x), rows, Rin, Kout, g, c.d.d,
                              c.at<void>(c.w.h), c.at<float>(c.w.rss), pv, c.st));
    c.rs.on = true;
    c.rs.rss = c.at<float>(c.w.rss);
    c.rs.rseg = (c.d.d + kFoldSeg - 1) / kFoldSeg;
  } else {
    HIP_TRY(launch_rmsnorm(c.d.dtype, c.at<float>(c.w.x), rows, Rin, Kout, g, c.d.eps, c.d.d,
                           c.at<void>(c.w.h), pv, c.st));
  }
  c.pend = Pending{};
  return DLLM_OK;
}

// Layer stack over R rows per sequence starting at absolute position r0, from layer l0
// (l0 > 0: x already holds the input of layer l0 in rows [0, B*R)).
dllm_status run_layers(const Ctx& c, int r0, int R, bool refresh, int l0 = 0) {
  const Dims& d = c.d;
  const int M = d.B * R;
  float* x = c.at<float>(c.w.x);
  void* h = c.at<void>(c.w.h);
  void* q = c.at<void>(c.w.q);
  void* o = c.at<void>(c.w.o);
  void* a = c.at<void>(c.w.a);
  if (l0 == 0) {
    ProfScope ps(DLLM_K_EMBED_NORM, c.st);
    HIP_TRY(launch_embed_norm(d.dtype, c.s->tokens, d.S, r0, R, d.B, c.m->embed,
                              c.m->attn_norm[0], d.eps, d.d, d.V, x, h, c.st));
  }
  AttnPlan ap = attn_plan(d.dtype, d.B, d.Hq, d.Hkv, R, d.S, d.D);
  if (ap.part_floats > c.w.apart_floats || ap.counters > c.w.acnt_n)
    return fail(DLLM_E_WORKSPACE, "internal: attention plan exceeds the workspace plan");
  const int Nqkv = (d.Hq + 2 * d.Hkv) * d.D;
  for (int l = l0; l < d.L; ++l) {
    if (l > 0) {
      dllm_status st = norm(c, M, R, R, c.m->attn_norm[l]);
      if (st) return st;
    }
    EpiArgs eq;
    eq.qo = q; eq.kc = c.cache_k(l); eq.vtc = c.cache_vt(l);
    eq.rcos = c.at<float>(c.w.rcos); eq.rsin = c.at<float>(c.w.rsin);
    eq.Hq = d.Hq; eq.Hkv = d.Hkv; eq.D = d.D; eq.R = R; eq.pos0 = r0; eq.Sp = d.Sp;
    dllm_status st = gemm(c, refresh ? DLLM_K_REF_QKV : DLLM_K_STEP_QKV, EPI_QKV, h, d.d,
                          c.m->w_qkv[l], M, Nqkv, d.d, eq);
    if (st) return st;
    if (refresh && l == d.L - 1) break;  // the last layer's attention and tail feed no K/V
    {
      ProfScope ps(refresh ? DLLM_K_REF_ATTN : DLLM_K_STEP_ATTN, c.st);
      HIP_TRY(launch_attention(d.dtype, ap, q, c.cache_k(l), c.cache_vt(l), o, d.B, d.Hq, d.Hkv,
                               R, d.S, d.Sp, d.D, c.at<float>(c.w.apart), c.at<int>(c.w.acnt),
                               c.st));
    }
    EpiArgs er;
    er.y = x; er.ldy = d.d;
    st = gemm(c, refresh ? DLLM_K_REF_O : DLLM_K_STEP_O, EPI_RESID, o, d.Hq * d.D, c.m->w_o[l], M,
              d.d, d.Hq * d.D, er);
    if (st) return st;
    st = norm(c, M, R, R, c.m->ffn_norm[l]);
    if (st) return st;
    EpiArgs eg;
    eg.y = a; eg.F = d.F;
    st = gemm(c, refresh ? DLLM_K_REF_GATE_UP : DLLM_K_STEP_GATE_UP, EPI_SWIGLU, h, d.d,
              c.m->w_gate_up[l], M, 2 * d.F, d.d, eg);
    if (st) return st;
    st = gemm(c, refresh ? DLLM_K_REF_DOWN : DLLM_K_STEP_DOWN, EPI_RESID, a, d.F, c.m->w_down[l], M,
              d.d, d.F, er);
    if (st) return st;
  }
  return DLLM_OK;
}

dllm_status do_refresh(const Ctx& c) {
  Range r("dllm refresh");
  dllm_status st = run_layers(c, 0, c.d.S, true);
  c.pend = Pending{};  // the last layer's tail is skipped: nothing is pending
  c.rs = RowScale{};
  return st;
}

dllm_status do_init(const Ctx& c) {
  const Dims& d = c.d;
  int ncnt = (int)((c.w.total - c.w.gcnt) / 4);
  HIP_TRY(launch_fill_i32(c.at<int>(c.w.gcnt), ncnt, 0, c.st));
  HIP_TRY(launch_rope_table(c.at<float>(c.w.rcos), c.at<float>(c.w.rsin), d.S, d.D, d.theta, c.st));
  return DLLM_OK;
}

// Final norm over the block rows (the first K of each sequence's R computed rows), LM
// head, confidence and threshold unmask.
dllm_status decode_tail(const Ctx& c, int b, int R, int* n_un, int* rem, float* logits,
                        float* conf, int* argmax) {
  const Dims& d = c.d;
  const int s0 = d.P + b * d.K;
  dllm_status st = norm(c, d.B * d.K, R, d.K, c.m->final_norm);
  if (st) return st;
  void* h = c.at<void>(c.w.h);
  float* lg = logits ? logits : c.at<float>(c.w.logits);
  EpiArgs el;
  el.y = lg; el.ldy = d.V; el.scale = d.lscale;
  ConfPlan cp = conf_plan(d.B * d.K, d.V, d.B);
  // A weight-streaming LM head leaves split partials: the confidence pass sums them
  // itself, so the fp32 logits go to memory only when the caller asked for them.
  Deferred df;
  st = gemm(c, DLLM_K_LM_HEAD, EPI_F32, h, d.d, c.m->lm_head, d.B * d.K, d.V, d.d, el,
            lm_conf_fusable(cp, d.V) ? &df : nullptr);
  if (st) return st;
  ProfScope ps(DLLM_K_CONF_UNMASK, c.st);
  float* cf = conf ? conf : c.at<float>(c.w.conf);
  int* am = argmax ? argmax : c.at<int>(c.w.argmax);
  if (df.on)
    HIP_TRY(launch_lm_conf_unmask(cp, df.pv, df.e, logits, d.B, d.K, d.V, d.mask, d.tau,
                                  c.s->tokens + s0, d.S, cf, am, n_un, rem, nullptr,
                                  c.at<float>(c.w.cpm), c.at<float>(c.w.cps), c.at<int>(c.w.cpi),
                                  c.st));
  else
    HIP_TRY(launch_conf_unmask(F32, cp, lg, d.B, d.K, d.V, d.mask, d.tau, c.s->tokens + s0, d.S,
                               cf, am, n_un, rem, nullptr, c.at<float>(c.w.cpm),
                               c.at<float>(c.w.cps), c.at<int>(c.w.cpi), c.st));
  return DLLM_OK;
}

dllm_status do_step(const Ctx& c, int b, int* n_un, int* rem, float* logits, float* conf,
                    int* argmax) {
  Range r("dllm step");
  const Dims& d = c.d;
  const int R = step_rows(d, b);
  dllm_status st = run_layers(c, d.P + b * d.K, R, false);
  if (st) return st;
  return decode_tail(c, b, R, n_un, rem, logits, conf, argmax);
}

// Staging room for the block rows of x: the FFN activation buffer, idle between layers.
bool refresh_step_fits(const Dims& d) {
  return (size_t)d.B * d.S * d.F * d.esz >= (size_t)d.B * d.K * d.d * sizeof(float);
}

// The block's first denoising step fused with its refresh (by property (a) the first
// step after a refresh equals the full forward): the full forward over all S rows
// writes every layer's K/V and leaves the last layer's input in x; the block rows of x
// move to the cached-step row layout, and only the last layer, over the block rows
// (attending to all S fresh keys), the final norm, LM head and unmask follow.  Saves
// the block-row recompute of layers 0 .. L-2 that a separate first step would do.
dllm_status do_refresh_step(const Ctx& c, int b, int* n_un, int* rem, float* logits,
                            float* conf, int* argmax) {
  Range r(b == 0 ? "dllm prefill+step" : "dllm refresh+step");
  const Dims& d = c.d;
  dllm_status st = (b == 0) ? do_init(c) : DLLM_OK;
  if (st) return st;
  st = do_refresh(c);
  if (st) return st;
  if (!refresh_step_fits(d)) return do_step(c, b, n_un, rem, logits, conf, argmax);
  const int s0 = d.P + b * d.K;
  const size_t row = (size_t)d.d * sizeof(float);
  float* x = c.at<float>(c.w.x);
  void* tmp = c.at<void>(c.w.a);
  HIP_TRY(hipMemcpy2DAsync(tmp, d.K * row, x + (size_t)s0 * d.d, (size_t)d.S * row, d.K * row,
                           d.B, hipMemcpyDeviceToDevice, c.st));
  HIP_TRY(hipMemcpyAsync(x, tmp, (size_t)d.B * d.K * row, hipMemcpyDeviceToDevice, c.st));
  st = run_layers(c, s0, d.K, false, d.L - 1);
  if (st) return st;
  return decode_tail(c, b, d.K, n_un, rem, logits, conf, argmax);
}

dllm_status setup(const dllm_model_desc* m, const dllm_seq_desc* s, Dims* d, Ws* w) {
  dllm_status st = dims_of(m, s, d);
  if (st) return st;
  return check_buffers(*d, s, w);
}

double now_ms() {
  return std::chrono::duration<double, std::milli>(
             std::chrono::steady_clock::now().time_since_epoch())
      .count();
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

size_t dllm_workspace_bytes(const dllm_model_desc* m, const dllm_seq_desc* s) {
  Dims d;
  if (dims_of(m, s, &d)) return 0;
  return plan_ws(d).total;
}

size_t dllm_kv_cache_bytes(const dllm_model_desc* m, const dllm_seq_desc* s) {
  Dims d;
  if (dims_of(m, s, &d)) return 0;
  return cache_bytes(d);
}

dllm_status dllm_prefill_cache(const dllm_model_desc* m, const dllm_seq_desc* s,
                               dllm_stream_t stream) {
  Dims d;
  Ws w;
  dllm_status st = setup(m, s, &d, &w);
  if (st) return st;
  Ctx c{d, m, s, w, (char*)s->workspace, (hipStream_t)stream};
  Range r("dllm prefill");
  st = do_init(c);
  if (st) return st;
  return do_refresh(c);
}

dllm_status dllm_refresh_cache(const dllm_model_desc* m, const dllm_seq_desc* s, int32_t block,
                               dllm_stream_t stream) {
  Dims d;
  Ws w;
  dllm_status st = setup(m, s, &d, &w);
  if (st) return st;
  if (block < 0 || block >= d.nblocks) return fail(DLLM_E_STATE, "block %d outside [0, %d)", block, d.nblocks);
  Ctx c{d, m, s, w, (char*)s->workspace, (hipStream_t)stream};
  return do_refresh(c);
}

dllm_status dllm_cache_staleness(const dllm_model_desc* m, const dllm_seq_desc* s, int32_t block,
                                 void* fresh_cache, size_t fresh_bytes, float* out,
                                 double* reuse, dllm_stream_t stream) {
  Dims d;
  Ws w;
  dllm_status st = setup(m, s, &d, &w);
  if (st) return st;
  if (block < 0 || block >= d.nblocks) return fail(DLLM_E_STATE, "block %d outside [0, %d)", block, d.nblocks);
  if (d.mode == DLLM_CACHE_NONE) return fail(DLLM_E_STATE, "no cache to compare in this mode");
  if (!fresh_cache || !out) return fail(DLLM_E_NULL, "fresh_cache/out is NULL");
  if (fresh_bytes < cache_bytes(d))
    return fail(DLLM_E_WORKSPACE, "fresh_bytes %zu < %zu", fresh_bytes, cache_bytes(d));
  // the per-(layer, K/V, sequence, head) partials go to the logits buffer, idle here
  const size_t part = (size_t)d.L * 2 * d.B * d.Hkv * 3 * sizeof(double);
  if (part > (size_t)d.B * d.K * d.V * 4)
    return fail(DLLM_E_UNSUPPORTED, "staleness partials exceed the logits buffer");
  // the exact K/V of the current tokens: a full forward into the fresh buffer
  dllm_seq_desc fs = *s;
  fs.kv_cache = fresh_cache;
  fs.kv_cache_bytes = fresh_bytes;
  const Ctx cf{d, m, &fs, w, (char*)s->workspace, (hipStream_t)stream};
  st = do_refresh(cf);
  if (st) return st;
  // the positions the next cached step of `block` takes from the cache: every one but
  // the block's (DualCache), those before the block (prefix)
  const int s0 = d.P + block * d.K;
  const int x1 = (d.mode == DLLM_CACHE_PREFIX) ? d.S : s0 + d.K;
  if (reuse) *reuse = (double)(d.S - (x1 - s0)) / d.S;
  HIP_TRY(launch_staleness(d.dtype, s->kv_cache, fresh_cache, d.L, d.B, d.Hkv, d.S, d.Sp, d.D,
                           s0, x1, cf.at<double>(w.logits), out, (hipStream_t)stream));
  return DLLM_OK;
}

dllm_status dllm_block_step(const dllm_model_desc* m, const dllm_seq_desc* s, int32_t block,
                            dllm_stream_t stream, int32_t* d_n_unmasked, int32_t* d_remaining,
                            float* d_logits, float* d_conf, int32_t* d_argmax) {
  Dims d;
  Ws w;
  dllm_status st = setup(m, s, &d, &w);
  if (st) return st;
  if (block < 0 || block >= d.nblocks) return fail(DLLM_E_STATE, "block %d outside [0, %d)", block, d.nblocks);
  if (!d_n_unmasked || !d_remaining) return fail(DLLM_E_NULL, "n_unmasked/remaining is NULL");
  Ctx c{d, m, s, w, (char*)s->workspace, (hipStream_t)stream};
  if (d.mode == DLLM_CACHE_NONE)
    return do_refresh_step(c, block, d_n_unmasked, d_remaining, d_logits, d_conf, d_argmax);
  return do_step(c, block, d_n_unmasked, d_remaining, d_logits, d_conf, d_argmax);
}

dllm_status dllm_refresh_step(const dllm_model_desc* m, const dllm_seq_desc* s, int32_t block,
                              dllm_stream_t stream, int32_t* d_n_unmasked, int32_t* d_remaining,
                              float* d_logits, float* d_conf, int32_t* d_argmax) {
  Dims d;
  Ws w;
  dllm_status st = setup(m, s, &d, &w);
  if (st) return st;
  if (block < 0 || block >= d.nblocks) return fail(DLLM_E_STATE, "block %d outside [0, %d)", block, d.nblocks);
  if (!d_n_unmasked || !d_remaining) return fail(DLLM_E_NULL, "n_unmasked/remaining is NULL");
  Ctx c{d, m, s, w, (char*)s->workspace, (hipStream_t)stream};
  return do_refresh_step(c, block, d_n_unmasked, d_remaining, d_logits, d_conf, d_argmax);
}

static dllm_status generate_impl(const dllm_model_desc* m, const dllm_seq_desc* s,
                                 dllm_stream_t stream, bool graphs, dllm_stats* out) {
  Dims d;
  Ws w;
  dllm_status st = setup(m, s, &d, &w);
  if (st) return st;
  if (graphs && g_prof.cls != DLLM_K_NONE)
    return fail(DLLM_E_UNSUPPORTED, "kernel-class timing is not available with graph replay");
  hipStream_t hs = (hipStream_t)stream;
  // The legacy null stream cannot be captured: graph replay then runs on a stream of its
  // own, after the null stream's pending work (the call is synchronous either way).
  hipStream_t own = nullptr;
  struct OwnStream {
    hipStream_t* s;
    ~OwnStream() { if (*s) { (void)hipStreamSynchronize(*s); (void)hipStreamDestroy(*s); } }
  } oguard{&own};
  if (graphs && hs == nullptr) {
    HIP_TRY(hipStreamSynchronize(nullptr));
    HIP_TRY(hipStreamCreateWithFlags(&own, hipStreamNonBlocking));
    hs = own;
  }
  Ctx c{d, m, s, w, (char*)s->workspace, hs};
  // Each step's outcome (mask tokens left per sequence) goes to one of two pinned host
  // slots, with an event behind the copy.  The host keeps the next step queued while it
  // waits for the previous outcome, so the device never waits for the host to launch a
  // step.  Every step decodes at least one token of each unfinished sequence, so a step
  // that follows an outcome of at most one token left per sequence finishes the block:
  // no further step is queued then.  With two or more left, the step after the one in
  // flight is queued on speculation; if the one in flight finishes the block, the
  // speculative step finds nothing masked and changes no token (its K/V writes are
  // overwritten by the next refresh), costing one step of device time.
  int32_t* host = nullptr;  // pinned: [2][B] remaining
  HIP_TRY(hipHostMalloc((void**)&host, sizeof(int32_t) * 2 * d.B, hipHostMallocDefault));
  struct Free { int32_t* p; ~Free() { if (p) (void)hipHostFree(p); } } guard{host};
  hipEvent_t ev[2] = {nullptr, nullptr};
  struct Ev { hipEvent_t* e; ~Ev() { for (int i = 0; i < 2; ++i) if (e[i]) (void)hipEventDestroy(e[i]); } } eguard{ev};
  for (int i = 0; i < 2; ++i) HIP_TRY(hipEventCreateWithFlags(&ev[i], hipEventDisableTiming));
  // Graph replay: a block's cached steps differ only in the tokens they read, so the
  // first one is captured (every kernel of the step, on this stream) and replayed for the
  // rest; the executable graphs live until the end of the call.
  std::vector<hipGraphExec_t> execs;
  struct Ex {
    std::vector<hipGraphExec_t>* v;
    hipStream_t s;
    ~Ex() {
      if (v->empty()) return;
      (void)hipStreamSynchronize(s);  // no replay may still be pending (error paths too)
      for (auto e : *v) (void)hipGraphExecDestroy(e);
    }
  } exguard{&execs, hs};
  const double t_start = now_ms();
  double ms_ref = 0, ms_step = 0;
  int steps = 0, refreshes = 0, wasted = 0;
  int64_t masked_seen = 0;  // masked block positions at the start of each step, summed
  for (int b = 0; b < d.nblocks; ++b) {
    int issued = 0;  // steps of this block enqueued (the first fused with the refresh)
    hipGraphExec_t exec = nullptr;
    auto issue = [&]() -> dllm_status {
      const bool full = issued == 0 || d.mode == DLLM_CACHE_NONE;
      dllm_status r = DLLM_OK;
      if (full) {
        r = do_refresh_step(c, b, c.at<int>(w.nun), c.at<int>(w.rem), nullptr, nullptr, nullptr);
      } else if (!graphs) {
        r = do_step(c, b, c.at<int>(w.nun), c.at<int>(w.rem), nullptr, nullptr, nullptr);
      } else {
        if (!exec) {
          HIP_TRY(hipStreamBeginCapture(hs, hipStreamCaptureModeThreadLocal));
          r = do_step(c, b, c.at<int>(w.nun), c.at<int>(w.rem), nullptr, nullptr, nullptr);
          hipGraph_t g = nullptr;
          const hipError_t e = hipStreamEndCapture(hs, &g);
          if (!r && e != hipSuccess) r = fail(DLLM_E_HIP, "stream capture: %s", hipGetErrorString(e));
          if (!r) {
            const hipError_t ei = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
            if (ei != hipSuccess) r = fail(DLLM_E_HIP, "graph instantiate: %s", hipGetErrorString(ei));
            else execs.push_back(exec);
          }
          if (g) (void)hipGraphDestroy(g);
        }
        if (!r) HIP_TRY(hipGraphLaunch(exec, hs));
      }
      if (r) return r;
      const int slot = issued & 1;
      HIP_TRY(hipMemcpyAsync(host + slot * d.B, c.at<int>(w.rem), d.B * sizeof(int32_t),
                             hipMemcpyDeviceToHost, hs));
      HIP_TRY(hipEventRecord(ev[slot], hs));
      ++issued;
      return DLLM_OK;
    };
    double t0 = now_ms();
    st = issue();
    if (st) return st;
    int confirmed = 0;  // steps whose outcome has been read
    int64_t masked_now = (int64_t)d.B * d.K;  // every block starts fully masked
    for (;;) {
      const int slot = confirmed & 1;
      HIP_TRY(hipEventSynchronize(ev[slot]));
      ++confirmed;
      masked_seen += masked_now;
      int left = 0;
      masked_now = 0;
      for (int i = 0; i < d.B; ++i) {
        left = std::max(left, (int)host[slot * d.B + i]);
        masked_now += host[slot * d.B + i];
      }
      if (confirmed == 1) {
        ms_ref += now_ms() - t0;
        t0 = now_ms();
      }
      if (left == 0) break;
      if (confirmed >= d.K) return fail(DLLM_E_STATE, "block %d did not finish in %d steps", b, d.K);
      if (issued == confirmed) {  // the next step is needed
        st = issue();
        if (st) return st;
      }
      if (left >= 2 && issued == confirmed + 1 && issued < d.K) {  // the one after, maybe
        st = issue();
        if (st) return st;
      }
    }
    ms_step += now_ms() - t0;
    const int n = confirmed;
    wasted += issued - confirmed;
    steps += n;
    ++refreshes;
    if (d.mode == DLLM_CACHE_NONE) refreshes += n - 1;  // every step was a full forward
    if (out && out->steps_per_block) out->steps_per_block[b] = n;
  }
  HIP_TRY(hipStreamSynchronize(hs));  // a speculative step may still be running
  if (out) {
    out->steps = steps;
    out->refreshes = refreshes;
    out->tokens = d.B * d.G;
    out->blocks = d.nblocks;
    out->ms_total = now_ms() - t_start;
    out->ms_refresh = ms_ref;
    out->ms_step = ms_step;
    out->speculative_steps = wasted;
    out->masked_at_step_start = masked_seen;
  }
  return DLLM_OK;
}

dllm_status dllm_generate(const dllm_model_desc* m, const dllm_seq_desc* s, dllm_stream_t stream,
                          dllm_stats* out) {
  return generate_impl(m, s, stream, false, out);
}

dllm_status dllm_generate_graphs(const dllm_model_desc* m, const dllm_seq_desc* s,
                                 dllm_stream_t stream, dllm_stats* out) {
  return generate_impl(m, s, stream, true, out);
}

// ---------------------------------------------------------------- kernel-level entries
// Workspace of the attention entry: the plan's counters and partials, the partials sized
// for every Hkv dividing Hq, since the workspace query does not take Hkv.
static size_t kw_attn(int B, int Hq, int Hkv, int R, int S, int D, int dtype, AttnPlan* p) {
  *p = attn_plan(dtype, B, Hq, Hkv, R, S, D);
  return up((size_t)p->counters * 4) + up(attn_part_floats_any_hkv(dtype, B, Hq, R, S, D) * 4);
}
static size_t kw_conf(int rows, int V, int B, ConfPlan* p) {
  *p = conf_plan(rows, V, B);
  return 3 * up(p->part_elems * 4);
}

size_t dllm_kernel_workspace_bytes(int32_t B, int32_t Hq, int32_t R, int32_t S, int32_t D,
                                   int32_t K, int32_t V) {
  AttnPlan ap;
  ConfPlan cp;
  if (B < 1) return 0;
  size_t a = (Hq > 0 && R > 0 && S > 0 && D > 0) ? kw_attn(B, Hq, Hq, R, S, D, DLLM_BF16, &ap) : 0;
  size_t c = (K > 0 && V > 0) ? kw_conf(B * K, V, B, &cp) : 0;
  return a > c ? a : c;
}

dllm_status dllm_kernel_block_attention(const void* q, const void* k, const void* vt, void* o,
                                        int32_t B, int32_t Hq, int32_t Hkv, int32_t R, int32_t S,
                                        int32_t Sp, int32_t D, int32_t dtype, void* ws,
                                        size_t ws_bytes, dllm_stream_t stream) {
  if (!q || !k || !vt || !o) return fail(DLLM_E_NULL, "q/k/vt/o is NULL");
  if (dtype != DLLM_F32 && dtype != DLLM_BF16) return fail(DLLM_E_ARG, "bad dtype");
  if (B < 1 || Hq < 1 || Hkv < 1 || R < 1 || S < 1 || D < 1 || Sp < S)
    return fail(DLLM_E_SHAPE, "sizes must be positive and Sp >= S");
  if (Hq % Hkv) return fail(DLLM_E_SHAPE, "Hq %% Hkv != 0");
  if (Sp % 32) return fail(DLLM_E_UNSUPPORTED, "Sp must be a multiple of 32 (32-key Vt blocks)");
  if (dtype == DLLM_BF16 && D != 128)
    return fail(DLLM_E_UNSUPPORTED, "bf16 attention needs D == 128");
  if (dtype == DLLM_F32 && (D > 128 || S > 12000))
    return fail(DLLM_E_UNSUPPORTED, "fp32 attention needs D <= 128 and S <= 12000");
  AttnPlan p;
  size_t need = kw_attn(B, Hq, Hkv, R, S, D, dtype, &p);
  if (need && (!ws || ws_bytes < need)) return fail(DLLM_E_WORKSPACE, "workspace %zu < %zu", ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  int* cnt = (int*)ws;
  float* part = need ? (float*)((char*)ws + up((size_t)p.counters * 4)) : nullptr;
  if (p.counters) HIP_TRY(launch_fill_i32(cnt, p.counters, 0, st));
  ProfScope ps(DLLM_K_STEP_ATTN, st);
  HIP_TRY(launch_attention(dtype, p, q, k, vt, o, B, Hq, Hkv, R, S, Sp, D, part, cnt, st));
  return DLLM_OK;
}

dllm_status dllm_kernel_confidence_unmask(const void* logits, int32_t logits_dtype, int32_t B,
                                          int32_t K, int32_t V, int32_t mask_id, float tau,
                                          int32_t* tokens_block, int32_t ld_tokens, float* conf,
                                          int32_t* argmax, int32_t* n_unmasked,
                                          int32_t* remaining, int32_t* unmasked_idx, void* ws,
                                          size_t ws_bytes, dllm_stream_t stream) {
  if (!logits || !tokens_block || !conf || !argmax || !n_unmasked || !remaining)
    return fail(DLLM_E_NULL, "a required pointer is NULL");
  if (logits_dtype != DLLM_F32 && logits_dtype != DLLM_BF16) return fail(DLLM_E_ARG, "bad dtype");
  if (B < 1 || K < 1 || V < 2 || ld_tokens < K) return fail(DLLM_E_SHAPE, "bad sizes");
  if (K > 64) return fail(DLLM_E_UNSUPPORTED, "K > 64");
  if (mask_id < 0 || mask_id >= V) return fail(DLLM_E_ARG, "mask_id outside [0, V)");
  if (std::isnan(tau)) return fail(DLLM_E_ARG, "tau is NaN");
  ConfPlan p;
  size_t need = kw_conf(B * K, V, B, &p);
  if (!ws || ws_bytes < need) return fail(DLLM_E_WORKSPACE, "workspace %zu < %zu", ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)ws;
  float* pm = (float*)base;
  float* ps_ = (float*)(base + up(p.part_elems * 4));
  int* pi = (int*)(base + 2 * up(p.part_elems * 4));
  ProfScope ps(DLLM_K_CONF_UNMASK, st);
  HIP_TRY(launch_conf_unmask(logits_dtype, p, logits, B, K, V, mask_id, tau, tokens_block,
                             ld_tokens, conf, argmax, n_unmasked, remaining, unmasked_idx, pm, ps_,
                             pi, st));
  return DLLM_OK;
}

// ---------------------------------------------------------------- no-allocation entry
// For callers that cannot allocate (code under graph capture, tight serving loops): the
// confidence pass's slice partials live in one file-scope device array per GPU instead
// of a caller workspace.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): its device address is looked up once per
// device with that device current and kept.
namespace {
constexpr size_t kScratchParts = 65536;  // (max, sum, argmax) slice triples: 768 KiB
static __device__ __align__(256) float scratch[3 * kScratchParts];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dllm_status scratch_for(hipStream_t st, char** out) {
  int cur = 0;
  HIP_TRY(hipGetDevice(&cur));
  int dev = cur;
  if (st != nullptr) HIP_TRY(hipStreamGetDevice(st, &dev));
  if (dev != cur)
    return fail(DLLM_E_ARG, "stream belongs to device %d, the current device is %d", dev, cur);
  if (dev < 0 || dev >= kMaxDevices) return fail(DLLM_E_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return fail(DLLM_E_HIP, "no device address for the scratch array");
    g_scratch_ptr[dev] = ptr;
  }
  *out = (char*)g_scratch_ptr[dev];
  return DLLM_OK;
}
}  // namespace

dllm_status dllm_kernel_confidence_unmask_noalloc(const void* logits, int32_t logits_dtype,
                                                  int32_t B, int32_t K, int32_t V,
                                                  int32_t mask_id, float tau,
                                                  int32_t* tokens_block, int32_t ld_tokens,
                                                  float* conf, int32_t* argmax,
                                                  int32_t* n_unmasked, int32_t* remaining,
                                                  int32_t* unmasked_idx, dllm_stream_t stream) {
  if (!logits || !tokens_block || !conf || !argmax || !n_unmasked || !remaining)
    return fail(DLLM_E_NULL, "a required pointer is NULL");
  if (logits_dtype != DLLM_F32 && logits_dtype != DLLM_BF16) return fail(DLLM_E_ARG, "bad dtype");
  if (B < 1 || K < 1 || V < 2 || ld_tokens < K) return fail(DLLM_E_SHAPE, "bad sizes");
  if (K > 64) return fail(DLLM_E_UNSUPPORTED, "K > 64");
  if (mask_id < 0 || mask_id >= V) return fail(DLLM_E_ARG, "mask_id outside [0, V)");
  if (std::isnan(tau)) return fail(DLLM_E_ARG, "tau is NaN");
  ConfPlan p = conf_plan(B * K, V, B);
  if (p.part_elems > kScratchParts)
    return fail(DLLM_E_UNSUPPORTED, "needs %zu slice partials, the static scratch holds %zu",
                p.part_elems, kScratchParts);
  hipStream_t st = (hipStream_t)stream;
  char* base = nullptr;
  dllm_status s = scratch_for(st, &base);
  if (s) return s;
  // every (row, slice) triple is written by pass 1 before pass 2 reads it: nothing to clear.
  // No kernel-class timing here: its events would be created on demand.
  float* pm = (float*)base;
  float* ps_ = pm + kScratchParts;
  int* pi = (int*)(pm + 2 * kScratchParts);
  HIP_TRY(launch_conf_unmask(logits_dtype, p, logits, B, K, V, mask_id, tau, tokens_block,
                             ld_tokens, conf, argmax, n_unmasked, remaining, unmasked_idx, pm, ps_,
                             pi, st));
  return DLLM_OK;
}

size_t dllm_linear_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t dtype) {
  if (M < 1 || N < 1 || K < 1) return 0;
  size_t best = 0;
  for (int epi : {EPI_STORE, EPI_F32, EPI_RESID}) {
    GemmPlan p = gemm_plan(dtype, M, N, K, epi);
    size_t b = up((size_t)p.counters * 4) + up(p.part_floats * 4) + kAlign;
    if (b > best) best = b;
  }
  return best;
}


dllm_status dllm_kernel_linear(const void* x, const void* w, void* y, int32_t M, int32_t N,
                               int32_t K, int32_t dtype, int32_t mode, float scale, void* ws,
                               size_t ws_bytes, dllm_stream_t stream) {
  if (!x || !w || !y) return fail(DLLM_E_NULL, "x/w/y is NULL");
  if (dtype != DLLM_F32 && dtype != DLLM_BF16) return fail(DLLM_E_ARG, "bad dtype");
  if (mode < 0 || mode > 2) return fail(DLLM_E_ARG, "bad mode");
  if (M < 1 || N < 1 || K < 1) return fail(DLLM_E_SHAPE, "sizes must be positive");
  if (dtype == DLLM_BF16 && (K % 256 || N % 8))
    return fail(DLLM_E_UNSUPPORTED, "bf16 needs K %% 256 == 0 and N %% 8 == 0");
  if (dtype == DLLM_F32 && K % 16) return fail(DLLM_E_UNSUPPORTED, "fp32 needs K %% 16 == 0");
  int epi = mode == 0 ? EPI_STORE : mode == 1 ? EPI_F32 : EPI_RESID;
  GemmPlan p = gemm_plan(dtype, M, N, K, epi);
  size_t need = up((size_t)p.counters * 4) + up(p.part_floats * 4);
  if (need && (!ws || ws_bytes < need)) return fail(DLLM_E_WORKSPACE, "workspace %zu < %zu", ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  int* cnt = (int*)ws;
  float* part = need ? (float*)((char*)ws + up((size_t)p.counters * 4)) : nullptr;
  if (p.counters) HIP_TRY(launch_fill_i32(cnt, p.counters, 0, st));
  EpiArgs e;
  e.y = y; e.ldy = N; e.scale = scale;
  HIP_TRY(launch_gemm(dtype, epi, p, x, K, w, M, N, K, e, part, cnt, st));
  if (p.deferred && epi == EPI_RESID) HIP_TRY(launch_fold_partials((float*)y, p.view(part, M, N), st));
  return DLLM_OK;
}

dllm_status dllm_synth_fill(void* dst, int64_t n, int32_t dtype, uint64_t seed,
                            uint32_t tensor_id, double stdv, int32_t mode, dllm_stream_t stream) {
  if (!dst && n > 0) return fail(DLLM_E_NULL, "dst is NULL");
  if (dtype != DLLM_F32 && dtype != DLLM_BF16) return fail(DLLM_E_ARG, "bad dtype");
  if (mode < 0 || mode > 2) return fail(DLLM_E_ARG, "bad mode");
  if (n < 0) return fail(DLLM_E_SHAPE, "n < 0");
  HIP_TRY(launch_synth_fill(dst, n, dtype, seed, tensor_id, stdv, mode, (hipStream_t)stream));
  return DLLM_OK;
}

const char* dllm_status_string(dllm_status st) {
  switch (st) {
    case DLLM_OK: return "ok";
    case DLLM_E_NULL: return "null pointer";
    case DLLM_E_SHAPE: return "inconsistent shape";
    case DLLM_E_UNSUPPORTED: return "unsupported configuration";
    case DLLM_E_WORKSPACE: return "buffer too small";
    case DLLM_E_HIP: return "HIP runtime error";
    case DLLM_E_STATE: return "bad block index or state";
    case DLLM_E_ARG: return "bad argument";
  }
  return "unknown status";
}

const char* dllm_last_error(void) { return g_err.c_str(); }

dllm_status dllm_profile_select_every(int32_t kernel_class, int32_t every) {
  if (kernel_class < DLLM_K_NONE || kernel_class >= DLLM_K_COUNT)
    return fail(DLLM_E_ARG, "bad kernel class %d", kernel_class);
  if (every < 1) return fail(DLLM_E_ARG, "bad sampling stride %d", every);
  g_prof.cls = kernel_class;
  g_prof.every = every;
  g_prof.seen = 0;
  g_prof.used = 0;
  return DLLM_OK;
}

dllm_status dllm_profile_select(int32_t kernel_class) {
  return dllm_profile_select_every(kernel_class, 1);
}

dllm_status dllm_profile_read(int32_t* launches, double* total_ms) {
  double tot = 0;
  for (size_t i = 0; i + 1 < g_prof.used; i += 2) {
    HIP_TRY(hipEventSynchronize(g_prof.ev[i + 1]));
    float ms = 0;
    HIP_TRY(hipEventElapsedTime(&ms, g_prof.ev[i], g_prof.ev[i + 1]));
    tot += ms;
  }
  if (launches) *launches = (int32_t)(g_prof.used / 2);
  if (total_ms) *total_ms = tot;
  g_prof.used = 0;
  return DLLM_OK;
}

}  // extern "C"
