// C ABI of the hybrid attention library: argument validation, workspace
// planning, host-side frame tables and dispatch to the kernel sequences.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/hyb_attn.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

hyb_status fail(hyb_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

hyb_status check_layout(const hyb_layout* L, bool tables_only) {
  if (!L) return fail(HYB_ERR_INVALID_ARGUMENT, "layout is NULL");
  if (L->frames < 1) return fail(HYB_ERR_INVALID_ARGUMENT, "frames must be >= 1 (got %d)", L->frames);
  if (L->chunk_frames < 1) return fail(HYB_ERR_INVALID_ARGUMENT, "chunk_frames must be >= 1");
  if (L->chunk_radius < 0) return fail(HYB_ERR_INVALID_ARGUMENT, "chunk_radius must be >= 0");
  if ((L->anchor_first != 0 && L->anchor_first != 1) || (L->anchor_last != 0 && L->anchor_last != 1))
    return fail(HYB_ERR_INVALID_ARGUMENT, "anchor flags must be 0 or 1");
  if (tables_only) return HYB_OK;
  if (L->batch < 1 || L->tokens_per_frame < 1 || L->heads < 1)
    return fail(HYB_ERR_INVALID_ARGUMENT, "batch, tokens_per_frame and heads must be >= 1");
  if (L->text_tokens < 0) return fail(HYB_ERR_INVALID_ARGUMENT, "text_tokens must be >= 0");
  if (L->head_dim != 32 && L->head_dim != 64 && L->head_dim != 128)
    return fail(HYB_ERR_UNSUPPORTED, "head_dim %d not supported (32, 64, 128)", L->head_dim);
  const long long N = (long long)L->frames * L->tokens_per_frame;
  if (N > (1LL << 30) || (long long)L->batch * N * L->heads > (1LL << 31) || L->text_tokens > (1 << 30))
    return fail(HYB_ERR_UNSUPPORTED, "problem too large for 32-bit work indexing");
  if ((long long)L->heads * L->head_dim > 65536) return fail(HYB_ERR_UNSUPPORTED, "hidden size too large");
  return HYB_OK;
}

hyb_status check_dtypes(const hyb_layout* L, hyb_dtype act, hyb_dtype soft) {
  if (act != HYB_F32 && act != HYB_BF16) return fail(HYB_ERR_UNSUPPORTED, "activation dtype must be F32 or BF16");
  if (soft != act && !((soft == HYB_FP8_E4M3 || soft == HYB_FP8_MX) && act == HYB_BF16))
    return fail(HYB_ERR_UNSUPPORTED,
                "softmax dtype must equal the activation dtype, or be FP8_E4M3 / FP8_MX with BF16");
  if (act == HYB_BF16 && L->head_dim == 32) return fail(HYB_ERR_UNSUPPORTED, "bf16 path needs head_dim 64 or 128");
  if (soft == HYB_FP8_MX && (L->heads * L->head_dim) % 256 != 0)
    return fail(HYB_ERR_UNSUPPORTED, "FP8_MX needs a hidden size that is a multiple of 256 (got %d)",
                L->heads * L->head_dim);
  return HYB_OK;
}

hyb::Dims make_dims(const hyb_layout* L) {
  hyb::Dims d;
  d.B = L->batch;
  d.T = L->frames;
  d.n = L->tokens_per_frame;
  d.L = L->text_tokens;
  d.H = L->heads;
  d.D = L->head_dim;
  d.N = (long long)d.T * d.n;
  d.hid = d.H * d.D;
  d.g.T = d.T;
  d.g.C = L->chunk_frames;
  d.g.R = L->chunk_radius;
  d.g.af = L->anchor_first;
  d.g.al = L->anchor_last;
  return d;
}

// State-build split.  Each split of a frame (and of the text) is one
// workgroup; two run per CU, 512 on the chip at once.  The time is about
// (rounds of 512 workgroups) x (bytes one workgroup moves: its keys and
// values read, its partial state written), so take the split that minimises
// that product (the smaller split on a tie: fewer partials for the scan).
void state_split(const hyb::Dims& d, int* split, int* ts, int* tsplit) {
  const long long tiles = (d.n + 63) / 64;
  const long long bht = (long long)d.B * d.H * d.T, bh = (long long)d.B * d.H;
  const long long part_bytes = ((long long)d.D * d.D + d.D) * 4;
  long long best_cost = -1;
  int best = 1;
  for (int sp = 1; sp <= 16 && sp <= tiles; ++sp) {
    const long long tss = 64 * ((tiles + sp - 1) / sp);
    const long long tsp = d.L > 0 ? (d.L + tss - 1) / tss : 0;
    const long long rounds = (bht * sp + bh * tsp + 511) / 512;
    const long long cost = rounds * (tss * 4 * d.D + part_bytes);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = sp;
    }
  }
  *split = best;
  *ts = (int)(64 * ((tiles + best - 1) / best));
  *tsplit = d.L > 0 ? (int)((d.L + *ts - 1) / *ts) : 0;
}

enum {
  W_OS, W_OL, W_SS, W_RINV, W_PART, W_PRE, W_CHI, W_CLO, W_CZ, W_AP, W_WG, W_WO,
  W_Q8, W_K8, W_V8, W_TK8, W_TV8, W_SC, W_AM, W_STATES, W_COMB, W_X8, W_XS, W_AS, W_WGS, W_WOS, W_COUNT
};

// Token rows of the MX exponent arrays: whole 256-token GEMM tiles.
size_t mx_rows(const hyb::Dims& d) { return ((size_t)d.B * d.N + 255) / 256 * 256; }

struct Plan {
  size_t off[W_COUNT];
  size_t total;
};

Plan make_plan(const hyb::Dims& d, hyb_dtype act, hyb_dtype soft) {
  Plan p;
  size_t sz[W_COUNT] = {0};
  const size_t BN = (size_t)d.B * d.N, hid = d.hid, D = d.D, BH = (size_t)d.B * d.H;
  // branch outputs: fp32 on the float32 path, fp16 on the bf16 path
  sz[W_OS] = BN * hid * (act == HYB_F32 ? 4 : 2);
  sz[W_OL] = BN * hid * (act == HYB_F32 ? 4 : 2);
  sz[W_SS] = BN * d.H * 4;
  if (act == HYB_F32) {
    sz[W_STATES] = BH * (d.T + 1) * D * (D + 1) * 4;
    sz[W_COMB] = BH * d.T * D * (D + 1) * 4;
    sz[W_AP] = BN * 2 * hid * 4;
  } else {
    int split, ts, tsplit;
    state_split(d, &split, &ts, &tsplit);
    const size_t slots = (size_t)d.T * split + tsplit;
    sz[W_PART] = BH * slots * (D * D + D) * 4;
    sz[W_PRE] = BH * d.T * (D * D + D) * 4;
    sz[W_CHI] = BH * d.T * D * D * 2;
    sz[W_CLO] = BH * d.T * D * D * 2;
    sz[W_CZ] = BH * d.T * D * 4;
    sz[W_RINV] = BN * 4;
    sz[W_AP] = BN * 2 * hid * 2;
    sz[W_WG] = 2 * hid * hid * 2;
    sz[W_WO] = 2 * hid * hid * 2;
    if (soft == HYB_FP8_MX) {  // e4m3 GEMM operands (codes reuse W_WG, W_WO, W_AP)
      const size_t mp = mx_rows(d);
      sz[W_X8] = BN * hid;
      sz[W_XS] = hid / 32 * mp;
      sz[W_AS] = 2 * hid / 32 * mp;
      sz[W_WGS] = hid / 32 * 2 * hid;
      sz[W_WOS] = 2 * hid / 32 * hid;
    }
    if (soft == HYB_FP8_E4M3 || soft == HYB_FP8_MX) {
      const size_t vt = (size_t)d.T * ((d.n + 63) / 64) * 64;  // per (b,h) padded video keys
      const size_t lt = (size_t)((d.L + 63) / 64) * 64;
      sz[W_Q8] = BN * hid;
      sz[W_K8] = BN * hid;
      sz[W_V8] = BH * vt * D;
      sz[W_TK8] = (size_t)d.B * d.L * hid;
      sz[W_TV8] = BH * lt * D;
      sz[W_SC] = 5 * BH * 4;
      sz[W_AM] = 5 * BH * 4;
    }
  }
  size_t o = 0;
  for (int i = 0; i < W_COUNT; ++i) {
    p.off[i] = o;
    o = align_up(o + sz[i], 256);
  }
  p.total = o;
  return p;
}

hyb_status check_tensor(const char* name, const hyb_tensor& t, size_t es, bool required) {
  if (!t.ptr) return required ? fail(HYB_ERR_INVALID_ARGUMENT, "%s.ptr is NULL", name) : HYB_OK;
  if (!aligned(t.ptr, 16)) return fail(HYB_ERR_INVALID_ARGUMENT, "%s.ptr is not 16-byte aligned", name);
  const int64_t q = (int64_t)(16 / es);
  if (t.stride_b < 0 || t.stride_tok < 0 || t.stride_head < 0)
    return fail(HYB_ERR_INVALID_ARGUMENT, "%s has a negative stride", name);
  if (t.stride_b % q || t.stride_tok % q || t.stride_head % q)
    return fail(HYB_ERR_INVALID_ARGUMENT, "%s strides must be multiples of %lld elements", name, (long long)q);
  if (t.stride_tok * (int64_t)es >= (1 << 18))
    return fail(HYB_ERR_UNSUPPORTED, "%s token stride too large (tile loads use 24-bit offsets)", name);
  return HYB_OK;
}

// Byte extent [lo, hi) of a strided tensor.
void extent(const hyb_tensor& t, long long B, long long T, long long H, long long D, size_t es, uintptr_t* lo,
            uintptr_t* hi) {
  *lo = (uintptr_t)t.ptr;
  *hi = *lo + (size_t)(((B - 1) * t.stride_b + (T - 1) * t.stride_tok + (H - 1) * t.stride_head + D) * es);
}

hyb::Tensor4 t4(const hyb_tensor& t) {
  hyb::Tensor4 r;
  r.p = t.ptr;
  r.sb = t.stride_b;
  r.st = t.stride_tok;
  r.sh = t.stride_head;
  return r;
}

}  // namespace

extern "C" {

const char* hyb_status_string(hyb_status s) {
  switch (s) {
    case HYB_OK: return "ok";
    case HYB_ERR_INVALID_ARGUMENT: return "invalid argument";
    case HYB_ERR_UNSUPPORTED: return "unsupported";
    case HYB_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case HYB_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* hyb_last_error(void) { return g_err; }

hyb_status hyb_layout_tables(const hyb_layout* layout, int32_t* soft_frames, int32_t* soft_count, int32_t* fwd,
                             int32_t* bwd) {
  g_err[0] = 0;
  hyb_status st = check_layout(layout, true);
  if (st != HYB_OK) return st;
  if (!soft_frames || !soft_count || !fwd || !bwd) return fail(HYB_ERR_INVALID_ARGUMENT, "table pointer is NULL");
  hyb::FrameGeom g{layout->frames, layout->chunk_frames, layout->chunk_radius, layout->anchor_first,
                   layout->anchor_last};
  const int T = g.T;
  for (int f = 0; f < T; ++f) {
    const hyb::SoftRanges sr = hyb::soft_ranges(g, f);
    int c = 0;
    for (int r = 0; r < sr.n; ++r)
      for (int x = sr.lo[r]; x < sr.hi[r]; ++x) soft_frames[(size_t)f * T + c++] = x;
    soft_count[f] = c;
    for (int i = c; i < T; ++i) soft_frames[(size_t)f * T + i] = -1;
    hyb::linear_ranges(g, f, &fwd[2 * f], &fwd[2 * f + 1], &bwd[2 * f], &bwd[2 * f + 1]);
  }
  return HYB_OK;
}

hyb_status hyb_workspace_size(const hyb_layout* layout, hyb_dtype act, hyb_dtype soft, size_t* bytes) {
  g_err[0] = 0;
  hyb_status st = check_layout(layout, false);
  if (st != HYB_OK) return st;
  st = check_dtypes(layout, act, soft);
  if (st != HYB_OK) return st;
  if (!bytes) return fail(HYB_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = make_plan(make_dims(layout), act, soft).total;
  return HYB_OK;
}

}  // extern "C"

namespace {

// The layer.  after_projection: called by hyb_block_forward, whose projection
// already ran (its stage events are recorded) and, with fp8, already wrote the
// absmax of q, k, v into the workspace.
// Forward values a training forward keeps for its backward (pointers into
// the caller's saved buffer); see hyb_attn_forward_train.
struct SavedPtrs {
  uint16_t *os, *ol, *ap, *gates16;
  float *rinv, *lse, *comb_z;
  hyb::bf16_t *comb_hi, *comb_lo;
};

hyb_status attn_forward_impl(const hyb_layout* layout, hyb_dtype act, hyb_dtype soft, const void* x, hyb_tensor q,
                             hyb_tensor k, hyb_tensor v, hyb_tensor text_k, hyb_tensor text_v,
                             const void* w_gate_soft, const void* w_gate_lin, const void* w_out_soft,
                             const void* w_out_lin, const void* rms_weight, float softmax_scale, float eps, void* y,
                             void* workspace, size_t workspace_bytes, void* stream, const hyb_debug* dbg,
                             bool after_projection, const SavedPtrs* keep = nullptr) {
  hyb_status st = check_layout(layout, false);
  if (st != HYB_OK) return st;
  st = check_dtypes(layout, act, soft);
  if (st != HYB_OK) return st;
  const size_t es = act == HYB_F32 ? 4 : 2;
  const hyb::Dims d = make_dims(layout);
  const bool has_text = d.L > 0;
  if ((st = check_tensor("q", q, es, true)) != HYB_OK) return st;
  if ((st = check_tensor("k", k, es, true)) != HYB_OK) return st;
  if ((st = check_tensor("v", v, es, true)) != HYB_OK) return st;
  if ((st = check_tensor("text_k", text_k, es, has_text)) != HYB_OK) return st;
  if ((st = check_tensor("text_v", text_v, es, has_text)) != HYB_OK) return st;
  const void* ptrs[] = {x, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin, rms_weight, y, workspace};
  const char* names[] = {"x", "w_gate_soft", "w_gate_lin", "w_out_soft", "w_out_lin", "rms_weight", "y", "workspace"};
  for (int i = 0; i < 8; ++i) {
    if (!ptrs[i]) return fail(HYB_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (!aligned(ptrs[i], i == 7 ? 256 : 16))
      return fail(HYB_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", names[i], i == 7 ? 256 : 16);
  }
  if (!(eps > 0.f) || !isfinite(eps)) return fail(HYB_ERR_INVALID_ARGUMENT, "eps must be finite and > 0");
  if (!(softmax_scale >= 0.f) || !isfinite(softmax_scale))
    return fail(HYB_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
  if (dbg) {
    const void* dp[] = {dbg->o_soft, dbg->o_lin, dbg->delta_f32, dbg->gates, dbg->scales};
    for (int i = 0; i < 5; ++i)
      if (dp[i] && !aligned(dp[i], 16)) return fail(HYB_ERR_INVALID_ARGUMENT, "debug buffer %d not 16-byte aligned", i);
  }
  {  // y must not overlap q, k, v
    const uintptr_t ylo = (uintptr_t)y, yhi = ylo + (size_t)d.B * d.N * d.hid * es;
    const hyb_tensor* ts[] = {&q, &k, &v};
    for (int i = 0; i < 3; ++i) {
      uintptr_t lo, hi;
      extent(*ts[i], d.B, d.N, d.H, d.D, es, &lo, &hi);
      if (ylo < hi && lo < yhi) return fail(HYB_ERR_INVALID_ARGUMENT, "y overlaps q, k or v");
    }
  }
  const Plan plan = make_plan(d, act, soft);
  if (workspace_bytes < plan.total)
    return fail(HYB_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, plan.total);

  char* ws = (char*)workspace;
  const float tau = softmax_scale > 0.f ? softmax_scale : 1.f / sqrtf((float)d.D);
  const float sl2 = tau * 1.4426950408889634f;
  hipStream_t s = (hipStream_t)stream;
  hipError_t he = hipSuccess;
  if (dbg && dbg->stage_events && !after_projection) {  // no projection stage here: empty interval
    hipEvent_t* ev = (hipEvent_t*)dbg->stage_events;
    he = hipEventRecord(ev[2 * HYB_STAGE_QKV], s);
    if (he == hipSuccess) he = hipEventRecord(ev[2 * HYB_STAGE_QKV + 1], s);
    if (he != hipSuccess) return fail(HYB_ERR_HIP, "HIP error: %s", hipGetErrorString(he));
  }
  if (act == HYB_F32) {
    hyb::F32Args a;
    a.q = t4(q); a.k = t4(k); a.v = t4(v);
    a.tk = t4(text_k); a.tv = t4(text_v);
    a.x = (const float*)x;
    a.wgs = (const float*)w_gate_soft; a.wgl = (const float*)w_gate_lin;
    a.wos = (const float*)w_out_soft; a.wol = (const float*)w_out_lin;
    a.rmsw = (const float*)rms_weight;
    a.scale_log2 = sl2;
    a.eps = eps;
    a.os = (float*)(ws + plan.off[W_OS]);
    a.ol = (float*)(ws + plan.off[W_OL]);
    a.ss = (float*)(ws + plan.off[W_SS]);
    a.states = (float*)(ws + plan.off[W_STATES]);
    a.comb = (float*)(ws + plan.off[W_COMB]);
    a.ap = (float*)(ws + plan.off[W_AP]);
    a.y = (float*)y;
    a.gates_dbg = dbg ? (float*)dbg->gates : nullptr;
    a.delta_dbg = dbg ? (float*)dbg->delta_f32 : nullptr;
    he = hyb::run_f32(d, a, s);
  } else {
    hyb::Bf16Args a;
    memset(&a, 0, sizeof(a));
    a.q = t4(q); a.k = t4(k); a.v = t4(v);
    a.tk = t4(text_k); a.tv = t4(text_v);
    a.x = (const hyb::bf16_t*)x;
    a.wgs = (const hyb::bf16_t*)w_gate_soft; a.wgl = (const hyb::bf16_t*)w_gate_lin;
    a.wos = (const hyb::bf16_t*)w_out_soft; a.wol = (const hyb::bf16_t*)w_out_lin;
    a.rmsw = (const hyb::bf16_t*)rms_weight;
    a.scale_log2 = sl2;
    a.eps = eps;
    a.fp8 = soft == HYB_FP8_E4M3 || soft == HYB_FP8_MX;
    a.qkv_absmax_ready = a.fp8 && after_projection;
    a.mx = soft == HYB_FP8_MX;
    a.mx_x_ready = a.mx && after_projection;
    a.mpad = (long long)mx_rows(d);
    a.x8 = (uint8_t*)(ws + plan.off[W_X8]);
    a.xs = (uint8_t*)(ws + plan.off[W_XS]);
    a.aps = (uint8_t*)(ws + plan.off[W_AS]);
    a.wgs8 = (uint8_t*)(ws + plan.off[W_WGS]);
    a.wos8 = (uint8_t*)(ws + plan.off[W_WOS]);
    a.os = (uint16_t*)(ws + plan.off[W_OS]);
    a.ol = (uint16_t*)(ws + plan.off[W_OL]);
    a.ss = (float*)(ws + plan.off[W_SS]);
    a.rinv = (float*)(ws + plan.off[W_RINV]);
    a.part = (float*)(ws + plan.off[W_PART]);
    a.pre = (float*)(ws + plan.off[W_PRE]);
    a.comb_hi = (hyb::bf16_t*)(ws + plan.off[W_CHI]);
    a.comb_lo = (hyb::bf16_t*)(ws + plan.off[W_CLO]);
    a.comb_z = (float*)(ws + plan.off[W_CZ]);
    a.ap = (uint16_t*)(ws + plan.off[W_AP]);
    a.wg_t = (hyb::bf16_t*)(ws + plan.off[W_WG]);
    a.wo_t = (uint16_t*)(ws + plan.off[W_WO]);
    a.q8 = (uint8_t*)(ws + plan.off[W_Q8]);
    a.k8 = (uint8_t*)(ws + plan.off[W_K8]);
    a.v8t = (uint8_t*)(ws + plan.off[W_V8]);
    a.tk8 = (uint8_t*)(ws + plan.off[W_TK8]);
    a.tv8t = (uint8_t*)(ws + plan.off[W_TV8]);
    a.scales = (float*)(ws + plan.off[W_SC]);
    a.absmax = (uint32_t*)(ws + plan.off[W_AM]);
    a.y = (hyb::bf16_t*)y;
    a.gates_dbg = dbg ? (float*)dbg->gates : nullptr;
    a.delta_dbg = dbg ? (float*)dbg->delta_f32 : nullptr;
    a.ev = dbg ? (hipEvent_t*)dbg->stage_events : nullptr;
    if (keep) {  // training forward: the backward's inputs go to the saved buffer
      a.os = keep->os; a.ol = keep->ol; a.ap = keep->ap; a.gates16 = keep->gates16;
      a.rinv = keep->rinv; a.lse = keep->lse;
      a.comb_hi = keep->comb_hi; a.comb_lo = keep->comb_lo; a.comb_z = keep->comb_z;
    }
    int split, ts, tsplit;
    state_split(d, &split, &ts, &tsplit);
    a.state_split = split;
    a.text_split = tsplit;
    a.state_slots = d.T * split + tsplit;
    he = hyb::run_bf16(d, a, s);
    if (he == hipSuccess && dbg && dbg->scales && a.fp8)
      he = hipMemcpyAsync(dbg->scales, a.scales, 5 * (size_t)d.B * d.H * 4, hipMemcpyDeviceToDevice, s);
    const long long nel = (long long)d.B * d.N * d.hid;
    if (he == hipSuccess && dbg && dbg->o_soft) he = hyb::launch_f16_to_f32(a.os, (float*)dbg->o_soft, nel, s);
    if (he == hipSuccess && dbg && dbg->o_lin) he = hyb::launch_f16_to_f32(a.ol, (float*)dbg->o_lin, nel, s);
  }
  if (act == HYB_F32) {
    const size_t bytes = (size_t)d.B * d.N * d.hid * 4;
    if (he == hipSuccess && dbg && dbg->o_soft)
      he = hipMemcpyAsync(dbg->o_soft, ws + plan.off[W_OS], bytes, hipMemcpyDeviceToDevice, s);
    if (he == hipSuccess && dbg && dbg->o_lin)
      he = hipMemcpyAsync(dbg->o_lin, ws + plan.off[W_OL], bytes, hipMemcpyDeviceToDevice, s);
  }
  if (he == hipSuccess && dbg && dbg->stage_events) {  // no feed-forward here: empty interval
    hipEvent_t* ev = (hipEvent_t*)dbg->stage_events;
    he = hipEventRecord(ev[2 * HYB_STAGE_FFN], s);
    if (he == hipSuccess) he = hipEventRecord(ev[2 * HYB_STAGE_FFN + 1], s);
  }
  if (he != hipSuccess) return fail(HYB_ERR_HIP, "HIP error: %s", hipGetErrorString(he));
  return HYB_OK;
}

// Workspace of the projection: [W_q | W_k | W_v] transposed, bf16.
size_t qkv_weight_bytes(const hyb::Dims& d) { return align_up((size_t)3 * d.hid * d.hid * 2, 256); }

hyb_status check_projection(const hyb_layout* layout) {
  hyb_status st = check_layout(layout, false);
  if (st != HYB_OK) return st;
  if (layout->head_dim != 64 && layout->head_dim != 128)
    return fail(HYB_ERR_UNSUPPORTED, "the projection needs head_dim 64 or 128");
  return HYB_OK;
}

// q, k, v = x [W_q | W_k | W_v] into contiguous [B*N][hid] bf16 buffers.
hipError_t run_projection(const hyb::Dims& d, const void* x, const void* w_q, const void* w_k, const void* w_v,
                          char* wt, void* q, void* k, void* v, uint32_t* absmax, hipStream_t s) {
  hipError_t e = hyb::launch_qkv_weights((const hyb::bf16_t*)w_q, (const hyb::bf16_t*)w_k,
                                         (const hyb::bf16_t*)w_v, d.hid, (hyb::bf16_t*)wt, s);
  if (e != hipSuccess) return e;
  return hyb::launch_qkv_gemm(d, (const hyb::bf16_t*)x, (const hyb::bf16_t*)wt, (hyb::bf16_t*)q,
                              (hyb::bf16_t*)k, (hyb::bf16_t*)v, absmax, s);
}

}  // namespace

extern "C" {

hyb_status hyb_attn_forward(const hyb_layout* layout, hyb_dtype act, hyb_dtype soft, const void* x, hyb_tensor q,
                            hyb_tensor k, hyb_tensor v, hyb_tensor text_k, hyb_tensor text_v,
                            const void* w_gate_soft, const void* w_gate_lin, const void* w_out_soft,
                            const void* w_out_lin, const void* rms_weight, float softmax_scale, float eps, void* y,
                            void* workspace, size_t workspace_bytes, void* stream, const hyb_debug* dbg) {
  g_err[0] = 0;
  return attn_forward_impl(layout, act, soft, x, q, k, v, text_k, text_v, w_gate_soft, w_gate_lin, w_out_soft,
                           w_out_lin, rms_weight, softmax_scale, eps, y, workspace, workspace_bytes, stream, dbg,
                           false);
}

}  // extern "C"

// Scratch of hyb_attn_forward_noalloc.  Each GPU the library runs on holds
// its own copy from the first use until the process ends.  In host code the
// name is only a handle for hipGetSymbolAddress: kernels and copies get the
// device address that call returns, kept per device below.
static __device__ __align__(256) unsigned char scratch[HYB_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the calling thread's current
// device, looked up once per device.
hyb_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HYB_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(HYB_ERR_UNSUPPORTED, "device index %d is beyond the %d devices the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(HYB_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HYB_OK;
}

}  // namespace

extern "C" {

hyb_status hyb_attn_forward_noalloc(const hyb_layout* layout, hyb_dtype act, hyb_dtype soft, const void* x,
                                    hyb_tensor q, hyb_tensor k, hyb_tensor v, hyb_tensor text_k, hyb_tensor text_v,
                                    const void* w_gate_soft, const void* w_gate_lin, const void* w_out_soft,
                                    const void* w_out_lin, const void* rms_weight, float softmax_scale, float eps,
                                    void* y, void* stream, const hyb_debug* dbg) {
  g_err[0] = 0;
  hyb_status st = check_layout(layout, false);
  if (st != HYB_OK) return st;
  if ((st = check_dtypes(layout, act, soft)) != HYB_OK) return st;
  const size_t need = make_plan(make_dims(layout), act, soft).total;
  if (need > (size_t)HYB_NOALLOC_SCRATCH_BYTES)
    return fail(HYB_ERR_WORKSPACE_TOO_SMALL,
                "this call needs %zu bytes of scratch, the built-in scratch of hyb_attn_forward_noalloc holds %zu; "
                "use hyb_attn_forward with a workspace",
                need, (size_t)HYB_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != HYB_OK) return st;
  return attn_forward_impl(layout, act, soft, x, q, k, v, text_k, text_v, w_gate_soft, w_gate_lin, w_out_soft,
                           w_out_lin, rms_weight, softmax_scale, eps, y, ws, (size_t)HYB_NOALLOC_SCRATCH_BYTES, stream,
                           dbg, false);
}

hyb_status hyb_qkv_workspace_size(const hyb_layout* layout, size_t* bytes) {
  g_err[0] = 0;
  hyb_status st = check_projection(layout);
  if (st != HYB_OK) return st;
  if (!bytes) return fail(HYB_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = qkv_weight_bytes(make_dims(layout));
  return HYB_OK;
}

hyb_status hyb_qkv_project(const hyb_layout* layout, const void* x, const void* w_q, const void* w_k,
                           const void* w_v, void* q, void* k, void* v, uint32_t* absmax, void* workspace,
                           size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  hyb_status st = check_projection(layout);
  if (st != HYB_OK) return st;
  const hyb::Dims d = make_dims(layout);
  const void* ptrs[] = {x, w_q, w_k, w_v, q, k, v, workspace};
  const char* names[] = {"x", "w_q", "w_k", "w_v", "q", "k", "v", "workspace"};
  for (int i = 0; i < 8; ++i) {
    if (!ptrs[i]) return fail(HYB_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (!aligned(ptrs[i], i == 7 ? 256 : 16))
      return fail(HYB_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", names[i], i == 7 ? 256 : 16);
  }
  if (absmax && !aligned(absmax, 4)) return fail(HYB_ERR_INVALID_ARGUMENT, "absmax is not 4-byte aligned");
  {  // outputs must not overlap x or each other
    const size_t bytes = (size_t)d.B * d.N * d.hid * 2;
    const uintptr_t lo[4] = {(uintptr_t)x, (uintptr_t)q, (uintptr_t)k, (uintptr_t)v};
    for (int i = 0; i < 4; ++i)
      for (int j = i + 1; j < 4; ++j)
        if (lo[i] < lo[j] + bytes && lo[j] < lo[i] + bytes)
          return fail(HYB_ERR_INVALID_ARGUMENT, "x, q, k and v must not overlap");
  }
  if (workspace_bytes < qkv_weight_bytes(d))
    return fail(HYB_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes,
                qkv_weight_bytes(d));
  const hipError_t he = run_projection(d, x, w_q, w_k, w_v, (char*)workspace, q, k, v, absmax, (hipStream_t)stream);
  if (he != hipSuccess) return fail(HYB_ERR_HIP, "HIP error: %s", hipGetErrorString(he));
  return HYB_OK;
}

}  // extern "C"

namespace {

// Block workspace: [layer plan | projection weights | q | k | v].
struct BlockPlan {
  Plan layer;
  size_t wt, q, k, v, wts, total;  // wts: MX exponents of the projection weights
};

BlockPlan make_block_plan(const hyb::Dims& d, hyb_dtype soft) {
  BlockPlan b;
  b.layer = make_plan(d, HYB_BF16, soft);
  const size_t act = align_up((size_t)d.B * d.N * d.hid * 2, 256);
  b.wt = b.layer.total;
  b.q = b.wt + qkv_weight_bytes(d);
  b.k = b.q + act;
  b.v = b.k + act;
  b.wts = b.v + act;
  b.total = b.wts + (soft == HYB_FP8_MX ? align_up((size_t)d.hid / 32 * 3 * d.hid, 256) : 0);
  return b;
}

}  // namespace

extern "C" {

hyb_status hyb_block_workspace_size(const hyb_layout* layout, hyb_dtype soft, size_t* bytes) {
  g_err[0] = 0;
  hyb_status st = check_projection(layout);
  if (st != HYB_OK) return st;
  st = check_dtypes(layout, HYB_BF16, soft);
  if (st != HYB_OK) return st;
  if (!bytes) return fail(HYB_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = make_block_plan(make_dims(layout), soft).total;
  return HYB_OK;
}

hyb_status hyb_block_forward(const hyb_layout* layout, hyb_dtype soft, const void* x, const void* w_q,
                             const void* w_k, const void* w_v, hyb_tensor text_k, hyb_tensor text_v,
                             const void* w_gate_soft, const void* w_gate_lin, const void* w_out_soft,
                             const void* w_out_lin, const void* rms_weight, float softmax_scale, float eps, void* y,
                             void* workspace, size_t workspace_bytes, void* stream, const hyb_debug* dbg) {
  g_err[0] = 0;
  hyb_status st = check_projection(layout);
  if (st != HYB_OK) return st;
  st = check_dtypes(layout, HYB_BF16, soft);
  if (st != HYB_OK) return st;
  const void* ptrs[] = {x, w_q, w_k, w_v, workspace};
  const char* names[] = {"x", "w_q", "w_k", "w_v", "workspace"};
  for (int i = 0; i < 5; ++i) {
    if (!ptrs[i]) return fail(HYB_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (!aligned(ptrs[i], i == 4 ? 256 : 16))
      return fail(HYB_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", names[i], i == 4 ? 256 : 16);
  }
  const hyb::Dims d = make_dims(layout);
  const BlockPlan bp = make_block_plan(d, soft);
  if (workspace_bytes < bp.total)
    return fail(HYB_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, bp.total);
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  // q, k, v views of the workspace buffers: contiguous [B, N, H, D]
  hyb_tensor tq, tk, tv;
  const int64_t sb = (int64_t)d.N * d.hid, stok = d.hid, sh = d.D;
  tq.ptr = ws + bp.q; tk.ptr = ws + bp.k; tv.ptr = ws + bp.v;
  tq.stride_b = tk.stride_b = tv.stride_b = sb;
  tq.stride_tok = tk.stride_tok = tv.stride_tok = stok;
  tq.stride_head = tk.stride_head = tv.stride_head = sh;
  // Validate the layer's own arguments before launching anything.
  {
    const bool has_text = d.L > 0;
    if ((st = check_tensor("text_k", text_k, 2, has_text)) != HYB_OK) return st;
    if ((st = check_tensor("text_v", text_v, 2, has_text)) != HYB_OK) return st;
    if ((st = check_tensor("q", tq, 2, true)) != HYB_OK) return st;
    const void* lp[] = {w_gate_soft, w_gate_lin, w_out_soft, w_out_lin, rms_weight, y};
    const char* ln[] = {"w_gate_soft", "w_gate_lin", "w_out_soft", "w_out_lin", "rms_weight", "y"};
    for (int i = 0; i < 6; ++i) {
      if (!lp[i]) return fail(HYB_ERR_INVALID_ARGUMENT, "%s is NULL", ln[i]);
      if (!aligned(lp[i], 16)) return fail(HYB_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", ln[i]);
    }
    if (!(eps > 0.f) || !isfinite(eps)) return fail(HYB_ERR_INVALID_ARGUMENT, "eps must be finite and > 0");
    if (!(softmax_scale >= 0.f) || !isfinite(softmax_scale))
      return fail(HYB_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
  }
  hipEvent_t* ev = dbg ? (hipEvent_t*)dbg->stage_events : nullptr;
  hipError_t he = hipSuccess;
  if (ev) he = hipEventRecord(ev[2 * HYB_STAGE_QKV], s);
  // fp8: the projection writes the absmax of q, k, v straight into the layer's absmax buffer
  uint32_t* amx = soft != HYB_BF16 ? (uint32_t*)(ws + bp.layer.off[W_AM]) : nullptr;
  if (soft == HYB_FP8_MX) {
    // MX projection: x is quantised once, into the layer's buffers, for this
    // GEMM and the gate GEMM
    uint8_t* x8 = (uint8_t*)(ws + bp.layer.off[W_X8]);
    uint8_t* xs = (uint8_t*)(ws + bp.layer.off[W_XS]);
    uint8_t* wt8 = (uint8_t*)(ws + bp.wt);
    uint8_t* wts = (uint8_t*)(ws + bp.wts);
    if (he == hipSuccess)
      he = hyb::launch_mx_weights(2, (const hyb::bf16_t*)w_q, (const hyb::bf16_t*)w_k, (const hyb::bf16_t*)w_v, d.hid,
                                  wt8, wts, s);
    if (he == hipSuccess)
      he = hyb::launch_mx_rows((const hyb::bf16_t*)x, (long long)d.B * d.N, d.hid, (long long)mx_rows(d), x8, xs, s);
    if (he == hipSuccess)
      he = hyb::launch_qkv_gemm_mx(d, x8, xs, (long long)mx_rows(d), wt8, wts, (hyb::bf16_t*)(ws + bp.q),
                                   (hyb::bf16_t*)(ws + bp.k), (hyb::bf16_t*)(ws + bp.v), amx, s);
  } else if (he == hipSuccess) {
    he = run_projection(d, x, w_q, w_k, w_v, ws + bp.wt, ws + bp.q, ws + bp.k, ws + bp.v, amx, s);
  }
  if (he == hipSuccess && ev) he = hipEventRecord(ev[2 * HYB_STAGE_QKV + 1], s);
  if (he != hipSuccess) return fail(HYB_ERR_HIP, "HIP error: %s", hipGetErrorString(he));
  return attn_forward_impl(layout, HYB_BF16, soft, x, tq, tk, tv, text_k, text_v, w_gate_soft, w_gate_lin,
                           w_out_soft, w_out_lin, rms_weight, softmax_scale, eps, y, workspace, bp.layer.total,
                           stream, dbg, true);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward pass.
namespace {

enum {
  B_LSE, B_G16, B_WO, B_WG, B_DYT, B_XT, B_APT, B_DZT, B_WPART, B_DOS, B_DZ, B_DR, B_TC, B_DOL, B_RMSP, B_DVR,
  B_DQS, B_DKS, B_DVS, B_DTKS, B_DTVS, B_DNUM, B_DDEN, B_LPART, B_DCF, B_DSH, B_DSL, B_DSZ, B_COUNT
};

constexpr int kWgradSplit = 4;

// Layout of the saved buffer of a training forward.
struct SavedPlan {
  size_t os, ol, ap, g16, rinv, lse, chi, clo, cz, total;
};

SavedPlan make_saved_plan(const hyb::Dims& d) {
  SavedPlan p;
  const size_t M = (size_t)d.B * d.N, hid = d.hid, D = d.D, BH = (size_t)d.B * d.H;
  size_t o = 0;
  p.os = o; o = align_up(o + M * hid * 2, 256);
  p.ol = o; o = align_up(o + M * hid * 2, 256);
  p.ap = o; o = align_up(o + M * 2 * hid * 2, 256);
  p.g16 = o; o = align_up(o + M * 2 * hid * 2, 256);
  p.rinv = o; o = align_up(o + M * 4, 256);
  p.lse = o; o = align_up(o + BH * d.N * 4 + 256, 256);  // padded like the backward's own copy
  p.chi = o; o = align_up(o + BH * d.T * D * D * 2, 256);
  p.clo = o; o = align_up(o + BH * d.T * D * D * 2, 256);
  p.cz = o; o = align_up(o + BH * d.T * D * 4, 256);
  p.total = o;
  return p;
}

SavedPtrs saved_ptrs(const SavedPlan& p, const void* saved) {
  char* b = (char*)saved;
  SavedPtrs k;
  k.os = (uint16_t*)(b + p.os);
  k.ol = (uint16_t*)(b + p.ol);
  k.ap = (uint16_t*)(b + p.ap);
  k.gates16 = (uint16_t*)(b + p.g16);
  k.rinv = (float*)(b + p.rinv);
  k.lse = (float*)(b + p.lse);
  k.comb_hi = (hyb::bf16_t*)(b + p.chi);
  k.comb_lo = (hyb::bf16_t*)(b + p.clo);
  k.comb_z = (float*)(b + p.cz);
  return k;
}

struct BwdPlan {
  Plan fwd;
  size_t off[B_COUNT];
  size_t total;
  long long mpad;
  int rms_blocks, lin_split;
};

BwdPlan make_bwd_plan(const hyb::Dims& d) {
  BwdPlan p;
  p.fwd = make_plan(d, HYB_BF16, HYB_BF16);
  const size_t M = (size_t)d.B * d.N, hid = d.hid, D = d.D, BH = (size_t)d.B * d.H, E = D * D + D;
  const size_t ML = (size_t)d.B * d.L;
  p.mpad = (long long)((M + 64 * kWgradSplit - 1) / (64 * kWgradSplit) * (64 * kWgradSplit));
  const long long rb = ((long long)M + 3) / 4;
  p.rms_blocks = (int)(rb < 512 ? rb : 512);
  int split, ts, tsplit;
  state_split(d, &split, &ts, &tsplit);
  p.lin_split = split;
  size_t sz[B_COUNT] = {0};
  sz[B_LSE] = BH * d.N * 4 + 256;  // padded: the key-centric kernel reads up to 31 rows past a frame
  sz[B_G16] = M * 2 * hid * 2;
  sz[B_WO] = 2 * hid * hid * 2;
  sz[B_WG] = 2 * hid * hid * 2;
  sz[B_DYT] = hid * (size_t)p.mpad * 2;
  sz[B_XT] = hid * (size_t)p.mpad * 2;
  sz[B_APT] = 2 * hid * (size_t)p.mpad * 2;
  sz[B_DZT] = 2 * hid * (size_t)p.mpad * 2;
  sz[B_WPART] = (size_t)kWgradSplit * 2 * hid * hid * 4;
  sz[B_DOS] = M * hid * 2;
  sz[B_DZ] = M * 2 * hid * 2;
  sz[B_DR] = M * hid * 2;
  sz[B_TC] = M * 4;
  sz[B_DOL] = M * hid * 4;
  sz[B_RMSP] = (size_t)p.rms_blocks * hid * 4;
  sz[B_DVR] = BH * d.N * 4 + 256;
  sz[B_DQS] = M * hid * 4;
  sz[B_DKS] = M * hid * 4;
  sz[B_DVS] = M * hid * 4;
  sz[B_DTKS] = ML * hid * 4;
  sz[B_DTVS] = ML * hid * 4;
  sz[B_DNUM] = M * hid * 2;
  sz[B_DDEN] = M * d.H * 4;
  sz[B_LPART] = BH * d.T * (size_t)split * E * 4;
  sz[B_DCF] = BH * d.T * E * 4;
  sz[B_DSH] = BH * (d.T + 1) * D * D * 2;
  sz[B_DSL] = BH * (d.T + 1) * D * D * 2;
  sz[B_DSZ] = BH * (d.T + 1) * D * 4;
  size_t o = p.fwd.total;
  for (int i = 0; i < B_COUNT; ++i) {
    p.off[i] = o;
    o = align_up(o + sz[i], 256);
  }
  p.total = o;
  return p;
}

hyb_status check_backward_layout(const hyb_layout* layout) {
  hyb_status st = check_layout(layout, false);
  if (st != HYB_OK) return st;
  if (layout->head_dim != 64 && layout->head_dim != 128)
    return fail(HYB_ERR_UNSUPPORTED, "the backward pass needs head_dim 64 or 128");
  if ((long long)layout->heads * layout->head_dim > 16384)
    return fail(HYB_ERR_UNSUPPORTED, "the backward pass supports hidden sizes up to 16384");
  return HYB_OK;
}

struct Range {
  uintptr_t lo, hi;
  const char* name;
};

}  // namespace

extern "C" {

hyb_status hyb_backward_workspace_size(const hyb_layout* layout, size_t* bytes) {
  g_err[0] = 0;
  hyb_status st = check_backward_layout(layout);
  if (st != HYB_OK) return st;
  if (!bytes) return fail(HYB_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = make_bwd_plan(make_dims(layout)).total;
  return HYB_OK;
}

}  // extern "C"

namespace {

// The backward pass.  ld_qkv: row stride of dq, dk, dv (hid for the public
// call; 3 hid when the block backward interleaves them into one [M][3 hid]
// operand, whose overlap the output check then skips).
hyb_status attn_backward_impl(const hyb_layout* layout, const void* x, hyb_tensor q, hyb_tensor k, hyb_tensor v,
                              hyb_tensor text_k, hyb_tensor text_v, const void* w_gate_soft, const void* w_gate_lin,
                              const void* w_out_soft, const void* w_out_lin, const void* rms_weight,
                              float softmax_scale, float eps, const void* dy, void* dx, void* dq, void* dk, void* dv,
                              int ld_qkv, void* dtext_k, void* dtext_v, float* dw_gate_soft, float* dw_gate_lin,
                              float* dw_out_soft, float* dw_out_lin, float* drms_weight, const void* saved,
                              size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream,
                              const hyb_bwd_debug* dbg) {
  hyb_status st = check_backward_layout(layout);
  if (st != HYB_OK) return st;
  const hyb::Dims d = make_dims(layout);
  const bool has_text = d.L > 0;
  if ((st = check_tensor("q", q, 2, true)) != HYB_OK) return st;
  if ((st = check_tensor("k", k, 2, true)) != HYB_OK) return st;
  if ((st = check_tensor("v", v, 2, true)) != HYB_OK) return st;
  if ((st = check_tensor("text_k", text_k, 2, has_text)) != HYB_OK) return st;
  if ((st = check_tensor("text_v", text_v, 2, has_text)) != HYB_OK) return st;
  {
    const void* req[] = {x, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin, rms_weight, dy, dx, dq, dk, dv,
                         has_text ? dtext_k : x, has_text ? dtext_v : x, workspace};
    const char* names[] = {"x", "w_gate_soft", "w_gate_lin", "w_out_soft", "w_out_lin", "rms_weight", "dy", "dx",
                           "dq", "dk", "dv", "dtext_k", "dtext_v", "workspace"};
    for (int i = 0; i < 14; ++i) {
      if (!req[i]) return fail(HYB_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
      if (!aligned(req[i], i == 13 ? 256 : 16))
        return fail(HYB_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", names[i], i == 13 ? 256 : 16);
    }
    const void* opt[] = {dw_gate_soft, dw_gate_lin, dw_out_soft, dw_out_lin, drms_weight};
    for (int i = 0; i < 5; ++i)
      if (opt[i] && !aligned(opt[i], 16)) return fail(HYB_ERR_INVALID_ARGUMENT, "weight gradient %d not 16-byte aligned", i);
  }
  if (!(eps > 0.f) || !isfinite(eps)) return fail(HYB_ERR_INVALID_ARGUMENT, "eps must be finite and > 0");
  if (!(softmax_scale >= 0.f) || !isfinite(softmax_scale))
    return fail(HYB_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
  const SavedPlan sp = make_saved_plan(d);
  if (saved) {
    if (!aligned(saved, 256)) return fail(HYB_ERR_INVALID_ARGUMENT, "saved is not 256-byte aligned");
    if (saved_bytes < sp.total)
      return fail(HYB_ERR_WORKSPACE_TOO_SMALL, "saved has %zu bytes, needs %zu", saved_bytes, sp.total);
  }
  if (dbg) {
    const void* dp[] = {dbg->d_os, dbg->d_ol, dbg->lse2};
    for (int i = 0; i < 3; ++i)
      if (dp[i] && !aligned(dp[i], 16)) return fail(HYB_ERR_INVALID_ARGUMENT, "debug buffer %d not 16-byte aligned", i);
  }
  if (ld_qkv == (int)d.hid) {  // outputs: no overlap with each other or with any input
    const size_t act = (size_t)d.B * d.N * d.hid * 2, tact = (size_t)d.B * d.L * d.hid * 2, ww = (size_t)d.hid * d.hid * 4;
    Range outs[] = {{(uintptr_t)dx, (uintptr_t)dx + act, "dx"}, {(uintptr_t)dq, (uintptr_t)dq + act, "dq"},
                    {(uintptr_t)dk, (uintptr_t)dk + act, "dk"}, {(uintptr_t)dv, (uintptr_t)dv + act, "dv"},
                    {(uintptr_t)dtext_k, (uintptr_t)dtext_k + tact, "dtext_k"},
                    {(uintptr_t)dtext_v, (uintptr_t)dtext_v + tact, "dtext_v"},
                    {(uintptr_t)dw_gate_soft, (uintptr_t)dw_gate_soft + ww, "dw_gate_soft"},
                    {(uintptr_t)dw_gate_lin, (uintptr_t)dw_gate_lin + ww, "dw_gate_lin"},
                    {(uintptr_t)dw_out_soft, (uintptr_t)dw_out_soft + ww, "dw_out_soft"},
                    {(uintptr_t)dw_out_lin, (uintptr_t)dw_out_lin + ww, "dw_out_lin"},
                    {(uintptr_t)drms_weight, (uintptr_t)drms_weight + (size_t)d.hid * 4, "drms_weight"}};
    const int nout = (int)(sizeof(outs) / sizeof(outs[0]));
    Range ins[10];
    int nin = 0;
    const hyb_tensor* ts[] = {&q, &k, &v};
    for (int i = 0; i < 3; ++i) {
      extent(*ts[i], d.B, d.N, d.H, d.D, 2, &ins[nin].lo, &ins[nin].hi);
      ins[nin++].name = "q/k/v";
    }
    if (has_text) {
      extent(text_k, d.B, d.L, d.H, d.D, 2, &ins[nin].lo, &ins[nin].hi);
      ins[nin++].name = "text_k";
      extent(text_v, d.B, d.L, d.H, d.D, 2, &ins[nin].lo, &ins[nin].hi);
      ins[nin++].name = "text_v";
    }
    ins[nin++] = {(uintptr_t)x, (uintptr_t)x + act, "x"};
    ins[nin++] = {(uintptr_t)dy, (uintptr_t)dy + act, "dy"};
    ins[nin++] = {(uintptr_t)workspace, (uintptr_t)workspace + workspace_bytes, "workspace"};
    if (saved) ins[nin++] = {(uintptr_t)saved, (uintptr_t)saved + sp.total, "saved"};
    for (int i = 0; i < nout; ++i) {
      if (!outs[i].lo || outs[i].hi == outs[i].lo) continue;
      for (int j = i + 1; j < nout; ++j)
        if (outs[j].lo && outs[j].hi > outs[j].lo && outs[i].lo < outs[j].hi && outs[j].lo < outs[i].hi)
          return fail(HYB_ERR_INVALID_ARGUMENT, "%s overlaps %s", outs[i].name, outs[j].name);
      for (int j = 0; j < nin; ++j)
        if (outs[i].lo < ins[j].hi && ins[j].lo < outs[i].hi)
          return fail(HYB_ERR_INVALID_ARGUMENT, "%s overlaps input %s", outs[i].name, ins[j].name);
    }
  }
  const BwdPlan plan = make_bwd_plan(d);
  if (workspace_bytes < plan.total)
    return fail(HYB_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, plan.total);

  char* ws = (char*)workspace;
  const float tau = softmax_scale > 0.f ? softmax_scale : 1.f / sqrtf((float)d.D);
  const float sl2 = tau * 1.4426950408889634f;
  hipStream_t s = (hipStream_t)stream;

  // forward recompute arguments (the forward plan sits at the workspace start)
  hyb::Bf16Args f;
  memset(&f, 0, sizeof(f));
  f.q = t4(q); f.k = t4(k); f.v = t4(v);
  f.tk = t4(text_k); f.tv = t4(text_v);
  f.x = (const hyb::bf16_t*)x;
  f.wgs = (const hyb::bf16_t*)w_gate_soft; f.wgl = (const hyb::bf16_t*)w_gate_lin;
  f.wos = (const hyb::bf16_t*)w_out_soft; f.wol = (const hyb::bf16_t*)w_out_lin;
  f.rmsw = (const hyb::bf16_t*)rms_weight;
  f.scale_log2 = sl2;
  f.eps = eps;
  const Plan& fp = plan.fwd;
  f.os = (uint16_t*)(ws + fp.off[W_OS]);
  f.ol = (uint16_t*)(ws + fp.off[W_OL]);
  f.ss = (float*)(ws + fp.off[W_SS]);
  f.rinv = (float*)(ws + fp.off[W_RINV]);
  f.part = (float*)(ws + fp.off[W_PART]);
  f.pre = (float*)(ws + fp.off[W_PRE]);
  f.comb_hi = (hyb::bf16_t*)(ws + fp.off[W_CHI]);
  f.comb_lo = (hyb::bf16_t*)(ws + fp.off[W_CLO]);
  f.comb_z = (float*)(ws + fp.off[W_CZ]);
  f.ap = (uint16_t*)(ws + fp.off[W_AP]);
  f.wg_t = (hyb::bf16_t*)(ws + fp.off[W_WG]);
  f.wo_t = (uint16_t*)(ws + fp.off[W_WO]);
  f.lse = (float*)(ws + plan.off[B_LSE]);
  f.gates16 = (uint16_t*)(ws + plan.off[B_G16]);
  {
    int split, ts, tsplit;
    state_split(d, &split, &ts, &tsplit);
    f.state_split = split;
    f.text_split = tsplit;
    f.state_slots = d.T * split + tsplit;
  }

  hyb::BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = f.q; a.k = f.k; a.v = f.v; a.tk = f.tk; a.tv = f.tv;
  a.x = f.x; a.wgs = f.wgs; a.wgl = f.wgl; a.wos = f.wos; a.wol = f.wol; a.rmsw = f.rmsw;
  a.dy = (const hyb::bf16_t*)dy;
  a.scale_log2 = sl2;
  a.tau = tau;
  a.eps = eps;
  a.os = f.os; a.ol = f.ol; a.ap = f.ap; a.gates16 = f.gates16;
  a.rinv = f.rinv; a.lse = f.lse;
  a.comb_hi = f.comb_hi; a.comb_lo = f.comb_lo; a.comb_z = f.comb_z;
  a.dx = (hyb::bf16_t*)dx; a.dq = (hyb::bf16_t*)dq; a.dk = (hyb::bf16_t*)dk; a.dv = (hyb::bf16_t*)dv;
  a.dtk = (hyb::bf16_t*)dtext_k; a.dtv = (hyb::bf16_t*)dtext_v;
  a.ld_qkv = ld_qkv;
  a.dwgs = dw_gate_soft; a.dwgl = dw_gate_lin; a.dwos = dw_out_soft; a.dwol = dw_out_lin; a.drmsw = drms_weight;
  a.wo_cat = (hyb::bf16_t*)(ws + plan.off[B_WO]);
  a.wg_cat = (hyb::bf16_t*)(ws + plan.off[B_WG]);
  a.dyT = (hyb::bf16_t*)(ws + plan.off[B_DYT]);
  a.xT = (hyb::bf16_t*)(ws + plan.off[B_XT]);
  a.apT = (hyb::bf16_t*)(ws + plan.off[B_APT]);
  a.dzT = (hyb::bf16_t*)(ws + plan.off[B_DZT]);
  a.mpad = plan.mpad;
  a.ksplit = kWgradSplit;
  a.wpart = (float*)(ws + plan.off[B_WPART]);
  a.dos = (hyb::bf16_t*)(ws + plan.off[B_DOS]);
  a.dz = (hyb::bf16_t*)(ws + plan.off[B_DZ]);
  a.dr = (hyb::bf16_t*)(ws + plan.off[B_DR]);
  a.tcoef = (float*)(ws + plan.off[B_TC]);
  a.dol = (float*)(ws + plan.off[B_DOL]);
  a.rms_part = (float*)(ws + plan.off[B_RMSP]);
  a.rms_blocks = plan.rms_blocks;
  a.dvr = (float*)(ws + plan.off[B_DVR]);
  a.dq_s = (float*)(ws + plan.off[B_DQS]);
  a.dk_s = (float*)(ws + plan.off[B_DKS]);
  a.dv_s = (float*)(ws + plan.off[B_DVS]);
  a.dtk_s = (float*)(ws + plan.off[B_DTKS]);
  a.dtv_s = (float*)(ws + plan.off[B_DTVS]);
  a.dnum = (hyb::bf16_t*)(ws + plan.off[B_DNUM]);
  a.dden = (float*)(ws + plan.off[B_DDEN]);
  a.lpart = (float*)(ws + plan.off[B_LPART]);
  a.lin_split = plan.lin_split;
  a.dcf = (float*)(ws + plan.off[B_DCF]);
  a.dsh = (hyb::bf16_t*)(ws + plan.off[B_DSH]);
  a.dsl = (hyb::bf16_t*)(ws + plan.off[B_DSL]);
  a.dsz = (float*)(ws + plan.off[B_DSZ]);
  a.ev = dbg ? (hipEvent_t*)dbg->stage_events : nullptr;
  a.recompute = saved == nullptr;
  if (saved) {  // the training forward's values instead of a recompute
    const SavedPtrs k = saved_ptrs(sp, saved);
    a.os = k.os; a.ol = k.ol; a.ap = k.ap; a.gates16 = k.gates16;
    a.rinv = k.rinv; a.lse = k.lse;
    a.comb_hi = k.comb_hi; a.comb_lo = k.comb_lo; a.comb_z = k.comb_z;
  }

  hipError_t he = hyb::run_bwd_bf16(d, f, a, s);
  const long long nel = (long long)d.B * d.N * d.hid;
  if (he == hipSuccess && dbg && dbg->d_os) he = hyb::launch_bf16_to_f32(a.dos, (float*)dbg->d_os, nel, s);
  if (he == hipSuccess && dbg && dbg->d_ol)
    he = hipMemcpyAsync(dbg->d_ol, a.dol, (size_t)nel * 4, hipMemcpyDeviceToDevice, s);
  if (he == hipSuccess && dbg && dbg->lse2)
    he = hipMemcpyAsync(dbg->lse2, a.lse, (size_t)d.B * d.H * d.N * 4, hipMemcpyDeviceToDevice, s);
  if (he != hipSuccess) return fail(HYB_ERR_HIP, "HIP error: %s", hipGetErrorString(he));
  return HYB_OK;
}

}  // namespace

extern "C" {

hyb_status hyb_attn_backward(const hyb_layout* layout, const void* x, hyb_tensor q, hyb_tensor k, hyb_tensor v,
                             hyb_tensor text_k, hyb_tensor text_v, const void* w_gate_soft, const void* w_gate_lin,
                             const void* w_out_soft, const void* w_out_lin, const void* rms_weight,
                             float softmax_scale, float eps, const void* dy, void* dx, void* dq, void* dk, void* dv,
                             void* dtext_k, void* dtext_v, float* dw_gate_soft, float* dw_gate_lin,
                             float* dw_out_soft, float* dw_out_lin, float* drms_weight, const void* saved,
                             size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream,
                             const hyb_bwd_debug* dbg) {
  g_err[0] = 0;
  hyb_status st = check_backward_layout(layout);
  if (st != HYB_OK) return st;
  return attn_backward_impl(layout, x, q, k, v, text_k, text_v, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin,
                            rms_weight, softmax_scale, eps, dy, dx, dq, dk, dv, layout->heads * layout->head_dim,
                            dtext_k, dtext_v, dw_gate_soft, dw_gate_lin, dw_out_soft, dw_out_lin, drms_weight,
                            saved, saved_bytes, workspace, workspace_bytes, stream, dbg);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// DiT block: projection + layer + feed-forward.
namespace {

struct DitPlan {
  BlockPlan block;
  size_t y, h, u, w1t, w2t, total;
  size_t h8, hs, us, w1s, w2s;  // MX operands of the feed-forward (HYB_FP8_MX)
};

DitPlan make_dit_plan(const hyb::Dims& d, hyb_dtype soft, int F) {
  DitPlan p;
  p.block = make_block_plan(d, soft);
  const size_t M = (size_t)d.B * d.N, hid = d.hid;
  size_t o = p.block.total;
  p.y = o; o = align_up(o + M * hid * 2, 256);
  p.h = o; o = align_up(o + M * hid * 2, 256);
  p.u = o; o = align_up(o + M * (size_t)F * 2, 256);
  p.w1t = o; o = align_up(o + (size_t)F * hid * 2, 256);
  p.w2t = o; o = align_up(o + (size_t)F * hid * 2, 256);
  p.h8 = p.hs = p.us = p.w1s = p.w2s = 0;
  if (soft == HYB_FP8_MX) {  // u, w1t, w2t hold the codes
    const size_t mp = mx_rows(d);
    p.h8 = o; o = align_up(o + M * hid, 256);
    p.hs = o; o = align_up(o + hid / 32 * mp, 256);
    p.us = o; o = align_up(o + (size_t)F / 32 * mp, 256);
    p.w1s = o; o = align_up(o + hid / 32 * (size_t)F, 256);
    p.w2s = o; o = align_up(o + (size_t)F / 32 * hid, 256);
  }
  p.total = o;
  return p;
}

hyb_status check_dit(const hyb_layout* layout, hyb_dtype soft, int32_t F) {
  hyb_status st = check_projection(layout);
  if (st != HYB_OK) return st;
  st = check_dtypes(layout, HYB_BF16, soft);
  if (st != HYB_OK) return st;
  if (F <= 0 || F % 64) return fail(HYB_ERR_INVALID_ARGUMENT, "ffn_hidden must be a positive multiple of 64 (got %d)", F);
  if (soft == HYB_FP8_MX && F % 256)
    return fail(HYB_ERR_UNSUPPORTED, "FP8_MX needs ffn_hidden to be a multiple of 256 (got %d)", F);
  return HYB_OK;
}

}  // namespace

extern "C" {

hyb_status hyb_dit_block_workspace_size(const hyb_layout* layout, hyb_dtype soft, int32_t ffn_hidden,
                                        size_t* bytes) {
  g_err[0] = 0;
  hyb_status st = check_dit(layout, soft, ffn_hidden);
  if (st != HYB_OK) return st;
  if (!bytes) return fail(HYB_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = make_dit_plan(make_dims(layout), soft, ffn_hidden).total;
  return HYB_OK;
}

hyb_status hyb_dit_block_forward(const hyb_layout* layout, hyb_dtype soft, const void* x, const void* w_q,
                                 const void* w_k, const void* w_v, hyb_tensor text_k, hyb_tensor text_v,
                                 const void* w_gate_soft, const void* w_gate_lin, const void* w_out_soft,
                                 const void* w_out_lin, const void* rms_weight, const void* ffn_norm_weight,
                                 const void* w_ff1, const void* w_ff2, int32_t ffn_hidden, float softmax_scale,
                                 float eps, void* z, void* workspace, size_t workspace_bytes, void* stream,
                                 const hyb_debug* dbg) {
  g_err[0] = 0;
  hyb_status st = check_dit(layout, soft, ffn_hidden);
  if (st != HYB_OK) return st;
  const void* ptrs[] = {ffn_norm_weight, w_ff1, w_ff2, z, workspace};
  const char* names[] = {"ffn_norm_weight", "w_ff1", "w_ff2", "z", "workspace"};
  for (int i = 0; i < 5; ++i) {
    if (!ptrs[i]) return fail(HYB_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (!aligned(ptrs[i], i == 4 ? 256 : 16))
      return fail(HYB_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", names[i], i == 4 ? 256 : 16);
  }
  const hyb::Dims d = make_dims(layout);
  const DitPlan p = make_dit_plan(d, soft, ffn_hidden);
  if (workspace_bytes < p.total)
    return fail(HYB_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, p.total);
  char* ws = (char*)workspace;
  // projection + layer into the workspace's y (validates the remaining arguments)
  st = hyb_block_forward(layout, soft, x, w_q, w_k, w_v, text_k, text_v, w_gate_soft, w_gate_lin, w_out_soft,
                         w_out_lin, rms_weight, softmax_scale, eps, ws + p.y, workspace, p.block.total, stream, dbg);
  if (st != HYB_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t* ev = dbg ? (hipEvent_t*)dbg->stage_events : nullptr;
  hipError_t he = hipSuccess;
  if (ev) he = hipEventRecord(ev[2 * HYB_STAGE_FFN], s);
  if (he == hipSuccess) {
    hyb::FfnArgs a;
    a.M = (long long)d.B * d.N;
    a.hid = d.hid;
    a.F = ffn_hidden;
    a.eps = eps;
    a.y = (const hyb::bf16_t*)(ws + p.y);
    a.wn = (const hyb::bf16_t*)ffn_norm_weight;
    a.w1 = (const hyb::bf16_t*)w_ff1;
    a.w2 = (const hyb::bf16_t*)w_ff2;
    a.h = (hyb::bf16_t*)(ws + p.h);
    a.u = (hyb::bf16_t*)(ws + p.u);
    a.w1t = (hyb::bf16_t*)(ws + p.w1t);
    a.w2t = (hyb::bf16_t*)(ws + p.w2t);
    a.z = (hyb::bf16_t*)z;
    a.mx = soft == HYB_FP8_MX;
    a.mpad = (long long)mx_rows(d);
    a.h8 = (uint8_t*)(ws + p.h8);
    a.hs = (uint8_t*)(ws + p.hs);
    a.us = (uint8_t*)(ws + p.us);
    a.w1s = (uint8_t*)(ws + p.w1s);
    a.w2s = (uint8_t*)(ws + p.w2s);
    he = hyb::run_ffn_bf16(a, s);
  }
  if (he == hipSuccess && ev) he = hipEventRecord(ev[2 * HYB_STAGE_FFN + 1], s);
  if (he != hipSuccess) return fail(HYB_ERR_HIP, "HIP error: %s", hipGetErrorString(he));
  return HYB_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Training forward: the layer plus the values its backward reads.
extern "C" {

hyb_status hyb_saved_size(const hyb_layout* layout, size_t* bytes) {
  g_err[0] = 0;
  hyb_status st = check_backward_layout(layout);
  if (st != HYB_OK) return st;
  if (!bytes) return fail(HYB_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = make_saved_plan(make_dims(layout)).total;
  return HYB_OK;
}

hyb_status hyb_attn_forward_train(const hyb_layout* layout, const void* x, hyb_tensor q, hyb_tensor k, hyb_tensor v,
                                  hyb_tensor text_k, hyb_tensor text_v, const void* w_gate_soft,
                                  const void* w_gate_lin, const void* w_out_soft, const void* w_out_lin,
                                  const void* rms_weight, float softmax_scale, float eps, void* y, void* saved,
                                  size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream,
                                  const hyb_debug* dbg) {
  g_err[0] = 0;
  hyb_status st = check_backward_layout(layout);
  if (st != HYB_OK) return st;
  const hyb::Dims d = make_dims(layout);
  const SavedPlan sp = make_saved_plan(d);
  if (!saved) return fail(HYB_ERR_INVALID_ARGUMENT, "saved is NULL");
  if (!aligned(saved, 256)) return fail(HYB_ERR_INVALID_ARGUMENT, "saved is not 256-byte aligned");
  if (saved_bytes < sp.total)
    return fail(HYB_ERR_WORKSPACE_TOO_SMALL, "saved has %zu bytes, needs %zu", saved_bytes, sp.total);
  {  // the saved buffer must not overlap y or the workspace
    const uintptr_t lo = (uintptr_t)saved, hi = lo + sp.total;
    const uintptr_t ylo = (uintptr_t)y, yhi = ylo + (size_t)d.B * d.N * d.hid * 2;
    const uintptr_t wlo = (uintptr_t)workspace, whi = wlo + workspace_bytes;
    if ((y && lo < yhi && ylo < hi) || (workspace && lo < whi && wlo < hi))
      return fail(HYB_ERR_INVALID_ARGUMENT, "saved overlaps y or the workspace");
  }
  const SavedPtrs keep = saved_ptrs(sp, saved);
  return attn_forward_impl(layout, HYB_BF16, HYB_BF16, x, q, k, v, text_k, text_v, w_gate_soft, w_gate_lin,
                           w_out_soft, w_out_lin, rms_weight, softmax_scale, eps, y, workspace, workspace_bytes,
                           stream, dbg, false, &keep);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward of the layer with its Q/K/V projection.
namespace {

struct BlockBwdPlan {
  size_t wt, q, k, v, layer, dxl, dqkv, wcat, xT, dqkvT, wpart, total;
  size_t layer_bytes;
  long long mpad;
};

BlockBwdPlan make_block_bwd_plan(const hyb::Dims& d) {
  BlockBwdPlan p;
  const BwdPlan lb = make_bwd_plan(d);
  const size_t M = (size_t)d.B * d.N, hid = d.hid;
  p.mpad = lb.mpad;
  size_t o = 0;
  p.wt = o; o = align_up(o + qkv_weight_bytes(d), 256);
  p.q = o; o = align_up(o + M * hid * 2, 256);
  p.k = o; o = align_up(o + M * hid * 2, 256);
  p.v = o; o = align_up(o + M * hid * 2, 256);
  p.layer = o; o = align_up(o + lb.total, 256);
  p.layer_bytes = lb.total;
  p.dxl = o; o = align_up(o + M * hid * 2, 256);
  p.dqkv = o; o = align_up(o + M * 3 * hid * 2, 256);
  p.wcat = o; o = align_up(o + 3 * hid * hid * 2, 256);
  p.xT = o; o = align_up(o + hid * (size_t)p.mpad * 2, 256);
  p.dqkvT = o; o = align_up(o + 3 * hid * (size_t)p.mpad * 2, 256);
  p.wpart = o; o = align_up(o + (size_t)kWgradSplit * 3 * hid * hid * 4, 256);
  p.total = o;
  return p;
}

}  // namespace

extern "C" {

hyb_status hyb_block_backward_workspace_size(const hyb_layout* layout, size_t* bytes) {
  g_err[0] = 0;
  hyb_status st = check_backward_layout(layout);
  if (st != HYB_OK) return st;
  if (!bytes) return fail(HYB_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = make_block_bwd_plan(make_dims(layout)).total;
  return HYB_OK;
}

hyb_status hyb_block_backward(const hyb_layout* layout, const void* x, const void* w_q, const void* w_k,
                              const void* w_v, hyb_tensor text_k, hyb_tensor text_v, const void* w_gate_soft,
                              const void* w_gate_lin, const void* w_out_soft, const void* w_out_lin,
                              const void* rms_weight, float softmax_scale, float eps, const void* dy, void* dx,
                              void* dtext_k, void* dtext_v, float* dw_q, float* dw_k, float* dw_v,
                              float* dw_gate_soft, float* dw_gate_lin, float* dw_out_soft, float* dw_out_lin,
                              float* drms_weight, void* workspace, size_t workspace_bytes, void* stream,
                              const hyb_bwd_debug* dbg) {
  g_err[0] = 0;
  hyb_status st = check_backward_layout(layout);
  if (st != HYB_OK) return st;
  const hyb::Dims d = make_dims(layout);
  const bool has_text = d.L > 0;
  {
    const void* req[] = {x, w_q, w_k, w_v, dy, dx, workspace};
    const char* names[] = {"x", "w_q", "w_k", "w_v", "dy", "dx", "workspace"};
    for (int i = 0; i < 7; ++i) {
      if (!req[i]) return fail(HYB_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
      if (!aligned(req[i], i == 6 ? 256 : 16))
        return fail(HYB_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", names[i], i == 6 ? 256 : 16);
    }
    const void* opt[] = {dw_q, dw_k, dw_v};
    for (int i = 0; i < 3; ++i)
      if (opt[i] && !aligned(opt[i], 16)) return fail(HYB_ERR_INVALID_ARGUMENT, "dw_q/k/v %d not 16-byte aligned", i);
    // dx and the projection-weight gradients must not overlap each other or x, dy
    const size_t act = (size_t)d.B * d.N * d.hid * 2, ww = (size_t)d.hid * d.hid * 4;
    Range r[] = {{(uintptr_t)dx, (uintptr_t)dx + act, "dx"}, {(uintptr_t)dw_q, (uintptr_t)dw_q + ww, "dw_q"},
                 {(uintptr_t)dw_k, (uintptr_t)dw_k + ww, "dw_k"}, {(uintptr_t)dw_v, (uintptr_t)dw_v + ww, "dw_v"},
                 {(uintptr_t)x, (uintptr_t)x + act, "x"}, {(uintptr_t)dy, (uintptr_t)dy + act, "dy"},
                 {(uintptr_t)workspace, (uintptr_t)workspace + workspace_bytes, "workspace"}};
    for (int i = 0; i < 4; ++i) {
      if (!r[i].lo) continue;
      for (int j = i + 1; j < 7; ++j)
        if (r[j].lo && r[i].lo < r[j].hi && r[j].lo < r[i].hi)
          return fail(HYB_ERR_INVALID_ARGUMENT, "%s overlaps %s", r[i].name, r[j].name);
    }
  }
  if ((st = check_tensor("text_k", text_k, 2, has_text)) != HYB_OK) return st;
  if ((st = check_tensor("text_v", text_v, 2, has_text)) != HYB_OK) return st;
  const BlockBwdPlan p = make_block_bwd_plan(d);
  if (workspace_bytes < p.total)
    return fail(HYB_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, p.total);
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  // q, k, v views of the workspace buffers: contiguous [B, N, H, D]
  hyb_tensor tq, tk, tv;
  const int64_t sb = (int64_t)d.N * d.hid, stok = d.hid, sh = d.D;
  tq.ptr = ws + p.q; tk.ptr = ws + p.k; tv.ptr = ws + p.v;
  tq.stride_b = tk.stride_b = tv.stride_b = sb;
  tq.stride_tok = tk.stride_tok = tv.stride_tok = stok;
  tq.stride_head = tk.stride_head = tv.stride_head = sh;
  hipError_t he = run_projection(d, x, w_q, w_k, w_v, ws + p.wt, ws + p.q, ws + p.k, ws + p.v, nullptr, s);
  if (he != hipSuccess) return fail(HYB_ERR_HIP, "HIP error: %s", hipGetErrorString(he));
  // the layer's gradients, dq | dk | dv interleaved per token row ([M][3 hid])
  char* dqkv = ws + p.dqkv;
  st = attn_backward_impl(layout, x, tq, tk, tv, text_k, text_v, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin,
                          rms_weight, softmax_scale, eps, dy, ws + p.dxl, dqkv, dqkv + (size_t)d.hid * 2,
                          dqkv + (size_t)d.hid * 4, 3 * d.hid, dtext_k, dtext_v, dw_gate_soft, dw_gate_lin,
                          dw_out_soft, dw_out_lin, drms_weight, nullptr, 0, ws + p.layer, p.layer_bytes, stream, dbg);
  if (st != HYB_OK) return st;
  hyb::QkvBwdArgs a;
  a.M = (long long)d.B * d.N;
  a.mpad = p.mpad;
  a.hid = d.hid;
  a.ksplit = kWgradSplit;
  a.x = (const hyb::bf16_t*)x;
  a.wq = (const hyb::bf16_t*)w_q; a.wk = (const hyb::bf16_t*)w_k; a.wv = (const hyb::bf16_t*)w_v;
  a.dxl = (const hyb::bf16_t*)(ws + p.dxl);
  a.dqkv = (const hyb::bf16_t*)dqkv;
  a.dx = (hyb::bf16_t*)dx;
  a.dwq = dw_q; a.dwk = dw_k; a.dwv = dw_v;
  a.wcat = (hyb::bf16_t*)(ws + p.wcat);
  a.xT = (hyb::bf16_t*)(ws + p.xT);
  a.dqkvT = (hyb::bf16_t*)(ws + p.dqkvT);
  a.wpart = (float*)(ws + p.wpart);
  he = hyb::run_qkv_backward(a, s);
  if (he != hipSuccess) return fail(HYB_ERR_HIP, "HIP error: %s", hipGetErrorString(he));
  return HYB_OK;
}

}  // extern "C"
