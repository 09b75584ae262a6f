// Host side of the C ABI declared in include/cfa.h: argument validation, workspace layout,
// work-list construction and kernel launch order. Every check runs before the first HIP call,
// so a rejected call launches nothing and writes nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "cfa.h"
#include "cfa_device.h"
#include "cfa_kernels.h"

namespace {

thread_local char g_err[512] = "";

// Optional per-kernel timing events (diagnostics), see cfa_set_kernel_events().
thread_local void* const* g_events = nullptr;
thread_local int g_event_pairs = 0;

void mark(int kernel, int end, hipStream_t st) {
  if (g_events && kernel < g_event_pairs && g_events[2 * kernel + end])
    (void)hipEventRecord((hipEvent_t)g_events[2 * kernel + end], st);
}

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

// CFA_SCHED=naive: documents in index order instead of longest first (a diagnostic that shows
// the scheduler's effect; results are bit-identical either way).
bool sched_naive() {
  const char* e = getenv("CFA_SCHED");
  return e && strcmp(e, "naive") == 0;
}

// CFA_DQ_MODE=fused: the bf16 backward at d = 128 sums dQ inside the dK/dV pass in key-tile order
// instead of running a separate dQ pass that recomputes S and dP (measured slower on MI355X: the
// hand-over of the fp32 sums between key tiles sits on each step's critical path).
bool dq_fused_requested() {
  const char* e = getenv("CFA_DQ_MODE");
  return e && strcmp(e, "fused") == 0;
}

// Compute units of the current device (the fused backward's persistent grid), looked up once per
// device.
int cu_count() {
  static int counts[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (counts[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    counts[dev] = n;
  }
  return counts[dev];
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CFA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return CFA_OK;
}

// Launches the plan kernel for a device cu_seqlens (`flag_ws`: the workspace region the plan and
// its check flag live in). CFA_DEBUG_CHECK=1 in the environment (a diagnostic) then reads the flag
// synchronously and fails the call before any other kernel runs when the device check raised it;
// without the switch the call goes on with every document empty, and cfa_device_error reads the
// flag later.
int run_plan(const int32_t* cu, int n, int total, void* flag_ws, hipStream_t st, const char* what) {
  if (int r = check_hip(cfa::launch_plan(cu, n, total, flag_ws, st, sched_naive()), what)) return r;
  const char* e = getenv("CFA_DEBUG_CHECK");
  if (!(e && strcmp(e, "1") == 0)) return CFA_OK;
  int flag = 0;
  if (int r = check_hip(hipMemcpyAsync(&flag, flag_ws, sizeof(int), hipMemcpyDeviceToHost, st), "read the plan flag"))
    return r;
  if (int r = check_hip(hipStreamSynchronize(st), "synchronize")) return r;
  if (flag) return fail(CFA_ERR_SHAPE, "%s: the device check of cu_seqlens failed (flag %d)", what, flag);
  return CFA_OK;
}

// Host mirror of cu_seqlens: cu[0] = 0, non-decreasing, cu[n] = total.
int check_cu_host(const int32_t* cu, int n_docs, int total, int max_seqlen) {
  if (!cu) return CFA_OK;
  if (cu[0] != 0) return fail(CFA_ERR_SHAPE, "cu_seqlens_host[0] = %d, expected 0", cu[0]);
  for (int n = 0; n < n_docs; ++n) {
    if (cu[n + 1] < cu[n])
      return fail(CFA_ERR_SHAPE, "cu_seqlens_host decreases at %d (%d -> %d)", n, cu[n], cu[n + 1]);
    if (max_seqlen > 0 && cu[n + 1] - cu[n] > max_seqlen)
      return fail(CFA_ERR_SHAPE, "document %d has length %d > max_seqlen %d", n, cu[n + 1] - cu[n], max_seqlen);
  }
  if (cu[n_docs] != total)
    return fail(CFA_ERR_SHAPE, "cu_seqlens_host[%d] = %d, expected total_tokens %d", n_docs, cu[n_docs], total);
  return CFA_OK;
}

struct Sizes {
  int T, n_docs, hq, hkv, d, dtype;
};

bool is_mx(int dtype) {
  return dtype == CFA_MXFP8 || dtype == CFA_MXFP4 || dtype == CFA_MXFP6 || dtype == CFA_MXFP6_E3M2;
}

int check_sizes(const Sizes& s, bool bwd) {
  if (s.T < 0) return fail(CFA_ERR_SHAPE, "total_tokens = %d < 0", s.T);
  if (s.n_docs < 1) return fail(CFA_ERR_SHAPE, "n_docs = %d < 1", s.n_docs);
  if (s.hq < 1 || s.hkv < 1) return fail(CFA_ERR_SHAPE, "hq = %d, hkv = %d must be >= 1", s.hq, s.hkv);
  if (s.hq % s.hkv) return fail(CFA_ERR_SHAPE, "hq = %d is not a multiple of hkv = %d", s.hq, s.hkv);
  if ((long)s.T * s.hq * s.d > 0x7fffffffL * 8L) return fail(CFA_ERR_SHAPE, "tensor too large");
  // the kernels address the rows of one staged tile as 32-bit offsets row·hq·d·2 bytes
  if (s.hq > 65536) return fail(CFA_ERR_UNSUPPORTED, "hq = %d above 65536", s.hq);
  if (s.dtype != CFA_F32 && s.dtype != CFA_BF16 && !is_mx(s.dtype))
    return fail(CFA_ERR_UNSUPPORTED, "dtype %d unknown", s.dtype);
  if (is_mx(s.dtype)) {
    if (s.d != 128) return fail(CFA_ERR_UNSUPPORTED, "the MX paths support d = 128 only (got %d)", s.d);
    // token-blocked rows are addressed as channel·t_pad + column in 32 bits
    if ((long)((s.T + 31) / 32 * 32 + 32L * s.n_docs) * s.d > 0x7fffffffL)
      return fail(CFA_ERR_UNSUPPORTED, "the MX paths need d·(32·ceil(T/32) + 32·n_docs) < 2^31 (T = %d, n_docs = %d)",
                  s.T, s.n_docs);
  } else if (s.dtype == CFA_F32 && s.d != 64 && s.d != 128) {
    return fail(CFA_ERR_UNSUPPORTED, "the fp32 path supports d = 64 or 128 (got %d)", s.d);
  } else if (s.d != 64 && s.d != 128 && s.d != 256) {
    return fail(CFA_ERR_UNSUPPORTED, "head dim %d unsupported (64, 128 or 256)", s.d);
  }
  if (bwd && s.dtype == CFA_F32) return fail(CFA_ERR_UNSUPPORTED, "the fp32 path is forward-only");
  return CFA_OK;
}

// An MX-quantised tensor: E4M3 codes and E8M0 scales, 256-byte aligned sections.
struct MxBuf {
  size_t codes, scales;
};

int t_pad_of(const Sizes& s) { return (s.T + 31) / 32 * 32 + 32 * s.n_docs; }

// element format of the score product's copies: 0 = E4M3, 1 = E2M1, 2 = E2M3, 3 = E3M2 (for the
// 6-bit types, the matrix instruction's format code)
int score_format(int dtype) {
  return dtype == CFA_MXFP4 ? 1 : dtype == CFA_MXFP6 ? 2 : dtype == CFA_MXFP6_E3M2 ? 3 : 0;
}

// d-blocked copy of a [T, h, d] tensor: codes [T, h, d] (E2M1: [T, h, d/2]; 6-bit: [T, h, 3d/4]),
// scales [T, h, d/32]
size_t add_mx_d(size_t off, const Sizes& s, int h, MxBuf& b, int qf = 0) {
  b.codes = off;
  off = cfa::align256(off + (size_t)s.T * h * (qf == 1 ? s.d / 2 : qf >= 2 ? 3 * s.d / 4 : s.d));
  b.scales = off;
  return cfa::align256(off + (size_t)s.T * h * (s.d / 32));
}

// token-blocked copy: codes [h, d, t_pad], scales [h, d, t_pad/32]
size_t add_mx_t(size_t off, const Sizes& s, int h, MxBuf& b) {
  const size_t tp = (size_t)t_pad_of(s);
  b.codes = off;
  off = cfa::align256(off + (size_t)h * s.d * tp);
  b.scales = off;
  return cfa::align256(off + (size_t)h * s.d * (tp / 32));
}

struct WsLayout {
  size_t plan_end;
  size_t delta;             // bwd: float [hq, T]
  size_t dkdv_part;         // bwd bf16 with a head split: float [2][n_split][T][hkv][d]
  size_t dq_acc, dq_cnt;    // bwd bf16 at d = 128, dQ inside the dK/dV pass: float [T][hq][d], int [t_pad/32][hq][8]
  size_t dq_kt;             // and the pass's Kᵀ operand slots (FUSED_KT_BYTES)
  long n_cnt;
  bool fused_dq;
  int n_split;
  MxBuf vt;                 // fwd MX: V along tokens
  MxBuf dod, dot;           // bwd MX
  size_t total;
};


// fused_dq: the bf16 backward at d = 128 sums dQ inside the dK/dV pass (its workspace holds the
// fp32 sums, their counts and Kᵀ operand slots); otherwise a separate dQ pass recomputes S and dP
WsLayout ws_layout(int pass, const Sizes& s, bool fused_dq = false) {
  WsLayout w{};
  cfa::PlanLayout pl(s.n_docs);
  w.plan_end = pl.end;
  size_t off = pl.end;
  w.n_split = 1;
  if (pass == 1) {
    w.delta = off;
    off = cfa::align256(off + sizeof(float) * (size_t)s.hq * (size_t)s.T);
    if (s.dtype == CFA_BF16) {
      w.n_split = cfa::dkdv_head_split(s.hq, s.hkv, s.d);
      if (w.n_split > 1) {
        w.dkdv_part = off;
        off = cfa::align256(off + sizeof(float) * 2 * (size_t)w.n_split * s.T * s.hkv * s.d);
      }
      if (fused_dq && s.d == 128) {
        w.fused_dq = true;
        w.dq_acc = off;
        off = cfa::align256(off + sizeof(float) * (size_t)s.T * s.hq * s.d);
        w.n_cnt = (long)(t_pad_of(s) / 32) * s.hq * 8;
        w.dq_cnt = off;
        off = cfa::align256(off + sizeof(int) * (size_t)w.n_cnt);
        w.dq_kt = off;
        off = cfa::align256(off + cfa::FUSED_KT_BYTES);
      }
    }
  }
  if (is_mx(s.dtype)) {
    if (pass == 0) {
      off = add_mx_t(off, s, s.hkv, w.vt);
    } else {
      off = add_mx_d(off, s, s.hq, w.dod);
      off = add_mx_t(off, s, s.hq, w.dot);
    }
  }
  w.total = off;
  return w;
}

// forward-to-backward buffer of the MX paths: Q_d and K_d (E4M3, E2M1 for CFA_MXFP4, E2M3 for CFA_MXFP6,
// E3M2 for CFA_MXFP6_E3M2) and V_d (E4M3, the dP operand), written by the forward's one pass over V
struct SavedLayout {
  MxBuf qd, kd, vd;
  size_t total;
};

SavedLayout saved_layout(const Sizes& s) {
  SavedLayout v{};
  size_t off = 0;
  const int qf = score_format(s.dtype);
  off = add_mx_d(off, s, s.hq, v.qd, qf);
  off = add_mx_d(off, s, s.hkv, v.kd, qf);
  off = add_mx_d(off, s, s.hkv, v.vd);
  v.total = off;
  return v;
}

cfa::Plan make_plan(void* ws, int n_docs) {
  cfa::PlanLayout pl(n_docs);
  char* b = (char*)ws;
  cfa::Plan p;
  p.header = (const int*)(b + pl.header);
  p.docinfo = (const int2*)(b + pl.docinfo);
  p.order = (const int*)(b + pl.order);
  p.pref = (const int*)(b + pl.pref);
  p.n_docs = n_docs;
  return p;
}

}  // namespace

extern "C" {

int cfa_version(void) { return (1 << 16) | 0; }

const char* cfa_status_string(int s) {
  switch (s) {
    case CFA_OK: return "CFA_OK";
    case CFA_ERR_NULL: return "CFA_ERR_NULL";
    case CFA_ERR_SHAPE: return "CFA_ERR_SHAPE";
    case CFA_ERR_UNSUPPORTED: return "CFA_ERR_UNSUPPORTED";
    case CFA_ERR_ALIGN: return "CFA_ERR_ALIGN";
    case CFA_ERR_WORKSPACE: return "CFA_ERR_WORKSPACE";
    case CFA_ERR_HIP: return "CFA_ERR_HIP";
    default: return "CFA_ERR_UNKNOWN";
  }
}

const char* cfa_last_error(void) { return g_err; }

size_t cfa_workspace_bytes(int pass, int total_tokens, int n_docs, int hq, int hkv, int d, int dtype) {
  Sizes s{total_tokens, n_docs, hq, hkv, d, dtype};
  if ((pass != 0 && pass != 1) || check_sizes(s, pass == 1) != CFA_OK) return 0;
  return ws_layout(pass, s, dq_fused_requested()).total;
}

size_t cfa_saved_bytes(int total_tokens, int n_docs, int hq, int hkv, int d, int dtype) {
  Sizes s{total_tokens, n_docs, hq, hkv, d, dtype};
  if (!is_mx(dtype) || check_sizes(s, false) != CFA_OK) return 0;
  return saved_layout(s).total;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens,
             const int32_t* cu_seqlens_host, int n_docs, int total_tokens, int max_seqlen, int hq, int hkv, int d,
             float scale, int causal, int dtype, void* saved, void* workspace, size_t workspace_bytes,
             void* stream) {
  g_err[0] = 0;
  const Sizes s{total_tokens, n_docs, hq, hkv, d, dtype};
  if (int st = check_sizes(s, false)) return st;
  if (!cu_seqlens || !workspace) return fail(CFA_ERR_NULL, "cu_seqlens and workspace must not be NULL");
  if (total_tokens > 0 && (!q || !k || !v || !o || !lse))
    return fail(CFA_ERR_NULL, "q, k, v, o and lse must not be NULL");
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(CFA_ERR_SHAPE, "scale must be finite and > 0");
  if (is_mx(dtype) && !saved) return fail(CFA_ERR_NULL, "the MX paths need the `saved` buffer");
  if (is_mx(dtype) && !aligned(saved, 256)) return fail(CFA_ERR_ALIGN, "saved must be 256-byte aligned");
  for (const void* p : {q, k, v, (const void*)o, (const void*)lse, (const void*)cu_seqlens})
    if (!aligned(p, 16)) return fail(CFA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(CFA_ERR_ALIGN, "workspace must be 256-byte aligned");
  const WsLayout wl = ws_layout(0, s);
  if (workspace_bytes < wl.total)
    return fail(CFA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, wl.total);
  if (int st = check_cu_host(cu_seqlens_host, n_docs, total_tokens, max_seqlen)) return st;

  hipStream_t st = (hipStream_t)stream;
  if (int r = run_plan(cu_seqlens, n_docs, total_tokens, workspace, st, "plan kernel")) return r;
  if (total_tokens == 0) return CFA_OK;
  const cfa::Plan plan = make_plan(workspace, n_docs);
  hipError_t e;
  if (is_mx(dtype)) {
    char* ws = (char*)workspace;
    char* sv = (char*)saved;
    const SavedLayout sl = saved_layout(s);
    const cfa::PlanLayout pl(n_docs);
    const int tp = t_pad_of(s);
    const int qf = score_format(dtype);
    auto S = [&](size_t off) { return (uint8_t*)sv + off; };
    cfa::MxPrepOut po{nullptr, nullptr, S(sl.kd.codes), S(sl.kd.scales), S(sl.vd.codes), S(sl.vd.scales),
                      (uint8_t*)ws + wl.vt.codes, (uint8_t*)ws + wl.vt.scales};
    mark(1, 0, st);
    if (int r = check_hip(cfa::launch_mx_prep_fwd(k, v, total_tokens, hkv, ws, n_docs, qf, po, tp, st),
                          "quantize K, V"))
      return r;
    mark(1, 1, st);
    mark(0, 0, st);
    e = cfa::launch_fwd_mx(q, S(sl.qd.codes), S(sl.qd.scales),
                           (const uint8_t*)sv + sl.kd.codes, (const uint8_t*)sv + sl.kd.scales,
                           (const uint8_t*)ws + wl.vt.codes, (const uint8_t*)ws + wl.vt.scales, v, o, lse, plan,
                           plan.pref, (const int*)(ws + pl.padoff), total_tokens, tp, hq, hkv, scale, causal, qf, st);
    mark(0, 1, st);
    return check_hip(e, "MX forward kernel");
  }
  mark(0, 0, st);
  if (dtype == CFA_F32)
    e = cfa::launch_fwd_f32(q, k, v, o, lse, plan, plan.pref, total_tokens, hq, hkv, d, scale, causal, st);
  else
    e = cfa::launch_fwd_bf16(q, k, v, o, lse, plan, plan.pref, total_tokens, hq, hkv, d, scale, causal, st);
  mark(0, 1, st);
  return check_hip(e, "forward kernel");
}

namespace {
int bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             const float* dlse, const void* saved, void* dq, void* dk, void* dv, const int32_t* cu_seqlens,
             const int32_t* cu_seqlens_host, int n_docs, int total_tokens, int max_seqlen, int hq, int hkv, int d,
             float scale, int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream,
             bool allow_fused) {
  g_err[0] = 0;
  const Sizes s{total_tokens, n_docs, hq, hkv, d, dtype};
  if (int st = check_sizes(s, true)) return st;
  if (!cu_seqlens || !workspace) return fail(CFA_ERR_NULL, "cu_seqlens and workspace must not be NULL");
  if (total_tokens > 0 && (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv))
    return fail(CFA_ERR_NULL, "q, k, v, o, lse, dout, dq, dk and dv must not be NULL");
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(CFA_ERR_SHAPE, "scale must be finite and > 0");
  // MX without `saved`: Q_d, K_d and V_d are quantised again into the workspace, after its own
  // sections (the quantisers give the bytes the forward wrote)
  const bool requant = is_mx(dtype) && !saved;
  if (is_mx(dtype) && saved && !aligned(saved, 256)) return fail(CFA_ERR_ALIGN, "saved must be 256-byte aligned");
  for (const void* p : {q, k, v, o, (const void*)lse, dout, (const void*)dlse, (const void*)dq, (const void*)dk,
                        (const void*)dv, (const void*)cu_seqlens})
    if (!aligned(p, 16)) return fail(CFA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(CFA_ERR_ALIGN, "workspace must be 256-byte aligned");
  const WsLayout wl = ws_layout(1, s, allow_fused);
  const size_t ws_need = wl.total + (requant ? saved_layout(s).total : 0);
  if (workspace_bytes < ws_need)
    return fail(CFA_ERR_WORKSPACE, "workspace %zu bytes < required %zu%s", workspace_bytes, ws_need,
                requant ? " (MX without saved: cfa_workspace_bytes + cfa_saved_bytes)" : "");
  if (int st = check_cu_host(cu_seqlens_host, n_docs, total_tokens, max_seqlen)) return st;

  hipStream_t st = (hipStream_t)stream;
  if (int r = run_plan(cu_seqlens, n_docs, total_tokens, workspace, st, "plan kernel")) return r;
  if (total_tokens == 0) return CFA_OK;
  const cfa::Plan plan = make_plan(workspace, n_docs);
  float* delta = (float*)((char*)workspace + wl.delta);
  if (!is_mx(dtype)) {
    mark(0, 0, st);
    if (int r = check_hip(cfa::launch_bwd_pre(o, dout, dlse, delta, total_tokens, hq, d, st), "bwd preprocess"))
      return r;
    mark(0, 1, st);
  }
  if (is_mx(dtype)) {
    char* ws = (char*)workspace;
    const char* sv = (const char*)saved;
    const SavedLayout sl = saved_layout(s);
    if (requant) {
      uint8_t* rq = (uint8_t*)ws + wl.total;
      const int qf = score_format(dtype);
      auto quant_d = [&](const void* x, int h, const MxBuf& b, int fmt) {
        const long n = (long)total_tokens * h * d;
        return fmt == 1 ? cfa::launch_mx_quantize_d_fp4(x, n, rq + b.codes, rq + b.scales, st)
             : fmt >= 2 ? cfa::launch_mx_quantize_d_fp6(x, n, d, fmt, rq + b.codes, rq + b.scales, st)
                        : cfa::launch_mx_quantize_d(x, n, rq + b.codes, rq + b.scales, st);
      };
      hipError_t e = quant_d(q, hq, sl.qd, qf);
      if (!e) e = quant_d(k, hkv, sl.kd, qf);
      if (!e) e = quant_d(v, hkv, sl.vd, 0);
      if (int r = check_hip(e, "backward requantisation of Q, K, V")) return r;
      sv = (const char*)rq;
    }
    const cfa::PlanLayout pl(n_docs);
    const int tp = t_pad_of(s);
    const int* padoff = (const int*)(ws + pl.padoff);
    auto U = [&](const MxBuf& b, bool codes) { return (uint8_t*)ws + (codes ? b.codes : b.scales); };
    // D and both dO copies in one pass over O and dO (V_d came with the forward's pass over V)
    cfa::MxPrepOut po{U(wl.dod, true), U(wl.dod, false), nullptr, nullptr, nullptr, nullptr, U(wl.dot, true),
                      U(wl.dot, false)};
    mark(0, 0, st);
    if (int r = check_hip(cfa::launch_mx_prep_bwd(o, dout, dlse, delta, total_tokens, hq, ws, n_docs, po, tp, st),
                          "backward preparation"))
      return r;
    mark(0, 1, st);
    cfa::MxOperands m;
    m.qd = (const uint8_t*)sv + sl.qd.codes; m.qd_sc = (const uint8_t*)sv + sl.qd.scales;
    m.kd = (const uint8_t*)sv + sl.kd.codes; m.kd_sc = (const uint8_t*)sv + sl.kd.scales;
    m.dod = U(wl.dod, true); m.dod_sc = U(wl.dod, false);
    m.vd = (const uint8_t*)sv + sl.vd.codes; m.vd_sc = (const uint8_t*)sv + sl.vd.scales;
    m.dot = U(wl.dot, true); m.dot_sc = U(wl.dot, false);
    mark(1, 0, st);
    if (int r = check_hip(cfa::launch_bwd_dkdv_mx(m, q, dout, lse, delta, dk, dv, plan, plan.pref, padoff, total_tokens,
                                                  tp, hq, hkv, scale, causal, score_format(dtype), st),
                          "MX dK/dV kernel"))
      return r;
    mark(1, 1, st);
    mark(2, 0, st);
    int r = check_hip(cfa::launch_bwd_dq_mx(m, k, lse, delta, dq, plan, plan.pref, total_tokens, hq, hkv, scale,
                                            causal, score_format(dtype), st),
                      "MX dQ kernel");
    mark(2, 1, st);
    return r;
  }
  if (wl.fused_dq) {
    char* ws = (char*)workspace;
    const cfa::PlanLayout pl(n_docs);
    mark(1, 0, st);
    int r = check_hip(cfa::launch_bwd_dkdv_dq(q, k, v, dout, lse, delta, dq, dk, dv, plan, total_tokens, hq, hkv, scale,
                                              causal, wl.n_split, (float*)(ws + wl.dkdv_part), (float*)(ws + wl.dq_acc),
                                              (int*)(ws + wl.dq_cnt), wl.n_cnt, (const int*)(ws + pl.padoff),
                                              (int*)(ws + pl.header), ws + wl.dq_kt, cu_count(), st),
                      "dK/dV/dQ kernel");
    mark(1, 1, st);
    return r;
  }
  mark(1, 0, st);
  if (int r = check_hip(cfa::launch_bwd_dkdv(q, k, v, dout, lse, delta, dk, dv, plan, plan.pref, total_tokens, hq,
                                             hkv, d, scale, causal, wl.n_split,
                                             (float*)((char*)workspace + wl.dkdv_part), st),
                        "dK/dV kernel"))
    return r;
  mark(1, 1, st);
  mark(2, 0, st);
  int r = check_hip(cfa::launch_bwd_dq(q, k, v, dout, lse, delta, dq, plan, plan.pref, total_tokens, hq, hkv, d,
                                       scale, causal, st),
                    "dQ kernel");
  mark(2, 1, st);
  return r;
}
}  // namespace

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             const float* dlse, const void* saved, void* dq, void* dk, void* dv, const int32_t* cu_seqlens,
             const int32_t* cu_seqlens_host, int n_docs, int total_tokens, int max_seqlen, int hq, int hkv, int d,
             float scale, int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, lse, dout, dlse, saved, dq, dk, dv, cu_seqlens, cu_seqlens_host, n_docs, total_tokens,
                  max_seqlen, hq, hkv, d, scale, causal, dtype, workspace, workspace_bytes, stream,
                  dq_fused_requested());
}

int mx_padded_tokens(int total_tokens, int n_docs) {
  if (total_tokens < 0 || n_docs < 0) return 0;
  return (total_tokens + 31) / 32 * 32 + 32 * n_docs;
}

size_t mx_workspace_bytes(int n_docs) { return n_docs >= 1 ? cfa::PlanLayout(n_docs).end : 0; }

size_t mx_quantize_bytes(int axis, int total_tokens, int n_docs, int h, int d, size_t* scale_bytes) {
  size_t codes = 0;
  if (total_tokens >= 0 && n_docs >= 1 && h >= 1 && (d == 64 || d == 128) && axis >= 0 && axis <= 2)
    codes = (size_t)h * d * (axis == 0 ? (size_t)total_tokens : (size_t)mx_padded_tokens(total_tokens, n_docs));
  if (scale_bytes) *scale_bytes = codes / 32;
  return codes;
}

int mx_quantize(const void* x, int total_tokens, int h, int d, const int32_t* cu_seqlens,
                const int32_t* cu_seqlens_host, int n_docs, int axis, uint8_t* codes, uint8_t* scales, int t_pad,
                void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (total_tokens < 0 || h < 1) return fail(CFA_ERR_SHAPE, "total_tokens = %d, h = %d", total_tokens, h);
  if (d != 64 && d != 128) return fail(CFA_ERR_UNSUPPORTED, "mx_quantize supports d = 64 or 128 (got %d)", d);
  if (axis < 0 || axis > 2) return fail(CFA_ERR_SHAPE, "axis must be 0, 1 or 2 (got %d)", axis);
  if (total_tokens > 0 && (!x || !codes || !scales)) return fail(CFA_ERR_NULL, "x, codes and scales must not be NULL");
  for (const void* p : {x, (const void*)codes})
    if (!aligned(p, 16)) return fail(CFA_ERR_ALIGN, "x and codes must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if (axis == 0) {
    if (total_tokens == 0) return CFA_OK;
    return check_hip(cfa::launch_mx_quantize_d(x, (long)total_tokens * h * d, codes, scales, st), "mx_quantize_d");
  }
  if (n_docs < 1) return fail(CFA_ERR_SHAPE, "n_docs = %d < 1", n_docs);
  if (!cu_seqlens || !workspace) return fail(CFA_ERR_NULL, "cu_seqlens and workspace must not be NULL for axes 1, 2");
  if ((long)t_pad * d > 0x7fffffffL) return fail(CFA_ERR_UNSUPPORTED, "t_pad·d must stay below 2^31");
  if (h > 65536) return fail(CFA_ERR_UNSUPPORTED, "axes 1 and 2 take h <= 65536 heads (got %d)", h);
  if ((long)((t_pad + 127) / 128) * h > 0x7fffffffL)
    return fail(CFA_ERR_UNSUPPORTED, "axes 1 and 2 need h·ceil(t_pad/128) < 2^31 workgroups");
  if (t_pad % 32 || t_pad < mx_padded_tokens(total_tokens, n_docs))
    return fail(CFA_ERR_SHAPE, "t_pad = %d must be a multiple of 32 and >= %d", t_pad,
                mx_padded_tokens(total_tokens, n_docs));
  if (!aligned(workspace, 256)) return fail(CFA_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < mx_workspace_bytes(n_docs))
    return fail(CFA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, mx_workspace_bytes(n_docs));
  if (int r = check_cu_host(cu_seqlens_host, n_docs, total_tokens, 0)) return r;
  if (int r = run_plan(cu_seqlens, n_docs, total_tokens, workspace, st, "plan kernel")) return r;
  if (total_tokens == 0) return CFA_OK;
  return check_hip(cfa::launch_mx_quantize_t(x, total_tokens, h, d, workspace, n_docs, codes, scales, t_pad, axis == 2,
                                             st),
                   "mx_quantize_t");
}

// ---------------------------------------------------------------- cross-attention (bf16)
namespace {
struct CrossLayout {
  size_t plan_k, delta, dkdv_part, total;
  int n_split;
};
// [plan on the query documents][plan on the key documents][bwd: D][bwd: head-split partial sums]
CrossLayout cross_layout(int pass, int Tq, int Tk, int n_docs, int hq, int hkv, int d) {
  CrossLayout l{};
  const cfa::PlanLayout pl(n_docs);
  l.plan_k = pl.end;
  size_t off = l.plan_k + pl.end;
  l.n_split = 1;
  if (pass == 1) {
    l.delta = off;
    off = cfa::align256(off + sizeof(float) * (size_t)hq * Tq);
    l.n_split = cfa::dkdv_head_split(hq, hkv, d);
    if (l.n_split > 1) {
      l.dkdv_part = off;
      off = cfa::align256(off + sizeof(float) * 2 * (size_t)l.n_split * Tk * hkv * d);
    }
  }
  l.total = off;
  return l;
}
int check_cross(int pass, int Tq, int Tk, int n_docs, int hq, int hkv, int d) {
  if (Tk < 0) return fail(CFA_ERR_SHAPE, "total_k = %d < 0", Tk);
  const Sizes s{Tq, n_docs, hq, hkv, d, CFA_BF16};
  if (int st = check_sizes(s, pass == 1)) return st;
  if ((long)Tk * hkv * d > 0x7fffffffL * 8L) return fail(CFA_ERR_SHAPE, "tensor too large");
  return CFA_OK;
}
cfa::Plan plan_at(void* ws, size_t off, int n_docs) { return make_plan((char*)ws + off, n_docs); }
}  // namespace

size_t cfa_cross_workspace_bytes(int pass, int total_q, int total_k, int n_docs, int hq, int hkv, int d) {
  if ((pass != 0 && pass != 1) || check_cross(pass, total_q, total_k, n_docs, hq, hkv, d) != CFA_OK) return 0;
  return cross_layout(pass, total_q, total_k, n_docs, hq, hkv, d).total;
}

int attn_fwd_cross(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens_q,
                   const int32_t* cu_seqlens_k, const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_k_host,
                   int n_docs, int total_q, int total_k, int hq, int hkv, int d, float scale, int causal,
                   void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (int st = check_cross(0, total_q, total_k, n_docs, hq, hkv, d)) return st;
  if (!cu_seqlens_q || !cu_seqlens_k || !workspace)
    return fail(CFA_ERR_NULL, "cu_seqlens_q, cu_seqlens_k and workspace must not be NULL");
  if (total_q > 0 && (!q || !o || !lse)) return fail(CFA_ERR_NULL, "q, o and lse must not be NULL");
  if (total_k > 0 && (!k || !v)) return fail(CFA_ERR_NULL, "k and v must not be NULL");
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(CFA_ERR_SHAPE, "scale must be finite and > 0");
  for (const void* p : {q, k, v, (const void*)o, (const void*)lse, (const void*)cu_seqlens_q, (const void*)cu_seqlens_k})
    if (!aligned(p, 16)) return fail(CFA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(CFA_ERR_ALIGN, "workspace must be 256-byte aligned");
  const CrossLayout cl = cross_layout(0, total_q, total_k, n_docs, hq, hkv, d);
  if (workspace_bytes < cl.total)
    return fail(CFA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, cl.total);
  if (int st = check_cu_host(cu_seqlens_q_host, n_docs, total_q, 0)) return st;
  if (int st = check_cu_host(cu_seqlens_k_host, n_docs, total_k, 0)) return st;
  hipStream_t st = (hipStream_t)stream;
  if (int r = run_plan(cu_seqlens_q, n_docs, total_q, workspace, st, "plan kernel (queries)")) return r;
  if (int r = run_plan(cu_seqlens_k, n_docs, total_k, (char*)workspace + cl.plan_k, st, "plan kernel (keys)"))
    return r;
  if (total_q == 0) return CFA_OK;
  const cfa::Plan pq = make_plan(workspace, n_docs);
  const cfa::Plan pk = plan_at(workspace, cl.plan_k, n_docs);
  mark(0, 0, st);
  hipError_t e = cfa::launch_fwd_bf16(q, k, v, o, lse, pq, pq.pref, total_q, hq, hkv, d, scale, causal, st, pk.docinfo);
  mark(0, 1, st);
  return check_hip(e, "cross-attention forward kernel");
}

int attn_bwd_cross(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   const float* dlse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q,
                   const int32_t* cu_seqlens_k, const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_k_host,
                   int n_docs, int total_q, int total_k, int hq, int hkv, int d, float scale, int causal,
                   void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (int st = check_cross(1, total_q, total_k, n_docs, hq, hkv, d)) return st;
  if (!cu_seqlens_q || !cu_seqlens_k || !workspace)
    return fail(CFA_ERR_NULL, "cu_seqlens_q, cu_seqlens_k and workspace must not be NULL");
  if (total_q > 0 && (!q || !o || !lse || !dout || !dq)) return fail(CFA_ERR_NULL, "q, o, lse, dout, dq must not be NULL");
  if (total_k > 0 && (!k || !v || !dk || !dv)) return fail(CFA_ERR_NULL, "k, v, dk, dv must not be NULL");
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(CFA_ERR_SHAPE, "scale must be finite and > 0");
  for (const void* p : {q, k, v, o, (const void*)lse, dout, (const void*)dlse, (const void*)dq, (const void*)dk,
                        (const void*)dv, (const void*)cu_seqlens_q, (const void*)cu_seqlens_k})
    if (!aligned(p, 16)) return fail(CFA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(CFA_ERR_ALIGN, "workspace must be 256-byte aligned");
  const CrossLayout cl = cross_layout(1, total_q, total_k, n_docs, hq, hkv, d);
  if (workspace_bytes < cl.total)
    return fail(CFA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, cl.total);
  if (int st = check_cu_host(cu_seqlens_q_host, n_docs, total_q, 0)) return st;
  if (int st = check_cu_host(cu_seqlens_k_host, n_docs, total_k, 0)) return st;
  hipStream_t st = (hipStream_t)stream;
  if (int r = run_plan(cu_seqlens_q, n_docs, total_q, workspace, st, "plan kernel (queries)")) return r;
  if (int r = run_plan(cu_seqlens_k, n_docs, total_k, (char*)workspace + cl.plan_k, st, "plan kernel (keys)"))
    return r;
  const cfa::Plan pq = make_plan(workspace, n_docs);
  const cfa::Plan pk = plan_at(workspace, cl.plan_k, n_docs);
  float* delta = (float*)((char*)workspace + cl.delta);
  mark(0, 0, st);
  if (int r = check_hip(cfa::launch_bwd_pre(o, dout, dlse, delta, total_q, hq, d, st), "bwd preprocess")) return r;
  mark(0, 1, st);
  mark(1, 0, st);
  if (total_k > 0) {   // dK/dV: key tiles; keys of an empty query document get zero gradients
    if (int r = check_hip(cfa::launch_bwd_dkdv(q, k, v, dout, lse, delta, dk, dv, pk, pk.pref, total_q, hq, hkv, d,
                                               scale, causal, cl.n_split, (float*)((char*)workspace + cl.dkdv_part),
                                               st, pq.docinfo, total_k),
                          "cross-attention dK/dV kernel"))
      return r;
  }
  mark(1, 1, st);
  mark(2, 0, st);
  hipError_t e = hipSuccess;
  if (total_q > 0)
    e = cfa::launch_bwd_dq(q, k, v, dout, lse, delta, dq, pq, pq.pref, total_q, hq, hkv, d, scale, causal, st,
                           pk.docinfo);
  mark(2, 1, st);
  return check_hip(e, "cross-attention dQ kernel");
}

int mx_quantize_fp4(const void* x, int total_tokens, int h, int d, uint8_t* codes, uint8_t* scales, void* stream) {
  g_err[0] = 0;
  if (total_tokens < 0 || h < 1) return fail(CFA_ERR_SHAPE, "total_tokens = %d, h = %d", total_tokens, h);
  if (d != 64 && d != 128) return fail(CFA_ERR_UNSUPPORTED, "mx_quantize_fp4 supports d = 64 or 128 (got %d)", d);
  if (total_tokens > 0 && (!x || !codes || !scales)) return fail(CFA_ERR_NULL, "x, codes and scales must not be NULL");
  for (const void* p : {x, (const void*)codes})
    if (!aligned(p, 16)) return fail(CFA_ERR_ALIGN, "x and codes must be 16-byte aligned");
  if (total_tokens == 0) return CFA_OK;
  return check_hip(cfa::launch_mx_quantize_d_fp4(x, (long)total_tokens * h * d, codes, scales, (hipStream_t)stream),
                   "mx_quantize_d_fp4");
}

namespace {
int quantize_fp6(const char* name, int fmt, const void* x, int total_tokens, int h, int d, uint8_t* codes,
                 uint8_t* scales, void* stream) {
  g_err[0] = 0;
  if (total_tokens < 0 || h < 1) return fail(CFA_ERR_SHAPE, "total_tokens = %d, h = %d", total_tokens, h);
  if (d != 64 && d != 128) return fail(CFA_ERR_UNSUPPORTED, "%s supports d = 64 or 128 (got %d)", name, d);
  if (total_tokens > 0 && (!x || !codes || !scales)) return fail(CFA_ERR_NULL, "x, codes and scales must not be NULL");
  for (const void* p : {x, (const void*)codes})
    if (!aligned(p, 16)) return fail(CFA_ERR_ALIGN, "x and codes must be 16-byte aligned");
  if (total_tokens == 0) return CFA_OK;
  return check_hip(
      cfa::launch_mx_quantize_d_fp6(x, (long)total_tokens * h * d, d, fmt, codes, scales, (hipStream_t)stream), name);
}
}  // namespace

int mx_quantize_fp6(const void* x, int total_tokens, int h, int d, uint8_t* codes, uint8_t* scales, void* stream) {
  return quantize_fp6("mx_quantize_fp6", 2, x, total_tokens, h, d, codes, scales, stream);
}

int mx_quantize_fp6_e3m2(const void* x, int total_tokens, int h, int d, uint8_t* codes, uint8_t* scales,
                         void* stream) {
  return quantize_fp6("mx_quantize_fp6_e3m2", 3, x, total_tokens, h, d, codes, scales, stream);
}

// ---------------------------------------------------------------- decoding over a KV cache
namespace {
struct DecLayout {
  size_t part_o, part_ml, total;
};
DecLayout dec_layout(int n_seqs, int total_k, int hq, int d) {
  DecLayout l{};
  const cfa::PlanLayout pl(n_seqs);
  const size_t slots = cfa::decode_partial_slots(total_k, n_seqs);
  l.part_o = pl.end;
  l.part_ml = cfa::align256(l.part_o + sizeof(float) * slots * hq * d);
  l.total = cfa::align256(l.part_ml + 2 * sizeof(float) * slots * hq);
  return l;
}
int check_decode_sizes(int n_seqs, int total_k, int hq, int hkv, int d, int kv_dtype) {
  if (total_k < 0) return fail(CFA_ERR_SHAPE, "total_k = %d < 0", total_k);
  if (n_seqs < 1) return fail(CFA_ERR_SHAPE, "n_seqs = %d < 1", n_seqs);
  if (hq < 1 || hkv < 1) return fail(CFA_ERR_SHAPE, "hq = %d, hkv = %d must be >= 1", hq, hkv);
  if (hq % hkv) return fail(CFA_ERR_SHAPE, "hq = %d is not a multiple of hkv = %d", hq, hkv);
  if ((long)total_k * hkv * d > 0x7fffffffL * 8L || (long)n_seqs * hq * d > 0x7fffffffL)
    return fail(CFA_ERR_SHAPE, "tensor too large");
  if (kv_dtype != CFA_BF16 && kv_dtype != CFA_MXFP8)
    return fail(CFA_ERR_UNSUPPORTED, "cache dtype %d unsupported (CFA_BF16 or CFA_MXFP8)", kv_dtype);
  if (d != 64 && d != 128) return fail(CFA_ERR_UNSUPPORTED, "decoding supports d = 64 or 128 (got %d)", d);
  return CFA_OK;
}
}  // namespace

size_t cfa_decode_workspace_bytes(int n_seqs, int total_k, int hq, int hkv, int d, int kv_dtype) {
  if (check_decode_sizes(n_seqs, total_k, hq, hkv, d, kv_dtype) != CFA_OK) return 0;
  return dec_layout(n_seqs, total_k, hq, d).total;
}

int attn_decode(const void* q, const void* k_cache, const void* v_cache, const uint8_t* k_scales,
                const uint8_t* v_scales, void* o, float* lse, const int32_t* cu_seqlens_k,
                const int32_t* cu_seqlens_k_host, int n_seqs, int total_k, int hq, int hkv, int d, float scale,
                int kv_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (int st = check_decode_sizes(n_seqs, total_k, hq, hkv, d, kv_dtype)) return st;
  if (!cu_seqlens_k || !workspace || !q || !o || !lse)
    return fail(CFA_ERR_NULL, "q, o, lse, cu_seqlens_k and workspace must not be NULL");
  if (total_k > 0 && (!k_cache || !v_cache)) return fail(CFA_ERR_NULL, "k_cache and v_cache must not be NULL");
  if (total_k > 0 && kv_dtype == CFA_MXFP8 && (!k_scales || !v_scales))
    return fail(CFA_ERR_NULL, "an MXFP8 cache needs k_scales and v_scales");
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(CFA_ERR_SHAPE, "scale must be finite and > 0");
  for (const void* p : {q, k_cache, v_cache, (const void*)o, (const void*)lse, (const void*)cu_seqlens_k})
    if (!aligned(p, 16)) return fail(CFA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (!aligned(workspace, 256)) return fail(CFA_ERR_ALIGN, "workspace must be 256-byte aligned");
  const DecLayout dl = dec_layout(n_seqs, total_k, hq, d);
  if (workspace_bytes < dl.total)
    return fail(CFA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, dl.total);
  if (int st = check_cu_host(cu_seqlens_k_host, n_seqs, total_k, 0)) return st;

  hipStream_t st = (hipStream_t)stream;
  if (int r = run_plan(cu_seqlens_k, n_seqs, total_k, workspace, st, "plan kernel")) return r;
  const cfa::Plan plan = make_plan(workspace, n_seqs);
  float* part_o = (float*)((char*)workspace + dl.part_o);
  void* part_ml = (char*)workspace + dl.part_ml;
  mark(0, 0, st);
  if (int r = check_hip(cfa::launch_decode(q, k_cache, v_cache, k_scales, v_scales, plan, plan.pref, n_seqs, total_k,
                                           hq, hkv, d, scale, kv_dtype == CFA_MXFP8, part_o, part_ml, st),
                        "decode kernel"))
    return r;
  mark(0, 1, st);
  mark(1, 0, st);
  int r = check_hip(cfa::launch_decode_combine(part_o, part_ml, o, lse, plan, n_seqs, hq, d, st), "decode combine");
  mark(1, 1, st);
  return r;
}

int cfa_set_kernel_events(void* const* events, int n_pairs) {
  g_err[0] = 0;
  if (n_pairs < 0 || (n_pairs > 0 && !events)) return fail(CFA_ERR_NULL, "events must hold 2*n_pairs handles");
  g_events = n_pairs ? events : nullptr;
  g_event_pairs = n_pairs;
  return CFA_OK;
}

int cfa_device_error(const void* workspace, void* stream, int* flag) {
  g_err[0] = 0;
  if (!workspace || !flag) return fail(CFA_ERR_NULL, "workspace and flag must not be NULL");
  hipStream_t st = (hipStream_t)stream;
  int host = 0;
  if (int r = check_hip(hipMemcpyAsync(&host, workspace, sizeof(int), hipMemcpyDeviceToHost, st), "read flag"))
    return r;
  if (int r = check_hip(hipStreamSynchronize(st), "synchronize")) return r;
  *flag = host;
  return CFA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- backward without allocation
namespace {
// Scratch of attn_bwd_noalloc: one copy per GPU the library runs on, held until the process ends.
// In host code this name is only a stand-in for the device array, never a device address: kernels
// get the pointer hipGetSymbolAddress returns for the current device.
constexpr size_t STATIC_SCRATCH_BYTES = size_t(64) << 20;
static __device__ __align__(256) char scratch[STATIC_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept.
int scratch_for_current_device(void** out) {
  int dev = 0;
  if (int r = check_hip(hipGetDevice(&dev), "hipGetDevice")) return r;
  if (dev < 0 || dev >= MAX_DEVICES) return fail(CFA_ERR_UNSUPPORTED, "device index %d >= %d", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (int r = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)")) return r;
    if (!p || !aligned(p, 256)) return fail(CFA_ERR_HIP, "scratch array address %p is not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CFA_OK;
}
}  // namespace

extern "C" {

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     const float* dlse, const void* saved, void* dq, void* dk, void* dv, const int32_t* cu_seqlens,
                     const int32_t* cu_seqlens_host, int n_docs, int total_tokens, int max_seqlen, int hq, int hkv,
                     int d, float scale, int causal, int dtype, void* stream) {
  g_err[0] = 0;
  const Sizes s{total_tokens, n_docs, hq, hkv, d, dtype};
  if (int st = check_sizes(s, true)) return st;
  // attn_bwd's own plan when it fits (then the results are attn_bwd's bit for bit), else dQ as
  // its own pass, which needs no fp32 dQ sums (results within rounding of attn_bwd's)
  const bool fused = dq_fused_requested() && ws_layout(1, s, true).total <= STATIC_SCRATCH_BYTES;
  const size_t need = ws_layout(1, s, fused).total + (is_mx(dtype) && !saved ? saved_layout(s).total : 0);
  if (need > STATIC_SCRATCH_BYTES)
    return fail(CFA_ERR_WORKSPACE, "attn_bwd_noalloc: these sizes need %zu bytes of scratch, above its fixed %zu",
                need, STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (int r = scratch_for_current_device(&ws)) return r;
  return bwd_impl(q, k, v, o, lse, dout, dlse, saved, dq, dk, dv, cu_seqlens, cu_seqlens_host, n_docs, total_tokens,
                  max_seqlen, hq, hkv, d, scale, causal, dtype, ws, STATIC_SCRATCH_BYTES, stream, fused);
}

}  // extern "C"
