// C ABI of libsparse_attn.so: argument checks, workspace layout and launches.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "sa_common.h"

namespace {

thread_local char g_msg[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_msg[0] = '\0';
  return SA_OK;
}

constexpr int kMaxDev = 64;
std::atomic<int> g_arch[kMaxDev];  // 0 unknown, 1 gfx950, 2 other

// The code objects are built for gfx950 only.
int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDev) return fail(SA_EUNSUPPORTED, "device index %d out of range", dev);
  int st = g_arch[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(SA_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(SA_EUNSUPPORTED, "libsparse_attn is built for gfx950 only");
  return SA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_mask(const sa_mask_t* m) {
  if (m == nullptr) return fail(SA_EINVAL, "mask is NULL");
  if (m->n_q < 1 || m->n_k < 1) return fail(SA_EINVAL, "n_q and n_k must be >= 1 (got %d, %d)", m->n_q, m->n_k);
  if ((int64_t)m->n_k > ((int64_t)1 << 24) * sa::BK - 1)
    return fail(SA_EINVAL, "n_k too large (%d)", m->n_k);
  switch (m->kind) {
    case SA_MASK_SEPLLM:
      if (m->n_q != m->n_k) return fail(SA_EINVAL, "SEPLLM needs n_q == n_k (got %d, %d)", m->n_q, m->n_k);
      if (m->a < 0) return fail(SA_EINVAL, "SEPLLM initial count a must be >= 0 (got %d)", m->a);
      if (m->w < 1) return fail(SA_EINVAL, "SEPLLM neighbour count w must be >= 1 (got %d)", m->w);
      if (m->sep_max < 0) return fail(SA_EINVAL, "SEPLLM separator bound sep_max must be >= 0 (got %d)", m->sep_max);
      break;
    case SA_MASK_LAMBDA:
      if (m->n_q != m->n_k) return fail(SA_EINVAL, "LAMBDA needs n_q == n_k (got %d, %d)", m->n_q, m->n_k);
      if (m->n_starting < 0) return fail(SA_EINVAL, "n_starting must be >= 0 (got %d)", m->n_starting);
      if (m->L_pretrain < 0) return fail(SA_EINVAL, "L_pretrain must be >= 0 (got %d)", m->L_pretrain);
      break;
    case SA_MASK_SEGMENT:
      if (m->prefix_len < 0) return fail(SA_EINVAL, "prefix_len must be >= 0 (got %d)", m->prefix_len);
      if ((int64_t)m->prefix_len + m->n_q != m->n_k)
        return fail(SA_EINVAL, "SEGMENT needs n_k == prefix_len + n_q (got %d != %d + %d)", m->n_k,
                    m->prefix_len, m->n_q);
      break;
    default:
      return fail(SA_EINVAL, "unknown mask kind %d", m->kind);
  }
  return SA_OK;
}

int check_tensor(const char* name, const void* p, const int64_t st[3], int esz) {
  if (p == nullptr) return fail(SA_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(SA_EINVAL, "%s must be 16-byte aligned", name);
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0 || (st[i] * esz) % 16 != 0)
      return fail(SA_EINVAL, "%s stride[%d] = %lld must be >= 0 and a multiple of 16 bytes", name, i,
                  (long long)st[i]);
  // rows of a 64-row block are addressed with 32-bit byte offsets
  if (st[2] * esz > (int64_t)1 << 26)
    return fail(SA_EUNSUPPORTED, "%s token stride = %lld elements exceeds 64 MiB", name, (long long)st[2]);
  return SA_OK;
}

int check_args(const sa_mask_t* m, const sa_fwd_args_t* a) {
  if (a == nullptr) return fail(SA_EINVAL, "args is NULL");
  if (a->dtype != SA_F32 && a->dtype != SA_BF16) return fail(SA_EINVAL, "unknown dtype %d", a->dtype);
  if (a->d != 64 && a->d != 128) return fail(SA_EUNSUPPORTED, "d must be 64 or 128 (got %d)", a->d);
  if (a->batch < 1 || a->h_q < 1 || a->h_kv < 1)
    return fail(SA_EINVAL, "batch, h_q and h_kv must be >= 1");
  if (a->h_q % a->h_kv != 0) return fail(SA_EINVAL, "h_q (%d) must be a multiple of h_kv (%d)", a->h_q, a->h_kv);
  if ((int64_t)a->batch * a->h_q * sa::ceil_div(m->n_q, sa::TQ) > 0x7fffffffLL)
    return fail(SA_EINVAL, "too many tiles");
  if (a->rope != SA_ROPE_NONE && a->rope != SA_ROPE_HALF && a->rope != SA_ALIBI)
    return fail(SA_EINVAL, "unknown position encoding %d", a->rope);
  if (a->rope == SA_ROPE_HALF && !(std::isfinite(a->rope_base) && a->rope_base > 1.0f))
    return fail(SA_EINVAL, "rope_base must be finite and > 1");
  if (a->rope == SA_ALIBI) {
    if (m->kind != SA_MASK_LAMBDA) return fail(SA_EUNSUPPORTED, "the ALiBi bias is supported with the LAMBDA mask only");
    if (!(std::isfinite(a->alibi_exp) && a->alibi_exp > 0.0f))
      return fail(SA_EINVAL, "ALiBi slope exponent alibi_exp must be finite and > 0");
  }
  if (!(std::isfinite(a->scale) && a->scale > 0.0f)) return fail(SA_EINVAL, "scale must be finite and > 0");
  const int esz = a->dtype == SA_BF16 ? 2 : 4;
  int r;
  if ((r = check_tensor("q", a->q, a->q_stride, esz)) != SA_OK) return r;
  if ((r = check_tensor("k", a->k, a->k_stride, esz)) != SA_OK) return r;
  if ((r = check_tensor("v", a->v, a->v_stride, esz)) != SA_OK) return r;
  if ((r = check_tensor("o", a->o, a->o_stride, esz)) != SA_OK) return r;
  return SA_OK;
}

// Workspace sections of sparse_attn_fwd (byte offsets from the base).
struct WsLayout {
  int64_t qrot = -1, krot = -1, ksep = -1, vsep = -1, kcap = -1;
  int64_t sep_rows = 0, cap_rows = 0;
  int n_cap = 0;
  int64_t total = 0;
};

// The rotated query copy: fp32 forwards with RoPE read it; the bf16 forward
// rotates and scales its queries in registers, so only the backward (which
// reads them pre-scaled) needs it there.
WsLayout ws_layout(const sa_mask_t& m, const sa_fwd_args_t& a, bool for_bwd = false) {
  WsLayout w;
  const int64_t esz = a.dtype == SA_BF16 ? 2 : 4;
  const int64_t row = esz * a.d;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off = sa::align_up(off + bytes, 256);
    return o;
  };
  if (a.dtype == SA_BF16 ? for_bwd : a.rope == SA_ROPE_HALF)
    w.qrot = take((int64_t)a.batch * a.h_q * m.n_q * row);
  if (a.rope == SA_ROPE_HALF) w.krot = take((int64_t)a.batch * a.h_kv * m.n_k * row);
  if (m.kind == SA_MASK_SEPLLM && m.sep != nullptr) {
    w.sep_rows = sa::align_up(sa::plan_layout(m).cap_sep, sa::BK);
    w.ksep = take((int64_t)a.batch * a.h_kv * w.sep_rows * row);
    w.vsep = take((int64_t)a.batch * a.h_kv * w.sep_rows * row);
  }
  if (m.kind == SA_MASK_LAMBDA && a.rope == SA_ROPE_HALF && m.n_starting > 0) {
    w.n_cap = m.n_starting < m.n_k ? m.n_starting : m.n_k;
    w.cap_rows = sa::align_up(w.n_cap, sa::BK);
    w.kcap = take((int64_t)a.batch * a.h_kv * w.cap_rows * row);
  }
  w.total = off;
  return w;
}

// Backward workspace: the forward's sections, then the fp32 gradient sections.
struct BwdLayout {
  WsLayout fwd;
  int64_t D = -1, dq_acc = -1, dq_cap = -1, dk_acc = -1, dv_acc = -1;
  int64_t dksep = -1, dvsep = -1, dkcap = -1, dvcap = -1;
  int64_t total = 0;
};

BwdLayout bwd_layout(const sa_mask_t& m, const sa_fwd_args_t& a) {
  BwdLayout L;
  L.fwd = ws_layout(m, a, true);
  int64_t off = sa::align_up(L.fwd.total, 256);
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off = sa::align_up(off + bytes, 256);
    return o;
  };
  const int64_t qrows = (int64_t)a.batch * a.h_q * m.n_q;
  const int64_t krows = (int64_t)a.batch * a.h_kv * m.n_k;
  const int64_t row = 4 * (int64_t)a.d;
  const bool use_cap = m.kind == SA_MASK_LAMBDA && a.rope == SA_ROPE_HALF && L.fwd.n_cap > 0;
  L.D = take(4 * qrows);
  L.dq_acc = take(row * qrows);
  if (use_cap) L.dq_cap = take(row * qrows);
  L.dk_acc = take(row * krows);
  L.dv_acc = take(row * krows);
  if (L.fwd.sep_rows > 0) {
    L.dksep = take(row * a.batch * a.h_kv * L.fwd.sep_rows);
    L.dvsep = take(row * a.batch * a.h_kv * L.fwd.sep_rows);
  }
  if (use_cap) {
    L.dkcap = take(row * a.batch * a.h_kv * L.fwd.cap_rows);
    L.dvcap = take(row * a.batch * a.h_kv * L.fwd.cap_rows);
  }
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

const char* sa_last_error(void) { return g_msg; }

int sa_plan_layout(const sa_mask_t* m, sa_plan_header_t* layout) {
  int r = check_mask(m);
  if (r != SA_OK) return r;
  if (layout == nullptr) return fail(SA_EINVAL, "layout is NULL");
  *layout = sa::plan_layout(*m);
  return ok();
}

int sa_plan_bytes(const sa_mask_t* m, size_t* bytes) {
  int r = check_mask(m);
  if (r != SA_OK) return r;
  if (bytes == nullptr) return fail(SA_EINVAL, "bytes is NULL");
  *bytes = (size_t)sa::plan_layout(*m).total_bytes;
  return ok();
}

int sparse_attn_plan(const sa_mask_t* m, void* plan, size_t plan_bytes, hipStream_t stream) {
  int r = check_mask(m);
  if (r != SA_OK) return r;
  if (plan == nullptr) return fail(SA_EINVAL, "plan is NULL");
  if (!aligned16(plan)) return fail(SA_EINVAL, "plan must be 16-byte aligned");
  const sa_plan_header_t lay = sa::plan_layout(*m);
  if (plan_bytes < (size_t)lay.total_bytes)
    return fail(SA_ENOSPACE, "plan buffer too small: %zu < %lld bytes", plan_bytes, (long long)lay.total_bytes);
  if ((r = check_device()) != SA_OK) return r;
  hipError_t e = sa::launch_plan(*m, lay, plan, stream);
  if (e != hipSuccess) return fail(SA_EHIP, "plan launch: %s", hipGetErrorString(e));
  return ok();
}

int sa_plan_status(const void* plan, size_t plan_bytes, hipStream_t stream, sa_plan_header_t* out) {
  if (plan == nullptr) return fail(SA_EINVAL, "plan is NULL");
  if (plan_bytes < sizeof(sa_plan_header_t)) return fail(SA_EINVAL, "plan buffer too small for a header");
  int r;
  if ((r = check_device()) != SA_OK) return r;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(SA_EHIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
  sa_plan_header_t h;
  e = hipMemcpy(&h, plan, sizeof(h), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SA_EHIP, "hipMemcpy of the plan header: %s", hipGetErrorString(e));
  if (h.magic != 0x31504153u || h.version != 1 || h.total_bytes > (int64_t)plan_bytes)
    return fail(SA_EINVAL, "the buffer does not hold a complete plan");
  if (out != nullptr) *out = h;
  if (h.n_sep > h.cap_sep)
    return fail(SA_ENOSPACE, "the mask has %d separators at j >= %d, the plan lists at most %d (sep_max)", h.n_sep,
                h.g0, h.cap_sep);
  return ok();
}

int sa_fwd_workspace_bytes(const sa_mask_t* m, const sa_fwd_args_t* a, size_t* bytes) {
  int r = check_mask(m);
  if (r != SA_OK) return r;
  if (a == nullptr || bytes == nullptr) return fail(SA_EINVAL, "args or bytes is NULL");
  *bytes = (size_t)ws_layout(*m, *a).total;
  return ok();
}

int sa_fwd_workspace_layout(const sa_mask_t* m, const sa_fwd_args_t* a, sa_fwd_ws_layout_t* out) {
  int r = check_mask(m);
  if (r != SA_OK) return r;
  if (a == nullptr || out == nullptr) return fail(SA_EINVAL, "args or layout is NULL");
  if ((r = check_args(m, a)) != SA_OK) return r;
  const WsLayout w = ws_layout(*m, *a);
  out->krot = w.krot;
  out->ksep = w.ksep;
  out->vsep = w.vsep;
  out->kcap = w.kcap;
  out->qrot = w.qrot;
  out->sep_rows = w.sep_rows;
  out->cap_rows = w.cap_rows;
  out->total = w.total;
  return ok();
}

}  // extern "C"

namespace {

enum { STAGE_ROPE = 1, STAGE_ATTEND = 2 };

int run_fwd(const sa_mask_t* m, const void* plan, size_t plan_bytes, const sa_fwd_args_t* a,
            void* ws, size_t ws_bytes, hipStream_t stream, int stages) {
  int r = check_mask(m);
  if (r != SA_OK) return r;
  if ((r = check_args(m, a)) != SA_OK) return r;
  if (plan == nullptr) return fail(SA_EINVAL, "plan is NULL");
  const sa_plan_header_t lay = sa::plan_layout(*m);
  if (plan_bytes < (size_t)lay.total_bytes)
    return fail(SA_ENOSPACE, "plan buffer too small: %zu < %lld bytes", plan_bytes, (long long)lay.total_bytes);
  const WsLayout w = ws_layout(*m, *a);
  if (ws_bytes < (size_t)w.total)
    return fail(SA_ENOSPACE, "workspace too small: %zu < %lld bytes", ws_bytes, (long long)w.total);
  if (w.total > 0 && (ws == nullptr || !aligned16(ws)))
    return fail(SA_EINVAL, "workspace must be a 16-byte aligned device pointer");
  if ((r = check_device()) != SA_OK) return r;
  char* base = static_cast<char*>(ws);
  sa::RopeOut ro;
  memset(&ro, 0, sizeof(ro));
  ro.qrot = w.qrot >= 0 ? base + w.qrot : nullptr;
  ro.krot = w.krot >= 0 ? base + w.krot : nullptr;
  ro.ksep = w.ksep >= 0 ? base + w.ksep : nullptr;
  ro.vsep = w.vsep >= 0 ? base + w.vsep : nullptr;
  ro.sep_rows = w.sep_rows;
  ro.kcap = w.kcap >= 0 ? base + w.kcap : nullptr;
  ro.cap_rows = w.cap_rows;
  ro.n_cap = w.n_cap;
  if (stages & STAGE_ROPE) {
    sa::ThetaTable th;
    memset(&th, 0, sizeof(th));
    if (a->rope == SA_ROPE_HALF)
      for (int c = 0; c < a->d / 2; ++c) th.th[c] = std::pow((double)a->rope_base, -2.0 * c / a->d);
    hipError_t e = sa::launch_rope(*m, lay, plan, *a, th, ro, stream);
    if (e != hipSuccess) return fail(SA_EHIP, "rope launch: %s", hipGetErrorString(e));
  }
  if (stages & STAGE_ATTEND) {
    hipError_t e = sa::launch_fwd(*m, lay, plan, *a, ro, stream);
    if (e != hipSuccess) return fail(SA_EHIP, "forward launch: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

int sparse_attn_fwd(const sa_mask_t* m, const void* plan, size_t plan_bytes, const sa_fwd_args_t* a,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_fwd(m, plan, plan_bytes, a, ws, ws_bytes, stream, STAGE_ROPE | STAGE_ATTEND);
}

int sparse_attn_rope(const sa_mask_t* m, const void* plan, size_t plan_bytes, const sa_fwd_args_t* a,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_fwd(m, plan, plan_bytes, a, ws, ws_bytes, stream, STAGE_ROPE);
}

int sparse_attn_attend(const sa_mask_t* m, const void* plan, size_t plan_bytes, const sa_fwd_args_t* a,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_fwd(m, plan, plan_bytes, a, ws, ws_bytes, stream, STAGE_ATTEND);
}

int sa_bwd_workspace_bytes(const sa_mask_t* m, const sa_fwd_args_t* a, size_t* bytes) {
  int r = check_mask(m);
  if (r != SA_OK) return r;
  if (a == nullptr || bytes == nullptr) return fail(SA_EINVAL, "args or bytes is NULL");
  *bytes = (size_t)bwd_layout(*m, *a).total;
  return ok();
}

int sparse_attn_bwd(const sa_mask_t* m, const void* plan, size_t plan_bytes, const sa_fwd_args_t* a,
                    const sa_bwd_args_t* g, void* ws, size_t ws_bytes, hipStream_t stream) {
  int r = check_mask(m);
  if (r != SA_OK) return r;
  if ((r = check_args(m, a)) != SA_OK) return r;
  if (a->lse == nullptr) return fail(SA_EINVAL, "the backward needs the forward's lse");
  if (!aligned16(a->lse)) return fail(SA_EINVAL, "lse must be 16-byte aligned");
  if (g == nullptr) return fail(SA_EINVAL, "grads is NULL");
  const int esz = a->dtype == SA_BF16 ? 2 : 4;
  if ((r = check_tensor("dout", g->dout, g->dout_stride, esz)) != SA_OK) return r;
  if ((r = check_tensor("dq", g->dq, g->dq_stride, esz)) != SA_OK) return r;
  if ((r = check_tensor("dk", g->dk, g->dk_stride, esz)) != SA_OK) return r;
  if ((r = check_tensor("dv", g->dv, g->dv_stride, esz)) != SA_OK) return r;
  if (plan == nullptr) return fail(SA_EINVAL, "plan is NULL");
  const sa_plan_header_t lay = sa::plan_layout(*m);
  if (plan_bytes < (size_t)lay.total_bytes)
    return fail(SA_ENOSPACE, "plan buffer too small: %zu < %lld bytes", plan_bytes, (long long)lay.total_bytes);
  const BwdLayout L = bwd_layout(*m, *a);
  if (ws_bytes < (size_t)L.total)
    return fail(SA_ENOSPACE, "workspace too small: %zu < %lld bytes", ws_bytes, (long long)L.total);
  if (ws == nullptr || !aligned16(ws)) return fail(SA_EINVAL, "workspace must be a 16-byte aligned device pointer");
  if ((r = check_device()) != SA_OK) return r;
  char* base = static_cast<char*>(ws);
  sa::RopeOut ro;
  memset(&ro, 0, sizeof(ro));
  ro.qrot = L.fwd.qrot >= 0 ? base + L.fwd.qrot : nullptr;
  ro.krot = L.fwd.krot >= 0 ? base + L.fwd.krot : nullptr;
  ro.ksep = L.fwd.ksep >= 0 ? base + L.fwd.ksep : nullptr;
  ro.vsep = L.fwd.vsep >= 0 ? base + L.fwd.vsep : nullptr;
  ro.sep_rows = L.fwd.sep_rows;
  ro.kcap = L.fwd.kcap >= 0 ? base + L.fwd.kcap : nullptr;
  ro.cap_rows = L.fwd.cap_rows;
  ro.n_cap = L.fwd.n_cap;
  sa::ThetaTable th;
  memset(&th, 0, sizeof(th));
  if (a->rope == SA_ROPE_HALF)
    for (int c = 0; c < a->d / 2; ++c) th.th[c] = std::pow((double)a->rope_base, -2.0 * c / a->d);
  hipError_t e = sa::launch_rope(*m, lay, plan, *a, th, ro, stream);
  if (e != hipSuccess) return fail(SA_EHIP, "rope launch: %s", hipGetErrorString(e));
  auto sec = [&](int64_t off) { return off >= 0 ? reinterpret_cast<float*>(base + off) : nullptr; };
  sa::BwdWs w;
  w.D = sec(L.D);
  w.dq_acc = sec(L.dq_acc);
  w.dq_cap = sec(L.dq_cap);
  w.dk_acc = sec(L.dk_acc);
  w.dv_acc = sec(L.dv_acc);
  w.dksep = sec(L.dksep);
  w.dvsep = sec(L.dvsep);
  w.dkcap = sec(L.dkcap);
  w.dvcap = sec(L.dvcap);
  e = sa::launch_bwd(*m, lay, plan, *a, *g, ro, w, th, stream);
  if (e != hipSuccess) return fail(SA_EHIP, "backward launch: %s", hipGetErrorString(e));
  return ok();
}

int sa_topk_workspace_bytes(int32_t n_heads, int32_t pool_len, size_t* bytes) {
  if (bytes == nullptr) return fail(SA_EINVAL, "bytes is NULL");
  if (n_heads < 1 || pool_len < 1) return fail(SA_EINVAL, "n_heads and pool_len must be >= 1");
  *bytes = sa::topk_workspace_bytes(n_heads, pool_len);
  return ok();
}

int topk_retrieve(int32_t dtype, int32_t n_heads, int32_t pool_len, int32_t d, int32_t k,
                  const void* q_score, int64_t q_head_stride, const void* pool_k, const void* pool_v,
                  int64_t pool_head_stride, int64_t pool_row_stride, int32_t* idx, double* score,
                  void* pref_k, void* pref_v, int64_t pref_head_stride, int64_t pref_row_stride,
                  void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dtype != SA_F32 && dtype != SA_BF16) return fail(SA_EINVAL, "unknown dtype %d", dtype);
  if (n_heads < 1 || pool_len < 1) return fail(SA_EINVAL, "n_heads and pool_len must be >= 1");
  if (d != 64 && d != 128) return fail(SA_EUNSUPPORTED, "d must be 64 or 128 (got %d)", d);
  if (k < 1 || k > pool_len) return fail(SA_EINVAL, "k must be in [1, pool_len] (got %d)", k);
  if (q_score == nullptr || pool_k == nullptr || idx == nullptr)
    return fail(SA_EINVAL, "q_score, pool_k and idx must not be NULL");
  if (q_head_stride < 0 || pool_head_stride < 0 || pool_row_stride < 0)
    return fail(SA_EINVAL, "strides must be >= 0");
  const int esz = dtype == SA_BF16 ? 2 : 4;
  if (!aligned16(pool_k) || (pool_head_stride * esz) % 16 || (pool_row_stride * esz) % 16)
    return fail(SA_EINVAL, "pool_k must be 16-byte aligned with strides that are multiples of 16 bytes");
  if (pool_v != nullptr) {
    if (pref_k == nullptr || pref_v == nullptr)
      return fail(SA_EINVAL, "pref_k and pref_v are required when pool_v is given");
    if (!aligned16(pool_k) || !aligned16(pool_v) || !aligned16(pref_k) || !aligned16(pref_v))
      return fail(SA_EINVAL, "pool and prefix buffers must be 16-byte aligned for the gather");
    if ((pool_head_stride * esz) % 16 || (pool_row_stride * esz) % 16 || (pref_head_stride * esz) % 16 ||
        (pref_row_stride * esz) % 16 || pref_head_stride < 0 || pref_row_stride < 0)
      return fail(SA_EINVAL, "pool and prefix strides must be multiples of 16 bytes");
  }
  const size_t need = sa::topk_workspace_bytes(n_heads, pool_len);
  if (ws_bytes < need) return fail(SA_ENOSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 7u))
    return fail(SA_EINVAL, "workspace must be an 8-byte aligned device pointer");
  int r = check_device();
  if (r != SA_OK) return r;
  hipError_t e = sa::launch_topk(dtype, n_heads, pool_len, d, k, q_score, q_head_stride, pool_k, pool_v,
                                 pool_head_stride, pool_row_stride, idx, score, pref_k, pref_v,
                                 pref_head_stride, pref_row_stride, ws, stream);
  if (e != hipSuccess) return fail(SA_EHIP, "top-k launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// Byte span of `rows` rows starting at row r0 of each of `heads` heads.
struct Span {
  uintptr_t lo, hi;
  bool dst;
};

void add_spans(std::vector<Span>& out, const void* base, int heads, int64_t hs, int64_t rs, int64_t r0,
               int64_t rows, int64_t row_bytes, int esz, bool dst) {
  if (rows <= 0) return;
  for (int h = 0; h < heads; ++h) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(base) + (uintptr_t)((h * hs + r0 * rs) * esz);
    out.push_back({lo, lo + (uintptr_t)((rows - 1) * rs * esz + row_bytes), dst});
  }
}

// True when some destination span meets any other span.
bool dst_overlap(std::vector<Span>& v) {
  std::sort(v.begin(), v.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
  uintptr_t end_all = 0, end_dst = 0;
  for (const Span& s : v) {
    if (s.lo < end_dst || (s.dst && s.lo < end_all)) return true;
    end_all = std::max(end_all, s.hi);
    if (s.dst) end_dst = std::max(end_dst, s.hi);
  }
  return false;
}

}  // namespace

extern "C" {

int sparse_attn_segment_carry(int32_t dtype, int32_t n_heads, int32_t n_local, int32_t d, int32_t prefix_len,
                              int32_t seg_len, int32_t tail_len, const void* k, const void* v,
                              int64_t kv_head_stride, int64_t kv_row_stride, void* tail_k, void* tail_v,
                              int64_t tail_head_stride, int64_t tail_row_stride, void* pool_k, void* pool_v,
                              int64_t pool_head_stride, int64_t pool_row_stride, int64_t pool_len,
                              int64_t pool_cap, hipStream_t stream) {
  if (dtype != SA_F32 && dtype != SA_BF16) return fail(SA_EINVAL, "unknown dtype %d", dtype);
  const int esz = dtype == SA_BF16 ? 2 : 4;
  if (n_heads < 1 || n_local < 0 || n_local > n_heads)
    return fail(SA_EINVAL, "need n_heads >= 1 and 0 <= n_local <= n_heads (got %d, %d)", n_heads, n_local);
  if (d < 1 || ((int64_t)d * esz) % 16 != 0) return fail(SA_EINVAL, "d * element size must be a multiple of 16 bytes");
  if (prefix_len < 0 || seg_len < 0 || tail_len < 0)
    return fail(SA_EINVAL, "prefix_len, seg_len and tail_len must be >= 0");
  if (pool_len < 0 || pool_cap < 0) return fail(SA_EINVAL, "pool_len and pool_cap must be >= 0");
  const int n_long = n_heads - n_local;
  const int keep = std::min<int64_t>(tail_len, (int64_t)prefix_len + seg_len);
  const bool do_tail = n_local > 0 && keep > 0;
  const bool do_pool = n_long > 0 && seg_len > 0;
  if (do_pool && pool_len + seg_len > pool_cap)
    return fail(SA_ENOSPACE, "pool too small: %lld + %d > %lld rows", (long long)pool_len, seg_len,
                (long long)pool_cap);
  if (!do_tail && !do_pool) return ok();
  if (k == nullptr || v == nullptr) return fail(SA_EINVAL, "k and v must not be NULL");
  auto bad_stride = [&](int64_t s) { return s < 0 || (s * esz) % 16 != 0; };
  if (!aligned16(k) || !aligned16(v) || bad_stride(kv_head_stride) || bad_stride(kv_row_stride))
    return fail(SA_EINVAL, "k and v must be 16-byte aligned with strides that are multiples of 16 bytes");
  if (do_tail && (tail_k == nullptr || tail_v == nullptr || !aligned16(tail_k) || !aligned16(tail_v) ||
                  bad_stride(tail_head_stride) || bad_stride(tail_row_stride) || tail_row_stride < d))
    return fail(SA_EINVAL, "tail buffers: 16-byte aligned, strides multiples of 16 bytes, row stride >= d");
  if (do_pool && (pool_k == nullptr || pool_v == nullptr || !aligned16(pool_k) || !aligned16(pool_v) ||
                  bad_stride(pool_head_stride) || bad_stride(pool_row_stride) || pool_row_stride < d))
    return fail(SA_EINVAL, "pool buffers: 16-byte aligned, strides multiples of 16 bytes, row stride >= d");
  const int64_t row_bytes = (int64_t)d * esz;
  std::vector<Span> spans;
  if (do_tail) {
    const int64_t r0 = (int64_t)prefix_len + seg_len - keep;
    add_spans(spans, k, n_local, kv_head_stride, kv_row_stride, r0, keep, row_bytes, esz, false);
    add_spans(spans, v, n_local, kv_head_stride, kv_row_stride, r0, keep, row_bytes, esz, false);
    add_spans(spans, tail_k, n_local, tail_head_stride, tail_row_stride, 0, keep, row_bytes, esz, true);
    add_spans(spans, tail_v, n_local, tail_head_stride, tail_row_stride, 0, keep, row_bytes, esz, true);
  }
  if (do_pool) {
    const char* kl = static_cast<const char*>(k) + (int64_t)n_local * kv_head_stride * esz;
    const char* vl = static_cast<const char*>(v) + (int64_t)n_local * kv_head_stride * esz;
    add_spans(spans, kl, n_long, kv_head_stride, kv_row_stride, prefix_len, seg_len, row_bytes, esz, false);
    add_spans(spans, vl, n_long, kv_head_stride, kv_row_stride, prefix_len, seg_len, row_bytes, esz, false);
    add_spans(spans, pool_k, n_long, pool_head_stride, pool_row_stride, pool_len, seg_len, row_bytes, esz, true);
    add_spans(spans, pool_v, n_long, pool_head_stride, pool_row_stride, pool_len, seg_len, row_bytes, esz, true);
  }
  if (dst_overlap(spans)) return fail(SA_EINVAL, "a destination of the carry overlaps a source or another destination");
  int r = check_device();
  if (r != SA_OK) return r;
  sa::CarryDesc c;
  c.esz = esz;
  c.n_local = n_local;
  c.n_pool_heads = do_pool ? n_long : 0;
  c.d = d;
  c.prefix_len = prefix_len;
  c.seg_len = seg_len;
  c.keep = do_tail ? keep : 0;
  c.k = k;
  c.v = v;
  c.kv_hs = kv_head_stride;
  c.kv_rs = kv_row_stride;
  c.tail_k = tail_k;
  c.tail_v = tail_v;
  c.t_hs = tail_head_stride;
  c.t_rs = tail_row_stride;
  c.pool_k = pool_k;
  c.pool_v = pool_v;
  c.p_hs = pool_head_stride;
  c.p_rs = pool_row_stride;
  c.pool_len = pool_len;
  hipError_t e = sa::launch_carry(c, stream);
  if (e != hipSuccess) return fail(SA_EHIP, "carry launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// The cache geometry a kernel sees: for LAMBDA, Initial = the starting span,
// Local = the window of L_pretrain + 1 slots, no Separator or Past part.
sa_stream_cfg_t stream_geometry(const sa_stream_cfg_t& c) {
  sa_stream_cfg_t g = c;
  if (c.kind == SA_MASK_LAMBDA) {
    g.s = 0;
    g.w = c.L_pretrain + 1;
    g.c = c.a + g.w;
  }
  return g;
}

int check_stream_cfg(const sa_stream_cfg_t* c) {
  if (c == nullptr) return fail(SA_EINVAL, "cfg is NULL");
  if (c->kind != SA_MASK_SEPLLM && c->kind != SA_MASK_LAMBDA)
    return fail(SA_EINVAL, "streaming decode kind must be SEPLLM or LAMBDA");
  if (c->kind == SA_MASK_LAMBDA) {
    if (c->a < 0 || c->L_pretrain < 0 || (int64_t)c->a + c->L_pretrain + 1 > 65536)
      return fail(SA_EINVAL, "LAMBDA decode needs n_starting >= 0, L_pretrain >= 0, n_starting + L_pretrain + 1 <= 65536");
    if (c->batch < 1 || c->h_q < 1 || c->h_kv < 1 || c->h_q % c->h_kv != 0)
      return fail(SA_EINVAL, "need batch, h_kv >= 1 and h_q a multiple of h_kv");
    if (c->h_q / c->h_kv > 8) return fail(SA_EUNSUPPORTED, "at most 8 query heads per kv head");
    if (c->d != 128) return fail(SA_EUNSUPPORTED, "streaming decode supports d = 128");
    if (c->rope != SA_ROPE_NONE && c->rope != SA_ROPE_HALF) return fail(SA_EINVAL, "unknown rope mode %d", c->rope);
    if (c->rope == SA_ROPE_HALF && !(std::isfinite(c->rope_base) && c->rope_base > 1.0f))
      return fail(SA_EINVAL, "rope_base must be finite and > 1");
    if (!(std::isfinite(c->scale) && c->scale > 0.0f)) return fail(SA_EINVAL, "scale must be finite and > 0");
    return SA_OK;
  }
  if (c->batch < 1 || c->h_q < 1 || c->h_kv < 1 || c->h_q % c->h_kv != 0)
    return fail(SA_EINVAL, "need batch, h_kv >= 1 and h_q a multiple of h_kv");
  if (c->h_q / c->h_kv > 8) return fail(SA_EUNSUPPORTED, "at most 8 query heads per kv head");
  if (c->d != 128) return fail(SA_EUNSUPPORTED, "streaming decode supports d = 128");
  if (c->a < 0 || c->s < 1 || c->w < 1 || (int64_t)c->c <= (int64_t)c->a + c->s + c->w)
    return fail(SA_EINVAL, "need a >= 0, s >= 1, w >= 1 and c > a + s + w");
  if (c->c > 4096) return fail(SA_EUNSUPPORTED, "c must be <= 4096");
  if (c->rope != SA_ROPE_NONE && c->rope != SA_ROPE_HALF) return fail(SA_EINVAL, "unknown rope mode %d", c->rope);
  if (c->rope == SA_ROPE_HALF && !(std::isfinite(c->rope_base) && c->rope_base > 1.0f))
    return fail(SA_EINVAL, "rope_base must be finite and > 1");
  if (!(std::isfinite(c->scale) && c->scale > 0.0f)) return fail(SA_EINVAL, "scale must be finite and > 0");
  return SA_OK;
}

}  // namespace

extern "C" {

int sa_stream_state_bytes(const sa_stream_cfg_t* cfg, size_t* bytes) {
  int r = check_stream_cfg(cfg);
  if (r != SA_OK) return r;
  if (bytes == nullptr) return fail(SA_EINVAL, "bytes is NULL");
  *bytes = (size_t)sa::stream_layout(stream_geometry(*cfg)).total;
  return ok();
}

int sa_decode_workspace_bytes(const sa_stream_cfg_t* cfg, size_t* bytes) {
  int r = check_stream_cfg(cfg);
  if (r != SA_OK) return r;
  if (bytes == nullptr) return fail(SA_EINVAL, "bytes is NULL");
  *bytes = (size_t)sa::stream_layout(stream_geometry(*cfg)).ws_total;
  return ok();
}

int sa_stream_layout(const sa_stream_cfg_t* cfg, int64_t offsets[5]) {
  int r = check_stream_cfg(cfg);
  if (r != SA_OK) return r;
  if (offsets == nullptr) return fail(SA_EINVAL, "offsets is NULL");
  const sa::StreamLayout L = sa::stream_layout(stream_geometry(*cfg));
  offsets[0] = L.k;
  offsets[1] = L.v;
  offsets[2] = L.pos;
  offsets[3] = L.flag;
  offsets[4] = L.ctrl;
  return ok();
}

int sparse_attn_stream_reset(const sa_stream_cfg_t* cfg, void* state, size_t state_bytes, hipStream_t stream) {
  int r = check_stream_cfg(cfg);
  if (r != SA_OK) return r;
  const sa_stream_cfg_t geo = stream_geometry(*cfg);
  const sa::StreamLayout L = sa::stream_layout(geo);
  if (state == nullptr || !aligned16(state)) return fail(SA_EINVAL, "state must be a 16-byte aligned device pointer");
  if (state_bytes < (size_t)L.total)
    return fail(SA_ENOSPACE, "state too small: %zu < %lld bytes", state_bytes, (long long)L.total);
  if ((r = check_device()) != SA_OK) return r;
  hipError_t e = sa::launch_stream_reset(geo, state, stream);
  if (e != hipSuccess) return fail(SA_EHIP, "reset launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// Checks shared by the two decode-step entry points (everything but the
// workspace).
int check_decode(const sa_stream_cfg_t* cfg, const void* state, size_t state_bytes, const void* q,
                 const void* k, const void* v, const uint8_t* is_sep, const void* o) {
  int r = check_stream_cfg(cfg);
  if (r != SA_OK) return r;
  const sa::StreamLayout L = sa::stream_layout(stream_geometry(*cfg));
  if (state == nullptr || !aligned16(state)) return fail(SA_EINVAL, "state must be a 16-byte aligned device pointer");
  if (state_bytes < (size_t)L.total)
    return fail(SA_ENOSPACE, "state too small: %zu < %lld bytes", state_bytes, (long long)L.total);
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr ||
      (is_sep == nullptr && cfg->kind == SA_MASK_SEPLLM))
    return fail(SA_EINVAL, "q, k, v, o (and is_sep for SEPLLM) must not be NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SA_EINVAL, "q, k, v and o must be 16-byte aligned");
  return SA_OK;
}

int launch_decode(const sa_stream_cfg_t* cfg, void* state, const void* q, const void* k, const void* v,
                  const uint8_t* is_sep, void* o, float* lse, void* ws, hipStream_t stream) {
  sa::ThetaTable th;
  memset(&th, 0, sizeof(th));
  if (cfg->rope == SA_ROPE_HALF)
    for (int c = 0; c < cfg->d / 2; ++c) th.th[c] = std::pow((double)cfg->rope_base, -2.0 * c / cfg->d);
  hipError_t e = sa::launch_decode_step(stream_geometry(*cfg), state, q, k, v, is_sep, o, lse, ws, th, stream);
  if (e != hipSuccess) return fail(SA_EHIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int sparse_attn_decode_step(const sa_stream_cfg_t* cfg, void* state, size_t state_bytes, const void* q,
                            const void* k, const void* v, const uint8_t* is_sep, void* o, float* lse, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  int r = check_decode(cfg, state, state_bytes, q, k, v, is_sep, o);
  if (r != SA_OK) return r;
  const sa::StreamLayout L = sa::stream_layout(stream_geometry(*cfg));
  if (ws == nullptr || !aligned16(ws)) return fail(SA_EINVAL, "workspace must be a 16-byte aligned device pointer");
  if (ws_bytes < (size_t)L.ws_total)
    return fail(SA_ENOSPACE, "workspace too small: %zu < %lld bytes", ws_bytes, (long long)L.ws_total);
  if ((r = check_device()) != SA_OK) return r;
  return launch_decode(cfg, state, q, k, v, is_sep, o, lse, ws, stream);
}

int sparse_attn_decode_step_static(const sa_stream_cfg_t* cfg, void* state, size_t state_bytes, const void* q,
                                   const void* k, const void* v, const uint8_t* is_sep, void* o, float* lse,
                                   hipStream_t stream) {
  int r = check_decode(cfg, state, state_bytes, q, k, v, is_sep, o);
  if (r != SA_OK) return r;
  const sa::StreamLayout L = sa::stream_layout(stream_geometry(*cfg));
  if (L.ws_total > (int64_t)SA_DECODE_STATIC_SCRATCH_BYTES)
    return fail(SA_ENOSPACE,
                "the step needs %lld bytes of scratch, more than the library's static %d bytes "
                "(use sparse_attn_decode_step with a workspace)",
                (long long)L.ws_total, (int)SA_DECODE_STATIC_SCRATCH_BYTES);
  if ((r = check_device()) != SA_OK) return r;
  void* ws = nullptr;
  hipError_t e = sa::decode_static_scratch(&ws);
  if (e != hipSuccess) return fail(SA_EHIP, "static scratch lookup: %s", hipGetErrorString(e));
  return launch_decode(cfg, state, q, k, v, is_sep, o, lse, ws, stream);
}

int sparse_attn_topk_middle(const sa_mask_t* m, const sa_fwd_args_t* a, int32_t k_mid, int32_t* sel,
                            float* score, hipStream_t stream) {
  int r = check_mask(m);
  if (r != SA_OK) return r;
  if ((r = check_args(m, a)) != SA_OK) return r;
  if (m->kind != SA_MASK_LAMBDA) return fail(SA_EINVAL, "top-k middle tokens apply to the LAMBDA mask");
  if (a->dtype != SA_BF16 || a->d != 128 || a->rope == SA_ALIBI)
    return fail(SA_EUNSUPPORTED, "top-k middle tokens: bf16, d = 128, RoPE or none");
  if (k_mid < 1 || k_mid > SA_TOPK_MIDDLE_MAX)
    return fail(SA_EINVAL, "k_mid must be in [1, %d] (got %d)", (int)SA_TOPK_MIDDLE_MAX, k_mid);
  if (a->lse == nullptr || sel == nullptr || score == nullptr)
    return fail(SA_EINVAL, "lse, sel and score must not be NULL");
  if ((r = check_device()) != SA_OK) return r;
  hipError_t e = sa::launch_topk_middle(*m, *a, k_mid, sel, score, stream);
  if (e != hipSuccess) return fail(SA_EHIP, "top-k middle launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

