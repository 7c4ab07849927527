// Internal declarations shared by the HIP sources of libsparse_attn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "sparse_attn.h"

namespace sa {

constexpr int TQ = SA_TQ;    // queries per tile
constexpr int BK = SA_BK;    // keys per block
constexpr int MAX_THETA = 64;  // d/2 for d <= 128

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t align_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Section offsets and capacities of the plan; depends on the mask scalars only.
inline sa_plan_header_t plan_layout(const sa_mask_t& m) {
  sa_plan_header_t h;
  memset(&h, 0, sizeof(h));
  h.magic = 0x31504153u;
  h.version = 1;
  h.kind = m.kind;
  h.tq = TQ;
  h.bk = BK;
  h.n_q = m.n_q;
  h.n_k = m.n_k;
  h.n_tiles = (int32_t)ceil_div(m.n_q, TQ);
  h.n_blocks = (int32_t)ceil_div(m.n_k, BK);
  int64_t per_tile;
  if (m.kind == SA_MASK_SEPLLM) {
    per_tile = ceil_div(m.a, BK) + ceil_div((int64_t)m.w + TQ - 1, BK) + 2;
    h.g0 = (int32_t)(BK * ceil_div(m.a, BK));
  } else if (m.kind == SA_MASK_LAMBDA) {
    per_tile = ceil_div(m.n_starting, BK) + ceil_div((int64_t)m.L_pretrain + TQ, BK) + 2;
  } else {
    per_tile = h.n_blocks;
  }
  if (per_tile > h.n_blocks) per_tile = h.n_blocks;
  h.max_items_per_tile = (int32_t)per_tile;
  h.cap_items = (int32_t)(per_tile * h.n_tiles);
  h.cap_sep = 0;
  if (m.kind == SA_MASK_SEPLLM) h.cap_sep = (m.sep_max > 0 && m.sep_max < m.n_k) ? m.sep_max : m.n_k;
  int64_t off = 256;  // header
  h.off_tile_ptr = off;  off = align_up(off + 4 * (int64_t)(h.n_tiles + 1), 256);
  h.off_items = off;     off = align_up(off + 4 * (int64_t)h.cap_items, 256);
  h.off_sep_count = off; off = align_up(off + 4 * (int64_t)h.n_tiles, 256);
  h.off_sep_idx = off;   off = align_up(off + 4 * (int64_t)h.cap_sep, 256);
  h.off_sep_bits = off;  off = align_up(off + 8 * (int64_t)h.n_blocks, 256);
  h.off_blk_sep = off;   off = align_up(off + 4 * (int64_t)(h.n_blocks + 1), 256);
  h.total_bytes = off;
  return h;
}

// ---------------------------------------------------------------------------
// Launchers (host functions defined next to their kernels).  They assume the
// arguments were validated by the C ABI layer.
// ---------------------------------------------------------------------------

hipError_t launch_plan(const sa_mask_t& m, const sa_plan_header_t& lay, void* plan, hipStream_t s);

// RoPE stage workspace description (element offsets from the workspace base).
struct RopeOut {
  void* qrot;  // [B, h_q, n_q, d] contiguous, or nullptr when rope is off
  void* krot;  // [B, h_kv, n_k, d] contiguous, or nullptr when rope is off
  void* ksep;  // [B, h_kv, cap_sep_rows, d] gathered separator keys (rotated)
  void* vsep;  // [B, h_kv, cap_sep_rows, d] gathered separator values
  int64_t sep_rows;  // rows per head in ksep / vsep (multiple of BK)
  void* kcap;  // [B, h_kv, cap_rows, d]: R(-L) k_j for j < n_cap (LM-Infinite)
  int64_t cap_rows;  // rows per head in kcap (multiple of BK)
  int n_cap;
};

struct ThetaTable {
  double th[MAX_THETA];
};

hipError_t launch_rope(const sa_mask_t& m, const sa_plan_header_t& lay, const void* plan,
                       const sa_fwd_args_t& a, const ThetaTable& theta, const RopeOut& ro,
                       hipStream_t s);

hipError_t launch_fwd(const sa_mask_t& m, const sa_plan_header_t& lay, const void* plan,
                      const sa_fwd_args_t& a, const RopeOut& ro, hipStream_t s);

hipError_t launch_topk(int dtype, int n_heads, int pool_len, int d, int k, const void* q,
                       int64_t q_hs, const void* pool_k, const void* pool_v, int64_t p_hs,
                       int64_t p_rs, int32_t* idx, double* score, void* pref_k, void* pref_v,
                       int64_t r_hs, int64_t r_rs, void* ws, hipStream_t s);

size_t topk_workspace_bytes(int n_heads, int pool_len);

// Segment carry: strides in elements, sizes validated by the caller.
struct CarryDesc {
  int esz, n_local, n_pool_heads, d, prefix_len, seg_len, keep;  // keep: tail rows (0: none)
  const void* k;
  const void* v;
  int64_t kv_hs, kv_rs;
  void* tail_k;
  void* tail_v;
  int64_t t_hs, t_rs;
  void* pool_k;
  void* pool_v;
  int64_t p_hs, p_rs;
  int64_t pool_len;
};

hipError_t launch_carry(const CarryDesc& c, hipStream_t s);

// Backward workspace sections (fp32), see sparse_attn_bwd.
struct BwdWs {
  float* D;        // [B, h_q, n_q]
  float* dq_acc;   // [B, h_q, n_q, d]
  float* dq_cap;   // [B, h_q, n_q, d] or null
  float* dk_acc;   // [B, h_kv, n_k, d]
  float* dv_acc;
  float* dksep;    // [B, h_kv, sep_rows, d] or null
  float* dvsep;
  float* dkcap;    // [B, h_kv, cap_rows, d] or null
  float* dvcap;
};

// Streaming decode state and workspace (byte offsets).
struct StreamLayout {
  int64_t k, v, pos, flag, ctrl, total;
  int n_split;
  int64_t ws_qrot, ws_capl, ws_part, ws_total;
};

StreamLayout stream_layout(const sa_stream_cfg_t& cfg);
hipError_t launch_stream_reset(const sa_stream_cfg_t& cfg, void* state, hipStream_t s);
hipError_t launch_decode_step(const sa_stream_cfg_t& cfg, void* state, const void* q, const void* k,
                              const void* v, const uint8_t* is_sep, void* o, float* lse, void* ws,
                              const ThetaTable& theta, hipStream_t s);

// The no-allocation decode step's scratch array on the current device (its
// device address, looked up once per device).
hipError_t decode_static_scratch(void** out);

hipError_t launch_topk_middle(const sa_mask_t& m, const sa_fwd_args_t& a, int kmid, int32_t* sel, float* score,
                              hipStream_t s);

hipError_t launch_bwd(const sa_mask_t& m, const sa_plan_header_t& lay, const void* plan,
                      const sa_fwd_args_t& a, const sa_bwd_args_t& g, const RopeOut& ro,
                      const BwdWs& w, const ThetaTable& theta, hipStream_t s);

}  // namespace sa
