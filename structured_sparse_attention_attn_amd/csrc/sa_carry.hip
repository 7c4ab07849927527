// Segment carry: the state one segment hands to the next (segmented-execution
// page, overall framework and key designs 2-3).  After a segment's forward,
// each local head keeps its latest `keep` keys and values (the tail the next
// segment attends to), and each long-range head's segment rows join the
// detached retrieval pool.  Both are plain row copies, so one launch moves
// them all: 16-byte pieces, four per thread, every load issued before the
// first store.
#include "sa_common.h"

namespace sa {
namespace {

struct CarryArgs {
  const char* k;  // [H, P+S, d]
  const char* v;
  int64_t kv_hs, kv_rs;  // bytes
  char* tail_k;   // [n_local, keep, d]
  char* tail_v;
  int64_t t_hs, t_rs;
  char* pool_k;   // [H - n_local, pool_cap, d]
  char* pool_v;
  int64_t p_hs, p_rs;
  int n_local, n_long;
  int src_tail_row0;  // first source row of the tail: P + S - keep
  int keep;           // tail rows
  int src_pool_row0;  // first source row of the segment: P
  int seg;            // segment rows S
  int64_t pool_row0;  // first pool row written: pool_len
  int pieces;         // 16-byte pieces per row
  int64_t n_tail;     // pieces of one tensor's tail copy: n_local * keep * pieces
  int64_t n_total;    // n_tail + n_long * seg * pieces
};

constexpr int CARRY_UNROLL = 4;

__global__ __launch_bounds__(256) void carry_rows(CarryArgs p) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t g0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  // blockIdx.y: 0 = keys, 1 = values
  const char* src = blockIdx.y ? p.v : p.k;
  char* tail = blockIdx.y ? p.tail_v : p.tail_k;
  char* pool = blockIdx.y ? p.pool_v : p.pool_k;
  uint4 x[CARRY_UNROLL];
  char* dst[CARRY_UNROLL];
#pragma unroll
  for (int u = 0; u < CARRY_UNROLL; ++u) {
    const int64_t g = g0 + u * stride;
    dst[u] = nullptr;
    if (g >= p.n_total) continue;
    int64_t piece, row, head;
    const char* s;
    if (g < p.n_tail) {
      piece = g % p.pieces;
      row = (g / p.pieces) % p.keep;
      head = g / ((int64_t)p.pieces * p.keep);
      s = src + head * p.kv_hs + (p.src_tail_row0 + row) * p.kv_rs + piece * 16;
      dst[u] = tail + head * p.t_hs + row * p.t_rs + piece * 16;
    } else {
      const int64_t h = g - p.n_tail;
      piece = h % p.pieces;
      row = (h / p.pieces) % p.seg;
      head = h / ((int64_t)p.pieces * p.seg);
      s = src + (p.n_local + head) * p.kv_hs + (p.src_pool_row0 + row) * p.kv_rs + piece * 16;
      dst[u] = pool + head * p.p_hs + (p.pool_row0 + row) * p.p_rs + piece * 16;
    }
    x[u] = *reinterpret_cast<const uint4*>(s);
  }
#pragma unroll
  for (int u = 0; u < CARRY_UNROLL; ++u)
    if (dst[u] != nullptr) *reinterpret_cast<uint4*>(dst[u]) = x[u];
}

}  // namespace

hipError_t launch_carry(const CarryDesc& c, hipStream_t s) {
  CarryArgs p;
  memset(&p, 0, sizeof(p));
  p.k = static_cast<const char*>(c.k);
  p.v = static_cast<const char*>(c.v);
  p.kv_hs = c.kv_hs * c.esz;
  p.kv_rs = c.kv_rs * c.esz;
  p.tail_k = static_cast<char*>(c.tail_k);
  p.tail_v = static_cast<char*>(c.tail_v);
  p.t_hs = c.t_hs * c.esz;
  p.t_rs = c.t_rs * c.esz;
  p.pool_k = static_cast<char*>(c.pool_k);
  p.pool_v = static_cast<char*>(c.pool_v);
  p.p_hs = c.p_hs * c.esz;
  p.p_rs = c.p_rs * c.esz;
  p.n_local = c.n_local;
  p.n_long = c.n_pool_heads;
  p.keep = c.keep;
  p.src_tail_row0 = c.prefix_len + c.seg_len - c.keep;
  p.seg = c.seg_len;
  p.src_pool_row0 = c.prefix_len;
  p.pool_row0 = c.pool_len;
  p.pieces = c.d * c.esz / 16;
  p.n_tail = (int64_t)p.n_local * p.keep * p.pieces;
  p.n_total = p.n_tail + (int64_t)p.n_long * p.seg * p.pieces;
  if (p.n_total == 0) return hipSuccess;
  const int64_t wgs = ceil_div(ceil_div(p.n_total, CARRY_UNROLL), 256);
  hipLaunchKernelGGL(carry_rows, dim3((unsigned)wgs, 2), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace sa
