// Plan kernels: per 128-query tile, the 64-key blocks that hold a visible pair
// and, for SepLLM, the compacted separator list.
//
// Key sets follow the pages' definitions: SepLLM page part 5 item 2 (initial
// a, separators before i, w neighbours), LM-Infinite page section "method"
// (Lambda mask j < n_starting or i-j <= L_pretrain), segmented-execution page
// method / overall framework (prefix fully visible, segment causal).  The
// kernels derive each tile's block list in closed form; the oracle derives it
// by evaluating the predicates pair by pair, and the two must agree exactly.
#include "sa_common.h"

namespace sa {
namespace {

struct PlanArgs {
  int kind, n_q, n_k, a, w, n_s, L, P;
  const uint8_t* sep;
  int n_tiles, n_blocks, g0;
  int* tile_ptr;
  int* items;
  int* sep_count;
  int* sep_idx;
  unsigned long long* sep_bits;
  int* blk_sep;
  sa_plan_header_t* hdr;
  sa_plan_header_t lay;
};

constexpr int FIN_THREADS = 1024;

// One wave per 64-key block: separator bits by a wavefront ballot, and the
// block's separator count (only blocks at or after g0 count toward the list).
__global__ __launch_bounds__(256) void plan_sep_blocks(PlanArgs p) {
  const int lane = threadIdx.x & 63;
  const int blk = (int)((blockIdx.x * 256u + threadIdx.x) >> 6);
  if (blk >= p.n_blocks) return;
  const int j = blk * BK + lane;
  const bool f = p.kind == SA_MASK_SEPLLM && p.sep != nullptr && j < p.n_k && p.sep[j] != 0;
  const unsigned long long word = __ballot(f);
  if (lane == 0) {
    p.sep_bits[blk] = word;
    p.blk_sep[blk] = (blk * BK >= p.g0) ? __popcll(word) : 0;
  }
}

// Exclusive scan over the 1024 threads of the block.  Returns the exclusive
// prefix of v and the block total in *total.
__device__ int block_excl_scan(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wave_tot[wid] = x;
  __syncthreads();
  if (wid == 0) {
    const int nw = FIN_THREADS / 64;
    int t = lane < nw ? wave_tot[lane] : 0;
    int s = t;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(s, o);
      if (lane >= o) s += y;
    }
    if (lane < nw) wave_tot[16 + lane] = s - t;  // exclusive wave offsets
    if (lane == nw - 1) wave_tot[32] = s;
  }
  __syncthreads();
  const int r = x - v + wave_tot[16 + wid];
  *total = wave_tot[32];
  __syncthreads();
  return r;
}

// Tile t visits blocks [0, lo_end) and [hi0, hi1] (lo_end <= hi0 <= hi1).
struct TileRange {
  int q0, q1, lo_end, hi0, hi1;
};

__device__ TileRange tile_range(const PlanArgs& p, int t) {
  TileRange r;
  r.q0 = t * TQ;
  r.q1 = min(p.n_q, r.q0 + TQ) - 1;
  if (p.kind == SA_MASK_SEGMENT) {
    r.lo_end = 0;
    r.hi0 = 0;
    r.hi1 = min(p.n_blocks - 1, (p.P + r.q1) / BK);
    return r;
  }
  int nsb, win_lo;
  if (p.kind == SA_MASK_SEPLLM) {
    nsb = (p.a + BK - 1) / BK;
    win_lo = max(0, r.q0 - p.w + 1);   // oldest key inside some query's window
  } else {
    nsb = (p.n_s + BK - 1) / BK;
    win_lo = max(0, r.q0 - p.L);
  }
  r.hi0 = win_lo / BK;
  r.hi1 = r.q1 / BK;
  r.lo_end = min(nsb, r.hi0);
  return r;
}

__device__ unsigned long long low_bits(int n) {  // bits r < n set, n clamped to [0, 64]
  if (n <= 0) return 0ull;
  if (n >= 64) return ~0ull;
  return (1ull << n) - 1ull;
}

__device__ int item_flags(const PlanArgs& p, const TileRange& r, int b) {
  const int k0 = b * BK;
  int fl = 0;
  const bool whole = k0 + BK <= p.n_k;
  if (p.kind == SA_MASK_SEGMENT) {
    if (whole && k0 + BK - 1 <= p.P + r.q0) fl |= SA_ITEM_FULL;
    return fl;
  }
  if (p.kind == SA_MASK_SEPLLM) {
    // key j is visible to every query of the tile iff j <= q0 and
    // (j < a or q1 - j < w or sep[j])
    const unsigned long long sink = low_bits(p.a - k0);
    const unsigned long long win = ~low_bits(r.q1 - p.w + 1 - k0);
    const unsigned long long all = sink | win | p.sep_bits[b];
    if (whole && k0 + BK - 1 <= r.q0 && all == ~0ull) fl |= SA_ITEM_FULL;
    return fl;
  }
  // LAMBDA: visible to all iff j <= q0 and (j < n_s or q1 - j <= L)
  const unsigned long long sink = low_bits(p.n_s - k0);
  const unsigned long long win = ~low_bits(r.q1 - p.L - k0);
  if (whole && k0 + BK - 1 <= r.q0 && (sink | win) == ~0ull) fl |= SA_ITEM_FULL;
  // some visible pair at distance > L: the block's first key is a starting
  // token seen by the tile's last query from farther than L
  if (k0 < p.n_s && r.q1 - k0 > p.L) fl |= SA_ITEM_CAPPED;
  return fl;
}

// One workgroup: scan of the per-block separator counts, the per-tile item
// offsets (CSR) and separator counts, and the header.
__global__ __launch_bounds__(FIN_THREADS) void plan_finish(PlanArgs p) {
  __shared__ int wave_tot[40];
  const int tid = threadIdx.x;
  int total;
  // 1. blk_sep: exclusive prefix of the per-block counts, plus the grand total
  //    (no separator flags: plan_sep_blocks did not run, every bit and count
  //    is zero)
  int carry = 0;
  if (p.sep == nullptr) {
    for (int b = tid; b < p.n_blocks; b += FIN_THREADS) {
      p.sep_bits[b] = 0ull;
      p.blk_sep[b] = 0;
    }
  } else {
    for (int base = 0; base < p.n_blocks; base += FIN_THREADS) {
      const int b = base + tid;
      const int v = b < p.n_blocks ? p.blk_sep[b] : 0;
      const int ex = block_excl_scan(v, wave_tot, &total);
      if (b < p.n_blocks) p.blk_sep[b] = carry + ex;
      carry += total;
    }
  }
  const int n_sep = carry;
  if (tid == 0) p.blk_sep[p.n_blocks] = n_sep;
  __syncthreads();
  // 2. tiles
  carry = 0;
  for (int base = 0; base < p.n_tiles; base += FIN_THREADS) {
    const int t = base + tid;
    TileRange r;
    int cnt = 0;
    if (t < p.n_tiles) {
      r = tile_range(p, t);
      cnt = r.lo_end + (r.hi1 - r.hi0 + 1);
    }
    const int ex = block_excl_scan(cnt, wave_tot, &total);
    if (t < p.n_tiles) {
      p.tile_ptr[t] = carry + ex;  // the items themselves: plan_lists
      int sc = 0;
      if (p.kind == SA_MASK_SEPLLM) {
        const int gh = r.hi0 * BK;  // first key of the first window block
        if (gh > p.g0) sc = min(p.blk_sep[r.hi0], p.lay.cap_sep);  // a broken sep_max bound: clamped
      }
      p.sep_count[t] = sc;
    }
    carry += total;
  }
  if (tid == 0) {
    p.tile_ptr[p.n_tiles] = carry;
    sa_plan_header_t h = p.lay;
    h.n_items = carry;
    h.n_sep = n_sep;
    *p.hdr = h;
  }
}

// Two jobs in one launch, both after plan_finish:
//  * work groups [0, n_item_wg): one wave per tile writes the tile's items,
//    leading blocks 0 .. lo_end-1 and then one run of consecutive blocks hi0 ..
//    hi1, a lane per item (the backward's key-major kernel finds a block's
//    item from this layout);
//  * the rest (SepLLM): one wave per block at or after g0 writes the block's
//    separator positions at their rank (block prefix + popcount of the lower
//    lanes' bits).
__global__ __launch_bounds__(256) void plan_lists(PlanArgs p, int n_item_wg) {
  const int lane = threadIdx.x & 63;
  if ((int)blockIdx.x < n_item_wg) {
    const int t = (int)((blockIdx.x * 256u + threadIdx.x) >> 6);
    if (t >= p.n_tiles) return;
    const TileRange r = tile_range(p, t);
    const int start = p.tile_ptr[t];
    const int cnt = r.lo_end + (r.hi1 - r.hi0 + 1);
    for (int i = lane; i < cnt; i += 64) {
      const int b = i < r.lo_end ? i : r.hi0 + (i - r.lo_end);
      p.items[start + i] = b | (item_flags(p, r, b) << 24);
    }
    return;
  }
  if (p.sep == nullptr) return;
  const int blk = (int)(((blockIdx.x - n_item_wg) * 256u + threadIdx.x) >> 6);
  if (blk >= p.n_blocks || blk * BK < p.g0) return;
  const unsigned long long word = p.sep_bits[blk];
  if ((word >> lane) & 1ull) {
    const int rank = p.blk_sep[blk] + __popcll(word & low_bits(lane));
    if (rank < p.lay.cap_sep) p.sep_idx[rank] = blk * BK + lane;
  }
}

}  // namespace

hipError_t launch_plan(const sa_mask_t& m, const sa_plan_header_t& lay, void* plan,
                       hipStream_t s) {
  char* base = static_cast<char*>(plan);
  PlanArgs p;
  p.kind = m.kind;
  p.n_q = m.n_q;
  p.n_k = m.n_k;
  p.a = m.a;
  p.w = m.w;
  p.n_s = m.n_starting;
  p.L = m.L_pretrain;
  p.P = m.prefix_len;
  p.sep = m.kind == SA_MASK_SEPLLM ? m.sep : nullptr;
  p.n_tiles = lay.n_tiles;
  p.n_blocks = lay.n_blocks;
  p.g0 = lay.g0;
  p.tile_ptr = reinterpret_cast<int*>(base + lay.off_tile_ptr);
  p.items = reinterpret_cast<int*>(base + lay.off_items);
  p.sep_count = reinterpret_cast<int*>(base + lay.off_sep_count);
  p.sep_idx = reinterpret_cast<int*>(base + lay.off_sep_idx);
  p.sep_bits = reinterpret_cast<unsigned long long*>(base + lay.off_sep_bits);
  p.blk_sep = reinterpret_cast<int*>(base + lay.off_blk_sep);
  p.hdr = reinterpret_cast<sa_plan_header_t*>(base);
  p.lay = lay;
  const unsigned wg = (unsigned)ceil_div(lay.n_blocks, 4);
  hipError_t e;
  if (p.sep != nullptr) {  // separator flags to read (otherwise plan_finish zeroes the bits)
    hipLaunchKernelGGL(plan_sep_blocks, dim3(wg), dim3(256), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(plan_finish, dim3(1), dim3(FIN_THREADS), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_item_wg = (int)ceil_div(lay.n_tiles, 4);
  const unsigned lists_wg = (unsigned)(n_item_wg + (p.sep != nullptr ? (int)wg : 0));
  hipLaunchKernelGGL(plan_lists, dim3(lists_wg), dim3(256), 0, s, p, n_item_wg);
  return hipGetLastError();
}

}  // namespace sa
