// Forward-only top-k retrieval of the prefix (segmented-execution page, key
// design 3: before the next segment the segment-end query selects R keys of a
// detached read-only pool for the long-range heads).
//
// 1. topk_score: s_j = fp64 fma chain over c = 0..d-1 for every pool key
//    (each bf16/fp32 product is exact in fp64, so the chain equals plain
//    multiply-then-add in the same order); stored as an order-preserving
//    64-bit key (+0 and -0 share one key).  Rows reach LDS by coalesced loads.
// 2. topk_select: one work group per head, its keys held in registers; radix
//    select of the k-th largest key T by 12-bit digits, stopping as soon as
//    the threshold bin holds exactly the keys still wanted; one block scan
//    then gives every selected index its output slot, so idx comes out in
//    ascending pool order with ties at T taken from the lowest indices.
// 3. topk_gather: copies the selected pool K/V rows into the prefix rows.
#include "sa_common.h"

namespace sa {
namespace {

constexpr int SEL_THREADS = 1024;

__device__ inline unsigned long long order_key(double s) {
  s = s + 0.0;  // -0 -> +0
  const unsigned long long b = (unsigned long long)__double_as_longlong(s);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ inline double key_value(unsigned long long k) {
  const unsigned long long b = (k >> 63) ? (k & 0x7fffffffffffffffull) : ~k;
  return __longlong_as_double((long long)b);
}

template <typename T>
__device__ inline double elem(const T* p, int c);
template <>
__device__ inline double elem<unsigned short>(const unsigned short* p, int c) {
  return (double)__uint_as_float(((unsigned)p[c]) << 16);
}
template <>
__device__ inline double elem<float>(const float* p, int c) {
  return (double)p[c];
}

// One work group scores ROWS = 256 consecutive pool keys of one head.  The
// rows are staged in LDS with coalesced 16-byte loads (a row's chunks come
// from consecutive lanes; rows padded by 16 bytes, so each thread's later
// reads of its own row are bank-conflict free), then thread t runs the fp64
// chain of key t in c order and stores its order-preserving key.
constexpr int SCORE_ROWS = 256;

template <typename T, int D>
__global__ __launch_bounds__(256) void topk_score(const T* q, int64_t q_hs, const T* pool,
                                                  int64_t p_hs, int64_t p_rs, int n,
                                                  unsigned long long* keys) {
  constexpr int ROW = D * (int)sizeof(T);  // bytes per row
  constexpr int CPR = ROW / 16;            // 16-byte chunks per row
  constexpr int PITCH = ROW + 16;
  __shared__ double qs[D];
  __shared__ __attribute__((aligned(16))) char rows[SCORE_ROWS * PITCH];
  const int h = blockIdx.y;
  const int t = threadIdx.x;
  const int j0 = blockIdx.x * SCORE_ROWS;
  if (t < D) qs[t] = elem<T>(q + h * q_hs, t);
  const char* base = reinterpret_cast<const char*>(pool + h * p_hs);
  const int64_t rs = p_rs * (int64_t)sizeof(T);
  uint4 x[CPR];
#pragma unroll
  for (int i = 0; i < CPR; ++i) {
    const int f = t + 256 * i;  // chunk f % CPR of row f / CPR
    const int r = min(j0 + f / CPR, n - 1);
    x[i] = *reinterpret_cast<const uint4*>(base + (int64_t)r * rs + (f % CPR) * 16);
  }
#pragma unroll
  for (int i = 0; i < CPR; ++i) {
    const int f = t + 256 * i;
    *reinterpret_cast<uint4*>(rows + (f / CPR) * PITCH + (f % CPR) * 16) = x[i];
  }
  __syncthreads();
  const int j = j0 + t;
  if (j >= n) return;
  const char* row = rows + t * PITCH;
  constexpr int PER = 16 / (int)sizeof(T);
  double acc = 0.0;
#pragma unroll
  for (int c0 = 0; c0 < D; c0 += PER) {
    const uint4 w = *reinterpret_cast<const uint4*>(row + c0 * (int)sizeof(T));
    const T* e = reinterpret_cast<const T*>(&w);
#pragma unroll
    for (int c = 0; c < PER; ++c) acc = fma(qs[c0 + c], elem<T>(e, c), acc);
  }
  keys[(int64_t)h * n + j] = order_key(acc);
}

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
    const int nw = SEL_THREADS / 64;
    const int t = lane < nw ? wave_tot[lane] : 0;
    int s = t;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(s, o);
      if (lane >= o) s += y;
    }
    if (lane < nw) wave_tot[16 + lane] = s - t;
    if (lane == nw - 1) wave_tot[32] = s;
  }
  __syncthreads();
  const int r = x - v + wave_tot[16 + wid];
  *total = wave_tot[32];
  __syncthreads();
  return r;
}

// One work group per head.  Thread t owns the contiguous run of keys
// [t*per, t*per + per), held in registers when per <= KPT (RESIDENT), read
// again from memory on every pass otherwise.  Radix select of the k-th
// largest key, 12-bit digits from the top (bits 63..52, 51..40, ..., 15..4,
// then 3..0): a digit's histogram counts the keys that match the prefix
// chosen so far; the bin holding the remaining-th largest extends the
// prefix.  The search stops early once that bin holds exactly the keys still
// wanted (all of them are taken).  Then one pass marks each selected key --
// a prefix above the chosen one, or equal to it (all of them, or the lowest
// indices when the full 64-bit key ties) -- and a block scan gives every
// selected index its output slot in ascending pool order.
constexpr int KPT = 32;

template <bool RESIDENT>
__global__ __launch_bounds__(SEL_THREADS) void topk_select(const unsigned long long* keys_all,
                                                           int n, int k, int32_t* idx_all,
                                                           double* score_all) {
  __shared__ int hist[4096];
  __shared__ int wave_tot[40];
  __shared__ unsigned long long sh_prefix;
  __shared__ int sh_remaining, sh_count;
  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const unsigned long long* keys = keys_all + (int64_t)h * n;
  const int per = (n + SEL_THREADS - 1) / SEL_THREADS;
  const int j0 = min(n, tid * per), j1 = min(n, j0 + per);
  const int cnt = j1 - j0;
  unsigned long long kr[RESIDENT ? KPT : 1];
  if constexpr (RESIDENT) {
#pragma unroll
    for (int e = 0; e < KPT; ++e) kr[e] = e < cnt ? keys[j0 + e] : 0ull;
  }
  // f(key, position in the run) over this thread's keys, in index order
  auto for_keys = [&](auto&& f) {
    if constexpr (RESIDENT) {
#pragma unroll
      for (int e = 0; e < KPT; ++e)
        if (e < cnt) f(kr[e], e);
    } else {
      for (int e = 0; e < cnt; ++e) f(keys[j0 + e], e);
    }
  };
  unsigned long long prefix = 0, pmask = 0;
  int remaining = k;  // keys with this prefix still to take
  bool all_eq = false;  // every key matching the prefix is taken
  for (int shift = 52; shift >= 0 && !all_eq; shift = shift >= 12 ? shift - 12 : (shift > 0 ? 0 : -1)) {
    const int bits = shift >= 4 ? 12 : 4;  // the last digit is bits 3..0
    const int nb = 1 << bits;
    for (int b = tid; b < 4096; b += SEL_THREADS) hist[b] = 0;
    __syncthreads();
    for_keys([&](unsigned long long key, int) {
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1);
    });
    __syncthreads();
    // thread t owns bins 4t .. 4t+3 (the first nb of them exist)
    const int b0 = 4 * tid;
    int mine = 0;
    if (b0 < nb)
      for (int e = 0; e < 4; ++e) mine += hist[b0 + e];
    int tot;
    const int below = block_excl_scan(mine, wave_tot, &tot);
    const int above = tot - below - mine;  // keys in higher bins
    if (b0 < nb && above < remaining && remaining <= above + mine) {
      int acc = above, sel = b0;
      for (int e = 3; e >= 0; --e) {
        if (acc + hist[b0 + e] >= remaining) { sel = b0 + e; break; }
        acc += hist[b0 + e];
      }
      sh_prefix = prefix | ((unsigned long long)sel << shift);
      sh_remaining = remaining - acc;
      sh_count = hist[sel];
    }
    __syncthreads();
    prefix = sh_prefix;
    remaining = sh_remaining;
    all_eq = sh_count == remaining;
    pmask |= (unsigned long long)(nb - 1) << shift;
    __syncthreads();
  }
  // selected: prefix above the chosen one, or equal to it (every such key
  // when all_eq, else the lowest `remaining` indices: the full key ties)
  int gt = 0, eq = 0;
  for_keys([&](unsigned long long key, int) {
    const unsigned long long m = key & pmask;
    gt += m > prefix;
    eq += m == prefix;
  });
  int tot;
  const int gt_pre = block_excl_scan(gt, wave_tot, &tot);
  const int eq_pre = block_excl_scan(eq, wave_tot, &tot);
  const int need = all_eq ? 0x7fffffff : remaining;
  int pos = gt_pre + min(eq_pre, need);
  int eq_seen = eq_pre;
  int32_t* idx = idx_all + (int64_t)h * k;
  double* score = score_all ? score_all + (int64_t)h * k : nullptr;
  for_keys([&](unsigned long long key, int e) {
    const unsigned long long m = key & pmask;
    bool take = m > prefix;
    if (m == prefix) {
      take = eq_seen < need;
      ++eq_seen;
    }
    if (take) {
      idx[pos] = j0 + e;
      if (score) score[pos] = key_value(key);
      ++pos;
    }
  });
}

// Thread = (prefix row r, 16-byte chunk): copy the pool row idx[h, r].
__global__ __launch_bounds__(256) void topk_gather(const int32_t* idx_all, int k, int row_bytes,
                                                   const char* pk, const char* pv, int64_t p_hs,
                                                   int64_t p_rs, char* rk, char* rv, int64_t r_hs,
                                                   int64_t r_rs) {
  const int h = blockIdx.y;
  const int cpr = row_bytes / 16;
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= k * cpr) return;
  const int r = x / cpr, ch = x % cpr;
  const int j = idx_all[(int64_t)h * k + r];
  const int64_t src = h * p_hs + (int64_t)j * p_rs + ch * 16;
  const int64_t dst = h * r_hs + (int64_t)r * r_rs + ch * 16;
  *reinterpret_cast<uint4*>(rk + dst) = *reinterpret_cast<const uint4*>(pk + src);
  *reinterpret_cast<uint4*>(rv + dst) = *reinterpret_cast<const uint4*>(pv + src);
}

}  // namespace

size_t topk_workspace_bytes(int n_heads, int pool_len) {
  return (size_t)align_up((int64_t)n_heads * pool_len * 8, 256);
}

hipError_t launch_topk(int dtype, int n_heads, int pool_len, int d, int k, const void* q,
                       int64_t q_hs, const void* pool_k, const void* pool_v, int64_t p_hs,
                       int64_t p_rs, int32_t* idx, double* score, void* pref_k, void* pref_v,
                       int64_t r_hs, int64_t r_rs, void* ws, hipStream_t s) {
  unsigned long long* keys = static_cast<unsigned long long*>(ws);
  const dim3 g1((unsigned)ceil_div(pool_len, SCORE_ROWS), (unsigned)n_heads);
  const dim3 b1(256);
  typedef unsigned short u16;
  if (dtype == SA_BF16 && d == 128)
    hipLaunchKernelGGL((topk_score<u16, 128>), g1, b1, 0, s, static_cast<const u16*>(q), q_hs,
                       static_cast<const u16*>(pool_k), p_hs, p_rs, pool_len, keys);
  else if (dtype == SA_BF16)
    hipLaunchKernelGGL((topk_score<u16, 64>), g1, b1, 0, s, static_cast<const u16*>(q), q_hs,
                       static_cast<const u16*>(pool_k), p_hs, p_rs, pool_len, keys);
  else if (d == 128)
    hipLaunchKernelGGL((topk_score<float, 128>), g1, b1, 0, s, static_cast<const float*>(q), q_hs,
                       static_cast<const float*>(pool_k), p_hs, p_rs, pool_len, keys);
  else
    hipLaunchKernelGGL((topk_score<float, 64>), g1, b1, 0, s, static_cast<const float*>(q), q_hs,
                       static_cast<const float*>(pool_k), p_hs, p_rs, pool_len, keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ceil_div(pool_len, SEL_THREADS) <= KPT)
    hipLaunchKernelGGL(topk_select<true>, dim3(n_heads), dim3(SEL_THREADS), 0, s, keys, pool_len, k,
                       idx, score);
  else
    hipLaunchKernelGGL(topk_select<false>, dim3(n_heads), dim3(SEL_THREADS), 0, s, keys, pool_len, k,
                       idx, score);
  e = hipGetLastError();
  if (e != hipSuccess || pool_v == nullptr) return e;
  const int esz = dtype == SA_BF16 ? 2 : 4;
  const int row_bytes = d * esz;
  const dim3 g3((unsigned)ceil_div((int64_t)k * (row_bytes / 16), 256), (unsigned)n_heads);
  hipLaunchKernelGGL(topk_gather, g3, dim3(256), 0, s, idx, k, row_bytes,
                     static_cast<const char*>(pool_k), static_cast<const char*>(pool_v),
                     p_hs * esz, p_rs * esz, static_cast<char*>(pref_k), static_cast<char*>(pref_v),
                     r_hs * esz, r_rs * esz);
  return hipGetLastError();
}

}  // namespace sa
