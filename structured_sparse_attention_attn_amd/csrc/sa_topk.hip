// Forward-only top-k retrieval of the prefix (segmented-execution page, key
// design 3: before the next segment the segment-end query selects R keys of a
// detached read-only pool for the long-range heads).
//
// 1. topk_score: one thread per pool key, s_j = fp64 fma chain over c = 0..d-1
//    (each bf16/fp32 product is exact in fp64, so the chain equals plain
//    multiply-then-add in the same order); stored as an order-preserving
//    64-bit key (+0 and -0 share one key).
// 2. topk_select: one work group per head; radix select (a 12-bit digit over
//    all keys, the rest over the keys sharing that prefix, in LDS when they
//    fit) finds the k-th largest key T; then each thread takes a contiguous run of
//    keys and one block scan gives every selected index its output slot, so
//    idx comes out in ascending pool order with ties at T taken from the
//    lowest indices.
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

// Thread = one pool key: its row in 16-byte pieces (rows are 16-byte
// aligned), the fp64 chain in c order.
template <typename T>
__global__ __launch_bounds__(256) void topk_score(const T* q, int64_t q_hs, const T* pool,
                                                  int64_t p_hs, int64_t p_rs, int n, int d,
                                                  unsigned long long* keys) {
  __shared__ double qs[128];
  const int h = blockIdx.y;
  if (threadIdx.x < d) qs[threadIdx.x] = elem<T>(q + h * q_hs, threadIdx.x);
  __syncthreads();
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  const T* row = pool + h * p_hs + (int64_t)j * p_rs;
  constexpr int PER = 16 / sizeof(T);
  double acc = 0.0;
  for (int c0 = 0; c0 < d; c0 += PER) {
    const uint4 w = *reinterpret_cast<const uint4*>(row + c0);
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

constexpr int SEL_CAND = 4096;  // candidates kept in LDS after the first digit

__global__ __launch_bounds__(SEL_THREADS) void topk_select(const unsigned long long* keys_all,
                                                           int n, int k, int32_t* idx_all,
                                                           double* score_all) {
  __shared__ int hist[4096];
  __shared__ unsigned long long cand[SEL_CAND];
  __shared__ int wave_tot[40];
  __shared__ unsigned long long sh_prefix;
  __shared__ int sh_remaining, sh_ncand;
  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const unsigned long long* keys = keys_all + (int64_t)h * n;
  // Radix select of the k-th largest key, most significant digit first: a
  // 12-bit digit over all keys, then 8-bit digits (a 4-bit one last).  After
  // the first digit the keys sharing the selected prefix are copied to LDS
  // when they fit, and the remaining digits run there.
  unsigned long long prefix = 0, pmask = 0;
  int remaining = k;  // how many of the largest keys with this prefix are still wanted
  // one digit: histogram of (key >> shift) & (nb-1) over the keys matching the
  // prefix, then the bin holding the remaining-th largest
  auto digit = [&](auto&& for_keys, int shift, int nb) {
    for (int b = tid; b < nb; b += SEL_THREADS) hist[b] = 0;
    __syncthreads();
    for_keys([&](unsigned long long key) {
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1);
    });
    __syncthreads();
    // thread t owns bins t*per .. t*per+per-1; counts above a thread's bins
    // come from an exclusive scan of the per-thread sums
    const int per = nb / SEL_THREADS > 0 ? nb / SEL_THREADS : 1;
    const int b0 = tid * per;
    int mine = 0;
    if (b0 < nb)
      for (int e = 0; e < per; ++e) mine += hist[b0 + e];
    int tot;
    const int below = block_excl_scan(mine, wave_tot, &tot);
    const int above = tot - below - mine;  // keys in bins above this thread's
    if (b0 < nb && above < remaining && remaining <= above + mine) {
      int acc = above, sel = b0;
      for (int e = per - 1; e >= 0; --e) {
        if (acc + hist[b0 + e] >= remaining) { sel = b0 + e; break; }
        acc += hist[b0 + e];
      }
      sh_prefix = prefix | ((unsigned long long)sel << shift);
      sh_remaining = remaining - acc;
    }
    __syncthreads();
    prefix = sh_prefix;
    remaining = sh_remaining;
    pmask |= (unsigned long long)(nb - 1) << shift;
    __syncthreads();
  };
  auto global_keys = [&](auto&& f) {
    for (int j = tid; j < n; j += SEL_THREADS) f(keys[j]);
  };
  digit(global_keys, 52, 4096);
  if (tid == 0) sh_ncand = 0;
  __syncthreads();
  const int n_match = hist[(int)((prefix >> 52) & 4095)];
  if (n_match <= SEL_CAND) {
    for (int j = tid; j < n; j += SEL_THREADS) {
      const unsigned long long key = keys[j];
      if ((key & pmask) == prefix) cand[atomicAdd(&sh_ncand, 1)] = key;
    }
    __syncthreads();
    const int nc = sh_ncand;
    auto lds_keys = [&](auto&& f) {
      for (int j = tid; j < nc; j += SEL_THREADS) f(cand[j]);
    };
    for (int shift = 44; shift >= 4; shift -= 8) digit(lds_keys, shift, 256);
    digit(lds_keys, 0, 16);
  } else {
    for (int shift = 44; shift >= 4; shift -= 8) digit(global_keys, shift, 256);
    digit(global_keys, 0, 16);
  }
  const unsigned long long T = prefix;
  const int need = remaining;  // keys equal to T to take, lowest indices first
  // contiguous run per thread
  const int per = (n + SEL_THREADS - 1) / SEL_THREADS;
  const int j0 = min(n, tid * per), j1 = min(n, j0 + per);
  int gt = 0, eq = 0;
  for (int j = j0; j < j1; ++j) {
    const unsigned long long key = keys[j];
    gt += key > T;
    eq += key == T;
  }
  int tot;
  const int gt_pre = block_excl_scan(gt, wave_tot, &tot);
  const int eq_pre = block_excl_scan(eq, wave_tot, &tot);
  int pos = gt_pre + min(eq_pre, need);
  int eq_seen = eq_pre;
  int32_t* idx = idx_all + (int64_t)h * k;
  double* score = score_all ? score_all + (int64_t)h * k : nullptr;
  for (int j = j0; j < j1; ++j) {
    const unsigned long long key = keys[j];
    bool take = key > T;
    if (key == T) {
      take = eq_seen < need;
      ++eq_seen;
    }
    if (take) {
      idx[pos] = j;
      if (score) score[pos] = key_value(key);
      ++pos;
    }
  }
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
  const dim3 g1((unsigned)ceil_div(pool_len, 256), (unsigned)n_heads);
  if (dtype == SA_BF16)
    hipLaunchKernelGGL(topk_score<unsigned short>, g1, dim3(256), 0, s,
                       static_cast<const unsigned short*>(q), q_hs,
                       static_cast<const unsigned short*>(pool_k), p_hs, p_rs, pool_len, d, keys);
  else
    hipLaunchKernelGGL(topk_score<float>, g1, dim3(256), 0, s, static_cast<const float*>(q), q_hs,
                       static_cast<const float*>(pool_k), p_hs, p_rs, pool_len, d, keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_select, dim3(n_heads), dim3(SEL_THREADS), 0, s, keys, pool_len, k, idx,
                     score);
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
