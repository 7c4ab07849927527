// Forward-only top-k retrieval of the prefix (segmented-execution page, key
// design 3: before the next segment the segment-end query selects R keys of a
// detached read-only pool for the long-range heads).
//
// 1. topk_score: s_j = fp64 fma chain over c = 0..d-1 for every pool key
//    (each bf16/fp32 product is exact in fp64, so the chain equals plain
//    multiply-then-add in the same order); stored as an order-preserving
//    64-bit key (+0 and -0 share one key) and a 14-bit bucket (the score
//    rounded to fp32: sign, exponent and 5 mantissa bits; monotone in the
//    key).  Rows reach LDS by coalesced loads, 64 keys per single-wave group.
// 2. topk_select: one work group per head.  A histogram of the buckets finds
//    the bucket holding the k-th largest key; the few keys of that bucket
//    are ranked exactly (key, then lower index first) to find the threshold
//    key T and the last index taken at T.  When that bucket is crowded (heavy
//    ties), a radix select of T by 12-bit digits of the full key decides
//    instead.  A ballot bitmap of the selection in index order and one block
//    scan give every selected index its output slot, so idx comes out in
//    ascending pool order with ties at T taken from the lowest indices.
// 3. topk_gather: the selected keys' scores, and copies of the selected pool
//    K/V rows into the prefix rows.
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

// One single-wave work group scores SCORE_ROWS = 64 consecutive pool keys of
// one head (small groups keep many in flight per CU, so the loads of one
// overlap the arithmetic of others).  The rows are staged in LDS with
// coalesced 16-byte loads (a row's chunks come from consecutive lanes; rows
// padded by 16 bytes, so each lane's later reads of its own row are
// bank-conflict free), then lane t runs the fp64 chain of key t in c order and
// stores its order-preserving key and its bucket (see bucket_of).
constexpr int SCORE_ROWS = 64;
constexpr int BUCKET_BITS = 14;
constexpr int NBUCKET = 1 << BUCKET_BITS;

// The bucket of a score: the top BUCKET_BITS bits of the order-preserving
// 32-bit key of the score rounded to fp32.  Rounding to nearest is monotone,
// so a higher bucket never holds a lower score; scores of one bucket are told
// apart by the full key.
__device__ inline unsigned short bucket_of(double s) {
  unsigned u = __float_as_uint((float)s + 0.0f);
  u = (u >> 31) ? ~u : (u | 0x80000000u);
  return (unsigned short)(u >> (32 - BUCKET_BITS));
}

template <typename T, int D>
__global__ __launch_bounds__(SCORE_ROWS) void topk_score(const T* q, int64_t q_hs, const T* pool,
                                                         int64_t p_hs, int64_t p_rs, int n,
                                                         unsigned long long* keys, unsigned short* buckets) {
  constexpr int ROW = D * (int)sizeof(T);  // bytes per row
  constexpr int CPR = ROW / 16;            // 16-byte chunks per row
  constexpr int PITCH = ROW + 16;
  __shared__ double qs[D];
  __shared__ __attribute__((aligned(16))) char rows[SCORE_ROWS * PITCH];
  const int h = blockIdx.y;
  const int t = threadIdx.x;
  const int j0 = blockIdx.x * SCORE_ROWS;
  for (int c = t; c < D; c += SCORE_ROWS) qs[c] = elem<T>(q + h * q_hs, c);
  const char* base = reinterpret_cast<const char*>(pool + h * p_hs);
  const int64_t rs = p_rs * (int64_t)sizeof(T);
  uint4 x[CPR];
#pragma unroll
  for (int i = 0; i < CPR; ++i) {
    const int f = t + SCORE_ROWS * i;  // chunk f % CPR of row f / CPR
    const int r = min(j0 + f / CPR, n - 1);
    x[i] = *reinterpret_cast<const uint4*>(base + (int64_t)r * rs + (f % CPR) * 16);
  }
#pragma unroll
  for (int i = 0; i < CPR; ++i) {
    const int f = t + SCORE_ROWS * i;
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
  buckets[(int64_t)h * n + j] = bucket_of(acc);
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

// One work group per head.  Thread t owns indices t + 1024 e (e = 0, 1, ...):
// every load instruction of the work group reads 1024 consecutive keys or
// buckets.  With n <= 1024 KPT (RESIDENT) the buckets are staged in LDS once;
// otherwise they are read again on every pass.  Keys are read only where a
// bucket does not decide (the threshold bucket).
//   * Bucket pass: a histogram of the buckets finds the one that holds the
//     k-th largest key; when it holds at most CAND_CAP keys they are ranked
//     exactly by (key descending, index ascending), which gives the threshold
//     key T and the index of the last key taken at T: a key is taken when its
//     bucket is higher, or it is in that bucket and above T, or equal to T
//     with an index up to that one.
//   * Otherwise (heavy ties) a radix select of T by 12-bit digits of the full
//     key (from the top; it stops once the threshold bin holds exactly the
//     keys still wanted), and the keys equal to T taken are the lowest-index
//     ones.
// Output slots follow the index order: for a batch of 32768 indices a ballot
// per wave and round writes the selection as a bitmap in index order (round
// e, wave w holds indices 1024 e + 64 w + lane), then thread t counts the 32
// bits of indices 32 t .. 32 t + 31 and one block scan gives every set bit its
// slot.
constexpr int KPT = 32;          // rounds of 1024 indices per batch (32768 indices)
constexpr int CAND_CAP = 2048;   // the exact ranking handles at most this many keys
constexpr int NWAVE = SEL_THREADS / 64;
// staged-bucket values past every bucket: a key of the threshold bucket once ranked
constexpr int MARK_TAKEN = 0xFFFF, MARK_LEFT = 0xFFFE;

template <bool RESIDENT>
__global__ __launch_bounds__(SEL_THREADS) void topk_select(const unsigned long long* keys_all,
                                                           const unsigned short* buckets_all,
                                                           int n, int k, int32_t* idx_all) {
  __shared__ int hist[NBUCKET];
  __shared__ int wave_tot[40];
  __shared__ unsigned long long bitmap[KPT * NWAVE];  // one batch of 32768 indices
  __shared__ unsigned long long sh_prefix;
  __shared__ int sh_remaining, sh_count, sh_tidx, sh_bsel;
  __shared__ unsigned long long ckey[CAND_CAP];
  __shared__ int cidx[CAND_CAP];
  __shared__ __attribute__((aligned(16))) unsigned short sb[RESIDENT ? KPT * SEL_THREADS : 1];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int h = blockIdx.x;
  const unsigned long long* keys = keys_all + (int64_t)h * n;
  const unsigned short* bks = buckets_all + (int64_t)h * n;
  if constexpr (RESIDENT) {  // 16-byte pieces of the bucket array
    const uint4* src = reinterpret_cast<const uint4*>(bks);
    uint4* dst = reinterpret_cast<uint4*>(sb);
    if ((reinterpret_cast<uintptr_t>(bks) & 15) == 0) {
      for (int i = tid; i < n / 8; i += SEL_THREADS) dst[i] = src[i];
      for (int j = (n / 8) * 8 + tid; j < n; j += SEL_THREADS) sb[j] = bks[j];
    } else {
      for (int j = tid; j < n; j += SEL_THREADS) sb[j] = bks[j];
    }
  }
  // bucket of index j, staged or loaded
  auto bucket_at = [&](int, int j) -> int {
    if constexpr (RESIDENT) return (int)sb[j];
    else return (int)bks[j];
  };
  // f(u, j) for every index of this thread, UNR at a time (j clamped to n - 1
  // by the callee's reads; the caller checks j < n)
  constexpr int UNR = 8;
  auto rounds = [&](auto&& f) {
    for (int j0 = 0; j0 < n; j0 += UNR * SEL_THREADS)
#pragma unroll
      for (int u = 0; u < UNR; ++u) f(u, j0 + tid + SEL_THREADS * u);
  };

  // 1. bucket histogram; thread t owns buckets BPT t .. BPT t + BPT - 1
  constexpr int BPT = NBUCKET / SEL_THREADS;
  for (int b = tid; b < NBUCKET; b += SEL_THREADS) hist[b] = 0;
  if (tid == 0) sh_count = 0;
  __syncthreads();
  rounds([&](int e, int j) { atomicAdd(&hist[bucket_at(e, min(j, n - 1))], j < n ? 1 : 0); });
  __syncthreads();
  int bsel, need, cnt;
  {
    int hv[BPT];
    int mine = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      hv[e] = hist[BPT * tid + e];
      mine += hv[e];
    }
    int tot;
    const int below = block_excl_scan(mine, wave_tot, &tot);
    const int above = tot - below - mine;  // keys in higher buckets
    if (above < k && k <= above + mine) {
      int acc = above, sel = BPT * tid, c = 0;
#pragma unroll
      for (int e = BPT - 1; e >= 0; --e) {
        if (acc + hv[e] >= k && c == 0) { sel = BPT * tid + e; c = hv[e]; }
        if (c == 0) acc += hv[e];
      }
      sh_bsel = sel;
      sh_remaining = k - acc;  // keys of bucket sel to take
      wave_tot[36] = c;
    }
    __syncthreads();
    bsel = sh_bsel;
    need = sh_remaining;
    cnt = wave_tot[36];
  }
  const bool fast = cnt <= CAND_CAP;
  unsigned long long prefix = 0, pmask = 0;
  int remaining = k;    // radix path: keys with this prefix still to take
  bool all_eq = false;  // radix path: every key matching the prefix is taken
  int t_idx = -1;       // keys equal to the threshold are taken up to this index
  if (fast) {
    // 2. the bucket's keys into LDS (any order; one LDS atomic per wave and
    //    round), each then ranked with G threads
    rounds([&](int e, int j) {
      const int jc = min(j, n - 1);
      const bool m = j < n && bucket_at(e, jc) == bsel;
      const unsigned long long bal = __ballot(m);
      if (bal != 0ull) {
        const int leader = __ffsll((long long)bal) - 1;
        int base = 0;
        if (lane == leader) base = atomicAdd(&sh_count, __popcll(bal));
        base = __shfl(base, leader);
        if (m) cidx[base + __popcll(bal & ((1ull << lane) - 1ull))] = j;
      }
    });
    __syncthreads();
    for (int c = tid; c < cnt; c += SEL_THREADS) ckey[c] = keys[cidx[c]];  // all at once
    __syncthreads();
    int G = 64;
    while (G > 1 && G * cnt > SEL_THREADS * 2) G >>= 1;
    for (int base = 0; base < cnt * G; base += SEL_THREADS) {
      const int x = base + tid;
      const int c = x / G, part = x % G;
      int rank = 0;
      unsigned long long kc = 0;
      int ic = 0;
      if (c < cnt) {
        kc = ckey[c];
        ic = cidx[c];
        for (int o = part; o < cnt; o += G) {
          const unsigned long long ko = ckey[o];
          rank += (ko > kc) | ((ko == kc) & (cidx[o] < ic));
        }
      }
      for (int m = 1; m < G; m <<= 1) rank += __shfl_xor(rank, m);  // G consecutive lanes share a key
      if (c < cnt && part == 0) {
        if (rank == need - 1) {
          sh_prefix = kc;
          sh_tidx = ic;
        }
        // the bucket no longer decides for this key: mark it taken or not
        if constexpr (RESIDENT) sb[ic] = rank < need ? MARK_TAKEN : MARK_LEFT;
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    t_idx = sh_tidx;
  } else {
    // 2'. radix select over the full keys
    for (int shift = 52; shift >= 0 && !all_eq; shift = shift >= 12 ? shift - 12 : (shift > 0 ? 0 : -1)) {
      const int bits = shift >= 4 ? 12 : 4;  // the last digit is bits 3..0
      const int nb = 1 << bits;
      for (int b = tid; b < 4096; b += SEL_THREADS) hist[b] = 0;
      __syncthreads();
      for (int j = tid; j < n; j += SEL_THREADS) {  // (rare path: keys read again)
        const unsigned long long key = keys[j];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1);
      }
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
  }

  // Slots in index order for the indices whose flag(e, j) holds: f(j, slot)
  // for each (flag is evaluated with j clamped to n - 1 past the end and then
  // discarded).
  auto ordered = [&](auto&& flag, auto&& f) {
    int carry = 0;
    for (int j0 = 0; j0 < n; j0 += KPT * SEL_THREADS) {
      {
        for (int e0 = 0; e0 < KPT; e0 += UNR) {
          bool fl[UNR];
#pragma unroll
          for (int u = 0; u < UNR; ++u) {
            const int j = j0 + tid + SEL_THREADS * (e0 + u);
            fl[u] = flag(u, min(j, n - 1)) && j < n;
          }
#pragma unroll
          for (int u = 0; u < UNR; ++u) {
            const unsigned long long bal = __ballot(fl[u]);
            if (lane == 0) bitmap[(e0 + u) * NWAVE + wid] = bal;
          }
        }
      }
      __syncthreads();
      // thread t: indices j0 + 32 t .. j0 + 32 t + 31
      const unsigned bits = (unsigned)(bitmap[tid >> 1] >> (32 * (tid & 1)));
      int tot;
      int slot = carry + block_excl_scan(__popc(bits), wave_tot, &tot);
      for (unsigned m = bits; m != 0; m &= m - 1) f(j0 + 32 * tid + __ffs(m) - 1, slot++);
      carry += tot;
    }
  };
  if (!fast && !all_eq) {
    // the `remaining` lowest-index keys equal to the threshold are taken
    if (tid == 0) sh_tidx = n;
    __syncthreads();
    const int rem = remaining;
    ordered([&](int, int j) { return (keys[j] & pmask) == prefix; },
            [&](int j, int slot) {
              if (slot == rem - 1) sh_tidx = j;
            });
    __syncthreads();
    t_idx = sh_tidx;
  }
  if (!fast && all_eq) t_idx = n;
  int32_t* idx = idx_all + (int64_t)h * k;
  auto emit = [&](int j, int slot) { idx[slot] = j; };  // scores: written by topk_gather
  if (fast) {
    ordered(
        [&](int e, int j) {
          const int b = bucket_at(e, j);
          if constexpr (RESIDENT) return b == MARK_TAKEN || (b < NBUCKET && b > bsel);
          if (b != bsel) return b > bsel;
          const unsigned long long key = keys[j];  // the threshold bucket: few keys
          return key > prefix || (key == prefix && j <= t_idx);
        },
        emit);
  } else {
    ordered(
        [&](int, int j) {
          const unsigned long long m = keys[j] & pmask;
          return m > prefix || (m == prefix && j <= t_idx);
        },
        emit);
  }
}

// Thread = (prefix row r, 16-byte chunk): the score of the selected key (chunk
// 0, when asked for) and, when rows are asked for, a copy of the pool row
// idx[h, r] into the prefix rows.
__global__ __launch_bounds__(256) void topk_gather(const int32_t* idx_all, int k, int n, int row_bytes,
                                                   const unsigned long long* keys_all, double* score_all,
                                                   const char* pk, const char* pv, int64_t p_hs,
                                                   int64_t p_rs, char* rk, char* rv, int64_t r_hs,
                                                   int64_t r_rs) {
  const int h = blockIdx.y;
  const int cpr = row_bytes / 16;
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= k * cpr) return;
  const int r = x / cpr, ch = x % cpr;
  const int j = idx_all[(int64_t)h * k + r];
  if (ch == 0 && score_all != nullptr) score_all[(int64_t)h * k + r] = key_value(keys_all[(int64_t)h * n + j]);
  if (pk == nullptr) return;
  const int64_t src = h * p_hs + (int64_t)j * p_rs + ch * 16;
  const int64_t dst = h * r_hs + (int64_t)r * r_rs + ch * 16;
  *reinterpret_cast<uint4*>(rk + dst) = *reinterpret_cast<const uint4*>(pk + src);
  *reinterpret_cast<uint4*>(rv + dst) = *reinterpret_cast<const uint4*>(pv + src);
}

}  // namespace

// Workspace: the order keys (8 bytes per pool key), then the buckets (2 bytes).
size_t topk_workspace_bytes(int n_heads, int pool_len) {
  return (size_t)(align_up((int64_t)n_heads * pool_len * 8, 256) + align_up((int64_t)n_heads * pool_len * 2, 256));
}

hipError_t launch_topk(int dtype, int n_heads, int pool_len, int d, int k, const void* q,
                       int64_t q_hs, const void* pool_k, const void* pool_v, int64_t p_hs,
                       int64_t p_rs, int32_t* idx, double* score, void* pref_k, void* pref_v,
                       int64_t r_hs, int64_t r_rs, void* ws, hipStream_t s) {
  unsigned long long* keys = static_cast<unsigned long long*>(ws);
  unsigned short* buckets =
      reinterpret_cast<unsigned short*>(static_cast<char*>(ws) + align_up((int64_t)n_heads * pool_len * 8, 256));
  const dim3 g1((unsigned)ceil_div(pool_len, SCORE_ROWS), (unsigned)n_heads);
  const dim3 b1(SCORE_ROWS);
  typedef unsigned short u16;
  if (dtype == SA_BF16 && d == 128)
    hipLaunchKernelGGL((topk_score<u16, 128>), g1, b1, 0, s, static_cast<const u16*>(q), q_hs,
                       static_cast<const u16*>(pool_k), p_hs, p_rs, pool_len, keys, buckets);
  else if (dtype == SA_BF16)
    hipLaunchKernelGGL((topk_score<u16, 64>), g1, b1, 0, s, static_cast<const u16*>(q), q_hs,
                       static_cast<const u16*>(pool_k), p_hs, p_rs, pool_len, keys, buckets);
  else if (d == 128)
    hipLaunchKernelGGL((topk_score<float, 128>), g1, b1, 0, s, static_cast<const float*>(q), q_hs,
                       static_cast<const float*>(pool_k), p_hs, p_rs, pool_len, keys, buckets);
  else
    hipLaunchKernelGGL((topk_score<float, 64>), g1, b1, 0, s, static_cast<const float*>(q), q_hs,
                       static_cast<const float*>(pool_k), p_hs, p_rs, pool_len, keys, buckets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ceil_div(pool_len, SEL_THREADS) <= KPT)
    hipLaunchKernelGGL(topk_select<true>, dim3(n_heads), dim3(SEL_THREADS), 0, s, keys, buckets, pool_len, k,
                       idx);
  else
    hipLaunchKernelGGL(topk_select<false>, dim3(n_heads), dim3(SEL_THREADS), 0, s, keys, buckets, pool_len, k,
                       idx);
  e = hipGetLastError();
  if (e != hipSuccess || (pool_v == nullptr && score == nullptr)) return e;
  const int esz = dtype == SA_BF16 ? 2 : 4;
  const int row_bytes = d * esz;
  const dim3 g3((unsigned)ceil_div((int64_t)k * (row_bytes / 16), 256), (unsigned)n_heads);
  hipLaunchKernelGGL(topk_gather, g3, dim3(256), 0, s, idx, k, pool_len, row_bytes, keys, score,
                     pool_v == nullptr ? nullptr : static_cast<const char*>(pool_k), static_cast<const char*>(pool_v),
                     p_hs * esz, p_rs * esz, static_cast<char*>(pref_k), static_cast<char*>(pref_v),
                     r_hs * esz, r_rs * esz);
  return hipGetLastError();
}

}  // namespace sa
