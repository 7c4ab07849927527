// Forward-only top-k retrieval of the prefix (segmented-execution page, key
// design 3: before the next segment the segment-end query selects R keys of a
// detached read-only pool for the long-range heads).
//
// 1. topk_score: s_j = fp64 fma chain over c = 0..d-1 for every pool key
//    (each bf16/fp32 product is exact in fp64, so the chain equals plain
//    multiply-then-add in the same order); stored as an order-preserving
//    64-bit key (+0 and -0 share one key) and a 14-bit bucket (the score
//    rounded to fp32: sign, exponent and 5 mantissa bits; monotone in the
//    key), counted in a histogram per head.  Rows reach LDS by coalesced
//    loads, 64 keys per single-wave group.
// 2. topk_pick: G work groups per head, each owning a chunk of the indices.
//    Each finds, from the head's histogram, the bucket holding the k-th
//    largest key, ranks that bucket's few keys exactly (key, then lower index
//    first) and so knows which of its own indices are taken and how many are
//    taken before its chunk; it writes their slots (idx comes out in
//    ascending pool order, ties at the threshold taken from the lowest
//    indices), their scores and copies of their pool K/V rows into the
//    prefix rows.  When that bucket is crowded (heavy ties), a radix select
//    of the threshold by 12-bit digits of the full key decides instead.
#include <algorithm>

#include "sa_common.h"

namespace sa {
namespace {

constexpr int PICK_THREADS = 1024;  // threads of a selection work group

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
// coalesced non-temporal 16-byte loads (a row's chunks come from consecutive
// lanes; rows padded by 16 bytes, so each lane's later reads of its own row
// are bank-conflict free), then lane t runs the fp64 chain of key t in c order and
// stores its order-preserving key and its bucket (see bucket_of); the first
// lane of every GROUP keys also stores their largest bucket.
constexpr int SCORE_ROWS = 64;
constexpr int GROUP = 16;  // keys per group maximum
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

// 16 bytes read once (non-temporal: the pool streams past the caches).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline uint4 ld16_stream(const char* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T, int D>
__global__ __launch_bounds__(SCORE_ROWS) void topk_score(const T* q, int64_t q_hs, const T* pool,
                                                         int64_t p_hs, int64_t p_rs, int n, int npad,
                                                         unsigned long long* keys, unsigned short* buckets,
                                                         unsigned short* gmax) {
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
    x[i] = ld16_stream(base + (int64_t)r * rs + (f % CPR) * 16);
  }
#pragma unroll
  for (int i = 0; i < CPR; ++i) {
    const int f = t + SCORE_ROWS * i;
    *reinterpret_cast<uint4*>(rows + (f / CPR) * PITCH + (f % CPR) * 16) = x[i];
  }
  __syncthreads();
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
  const int j = j0 + t;
  const bool valid = j < n;
  const unsigned short b = bucket_of(acc);
  int m = valid ? (int)b : 0;  // bucket 0 is below every bucket: a group's largest is unchanged
#pragma unroll
  for (int o = 1; o < GROUP; o <<= 1) m = max(m, __shfl_xor(m, o));
  if (!valid) return;
  keys[(int64_t)h * npad + j] = order_key(acc);
  buckets[(int64_t)h * npad + j] = b;
  if ((t & (GROUP - 1)) == 0) gmax[(int64_t)h * (npad / GROUP) + j / GROUP] = (unsigned short)m;
}

// Inclusive sum over lanes 0..lane of the wave: shifts within rows of 16
// lanes, then each row's total broadcast into the later rows (DPP).
__device__ inline int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2 and 3
  return x;
}

constexpr int NWAVE = PICK_THREADS / 64;

// Exclusive prefix of v over the work group's threads and its total, with one
// barrier.  wave_tot (NWAVE ints) must not be in use by the previous call:
// alternate two of them.
__device__ inline int block_excl_scan(int v, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int x = wave_incl_sum(v);
  if (lane == 63) wave_tot[wid] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) {
    const int t = wave_tot[w];
    all += t;
    before += w < wid ? t : 0;
  }
  *total = all;
  return before + x - v;
}

// Two buckets per 32-bit word (buckets < 2^14): bit 15 (bit 31) set where the
// low (high) bucket is >= v, v2 = v * 0x10001 with v < 2^15; or equal to v.
__device__ inline unsigned ge2(unsigned w, unsigned v2) { return ((w | 0x80008000u) - v2) & 0x80008000u; }
__device__ inline unsigned eq2(unsigned w, unsigned v2) {
  return ~(((w ^ v2) | 0x80008000u) - 0x00010001u) & 0x80008000u;
}

// The LDS histogram keeps bin b in word hbin(b): within every 64 bins the four
// 16-byte slots of each 64-byte run are permuted, so that the threads of a
// quarter wave, each reading its 16 contiguous bins a slot at a time, read 16
// different slots of a 256-byte span (bank-conflict free).
__device__ inline int hbin(int b) { return b ^ (((b >> 6) & 3) << 2); }

// The selection runs on G work groups per head.  Work group (h, g) owns the
// indices [g C, g C + C) of head h (C = chunk) and writes the output slots of
// the selected ones among them.  Every work group of a head derives the same
// threshold from data of the whole head, so none waits for another:
//   1. A lower bound L of the threshold bucket: the k-th largest of the
//      head's group maxima (k groups have a key in bucket L or higher, so the
//      k-th largest key is there too); 0 when k exceeds the group count.
//   2. One pass over the head's buckets lists the keys in buckets >= L (about
//      1400 of 32768 at the segment workload, k = 1024) with a histogram of
//      their buckets, which gives the bucket bsel that holds the k-th largest
//      key and how many of its keys are taken (need = k - the keys of higher
//      buckets).  The keys of higher buckets before the chunk and the keys of
//      bsel (the candidates) are all on the list; when it overflows, one more
//      pass over the buckets finds them.
//   3. The candidates are ranked exactly by (key descending, index ascending);
//      the first `need` are taken.  When bsel holds more than CAND_CAP keys
//      (heavy ties), a radix select of the threshold key T by 12-bit digits of
//      the full key decides instead (from the top; it stops once the threshold
//      bin holds exactly the keys still wanted), and of the keys equal to T
//      the lowest-index ones are taken.
//   4. The chunk's selected indices, in ascending order, take the slots after
//      those selected before the chunk; each one's score and, when asked for,
//      its K/V rows follow.
constexpr int CHUNK_MAX = 4 * PICK_THREADS;  // indices per work group
constexpr int CAND_CAP = 2048;               // the exact ranking handles at most this many keys
constexpr int LIST_CAP = 4 * PICK_THREADS;   // listed keys (bucket >= L)
constexpr int BR = 4;                        // 16-byte bucket pieces per thread and pass (32 buckets)
// staged-bucket values past every bucket, for keys whose bucket does not decide
constexpr int MARK_TAKEN = 0xFFFF, MARK_LEFT = 0xFFFE;

struct PickArgs {
  const unsigned long long* keys;  // [n_heads][npad] order keys
  const unsigned short* buckets;   // [n_heads][npad]
  const unsigned short* gmax;      // [n_heads][npad / GROUP] group maxima
  int n, npad, k, chunk, n_heads;
  int32_t* idx;                    // [n_heads][k]
  double* score;                   // [n_heads][k] or null
  const char* pk;                  // pool K and V (null: no row copies)
  const char* pv;
  int64_t p_hs, p_rs;              // bytes
  char* rk;                        // prefix K and V
  char* rv;
  int64_t r_hs, r_rs;              // bytes
  int row_bytes;
};

__global__ __launch_bounds__(PICK_THREADS) void topk_pick(PickArgs a) {
  __shared__ int wave_tot[2][NWAVE];
  __shared__ int sh_bin, sh_need, sh_cnt, sh_count, sh_before, sh_remaining, sh_hcount;
  __shared__ unsigned long long sh_prefix;
  __shared__ __attribute__((aligned(16))) int hist[NBUCKET];  // (later: the radix bins; the chunk's selection)
  __shared__ int lj[LIST_CAP];                                // listed indices
  __shared__ unsigned short lb[LIST_CAP];                     // and their buckets
  __shared__ unsigned long long ckey[CAND_CAP];
  __shared__ int cidx[CAND_CAP];
  __shared__ __attribute__((aligned(16))) unsigned short sb[CHUNK_MAX];  // the chunk's buckets
  const int tid = threadIdx.x, lane = tid & 63;
  const int h = blockIdx.x % a.n_heads, g = blockIdx.x / a.n_heads;
  const int n = a.n, k = a.k;
  const int s0 = g * a.chunk, len = min(n - s0, a.chunk);
  const int n_groups = (n + GROUP - 1) / GROUP;
  const unsigned long long* keys = a.keys + (int64_t)h * a.npad;
  const unsigned short* bks = a.buckets + (int64_t)h * a.npad;
  const unsigned* gm2 = reinterpret_cast<const unsigned*>(a.gmax + (int64_t)h * (a.npad / GROUP));
  int slot = 0;  // alternates the block scans' wave totals
  auto scan = [&](int v, int* total) {
    const int r = block_excl_scan(v, wave_tot[slot], total);
    slot ^= 1;
    return r;
  };

  // Loads first, in flight together: the head's buckets when one pass of BR
  // pieces per thread holds them (else they are read once per pass), the
  // group maxima in pairs, the chunk's buckets (s0 is a multiple of 1024:
  // 16-byte pieces; the pad past n lies inside the head's npad entries).
  const bool one_pass = n <= BR * 8 * PICK_THREADS;
  uint4 bv[BR];
  auto load_pass = [&](int base) {
#pragma unroll
    for (int r = 0; r < BR; ++r) {
      const int j0 = base + 8 * (tid + PICK_THREADS * r);
      bv[r] = j0 < n ? *reinterpret_cast<const uint4*>(bks + j0) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  if (one_pass) load_pass(0);
  const bool bounded = k <= n_groups;
  unsigned gv[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = tid + PICK_THREADS * r;  // groups 2i, 2i + 1
    gv[r] = bounded && 2 * i < n_groups ? gm2[i] : 0u;
  }
  for (int i = tid; i < (len + 7) / 8; i += PICK_THREADS)
    reinterpret_cast<uint4*>(sb)[i] = reinterpret_cast<const uint4*>(bks + s0)[i];
  for (int b = tid; b < NBUCKET; b += PICK_THREADS) hist[b] = 0;
  if (tid == 0) {
    sh_bin = 0;
    sh_need = 0;
    sh_cnt = 0;
    sh_count = 0;
    sh_before = 0;
  }
  // f(j0, w, vm): the 8 buckets of indices j0 .. j0 + 7, packed two to a word
  // in w, vm[q] the halves of word q inside the head; every index once
  auto visit = [&](auto&& f) {
    for (int base = 0; base < n; base += BR * 8 * PICK_THREADS) {
      if (!one_pass) load_pass(base);
#pragma unroll
      for (int r = 0; r < BR; ++r) {
        const int j0 = base + 8 * (tid + PICK_THREADS * r);
        const unsigned w[4] = {bv[r].x, bv[r].y, bv[r].z, bv[r].w};
        unsigned vm[4] = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        if (j0 + 8 > n) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            vm[q] = (j0 + 2 * q < n ? 0x8000u : 0u) | (j0 + 2 * q + 1 < n ? 0x80000000u : 0u);
        }
        f(j0, w, vm);
      }
    }
  };
  // The bin holding the want-th largest counted key (thread t owns bins
  // BPT t .. BPT t + BPT - 1): sh_bin, sh_need = want - the keys of higher
  // bins, sh_cnt = its count.  clear: the bins are zeroed after reading.
  constexpr int BPT = NBUCKET / PICK_THREADS;
  auto find_bin = [&](int want, bool clear) {
    int hv[BPT];
#pragma unroll
    for (int i = 0; i < BPT / 4; ++i) {
      int4* p = reinterpret_cast<int4*>(hist + hbin(BPT * tid + 4 * i));
      const int4 v = *p;
      hv[4 * i] = v.x;
      hv[4 * i + 1] = v.y;
      hv[4 * i + 2] = v.z;
      hv[4 * i + 3] = v.w;
      if (clear) *p = make_int4(0, 0, 0, 0);
    }
    int mine = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) mine += hv[e];
    int tot;
    const int below = scan(mine, &tot);
    const int above = tot - below - mine;  // counted keys in higher bins
    if (above < want && want <= above + mine) {
      int acc = above, s = BPT * tid, c = 0;
#pragma unroll
      for (int e = BPT - 1; e >= 0; --e) {
        if (c == 0 && acc + hv[e] >= want) {
          s = BPT * tid + e;
          c = hv[e];
        }
        if (c == 0) acc += hv[e];
      }
      sh_bin = s;
      sh_need = want - acc;
      sh_cnt = c;
    }
    __syncthreads();
  };
  __syncthreads();

  // 1. lower bound of the threshold bucket
  int low = 0;
  if (bounded) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = tid + PICK_THREADS * r;
      if (2 * i < n_groups) atomicAdd(&hist[hbin(gv[r] & 0xFFFFu)], 1);
      if (2 * i + 1 < n_groups) atomicAdd(&hist[hbin(gv[r] >> 16)], 1);
    }
    for (int i = tid + 2 * PICK_THREADS; 2 * i < n_groups; i += PICK_THREADS) {  // beyond 4096 groups
      const unsigned v = gm2[i];
      atomicAdd(&hist[hbin(v & 0xFFFFu)], 1);
      if (2 * i + 1 < n_groups) atomicAdd(&hist[hbin(v >> 16)], 1);
    }
    __syncthreads();
    find_bin(k, true);
    low = sh_bin;
  }
  // 2. the keys in buckets >= low: listed (up to LIST_CAP) with their
  //    buckets, and every one of them counted in the histogram
  const unsigned low2 = (unsigned)low * 0x10001u;
  int n_list = 0;
  for (int base = 0; base < n; base += BR * 8 * PICK_THREADS) {
    if (!one_pass) load_pass(base);
    unsigned hit = 0;  // bit 8 r + e: element e of piece r
#pragma unroll
    for (int r = 0; r < BR; ++r) {
      const int j0 = base + 8 * (tid + PICK_THREADS * r);
      const unsigned w[4] = {bv[r].x, bv[r].y, bv[r].z, bv[r].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        unsigned f = ge2(w[q], low2);
        if (j0 + 8 > n) f &= (j0 + 2 * q < n ? 0x8000u : 0u) | (j0 + 2 * q + 1 < n ? 0x80000000u : 0u);
        hit |= (((f >> 15) & 1u) | ((f >> 30) & 2u)) << (8 * r + 2 * q);
      }
    }
    int tot;
    int pos = n_list + scan(__popc(hit), &tot);
#pragma unroll
    for (int r = 0; r < BR; ++r) {
      const unsigned w[4] = {bv[r].x, bv[r].y, bv[r].z, bv[r].w};
      for (unsigned hr = (hit >> (8 * r)) & 0xFFu; hr != 0u; hr &= hr - 1u) {
        const int e = __ffs(hr) - 1;  // element e of piece r
        const unsigned wq = e < 2 ? w[0] : e < 4 ? w[1] : e < 6 ? w[2] : w[3];
        const int bkt = (int)((wq >> (16 * (e & 1))) & 0xFFFFu);
        atomicAdd(&hist[hbin(bkt)], 1);
        if (pos < LIST_CAP) {
          lj[pos] = base + 8 * (tid + PICK_THREADS * r) + e;
          lb[pos] = (unsigned short)bkt;
        }
        ++pos;
      }
    }
    n_list += tot;
  }
  __syncthreads();
  const bool listed = n_list <= LIST_CAP;
  constexpr int LPT = LIST_CAP / PICK_THREADS;
  find_bin(k, false);
  int bsel = sh_bin;
  const int need = sh_need, cnt = sh_cnt;
  const bool fast = cnt <= CAND_CAP;
  int before;  // selected indices before the chunk
  if (fast) {
    // the candidates (any order) and the higher-bucket count before the chunk
    int ab = 0;
    if (listed) {
#pragma unroll
      for (int r = 0; r < LPT; ++r) {
        const int i = tid + PICK_THREADS * r;
        if (i < n_list) {
          const int b = lb[i], j = lj[i];
          ab += (b > bsel && j < s0) ? 1 : 0;
          if (b == bsel) {
            const int c = atomicAdd(&sh_count, 1);
            cidx[c] = j;
            ckey[c] = keys[j];
          }
        }
      }
    } else {
      const unsigned gt2 = (unsigned)(bsel + 1) * 0x10001u, eq = (unsigned)bsel * 0x10001u;
      visit([&](int j0, const unsigned* w, const unsigned* vm) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (j0 + 8 <= s0) ab += __popc(ge2(w[q], gt2) & vm[q]);
          for (unsigned m = eq2(w[q], eq) & vm[q]; m != 0u; m &= m - 1u) {
            const int j = j0 + 2 * q + ((__ffs(m) - 1) >> 4);
            const int c = atomicAdd(&sh_count, 1);
            cidx[c] = j;
            ckey[c] = keys[j];
          }
        }
      });
    }
    int ab_tot;
    scan(ab, &ab_tot);  // (its barrier also publishes the candidates)
    // 3. rank the candidates, G threads per candidate
    int lg = 6;  // G = 2^lg threads per candidate, one pass of the work group when cnt <= 1024
    while (lg > 0 && (cnt << lg) > PICK_THREADS) --lg;
    const int G = 1 << lg;
    for (int base = 0; base < cnt * G; base += PICK_THREADS) {
      const int x = base + tid;
      const int c = x >> lg, part = x & (G - 1);
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
        const bool take = rank < need;
        if (ic < s0) {
          if (take) atomicAdd(&sh_before, 1);
        } else if (ic < s0 + len) {
          sb[ic - s0] = take ? MARK_TAKEN : MARK_LEFT;
        }
      }
    }
    __syncthreads();
    before = ab_tot + sh_before;
  } else {
    // 3'. radix select of the threshold over the head's full keys
    unsigned long long prefix = 0, pmask = 0;
    int remaining = k;    // keys with this prefix still to take
    bool all_eq = false;  // every key matching the prefix is taken
    for (int shift = 52; shift >= 0 && !all_eq; shift = shift >= 12 ? shift - 12 : (shift > 0 ? 0 : -1)) {
      const int bits = shift >= 4 ? 12 : 4;  // the last digit is bits 3..0
      const int nb = 1 << bits;
      for (int b = tid; b < 4096; b += PICK_THREADS) hist[b] = 0;
      __syncthreads();
      for (int j = tid; j < n; j += PICK_THREADS) {
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
      const int below = scan(mine, &tot);
      const int above = tot - below - mine;  // keys in higher bins
      if (b0 < nb && above < remaining && remaining <= above + mine) {
        int acc = above, s = b0;
        for (int e = 3; e >= 0; --e) {
          if (acc + hist[b0 + e] >= remaining) {
            s = b0 + e;
            break;
          }
          acc += hist[b0 + e];
        }
        sh_prefix = prefix | ((unsigned long long)s << shift);
        sh_remaining = remaining - acc;
        sh_hcount = hist[s];
      }
      __syncthreads();
      prefix = sh_prefix;
      remaining = sh_remaining;
      all_eq = sh_hcount == remaining;
      pmask |= (unsigned long long)(nb - 1) << shift;
      __syncthreads();
    }
    // keys above the threshold and equal to it before the chunk
    int ab = 0, eq = 0;
    for (int j = tid; j < s0; j += PICK_THREADS) {
      const unsigned long long m = keys[j] & pmask;
      ab += m > prefix ? 1 : 0;
      eq += m == prefix ? 1 : 0;
    }
    int ab_tot, eq_tot;
    scan(ab, &ab_tot);
    scan(eq, &eq_tot);
    // the chunk, E contiguous indices per thread: of the keys equal to the
    // threshold the `remaining` lowest-index ones are taken
    const int E = a.chunk / PICK_THREADS;
    int gt = 0, eqm = 0;
    for (int e = 0; e < E; ++e) {
      const int i = E * tid + e;
      if (i < len) {
        const unsigned long long m = keys[s0 + i] & pmask;
        gt |= (m > prefix ? 1 : 0) << e;
        eqm |= (m == prefix ? 1 : 0) << e;
      }
    }
    int eq_chunk;
    int r = eq_tot + scan(__popc(eqm), &eq_chunk);
    for (int e = 0; e < E; ++e) {
      const int i = E * tid + e;
      if (i < len) {
        bool take = (gt >> e) & 1;
        if ((eqm >> e) & 1) take = all_eq || r++ < remaining;
        sb[i] = take ? MARK_TAKEN : MARK_LEFT;
      }
    }
    __syncthreads();
    before = ab_tot + (all_eq ? eq_tot : min(eq_tot, remaining));
    bsel = NBUCKET - 1;  // every index of the chunk is decided by its mark
  }

  // 4. the chunk's selected indices in ascending order, E contiguous ones per thread
  const int E = a.chunk / PICK_THREADS;
  int fl = 0;
  for (int e = 0; e < E; ++e) {
    const int i = E * tid + e;
    if (i < len) {
      const int b = sb[i];
      fl |= ((b == MARK_TAKEN || (b > bsel && b < NBUCKET)) ? 1 : 0) << e;
    }
  }
  int tot;
  int r = scan(__popc(fl), &tot);  // (every earlier use of hist is behind its barrier)
  int* sel = hist;
  int32_t* idx = a.idx + (int64_t)h * k + before;
  for (int e = 0; e < E; ++e)
    if ((fl >> e) & 1) {
      const int j = s0 + E * tid + e;
      idx[r] = j;
      sel[r++] = j;
    }
  __syncthreads();
  if (a.score != nullptr)
    for (int x = tid; x < tot; x += PICK_THREADS)
      a.score[(int64_t)h * k + before + x] = key_value(keys[sel[x]]);
  if (a.pk != nullptr) {
    const int cpr = a.row_bytes / 16;
    for (int x = tid; x < tot * cpr; x += PICK_THREADS) {
      const int rr = x / cpr, ch = x % cpr;
      const int64_t src = h * a.p_hs + (int64_t)sel[rr] * a.p_rs + ch * 16;
      const int64_t dst = h * a.r_hs + (int64_t)(before + rr) * a.r_rs + ch * 16;
      *reinterpret_cast<uint4*>(a.rk + dst) = *reinterpret_cast<const uint4*>(a.pk + src);
      *reinterpret_cast<uint4*>(a.rv + dst) = *reinterpret_cast<const uint4*>(a.pv + src);
    }
  }
}

}  // namespace

// Workspace (from its first 256-byte boundary): the order keys
// [n_heads][npad], the buckets [n_heads][npad] and the group maxima
// [n_heads][npad / GROUP], npad = pool_len rounded up to 64.
size_t topk_workspace_bytes(int n_heads, int pool_len) {
  const int64_t npad = align_up(pool_len, 64);
  return (size_t)(256 + align_up((int64_t)n_heads * npad * 8, 256) + align_up((int64_t)n_heads * npad * 2, 256) +
                  align_up((int64_t)n_heads * (npad / GROUP) * 2, 256));
}

hipError_t launch_topk(int dtype, int n_heads, int pool_len, int d, int k, const void* q,
                       int64_t q_hs, const void* pool_k, const void* pool_v, int64_t p_hs,
                       int64_t p_rs, int32_t* idx, double* score, void* pref_k, void* pref_v,
                       int64_t r_hs, int64_t r_rs, void* ws, hipStream_t s) {
  const int npad = (int)align_up(pool_len, 64);
  char* base = reinterpret_cast<char*>(align_up((int64_t)reinterpret_cast<uintptr_t>(ws), 256));
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(base);
  base += align_up((int64_t)n_heads * npad * 8, 256);
  unsigned short* buckets = reinterpret_cast<unsigned short*>(base);
  base += align_up((int64_t)n_heads * npad * 2, 256);
  unsigned short* gmax = reinterpret_cast<unsigned short*>(base);

  const dim3 g1((unsigned)ceil_div(pool_len, SCORE_ROWS), (unsigned)n_heads);
  const dim3 b1(SCORE_ROWS);
  typedef unsigned short u16;
  if (dtype == SA_BF16 && d == 128)
    hipLaunchKernelGGL((topk_score<u16, 128>), g1, b1, 0, s, static_cast<const u16*>(q), q_hs,
                       static_cast<const u16*>(pool_k), p_hs, p_rs, pool_len, npad, keys, buckets, gmax);
  else if (dtype == SA_BF16)
    hipLaunchKernelGGL((topk_score<u16, 64>), g1, b1, 0, s, static_cast<const u16*>(q), q_hs,
                       static_cast<const u16*>(pool_k), p_hs, p_rs, pool_len, npad, keys, buckets, gmax);
  else if (d == 128)
    hipLaunchKernelGGL((topk_score<float, 128>), g1, b1, 0, s, static_cast<const float*>(q), q_hs,
                       static_cast<const float*>(pool_k), p_hs, p_rs, pool_len, npad, keys, buckets, gmax);
  else
    hipLaunchKernelGGL((topk_score<float, 64>), g1, b1, 0, s, static_cast<const float*>(q), q_hs,
                       static_cast<const float*>(pool_k), p_hs, p_rs, pool_len, npad, keys, buckets, gmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // chunk: about enough work groups to give each of the 256 CUs one, 1024 to
  // CHUNK_MAX indices each
  const int per_head = std::max(1, 256 / n_heads);
  const int chunk = (int)std::min<int64_t>(
      std::max<int64_t>(align_up(ceil_div(pool_len, per_head), PICK_THREADS), PICK_THREADS), CHUNK_MAX);
  const int n_chunks = (int)ceil_div(pool_len, chunk);
  const int esz = dtype == SA_BF16 ? 2 : 4;
  PickArgs a;
  a.keys = keys;
  a.buckets = buckets;
  a.gmax = gmax;
  a.n = pool_len;
  a.npad = npad;
  a.k = k;
  a.chunk = chunk;
  a.n_heads = n_heads;
  a.idx = idx;
  a.score = score;
  a.pk = pool_v == nullptr ? nullptr : static_cast<const char*>(pool_k);
  a.pv = static_cast<const char*>(pool_v);
  a.p_hs = p_hs * esz;
  a.p_rs = p_rs * esz;
  a.rk = static_cast<char*>(pref_k);
  a.rv = static_cast<char*>(pref_v);
  a.r_hs = r_hs * esz;
  a.r_rs = r_rs * esz;
  a.row_bytes = d * esz;
  hipLaunchKernelGGL(topk_pick, dim3((unsigned)(n_chunks * n_heads)), dim3(PICK_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
