// Streaming decode with the generation-time cache (SepLLM page, part 6.2,
// generation): Initial (the first a tokens), Separator (at most s separators),
// Local window (the last w tokens) and Past (tokens that left the local window
// since the last compression).  When a + s + w + |Past| reaches c, Past's
// separators join the Separator part in order, its oldest beyond s dropped,
// and Past is emptied; then the new query attends to every held token.
//
// Slot layout per (sequence, kv head): [0, a) Initial, [a, a+s) Separator
// ring, [a+s, a+s+P) Past (P = c - a - s - w), [a+s+P, c) Local ring.  Both
// rings fill from slot 0 and start to wrap only once full, so the held slots
// are always four contiguous ranges.  Keys are stored rotated at their
// original positions; a query never needs them moved again.
//
// Per step: stream_insert (one work group per (sequence, kv head): the moved
// and compressed rows, the new key and value, the rotated queries), then
// decode_attn (split over slots: partial softmax per 64 slots, over the held
// ranges the step leaves) and decode_combine (the splits merged; its extra
// work groups, one per sequence, record each slot's token index and
// separator flag and advance the counters).
#include <atomic>

#include "sa_common.h"

namespace sa {
namespace {

typedef unsigned short u16;

enum { C_T = 0, C_NINIT = 1, C_NSEP = 2, C_SEPHEAD = 3, C_NPAST = 4, C_NLOCAL = 5, C_LOCALHEAD = 6 };
constexpr int SPLIT = 64;   // slots per decode work group
constexpr int MAX_G = 8;    // query heads per kv head

struct StreamArgs {
  char* kc;                  // [B, h_kv, c, d] bf16 rows
  char* vc;
  int* pos;                  // [B, c] token index of each slot
  unsigned char* flag;       // [B, c] separator flag of each slot
  int* ctrl;                 // [B, 8] counters
  const u16* q;              // [B, h_q, d]
  const u16* k;              // [B, h_kv, d]
  const u16* v;
  const unsigned char* is_sep;  // [B]
  float* qrot;               // [B, h_q, d] rotated, scaled by scale * log2(e)
  float* capl;               // [B, h_q, a] LAMBDA: base-2 logits of the capped starting keys
  float* part;               // [B, h_q, n_split, d + 2]
  u16* o;                    // [B, h_q, d]
  float* lse;                // [B, h_q] or null
  int B, h_q, h_kv, d, a, s, w, c, P, group, rotate, n_split;
  int lambda, L;             // LAMBDA: no Separator or Past part; starting keys capped at L
  float scale_log2;
  ThetaTable theta;
};

__device__ inline float bf2f(u16 x) { return __uint_as_float(((unsigned)x) << 16); }
// element e (0..7, compile-time) of 8 packed bf16 values, widened to fp32
__device__ inline float bf_at(const uint4& x, int e) {
  const unsigned w = (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}
__device__ inline u16 f2bf(float f) {  // round to nearest even (finite inputs)
  const unsigned u = __float_as_uint(f);
  return (u16)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ inline void angle_sincos(double pos, double th, float* c, float* s) {
  const double TWO_PI_HI = 6.283185307179586232;
  const double TWO_PI_LO = 2.4492935982947064e-16;
  const double INV_TWO_PI = 0.15915494309189535;
  const double ang = pos * th;
  const double kq = rint(ang * INV_TWO_PI);
  double r = fma(-kq, TWO_PI_HI, ang);
  r = fma(-kq, TWO_PI_LO, r);
  sincosf((float)r, s, c);
}

// What this step does to one sequence's cache, from its counters.
struct StepPlan {
  int t, ns;          // new token index and slot
  bool evict;         // the oldest local token leaves the window (slot ms)
  int ms;
  bool compress;      // ... and fills Past: compression
  int n_past;         // Past size before the step
};

__device__ inline StepPlan plan_step(const StreamArgs& p, const int* ct) {
  StepPlan sp;
  sp.t = ct[C_T];
  sp.n_past = ct[C_NPAST];
  const int n_local = ct[C_NLOCAL], head = ct[C_LOCALHEAD];
  const int L0 = p.a + p.s + p.P;
  sp.evict = false;
  sp.compress = false;
  sp.ms = 0;
  if (sp.t < p.a) {
    sp.ns = sp.t;
  } else if (n_local < p.w) {
    sp.ns = L0 + n_local;
  } else {
    sp.evict = true;
    sp.ms = L0 + head;
    sp.ns = sp.ms;
    sp.compress = sp.n_past + 1 == p.P;
  }
  return sp;
}

// Compression of one sequence, computed by one wave: Past items i < P are the
// Past slots a+s+i (i < n_past) and the evicted local token (i = n_past).  The
// separators among them, in order, are appended to the Separator ring; the
// k-th goes to ring slot (head + n_sep + k) mod s and survives only if it is
// among the last s appended.  Writes the survivors' (source slot, ring slot)
// to list[] and returns their count; n_new receives the separator count.
__device__ inline int compress_list(const StreamArgs& p, int b, const int* ct, const StepPlan& sp, int lane,
                                    int* list_src, int* list_dst, int* n_new_out) {
  const unsigned char* fl = p.flag + (int64_t)b * p.c;
  auto src_of = [&](int i) { return i < sp.n_past ? p.a + p.s + i : sp.ms; };
  int n_new = 0;
  for (int i0 = 0; i0 < p.P; i0 += 64) {
    const int i = i0 + lane;
    const bool f = i < p.P && fl[src_of(i)] != 0;
    n_new += __popcll(__ballot(f));
  }
  const int n_sep = ct[C_NSEP], head = ct[C_SEPHEAD];
  const int first = max(0, n_new - p.s);  // appends before this one are overwritten
  int rank0 = 0;
  for (int i0 = 0; i0 < p.P; i0 += 64) {
    const int i = i0 + lane;
    const bool f = i < p.P && fl[src_of(i)] != 0;
    const unsigned long long m = __ballot(f);
    const int k = rank0 + __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
    if (f && k >= first) {
      list_src[k - first] = src_of(i);
      list_dst[k - first] = p.a + (head + n_sep + k) % p.s;
    }
    rank0 += __popcll(m);
  }
  *n_new_out = n_new;
  return n_new - first;
}

__global__ __launch_bounds__(256) void stream_insert(StreamArgs p) {
  __shared__ int list_src[4096];
  __shared__ int list_dst[4096];
  __shared__ int n_list;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = blockIdx.x / p.h_kv, g = blockIdx.x % p.h_kv;
  const int* ct = p.ctrl + b * 8;
  const StepPlan sp = plan_step(p, ct);
  char* K = p.kc + ((int64_t)b * p.h_kv + g) * p.c * 256;
  char* V = p.vc + ((int64_t)b * p.h_kv + g) * p.c * 256;

  // phase A: every read of a slot this step overwrites
  if (sp.compress && wid == 0) {
    int n_new;
    const int n = compress_list(p, b, ct, sp, lane, list_src, list_dst, &n_new);
    if (lane == 0) n_list = n;
  }
  __syncthreads();
  if (sp.compress) {
    // survivors to the Separator ring (ring slots are read by nobody here)
    const int n = n_list;
    for (int e = tid; e < n * 32; e += 256) {
      const int r = e >> 5, piece = e & 31;
      const char* srcb = piece < 16 ? K : V;
      char* dstb = piece < 16 ? K : V;
      const int pc = piece & 15;
      *reinterpret_cast<uint4*>(dstb + (int64_t)list_dst[r] * 256 + pc * 16) =
          *reinterpret_cast<const uint4*>(srcb + (int64_t)list_src[r] * 256 + pc * 16);
    }
  } else if (sp.evict && tid < 32 && !p.lambda) {
    // the evicted local token enters Past (LAMBDA: it is dropped)
    const int pc = tid & 15;
    char* base = tid < 16 ? K : V;
    *reinterpret_cast<uint4*>(base + (int64_t)(p.a + p.s + sp.n_past) * 256 + pc * 16) =
        *reinterpret_cast<const uint4*>(base + (int64_t)sp.ms * 256 + pc * 16);
  }
  __syncthreads();

  // phase B: the new token's key (rotated at t) and value, and the rotated queries
  const int half = p.d / 2;
  if (tid < half) {
    const int c0 = tid;
    const u16* kr = p.k + ((int64_t)b * p.h_kv + g) * p.d;
    float x1 = bf2f(kr[c0]), x2 = bf2f(kr[c0 + half]);
    if (p.rotate) {
      float cs, sn;
      angle_sincos((double)sp.t, p.theta.th[c0], &cs, &sn);
      const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
      x1 = y1;
      x2 = y2;
    }
    u16* dst = reinterpret_cast<u16*>(K + (int64_t)sp.ns * 256);
    dst[c0] = f2bf(x1);
    dst[c0 + half] = f2bf(x2);
  } else if (tid < half + 16) {
    const int pc = tid - half;
    const char* vr = reinterpret_cast<const char*>(p.v + ((int64_t)b * p.h_kv + g) * p.d);
    *reinterpret_cast<uint4*>(V + (int64_t)sp.ns * 256 + pc * 16) = *reinterpret_cast<const uint4*>(vr + pc * 16);
  }
  for (int e = tid; e < p.group * half; e += 256) {
    const int gq = e / half, c0 = e % half;
    const int hq = g * p.group + gq;
    const u16* qr = p.q + ((int64_t)b * p.h_q + hq) * p.d;
    float x1 = bf2f(qr[c0]), x2 = bf2f(qr[c0 + half]);
    if (p.rotate) {
      float cs, sn;
      angle_sincos((double)sp.t, p.theta.th[c0], &cs, &sn);
      const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
      x1 = y1;
      x2 = y2;
    }
    float* qd = p.qrot + ((int64_t)b * p.h_q + hq) * p.d;
    qd[c0] = x1 * p.scale_log2;
    qd[c0 + half] = x2 * p.scale_log2;
  }
  // LAMBDA: the starting keys j with t - j > L take scale <R(L) q, k_j> =
  // scale <R(L + j) q, R(j) k_j> (keys are stored rotated at their index).
  // One wave per starting key, one lane per rotation pair, a wave sum per head.
  if (p.lambda && half == 64) {
    for (int jj = wid; jj < min(p.a, sp.t); jj += 4) {
      if (sp.t - jj <= p.L) continue;
      const int c0 = lane;
      float cs = 1.f, sn = 0.f;
      if (p.rotate) angle_sincos((double)(p.L + jj), p.theta.th[c0], &cs, &sn);
      const u16* kr = reinterpret_cast<const u16*>(K + (int64_t)jj * 256);
      const float k1 = bf2f(kr[c0]), k2 = bf2f(kr[c0 + 64]);
      for (int gq = 0; gq < p.group; ++gq) {
        const int hq = g * p.group + gq;
        const u16* qr = p.q + ((int64_t)b * p.h_q + hq) * p.d;
        const float x1 = bf2f(qr[c0]), x2 = bf2f(qr[c0 + 64]);
        float acc = k1 * (x1 * cs - x2 * sn) + k2 * (x2 * cs + x1 * sn);
        for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
        if (lane == 0) p.capl[((int64_t)b * p.h_q + hq) * p.a + jj] = acc * p.scale_log2;
      }
    }
  }
}

// Token index, flag and counters of sequence b after the step.  Called by
// every thread of a work group (its barriers are uniform); wave 0 works.  On
// compression the survivors' token indices and flags are copied straight to
// their ring slots: the ring and the Past / evicted-local slots they come
// from are disjoint, so no copy reads a slot another has written.
__device__ inline void update_ctrl(const StreamArgs& p, int b) {
  const int lane = threadIdx.x & 63;
  const bool w0 = threadIdx.x < 64;
  int* ct = p.ctrl + b * 8;
  const StepPlan sp = plan_step(p, ct);
  int* pos = p.pos + (int64_t)b * p.c;
  unsigned char* fl = p.flag + (int64_t)b * p.c;
  int n_sep = ct[C_NSEP], head = ct[C_SEPHEAD], n_past = ct[C_NPAST];
  int n_local = ct[C_NLOCAL], lhead = ct[C_LOCALHEAD], n_init = ct[C_NINIT];
  if (sp.compress) {
    auto src_of = [&](int i) { return i < sp.n_past ? p.a + p.s + i : sp.ms; };
    int n_new = 0;
    if (w0) {
      for (int i0 = 0; i0 < p.P; i0 += 64) {
        const int i = i0 + lane;
        n_new += __popcll(__ballot(i < p.P && fl[src_of(i)] != 0));
      }
      const int first = max(0, n_new - p.s);  // appends before this one are overwritten
      int rank0 = 0;
      for (int i0 = 0; i0 < p.P; i0 += 64) {
        const int i = i0 + lane;
        const bool f = i < p.P && fl[src_of(i)] != 0;
        const unsigned long long m = __ballot(f);
        const int k = rank0 + __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        if (f && k >= first) {
          const int dst = p.a + (head + n_sep + k) % p.s;
          pos[dst] = pos[src_of(i)];
          fl[dst] = fl[src_of(i)];
        }
        rank0 += __popcll(m);
      }
    }
    __syncthreads();  // (only thread 0 uses the counts below; wave 0's lanes agree on n_new)
    head = (head + max(0, n_sep + n_new - p.s)) % p.s;
    n_sep = min(p.s, n_sep + n_new);
    n_past = 0;
  } else if (sp.evict && !p.lambda) {
    if (threadIdx.x == 0) {
      pos[p.a + p.s + n_past] = pos[sp.ms];
      fl[p.a + p.s + n_past] = fl[sp.ms];
    }
    n_past += 1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (sp.t < p.a) {
      n_init = sp.t + 1;
    } else if (!sp.evict) {
      n_local += 1;
    } else {
      lhead = (lhead + 1) % p.w;
    }
    pos[sp.ns] = sp.t;
    fl[sp.ns] = (p.is_sep != nullptr && p.is_sep[b] != 0) ? 1 : 0;
    ct[C_T] = sp.t + 1;
    ct[C_NINIT] = n_init;
    ct[C_NSEP] = n_sep;
    ct[C_SEPHEAD] = head;
    ct[C_NPAST] = n_past;
    ct[C_NLOCAL] = n_local;
    ct[C_LOCALHEAD] = lhead;
  }
}

// Held slots per part after a step.
struct Held {
  int n_init, n_sep, n_past, n_local;
};

// Partial softmax of the group's queries over 64 held slots: (m, l, o) per
// query head in base 2, over 64 consecutive physical slots (the held ones
// among them).  Every K and V byte of the slots, and the group's queries, are
// requested first, before the counters say which slots are held: thread (slot r, quarter qq) holds a
// quarter of r's key for the logits; thread (slot group sg, column chunk cc)
// holds columns 8 cc .. +7 of the values of slots 4 sg .. 4 sg + 3 for the
// weighted sum, reduced over the 16 slot groups by shuffles within a wave and
// LDS across the 4 waves.  Slots not held take no part: their logits are
// -inf and their values are replaced by zeros (never-written slots may hold
// any bits).
template <bool LAM>
__global__ __launch_bounds__(256) void decode_attn(StreamArgs p) {
  __shared__ float qs[MAX_G][128];
  __shared__ float ps[MAX_G][SPLIT];
  __shared__ float mrow[MAX_G], lrow[MAX_G];
  __shared__ float ored[4][MAX_G][128];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bg = blockIdx.x / p.n_split, spl = blockIdx.x % p.n_split;
  const int b = bg / p.h_kv, g = bg % p.h_kv;
  const int v0 = spl * SPLIT;                      // first physical slot
  const int nslot = min(SPLIT, p.c - v0);          // slots of this work group
  const char* K = p.kc + ((int64_t)b * p.h_kv + g) * p.c * 256;
  const char* V = p.vc + ((int64_t)b * p.h_kv + g) * p.c * 256;
  const int r = tid >> 2, qq = tid & 3;
  uint4 kx4[4];
  {
    const uint4* kp = reinterpret_cast<const uint4*>(K + (int64_t)(v0 + (r < nslot ? r : 0)) * 256 + qq * 64);
#pragma unroll
    for (int e = 0; e < 4; ++e) kx4[e] = kp[e];
  }
  const int sg = tid >> 4, cc = tid & 15;
  uint4 vx4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 4 * sg + i;
    vx4[i] = *reinterpret_cast<const uint4*>(V + (int64_t)(v0 + (rr < nslot ? rr : 0)) * 256 + cc * 16);
  }
  // the group's rotated queries (up to MAX_G * 128 floats: 4 per thread),
  // requested with the rows
  float qv[MAX_G * 128 / 256];
#pragma unroll
  for (int i = 0; i < MAX_G * 128 / 256; ++i) {
    const int e = tid + 256 * i;
    qv[i] = e < p.group * 128 ? p.qrot[((int64_t)b * p.h_q + g * p.group + (e >> 7)) * 128 + (e & 127)] : 0.f;
  }
  // the held ranges after this step, from the counters before it (they are
  // updated by decode_combine, after every read of them in this step)
  __shared__ int n_new_s;
  const int* ct = p.ctrl + b * 8;
  const StepPlan sp = plan_step(p, ct);
  Held h;
  h.n_init = ct[C_NINIT];
  h.n_sep = ct[C_NSEP];
  h.n_past = ct[C_NPAST];
  h.n_local = ct[C_NLOCAL];
  if (sp.t < p.a) h.n_init = sp.t + 1;
  else if (!sp.evict) h.n_local += 1;
  if (sp.compress) {
    if (wv == 0) {
      const unsigned char* fl = p.flag + (int64_t)b * p.c;
      int n_new = 0;
      for (int i0 = 0; i0 < p.P; i0 += 64) {
        const int i = i0 + lane;
        const bool f = i < p.P && fl[i < sp.n_past ? p.a + p.s + i : sp.ms] != 0;
        n_new += __popcll(__ballot(f));
      }
      if (lane == 0) n_new_s = n_new;
    }
    __syncthreads();
    h.n_sep = min(p.s, h.n_sep + n_new_s);
    h.n_past = 0;
  } else if (sp.evict && !p.lambda) {
    h.n_past += 1;
  }
  // Initial [0, n_init), Separator [a, a + n_sep), Past [a + s, a + s + n_past),
  // Local [a + s + P, a + s + P + n_local): the rings fill from their first slot
  auto held = [&](int x) {
    const int x1 = x - p.a, x2 = x1 - p.s, x3 = x2 - p.P;
    return (x < h.n_init) | ((x1 >= 0) & (x1 < h.n_sep)) | ((x2 >= 0) & (x2 < h.n_past)) |
           ((x3 >= 0) & (x3 < h.n_local));
  };
  const bool kok = (r < nslot) && held(v0 + r);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 4 * sg + i;
    if (!((rr < nslot) && held(v0 + rr))) vx4[i] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < MAX_G * 128 / 256; ++i) {
    const int e = tid + 256 * i;
    if (e < p.group * 128) qs[e >> 7][e & 127] = qv[i];
  }
  __syncthreads();
  // logits (bf16 elements widened where they are used: fewer live registers)
  {
    // LAMBDA: a starting key j (its slot index) farther than L from t takes the
    // capped logit computed by stream_insert
    const int jslot = v0 + r;
    const bool capped = LAM && kok && jslot < p.a && sp.t - jslot > p.L;
    for (int gq = 0; gq < p.group; ++gq) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) acc = fmaf(bf_at(kx4[e >> 3], e & 7), qs[gq][qq * 32 + e], acc);
      acc += __shfl_xor(acc, 1, 4);
      acc += __shfl_xor(acc, 2, 4);
      if (capped) acc = p.capl[((int64_t)b * p.h_q + g * p.group + gq) * p.a + jslot];
      if (qq == 0) ps[gq][r] = kok ? acc : -__builtin_huge_valf();
    }
  }
  __syncthreads();
  // softmax pieces: wave gq % 4 handles query head gq
  for (int gq = wv; gq < p.group; gq += 4) {
    const float x = ps[gq][lane];
    float m = x;
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float e = x == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(x - m);
    float l = e;
    for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
    ps[gq][lane] = e;
    if (lane == 0) {
      mrow[gq] = m;  // -inf when no slot of the group is held
      lrow[gq] = l;
    }
  }
  __syncthreads();
  // weighted values: this thread's 4 slots x 8 columns, then the reductions
  for (int gq = 0; gq < p.group; ++gq) {
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pw = ps[gq][4 * sg + i];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = fmaf(pw, bf_at(vx4[i], c), acc[c]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      acc[c] += __shfl_xor(acc[c], 16);
      acc[c] += __shfl_xor(acc[c], 32);
    }
    if (lane < 16) {
#pragma unroll
      for (int c = 0; c < 8; ++c) ored[wv][gq][cc * 8 + c] = acc[c];
    }
  }
  __syncthreads();
  for (int e = tid; e < p.group * 128; e += 256) {
    const int gq = e >> 7, col = e & 127;
    const int hq = g * p.group + gq;
    float* dst = p.part + (((int64_t)b * p.h_q + hq) * p.n_split + spl) * (128 + 2);
    dst[2 + col] = ored[0][gq][col] + ored[1][gq][col] + ored[2][gq][col] + ored[3][gq][col];
    if (col == 0) {
      dst[0] = mrow[gq];
      dst[1] = lrow[gq];
    }
  }
}

// o = sum_i 2^(m_i - m) o_i / sum_i 2^(m_i - m) l_i over the splits, one
// work group per (sequence, query head): the split weights go to LDS, then
// wave w sums splits w, w + 4, ... over all 128 columns (two per lane, eight
// splits' loads in flight), and the four waves' sums are added.  Work groups
// past the last row each advance one sequence's counters.
constexpr int MAX_SPLIT = 1024;  // 65536 slots / SPLIT

__global__ __launch_bounds__(256) void decode_combine(StreamArgs p) {
  __shared__ float wgt[MAX_SPLIT];
  __shared__ float red[4][128];
  __shared__ float rm[4], rl[4];
  const int n_rows = p.B * p.h_q;
  if ((int)blockIdx.x >= n_rows) {
    update_ctrl(p, blockIdx.x - n_rows);
    return;
  }
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ns = p.n_split;
  const float* pr = p.part + (int64_t)row * ns * 130;
  float m = -__builtin_huge_valf();
  for (int i = tid; i < ns; i += 256) m = fmaxf(m, pr[i * 130]);
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) rm[wv] = m;
  __syncthreads();
  m = fmaxf(fmaxf(rm[0], rm[1]), fmaxf(rm[2], rm[3]));
  float l = 0.f;
  for (int i = tid; i < ns; i += 256) {
    const float mi = pr[i * 130];
    const float f = mi == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(mi - m);
    wgt[i] = f;
    l = fmaf(pr[i * 130 + 1], f, l);
  }
  for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
  if (lane == 0) rl[wv] = l;
  __syncthreads();
  l = rl[0] + rl[1] + rl[2] + rl[3];
  float2 acc = make_float2(0.f, 0.f);
  const float* col = pr + 2 + 2 * lane;
  int i = wv;
  for (; i + 28 < ns; i += 32) {  // eight splits per round
    float2 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const float2*>(col + (int64_t)(i + 4 * u) * 130);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float f = wgt[i + 4 * u];
      acc.x = fmaf(f, x[u].x, acc.x);
      acc.y = fmaf(f, x[u].y, acc.y);
    }
  }
  for (; i < ns; i += 4) {
    const float2 x = *reinterpret_cast<const float2*>(col + (int64_t)i * 130);
    const float f = wgt[i];
    acc.x = fmaf(f, x.x, acc.x);
    acc.y = fmaf(f, x.y, acc.y);
  }
  red[wv][2 * lane] = acc.x;
  red[wv][2 * lane + 1] = acc.y;
  __syncthreads();
  if (tid < 128) {
    const float sum = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
    p.o[(int64_t)row * 128 + tid] = f2bf(sum / l);
    if (p.lse != nullptr && tid == 0) p.lse[row] = (m + __log2f(l)) * 0.6931471805599453f;
  }
}

__global__ void stream_zero(int* ctrl, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) ctrl[i] = 0;
}

}  // namespace

StreamLayout stream_layout(const sa_stream_cfg_t& cfg) {
  StreamLayout L;
  const int64_t rows = (int64_t)cfg.batch * cfg.h_kv * cfg.c;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  L.k = take(rows * cfg.d * 2);
  L.v = take(rows * cfg.d * 2);
  L.pos = take((int64_t)cfg.batch * cfg.c * 4);
  L.flag = take((int64_t)cfg.batch * cfg.c);
  L.ctrl = take((int64_t)cfg.batch * 8 * 4);
  L.total = off;
  L.n_split = (int)ceil_div(cfg.c, SPLIT);
  L.ws_qrot = 0;
  L.ws_capl = align_up((int64_t)cfg.batch * cfg.h_q * cfg.d * 4, 256);
  L.ws_part = L.ws_capl + align_up((int64_t)cfg.batch * cfg.h_q * (cfg.a > 0 ? cfg.a : 1) * 4, 256);
  L.ws_total = L.ws_part + (int64_t)cfg.batch * cfg.h_q * L.n_split * (cfg.d + 2) * 4;
  return L;
}

hipError_t launch_stream_reset(const sa_stream_cfg_t& cfg, void* state, hipStream_t s) {
  const StreamLayout L = stream_layout(cfg);
  int* ctrl = reinterpret_cast<int*>(static_cast<char*>(state) + L.ctrl);
  const int n = cfg.batch * 8;
  hipLaunchKernelGGL(stream_zero, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, ctrl, n);
  return hipGetLastError();
}

hipError_t launch_decode_step(const sa_stream_cfg_t& cfg, void* state, const void* q, const void* k,
                              const void* v, const uint8_t* is_sep, void* o, float* lse, void* ws,
                              const ThetaTable& theta, hipStream_t s) {
  const StreamLayout L = stream_layout(cfg);
  char* st = static_cast<char*>(state);
  char* w = static_cast<char*>(ws);
  StreamArgs p;
  memset(&p, 0, sizeof(p));
  p.kc = st + L.k;
  p.vc = st + L.v;
  p.pos = reinterpret_cast<int*>(st + L.pos);
  p.flag = reinterpret_cast<unsigned char*>(st + L.flag);
  p.ctrl = reinterpret_cast<int*>(st + L.ctrl);
  p.q = static_cast<const u16*>(q);
  p.k = static_cast<const u16*>(k);
  p.v = static_cast<const u16*>(v);
  p.is_sep = is_sep;
  p.qrot = reinterpret_cast<float*>(w + L.ws_qrot);
  p.capl = reinterpret_cast<float*>(w + L.ws_capl);
  p.part = reinterpret_cast<float*>(w + L.ws_part);
  p.o = static_cast<u16*>(o);
  p.lse = lse;
  p.B = cfg.batch;
  p.h_q = cfg.h_q;
  p.h_kv = cfg.h_kv;
  p.d = cfg.d;
  p.a = cfg.a;
  p.s = cfg.s;
  p.w = cfg.w;
  p.c = cfg.c;
  p.P = cfg.c - cfg.a - cfg.s - cfg.w;
  p.lambda = cfg.kind == SA_MASK_LAMBDA ? 1 : 0;
  p.L = cfg.L_pretrain;
  p.group = cfg.h_q / cfg.h_kv;
  p.rotate = cfg.rope == SA_ROPE_HALF ? 1 : 0;
  p.n_split = L.n_split;
  p.scale_log2 = cfg.scale * 1.4426950408889634f;
  p.theta = theta;
  hipLaunchKernelGGL(stream_insert, dim3((unsigned)(cfg.batch * cfg.h_kv)), dim3(256), 0, s, p);
  if (p.lambda)
    hipLaunchKernelGGL(decode_attn<true>, dim3((unsigned)(cfg.batch * cfg.h_kv * L.n_split)), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(decode_attn<false>, dim3((unsigned)(cfg.batch * cfg.h_kv * L.n_split)), dim3(256), 0, s, p);
  hipLaunchKernelGGL(decode_combine, dim3((unsigned)(cfg.batch * cfg.h_q + cfg.batch)), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Per-step scratch of the no-allocation decode step: one array in each GPU's
// memory, held until the process ends.  Host code never passes the array's
// name to a kernel; it uses the device address hipGetSymbolAddress returns,
// looked up once per device (with that device current) and kept.  Every
// value a step reads from it is written earlier in the same step (rotated
// queries, capped logits, per-split partial sums), so nothing is cleared.
static __device__ __align__(256) char scratch[SA_DECODE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDev = 64;
std::atomic<void*> g_scratch[kMaxScratchDev];
}  // namespace

hipError_t decode_static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDev) return hipErrorInvalidDevice;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return hipSuccess;
}

}  // namespace sa
