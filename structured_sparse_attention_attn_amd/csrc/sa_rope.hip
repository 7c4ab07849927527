// RoPE stage: rotate queries and keys at their positions, gather the SepLLM
// separator rows and precompute the LM-Infinite capped keys.
//
// Rotary embedding: rotate-half pairs (c, c + d/2), theta_c = base^(-2c/d);
// the angle pos * theta_c is formed in fp64 and reduced to a fraction of a
// turn, then the hardware sine and cosine.  Positions (segmented-execution page, method / overall
// framework): keys at their index (the prefix re-indexed to 0..P-1), queries
// at P + i in a segment and at i otherwise.  LM-Infinite page, section
// "method": starting-span keys outside the window keep the raw key and take
// the query rotated to distance L_pretrain; <R(L) q, k> = <q, R(-L) k>, so the
// stage stores R(-L) k_j for j < n_starting and the forward pairs it with the
// raw query.  SepLLM page, part 6.2: only kept keys take part, so the
// separator rows a tile gathers are copied here into one compact array per
// kv head (rotated keys and raw values), in ascending position order.
#include "sa_common.h"

namespace sa {
namespace {

typedef unsigned short u16;

struct RopeArgs {
  const void* q;
  int64_t qsB, qsH, qsT;
  void* qrot;
  int n_q, h_q, q_pos0;
  const void* k;
  int64_t ksB, ksH, ksT;
  void* krot;
  int n_k, h_kv;
  const void* v;
  int64_t vsB, vsH, vsT;
  int B, d, rotate;
  const unsigned long long* sep_bits;
  const int* blk_sep;
  int g0, gather;
  void* ksep;
  void* vsep;
  int64_t sep_rows;
  void* kcap;
  int64_t cap_rows;
  int n_cap, L;
  int n_pos;
  int row0;         // first row handled: B*h_kv when no key row needs work
  int write_q;      // write the query copy (rotated when rotate is set)
  float q_scale;    // factor applied to the stored queries
  float cap_scale;  // factor applied to the stored capped keys
  ThetaTable theta;
};

__device__ inline float bf2f(u16 x) { return __uint_as_float(((unsigned)x) << 16); }

__device__ inline u16 f2bf(float f) {  // round to nearest even (inputs are finite)
  const unsigned u = __float_as_uint(f);
  return (u16)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// cos and sin of an angle given in turns: reduced in fp64 to [-1/2, 1/2],
// then the hardware sine and cosine (whose argument is in turns).
__device__ inline void turn_sincos(double rev, float* c, float* s) {
  const float f = (float)(rev - rint(rev));
  *c = __builtin_amdgcn_cosf(f);
  *s = __builtin_amdgcn_sinf(f);
}

// 8 consecutive elements of a row: 16 bytes (bf16) or 32 bytes (fp32).
template <typename T>
struct Row8;
template <>
struct Row8<u16> {
  uint4 w;
  __device__ void load(const void* p) { w = *reinterpret_cast<const uint4*>(p); }
  __device__ void store(void* p) const { *reinterpret_cast<uint4*>(p) = w; }
  __device__ void get(float* x) const {
    const unsigned u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf2f((u16)(u[e] & 0xffffu));
      x[2 * e + 1] = bf2f((u16)(u[e] >> 16));
    }
  }
  __device__ void set(const float* x) {
    unsigned u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = (unsigned)f2bf(x[2 * e]) | ((unsigned)f2bf(x[2 * e + 1]) << 16);
    w = make_uint4(u[0], u[1], u[2], u[3]);
  }
};
template <>
struct Row8<float> {
  float4 a, b;
  __device__ void load(const void* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ void store(void* p) const {
    reinterpret_cast<float4*>(p)[0] = a;
    reinterpret_cast<float4*>(p)[1] = b;
  }
  __device__ void get(float* x) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  __device__ void set(const float* x) {
    a = make_float4(x[0], x[1], x[2], x[3]);
    b = make_float4(x[4], x[5], x[6], x[7]);
  }
};

constexpr int ROPE_ROWS = 8;  // rows (batch x head) per thread

// Thread = (position, group of 8 rotation pairs, chunk of ROPE_ROWS rows).
// Rows 0 .. B*h_kv-1 are the key rows of the position, the rest its query
// rows; chunks start at row0, past the key rows when they need no work (no
// rotation and no separator gather).  The sincos values are computed once per thread and reused for its
// rows; all of a thread's row loads are issued before its first store.
template <typename T>
__global__ __launch_bounds__(256) void rope_qk(RopeArgs p) {
  const int esz = sizeof(T);
  const int tpr = p.d / 16;  // threads per position: d/2 pairs, 8 per thread
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int pos = (int)(gid / tpr);
  if (pos >= p.n_pos) return;
  const int c0 = (int)(gid % tpr) * 8;
  const int half = p.d / 2;
  const int n_krows = pos < p.n_k ? p.B * p.h_kv : 0;
  const int i = pos - p.q_pos0;
  const int n_qrows = (p.write_q && i >= 0 && i < p.n_q) ? p.B * p.h_q : 0;
  const int r_begin = p.row0 + blockIdx.y * ROPE_ROWS;
  if (r_begin >= p.B * (p.h_kv + p.h_q)) return;
  // key-row extras of this position: separator rank (its plan reads go out
  // before the row loads, so waiting for them does not wait for the rows)
  bool is_sep = false;
  int64_t rank = 0;
  if (pos < p.n_k && p.gather && pos >= p.g0) {
    const int blk = pos / BK;
    const unsigned long long word = p.sep_bits[blk];
    const int r = pos - blk * BK;
    if ((word >> r) & 1ull) {
      is_sep = true;
      rank = p.blk_sep[blk] + __popcll(word & ((r == 0) ? 0ull : (~0ull >> (64 - r))));
    }
  }
  const int hk = p.B * p.h_kv;
  Row8<T> in1[ROPE_ROWS], in2[ROPE_ROWS];
#pragma unroll
  for (int rr = 0; rr < ROPE_ROWS; ++rr) {
    const int r = r_begin + rr;
    const char* src = nullptr;
    if (r < hk) {
      if (r < n_krows) {
        const int b = r / p.h_kv, h = r - b * p.h_kv;
        src = static_cast<const char*>(p.k) + (b * p.ksB + h * p.ksH + pos * p.ksT) * esz;
      }
    } else if (r - hk < n_qrows) {
      const int b = (r - hk) / p.h_q, h = (r - hk) - b * p.h_q;
      src = static_cast<const char*>(p.q) + (b * p.qsB + h * p.qsH + (int64_t)i * p.qsT) * esz;
    }
    if (src) {
      in1[rr].load(src + c0 * esz);
      in2[rr].load(src + (c0 + half) * esz);
    }
  }
  // cos and sin of pos * theta_c, c = c0 .. c0+7 (and of -L * theta_c for the
  // capped keys), after the row loads are in flight: theta_c / (2 pi) from
  // theta_{c0} times powers of base^(-2/d) in fp64, the angle reduced in fp64
  // to a fraction of a turn, then the hardware sine and cosine (which take
  // turns)
  const bool is_cap = p.rotate && pos < p.n_cap;
  float cs[8], sn[8], ccs[8], csn[8];
  if (p.rotate) {
    // theta_{c0} = (base^(-16/d))^(c0/8) from table entries 8, 16, 32 (uniform
    // loads, no per-lane memory read); th[0] = 1
    const int e8 = c0 >> 3;
    double t = ((e8 & 1) ? p.theta.th[8] : 1.0) * ((e8 & 2) ? p.theta.th[16] : 1.0) *
               ((e8 & 4) ? p.theta.th[32] : 1.0) * 0.15915494309189535;
    const double r1 = p.theta.th[1];  // base^(-2/d)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      turn_sincos((double)pos * t, &cs[e], &sn[e]);
      if (is_cap) turn_sincos(-(double)p.L * t, &ccs[e], &csn[e]);
      t *= r1;
    }
  }
#pragma unroll
  for (int rr = 0; rr < ROPE_ROWS; ++rr) {
    const int r = r_begin + rr;
    float x1[8], x2[8], y1[8], y2[8];
    if (r < hk) {
      if (r >= n_krows) continue;
      const int b = r / p.h_kv, h = r - b * p.h_kv;
      in1[rr].get(x1);
      in2[rr].get(x2);
      const int64_t orow = ((int64_t)b * p.h_kv + h) * p.n_k + pos;
      if (p.rotate) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          y1[e] = x1[e] * cs[e] - x2[e] * sn[e];
          y2[e] = x2[e] * cs[e] + x1[e] * sn[e];
        }
        Row8<T> o1, o2;
        o1.set(y1);
        o2.set(y2);
        char* dst = static_cast<char*>(p.krot) + orow * p.d * esz;
        o1.store(dst + c0 * esz);
        o2.store(dst + (c0 + half) * esz);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { y1[e] = x1[e]; y2[e] = x2[e]; }
      }
      if (is_sep && rank < p.sep_rows) {  // rows past a broken sep_max bound are dropped
        const int64_t srow = ((int64_t)b * p.h_kv + h) * p.sep_rows + rank;
        char* kd = static_cast<char*>(p.ksep) + srow * p.d * esz;
        Row8<T> o1, o2;
        o1.set(y1);
        o2.set(y2);
        o1.store(kd + c0 * esz);
        o2.store(kd + (c0 + half) * esz);
        const char* vs = static_cast<const char*>(p.v) + (b * p.vsB + h * p.vsH + pos * p.vsT) * esz;
        char* vd = static_cast<char*>(p.vsep) + srow * p.d * esz;
        Row8<T> v1, v2;
        v1.load(vs + c0 * esz);
        v2.load(vs + (c0 + half) * esz);
        v1.store(vd + c0 * esz);
        v2.store(vd + (c0 + half) * esz);
      }
      if (is_cap) {
        float z1[8], z2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          z1[e] = (x1[e] * ccs[e] - x2[e] * csn[e]) * p.cap_scale;
          z2[e] = (x2[e] * ccs[e] + x1[e] * csn[e]) * p.cap_scale;
        }
        const int64_t crow = ((int64_t)b * p.h_kv + h) * p.cap_rows + pos;
        char* cd = static_cast<char*>(p.kcap) + crow * p.d * esz;
        Row8<T> o1, o2;
        o1.set(z1);
        o2.set(z2);
        o1.store(cd + c0 * esz);
        o2.store(cd + (c0 + half) * esz);
      }
    } else {
      if (r - hk >= n_qrows) continue;
      const int b = (r - hk) / p.h_q, h = (r - hk) - b * p.h_q;
      in1[rr].get(x1);
      in2[rr].get(x2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (p.rotate) {
          y1[e] = (x1[e] * cs[e] - x2[e] * sn[e]) * p.q_scale;
          y2[e] = (x2[e] * cs[e] + x1[e] * sn[e]) * p.q_scale;
        } else {
          y1[e] = x1[e] * p.q_scale;
          y2[e] = x2[e] * p.q_scale;
        }
      }
      const int64_t orow = ((int64_t)b * p.h_q + h) * p.n_q + i;
      char* dst = static_cast<char*>(p.qrot) + orow * p.d * esz;
      Row8<T> o1, o2;
      o1.set(y1);
      o2.set(y2);
      o1.store(dst + c0 * esz);
      o2.store(dst + (c0 + half) * esz);
    }
  }
}

}  // namespace

hipError_t launch_rope(const sa_mask_t& m, const sa_plan_header_t& lay, const void* plan,
                       const sa_fwd_args_t& a, const ThetaTable& theta, const RopeOut& ro,
                       hipStream_t s) {
  RopeArgs p;
  memset(&p, 0, sizeof(p));
  const bool rotate = a.rope == SA_ROPE_HALF;
  const bool gather = m.kind == SA_MASK_SEPLLM && m.sep != nullptr;
  // The query copy is written where the caller provides one: the fp32
  // forward reads rotated queries (it keeps the scale itself); the bf16
  // backward reads them rotated and pre-multiplied by scale * log2(e).  The
  // bf16 forward prepares its queries in registers and passes no copy.
  const bool write_q = ro.qrot != nullptr && (rotate || a.dtype == SA_BF16);
  if (!write_q && !gather && !rotate) return hipSuccess;
  const char* pb = static_cast<const char*>(plan);
  p.q = a.q;
  p.qsB = a.q_stride[0]; p.qsH = a.q_stride[1]; p.qsT = a.q_stride[2];
  p.qrot = ro.qrot;
  p.n_q = m.n_q;
  p.h_q = a.h_q;
  p.q_pos0 = m.kind == SA_MASK_SEGMENT ? m.prefix_len : 0;
  p.k = a.k;
  p.ksB = a.k_stride[0]; p.ksH = a.k_stride[1]; p.ksT = a.k_stride[2];
  p.krot = ro.krot;
  p.n_k = m.n_k;
  p.h_kv = a.h_kv;
  p.v = a.v;
  p.vsB = a.v_stride[0]; p.vsH = a.v_stride[1]; p.vsT = a.v_stride[2];
  p.B = a.batch;
  p.d = a.d;
  p.rotate = rotate ? 1 : 0;
  p.sep_bits = reinterpret_cast<const unsigned long long*>(pb + lay.off_sep_bits);
  p.blk_sep = reinterpret_cast<const int*>(pb + lay.off_blk_sep);
  p.g0 = lay.g0;
  p.gather = gather ? 1 : 0;
  p.ksep = ro.ksep;
  p.vsep = ro.vsep;
  p.sep_rows = ro.sep_rows;
  p.kcap = ro.kcap;
  p.cap_rows = ro.cap_rows;
  p.n_cap = ro.n_cap;
  p.L = m.L_pretrain;
  p.write_q = write_q ? 1 : 0;
  p.q_scale = a.dtype == SA_BF16 ? a.scale * 1.4426950408889634f : 1.0f;
  p.cap_scale = p.q_scale;
  p.n_pos = m.n_k;
  if (write_q && p.q_pos0 + m.n_q > p.n_pos) p.n_pos = p.q_pos0 + m.n_q;
  p.theta = theta;
  const int64_t threads = (int64_t)p.n_pos * (a.d / 16);
  const unsigned wg = (unsigned)ceil_div(threads, 256);
  p.row0 = (rotate || gather) ? 0 : a.batch * a.h_kv;
  // rows past the key rows are query rows: only when the query copy is written
  const int64_t rows = (int64_t)a.batch * a.h_kv + (write_q ? (int64_t)a.batch * a.h_q : 0);
  const unsigned chunks = (unsigned)ceil_div(rows - p.row0, ROPE_ROWS);
  if (a.dtype == SA_BF16)
    hipLaunchKernelGGL(rope_qk<unsigned short>, dim3(wg, chunks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(rope_qk<float>, dim3(wg, chunks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace sa
