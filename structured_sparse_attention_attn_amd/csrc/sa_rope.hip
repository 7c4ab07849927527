// RoPE stage: rotate queries and keys at their positions, gather the SepLLM
// separator rows and precompute the LM-Infinite capped keys.
//
// Rotary embedding: rotate-half pairs (c, c + d/2), theta_c = base^(-2c/d);
// the angle pos * theta_c is formed and reduced modulo 2*pi in fp64, then one
// fp32 sincos.  Positions (segmented-execution page, method / overall
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

template <typename T>
struct Vec4;
template <>
struct Vec4<float> {
  __device__ static void load(const void* p, float* x) {
    const float4 t = *reinterpret_cast<const float4*>(p);
    x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
  }
  __device__ static void store(void* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
  __device__ static void copy(void* dst, const void* src) {
    *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(src);
  }
};
template <>
struct Vec4<u16> {
  __device__ static void load(const void* p, float* x) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    x[0] = bf2f((u16)(t.x & 0xffffu)); x[1] = bf2f((u16)(t.x >> 16));
    x[2] = bf2f((u16)(t.y & 0xffffu)); x[3] = bf2f((u16)(t.y >> 16));
  }
  __device__ static void store(void* p, const float* x) {
    uint2 t;
    t.x = (unsigned)f2bf(x[0]) | ((unsigned)f2bf(x[1]) << 16);
    t.y = (unsigned)f2bf(x[2]) | ((unsigned)f2bf(x[3]) << 16);
    *reinterpret_cast<uint2*>(p) = t;
  }
  __device__ static void copy(void* dst, const void* src) {
    *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
  }
};

// cos and sin of pos * theta: fp64 product and reduction, fp32 sincos.
__device__ inline void angle_sincos(double pos, double th, float* c, float* s) {
  const double TWO_PI_HI = 6.283185307179586232;     // nearest double to 2*pi
  const double TWO_PI_LO = 2.4492935982947064e-16;   // 2*pi - TWO_PI_HI
  const double INV_TWO_PI = 0.15915494309189535;
  const double ang = pos * th;
  const double kq = rint(ang * INV_TWO_PI);
  double r = fma(-kq, TWO_PI_HI, ang);
  r = fma(-kq, TWO_PI_LO, r);
  sincosf((float)r, s, c);
}

// Thread = (position p, group of 4 rotation pairs).  The sincos values are
// computed once per thread and reused for every batch row and head.
template <typename T>
__global__ __launch_bounds__(256) void rope_qk(RopeArgs p) {
  const int esz = sizeof(T);
  const int tpr = p.d / 8;  // threads per position: d/2 pairs, 4 per thread
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int pos = (int)(gid / tpr);
  if (pos >= p.n_pos) return;
  const int c0 = (int)(gid % tpr) * 4;
  const int half = p.d / 2;
  float cs[4], sn[4];
  if (p.rotate) {
#pragma unroll
    for (int e = 0; e < 4; ++e) angle_sincos((double)pos, p.theta.th[c0 + e], &cs[e], &sn[e]);
  }
  // keys
  if (pos < p.n_k) {
    const int blk = pos / BK;
    bool is_sep = false;
    int64_t rank = 0;
    if (p.gather && pos >= p.g0) {
      const unsigned long long word = p.sep_bits[blk];
      const int r = pos - blk * BK;
      if ((word >> r) & 1ull) {
        is_sep = true;
        rank = p.blk_sep[blk] + __popcll(word & ((r == 0) ? 0ull : (~0ull >> (64 - r))));
      }
    }
    const bool is_cap = p.rotate && pos < p.n_cap;
    float ccs[4], csn[4];
    if (is_cap) {
#pragma unroll
      for (int e = 0; e < 4; ++e) angle_sincos(-(double)p.L, p.theta.th[c0 + e], &ccs[e], &csn[e]);
    }
    for (int b = 0; b < p.B; ++b) {
      for (int h = 0; h < p.h_kv; ++h) {
        const char* src = static_cast<const char*>(p.k) + (b * p.ksB + h * p.ksH + pos * p.ksT) * esz;
        const int64_t orow = ((int64_t)b * p.h_kv + h) * p.n_k + pos;
        float x1[4], x2[4], y1[4], y2[4];
        Vec4<T>::load(src + c0 * esz, x1);
        Vec4<T>::load(src + (c0 + half) * esz, x2);
        if (p.rotate) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y1[e] = x1[e] * cs[e] - x2[e] * sn[e];
            y2[e] = x2[e] * cs[e] + x1[e] * sn[e];
          }
          char* dst = static_cast<char*>(p.krot) + orow * p.d * esz;
          Vec4<T>::store(dst + c0 * esz, y1);
          Vec4<T>::store(dst + (c0 + half) * esz, y2);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) { y1[e] = x1[e]; y2[e] = x2[e]; }
        }
        if (is_sep) {
          const int64_t srow = ((int64_t)b * p.h_kv + h) * p.sep_rows + rank;
          char* kd = static_cast<char*>(p.ksep) + srow * p.d * esz;
          Vec4<T>::store(kd + c0 * esz, y1);
          Vec4<T>::store(kd + (c0 + half) * esz, y2);
          const char* vs = static_cast<const char*>(p.v) + (b * p.vsB + h * p.vsH + pos * p.vsT) * esz;
          char* vd = static_cast<char*>(p.vsep) + srow * p.d * esz;
          Vec4<T>::copy(vd + c0 * esz, vs + c0 * esz);
          Vec4<T>::copy(vd + (c0 + half) * esz, vs + (c0 + half) * esz);
        }
        if (is_cap) {
          float z1[4], z2[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            z1[e] = (x1[e] * ccs[e] - x2[e] * csn[e]) * p.cap_scale;
            z2[e] = (x2[e] * ccs[e] + x1[e] * csn[e]) * p.cap_scale;
          }
          const int64_t crow = ((int64_t)b * p.h_kv + h) * p.cap_rows + pos;
          char* cd = static_cast<char*>(p.kcap) + crow * p.d * esz;
          Vec4<T>::store(cd + c0 * esz, z1);
          Vec4<T>::store(cd + (c0 + half) * esz, z2);
        }
      }
    }
  }
  // queries
  const int i = pos - p.q_pos0;
  if (p.write_q && i >= 0 && i < p.n_q) {
    for (int b = 0; b < p.B; ++b) {
      for (int h = 0; h < p.h_q; ++h) {
        const char* src = static_cast<const char*>(p.q) + (b * p.qsB + h * p.qsH + i * p.qsT) * esz;
        float x1[4], x2[4], y1[4], y2[4];
        Vec4<T>::load(src + c0 * esz, x1);
        Vec4<T>::load(src + (c0 + half) * esz, x2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
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
        Vec4<T>::store(dst + c0 * esz, y1);
        Vec4<T>::store(dst + (c0 + half) * esz, y2);
      }
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
  // bf16: the forward reads queries pre-multiplied by scale * log2(e) (its
  // logits come out of the MFMA in base-2 units), so the query copy is always
  // written; fp32 keeps the scale in the forward.
  const bool write_q = rotate || a.dtype == SA_BF16;
  if (!write_q && !gather) return hipSuccess;
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
  const int64_t threads = (int64_t)p.n_pos * (a.d / 8);
  const unsigned wg = (unsigned)ceil_div(threads, 256);
  if (a.dtype == SA_BF16)
    hipLaunchKernelGGL(rope_qk<unsigned short>, dim3(wg), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(rope_qk<float>, dim3(wg), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace sa
