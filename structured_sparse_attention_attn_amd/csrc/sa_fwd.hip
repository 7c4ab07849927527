// Fused sparse attention forward over the plan's live blocks.
//
// What is computed (SepLLM page part 6.1 and 6.2; LM-Infinite page section
// "method"; segmented-execution page method / overall framework): for each
// query i, O_i = sum_{j in A_i} softmax_j(scale * <q_i, k_j>) v_j over the
// rotated queries and keys, with masked pairs excluded (-inf); LM-Infinite
// pairs farther than L_pretrain use <q_i raw, R(-L) k_j>.  Only the blocks of
// Q K^T that hold a visible pair are computed: the plan lists them per
// 128-query tile, and SepLLM tiles read their far separators from the
// compacted rows gathered by the RoPE stage.
//
// Work units of a tile, all folded into one fp32 online softmax (base-2, the
// scale times log2(e) applied to the logits):
//   1. LM-Infinite CAPPED blocks, capped pairs only: raw Q against R(-L) K;
//   2. SepLLM gathered separator chunks of 64 rows (no mask but the count);
//   3. the plan's blocks: unmasked when FULL, otherwise the key-set predicate
//      (LM-Infinite CAPPED blocks exclude their capped pairs here).
#include "sa_common.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct FwdArgs {
  const void* q;      // rotated queries (raw when rope is off)
  int64_t qsB, qsH, qsT;
  const void* qraw;   // raw queries, for the capped pass
  int64_t qrB, qrH, qrT;
  const void* k;      // rotated keys (raw when rope is off)
  int64_t ksB, ksH, ksT;
  const void* v;
  int64_t vsB, vsH, vsT;
  const void* ksep;   // [B, h_kv, sep_rows, d]
  const void* vsep;
  int64_t sep_rows;
  const void* kcap;   // [B, h_kv, cap_rows, d]
  int64_t cap_rows;
  void* o;
  int64_t osB, osH, osT;
  float* lse;
  const int* tile_ptr;
  const int* items;
  const int* sep_count;
  const unsigned long long* sep_bits;
  int kind, B, h_q, h_kv, n_q, n_k, n_tiles, group;
  int a, w, n_s, L, P, n_cap;
  int use_cap, gather;
  float scale_log2;
};

enum MaskKind : int {
  MK_NONE = 0,    // every pair visible
  MK_COUNT = 1,   // key slot < count
  MK_SEPLLM = 2,  // j <= i and (j < a or i-j < w or sep[j])
  MK_LALL = 3,    // j <= i and (j < n_s or i-j <= L)
  MK_LNORM = 4,   // j <= i and i-j <= L (capped pairs excluded)
  MK_LCAP = 5,    // j < n_s and i-j > L (capped pairs only)
  MK_SEG = 6,     // j <= P + i
};

struct Unit {
  const char* kbase;  // row 0 of the unit's keys
  int64_t kstride;    // bytes between key rows
  int kvalid;         // rows < kvalid are loaded, the rest read as zero
  const char* vbase;
  int64_t vstride;
  int vvalid;
  int key0;           // key index of row 0 (dense blocks)
  int mk;             // MaskKind
  int count;          // MK_COUNT
  unsigned long long sbits;  // MK_SEPLLM: separator bits of the block
};

__device__ inline bool visible(const FwdArgs& p, const Unit& u, int i, int kk) {
  const int j = u.key0 + kk;
  switch (u.mk) {
    case MK_NONE: return true;
    case MK_COUNT: return kk < u.count;
    case MK_SEPLLM:
      return j <= i && j < p.n_k && (j < p.a || i - j < p.w || ((u.sbits >> kk) & 1ull));
    case MK_LALL: return j <= i && j < p.n_k && (j < p.n_s || i - j <= p.L);
    case MK_LNORM: return j <= i && j < p.n_k && i - j <= p.L;
    case MK_LCAP: return j < p.n_s && j < p.n_k && i - j > p.L;
    default: return j <= p.P + i && j < p.n_k;
  }
}

// Work-group id -> (batch, kv head, tile, query head in group).  Work groups
// are dealt to the 8 XCDs round-robin; each XCD gets one contiguous range of
// units so the tiles sharing K/V rows (same kv head, neighbouring tiles, the
// query heads of a group) meet in that XCD's L2.  Within a range, tiles run
// from the last (most keys) to the first.
__device__ inline void map_unit(const FwdArgs& p, int& b, int& kvh, int& t, int& hq) {
  const int U = p.B * p.h_q * p.n_tiles;
  const int g = blockIdx.x;
  const int x = g & 7, kx = g >> 3;
  const int qu = U >> 3, r = U & 7;
  const int u = x * qu + min(x, r) + kx;
  const int gq = u % p.group;
  int rest = u / p.group;
  const int tt = rest % p.n_tiles;
  rest /= p.n_tiles;
  kvh = rest % p.h_kv;
  b = rest / p.h_kv;
  t = p.n_tiles - 1 - tt;
  hq = kvh * p.group + gq;
}

// Iterate the units of tile t in order; F(unit, use_raw_q) is called for each.
// row_bytes: bytes of one row of the compact arrays (d * element size).
template <class F>
__device__ inline void for_each_unit(const FwdArgs& p, int b, int kvh, int t, int esz,
                                     int64_t row_bytes, F&& f) {
  const int it0 = p.tile_ptr[t], it1 = p.tile_ptr[t + 1];
  const char* kb = static_cast<const char*>(p.k) + (b * p.ksB + kvh * p.ksH) * esz;
  const char* vb = static_cast<const char*>(p.v) + (b * p.vsB + kvh * p.vsH) * esz;
  const int64_t kst = p.ksT * esz, vst = p.vsT * esz;
  // 1. capped pairs (LM-Infinite with RoPE): raw queries against R(-L) K
  if (p.use_cap) {
    const char* cb = static_cast<const char*>(p.kcap) +
                     ((int64_t)b * p.h_kv + kvh) * p.cap_rows * row_bytes;
    for (int it = it0; it < it1; ++it) {
      const int item = p.items[it];
      if (!((item >> 24) & SA_ITEM_CAPPED)) continue;
      const int blk = item & 0xffffff;
      Unit u;
      u.kbase = cb + (int64_t)blk * BK * row_bytes;
      u.kstride = row_bytes;
      u.kvalid = min(BK, p.n_cap - blk * BK);
      u.vbase = vb + (int64_t)blk * BK * vst;
      u.vstride = vst;
      u.vvalid = min(BK, p.n_k - blk * BK);
      u.key0 = blk * BK;
      u.mk = MK_LCAP;
      u.count = 0;
      u.sbits = 0;
      f(u, true);
    }
  }
  // 2. gathered separators: every row precedes the tile and lies outside all
  //    of its windows, so only the count masks
  if (p.gather) {
    const int nsep = p.sep_count[t];
    const int64_t hb = ((int64_t)b * p.h_kv + kvh) * p.sep_rows * row_bytes;
    const char* ksb = static_cast<const char*>(p.ksep) + hb;
    const char* vsb = static_cast<const char*>(p.vsep) + hb;
    for (int c0 = 0; c0 < nsep; c0 += BK) {
      Unit u;
      u.kbase = ksb + (int64_t)c0 * row_bytes;
      u.kstride = row_bytes;
      u.kvalid = min(BK, nsep - c0);
      u.vbase = vsb + (int64_t)c0 * row_bytes;
      u.vstride = row_bytes;
      u.vvalid = u.kvalid;
      u.key0 = 0;
      u.mk = u.kvalid == BK ? MK_NONE : MK_COUNT;
      u.count = u.kvalid;
      u.sbits = 0;
      f(u, false);
    }
  }
  // 3. the plan's blocks
  for (int it = it0; it < it1; ++it) {
    const int item = p.items[it];
    const int blk = item & 0xffffff;
    const int fl = item >> 24;
    Unit u;
    u.kbase = kb + (int64_t)blk * BK * kst;
    u.kstride = kst;
    u.kvalid = min(BK, p.n_k - blk * BK);
    u.vbase = vb + (int64_t)blk * BK * vst;
    u.vstride = vst;
    u.vvalid = u.kvalid;
    u.key0 = blk * BK;
    u.count = 0;
    u.sbits = 0;
    if (p.use_cap && (fl & SA_ITEM_CAPPED)) {
      u.mk = MK_LNORM;
    } else if (fl & SA_ITEM_FULL) {
      u.mk = MK_NONE;
    } else if (p.kind == SA_MASK_SEPLLM) {
      u.mk = MK_SEPLLM;
      u.sbits = p.sep_bits[blk];
    } else if (p.kind == SA_MASK_LAMBDA) {
      u.mk = MK_LALL;
    } else {
      u.mk = MK_SEG;
    }
    f(u, false);
  }
}

// ===========================================================================
// bf16, d = 128: MFMA 32x32x16.  4 waves x 32 queries = one 128-query tile.
// S^T = K Q^T (keys as rows) so every lane owns one query's logits; then
// O^T += V^T P^T with the key order permuted to match the logits' registers.
// ===========================================================================

constexpr int D128 = 128;
constexpr int KS_BYTES = BK * 256;        // K block, 256 B per row, 16 B chunks XOR-swizzled
constexpr int VT_ROW = 68;                // V^T row: 64 keys + 4 pad (bf16 elements)
constexpr int VT_BYTES = D128 * VT_ROW * 2;

__device__ inline uint4 ld16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

__global__ __launch_bounds__(256, 2) void fwd_bf16_d128(FwdArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[KS_BYTES + VT_BYTES];
  char* Ks = smem;
  unsigned short* Vt = reinterpret_cast<unsigned short*>(smem + KS_BYTES);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  int b, kvh, t, hq;
  map_unit(p, b, kvh, t, hq);
  const int q0 = t * TQ;
  const int qi = q0 + wid * 32 + l32;  // this lane's query
  const bool qok = qi < p.n_q;

  bf16x8 qf[8];
  auto load_q = [&](const void* base, int64_t sB, int64_t sH, int64_t sT) {
    const char* row = static_cast<const char*>(base) + (b * sB + hq * sH + (int64_t)qi * sT) * 2;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (qok) x = ld16(row + (16 * s + 8 * hl) * 2);
      qf[s] = __builtin_bit_cast(bf16x8, x);
    }
  };
  load_q(p.q, p.qsB, p.qsH, p.qsT);
  bool q_is_raw = false;

  float m_run = NEG_INF, l_run = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};

  auto unit = [&](const Unit& u, bool raw_q) {
    if (raw_q != q_is_raw) {
      if (raw_q) load_q(p.qraw, p.qrB, p.qrH, p.qrT);
      else load_q(p.q, p.qsB, p.qsH, p.qsT);
      q_is_raw = raw_q;
    }
    // --- global -> LDS: K row-major swizzled, V transposed ---
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = it * 16 + (tid >> 4), ch = tid & 15;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row < u.kvalid) x = ld16(u.kbase + row * u.kstride + ch * 16);
      *reinterpret_cast<uint4*>(Ks + row * 256 + ((ch ^ (row & 15)) * 16)) = x;
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int key = lane, ch = wid + 4 * it;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (key < u.vvalid) x = ld16(u.vbase + key * u.vstride + ch * 16);
      const unsigned w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[(ch * 8 + 2 * e) * VT_ROW + key] = (unsigned short)(w4[e] & 0xffffu);
        Vt[(ch * 8 + 2 * e + 1) * VT_ROW + key] = (unsigned short)(w4[e] >> 16);
      }
    }
    __syncthreads();
    // --- S^T = K Q^T : two 32-key halves ---
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16 c = f32x16{};
      const int row = mb * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int ch = 2 * ks + hl;
        const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Ks + row * 256 + ((ch ^ (row & 15)) * 16)));
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], c, 0, 0, 0);
      }
      s[mb] = c;
    }
    // --- scale, mask, online softmax ---
    float mx = NEG_INF;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 32 * mb + 8 * (r >> 2) + 4 * hl + (r & 3);
        float x = s[mb][r] * p.scale_log2;
        if (u.mk != MK_NONE && !visible(p, u, qi, kk)) x = NEG_INF;
        s[mb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == NEG_INF ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2f(s[mb][r] - m_use);
        s[mb][r] = e;
        psum += e;
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dm = 0; dm < 4; ++dm) acc[dm] *= alpha;
    // --- O^T += V^T P^T ---
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
      const int mb = kstep >> 1, uu = kstep & 1;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const f32x2 two = {s[mb][8 * uu + e], s[mb][8 * uu + e + 1]};
        const bf16x2 c2 = __builtin_convertvector(two, bf16x2);
        pb[e] = c2[0];
        pb[e + 1] = c2[1];
      }
      const int kA = 32 * mb + 16 * uu + 4 * hl;
#pragma unroll
      for (int dm = 0; dm < 4; ++dm) {
        const unsigned short* vr = Vt + (dm * 32 + l32) * VT_ROW;
        const uint2 lo = *reinterpret_cast<const uint2*>(vr + kA);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + kA + 8);
        const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        acc[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[dm], 0, 0, 0);
      }
    }
    __syncthreads();
  };

  for_each_unit(p, b, kvh, t, 2, (int64_t)D128 * 2, unit);

  // --- epilogue ---
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    char* orow = static_cast<char*>(p.o) + (b * p.osB + hq * p.osH + (int64_t)qi * p.osT) * 2;
#pragma unroll
    for (int dm = 0; dm < 4; ++dm) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dm + 8 * g + 4 * hl;
        const f32x2 x01 = {acc[dm][4 * g] * inv, acc[dm][4 * g + 1] * inv};
        const f32x2 x23 = {acc[dm][4 * g + 2] * inv, acc[dm][4 * g + 3] * inv};
        const bf16x2 y01 = __builtin_convertvector(x01, bf16x2);
        const bf16x2 y23 = __builtin_convertvector(x23, bf16x2);
        uint2 w;
        w.x = __builtin_bit_cast(unsigned, y01);
        w.y = __builtin_bit_cast(unsigned, y23);
        *reinterpret_cast<uint2*>(orow + d0 * 2) = w;
      }
    }
    if (p.lse != nullptr && hl == 0)
      p.lse[((int64_t)b * p.h_q + hq) * p.n_q + qi] = (m_run + log2f(l_tot)) * LN2;
  }
}

// ===========================================================================
// fp32 (no bf16 rounding anywhere): one thread per query row, K/V staged in
// LDS; every product and sum in fp32.
// ===========================================================================

template <int D>
__global__ __launch_bounds__(128) void fwd_f32(FwdArgs p) {
  __shared__ __attribute__((aligned(16))) float Ks[BK][D];
  __shared__ __attribute__((aligned(16))) float Vs[BK][D];
  const int tid = threadIdx.x;
  int b, kvh, t, hq;
  map_unit(p, b, kvh, t, hq);
  const int qi = t * TQ + tid;
  const bool qok = qi < p.n_q;
  float q[D];
  auto load_q = [&](const void* base, int64_t sB, int64_t sH, int64_t sT) {
    const float* row = static_cast<const float*>(base) + (b * sB + hq * sH + (int64_t)qi * sT);
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (qok) x = *reinterpret_cast<const float4*>(row + c);
      q[c] = x.x; q[c + 1] = x.y; q[c + 2] = x.z; q[c + 3] = x.w;
    }
  };
  load_q(p.q, p.qsB, p.qsH, p.qsT);
  bool q_is_raw = false;
  float m_run = NEG_INF, l_run = 0.f;
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;

  auto unit = [&](const Unit& u, bool raw_q) {
    if (raw_q != q_is_raw) {
      if (raw_q) load_q(p.qraw, p.qrB, p.qrH, p.qrT);
      else load_q(p.q, p.qsB, p.qsH, p.qsT);
      q_is_raw = raw_q;
    }
    constexpr int CH = D / 4;  // float4 chunks per row
    for (int x = tid; x < BK * CH; x += 128) {
      const int row = x / CH, ch = x % CH;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (row < u.kvalid) kv = *reinterpret_cast<const float4*>(u.kbase + row * u.kstride + ch * 16);
      if (row < u.vvalid) vv = *reinterpret_cast<const float4*>(u.vbase + row * u.vstride + ch * 16);
      *reinterpret_cast<float4*>(&Ks[row][ch * 4]) = kv;
      *reinterpret_cast<float4*>(&Vs[row][ch * 4]) = vv;
    }
    __syncthreads();
    float s[BK];
    float mx = NEG_INF;
    for (int r = 0; r < BK; ++r) {
      float acc_s = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) acc_s = fmaf(q[c], Ks[r][c], acc_s);
      float x = acc_s * p.scale_log2;
      if (u.mk != MK_NONE && !visible(p, u, qi, r)) x = NEG_INF;
      s[r] = x;
      mx = fmaxf(mx, x);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == NEG_INF ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] *= alpha;
    for (int r = 0; r < BK; ++r) {
      const float e = exp2f(s[r] - m_use);
      psum += e;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(e, Vs[r][c], acc[c]);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    __syncthreads();
  };

  for_each_unit(p, b, kvh, t, 4, (int64_t)D * 4, unit);

  if (qok) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* orow = static_cast<float*>(p.o) + (b * p.osB + hq * p.osH + (int64_t)qi * p.osT);
#pragma unroll
    for (int c = 0; c < D; c += 4)
      *reinterpret_cast<float4*>(orow + c) =
          make_float4(acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv);
    if (p.lse != nullptr) p.lse[((int64_t)b * p.h_q + hq) * p.n_q + qi] = (m_run + log2f(l_run)) * LN2;
  }
}

}  // namespace

hipError_t launch_fwd(const sa_mask_t& m, const sa_plan_header_t& lay, const void* plan,
                      const sa_fwd_args_t& a, const RopeOut& ro, hipStream_t s) {
  const char* pb = static_cast<const char*>(plan);
  FwdArgs p;
  memset(&p, 0, sizeof(p));
  const bool rope = a.rope == SA_ROPE_HALF;
  if (rope) {
    p.q = ro.qrot;
    p.qsT = a.d; p.qsH = (int64_t)m.n_q * a.d; p.qsB = p.qsH * a.h_q;
    p.k = ro.krot;
    p.ksT = a.d; p.ksH = (int64_t)m.n_k * a.d; p.ksB = p.ksH * a.h_kv;
  } else {
    p.q = a.q;
    p.qsB = a.q_stride[0]; p.qsH = a.q_stride[1]; p.qsT = a.q_stride[2];
    p.k = a.k;
    p.ksB = a.k_stride[0]; p.ksH = a.k_stride[1]; p.ksT = a.k_stride[2];
  }
  p.qraw = a.q;
  p.qrB = a.q_stride[0]; p.qrH = a.q_stride[1]; p.qrT = a.q_stride[2];
  p.v = a.v;
  p.vsB = a.v_stride[0]; p.vsH = a.v_stride[1]; p.vsT = a.v_stride[2];
  p.ksep = ro.ksep;
  p.vsep = ro.vsep;
  p.sep_rows = ro.sep_rows;
  p.kcap = ro.kcap;
  p.cap_rows = ro.cap_rows;
  p.o = a.o;
  p.osB = a.o_stride[0]; p.osH = a.o_stride[1]; p.osT = a.o_stride[2];
  p.lse = a.lse;
  p.tile_ptr = reinterpret_cast<const int*>(pb + lay.off_tile_ptr);
  p.items = reinterpret_cast<const int*>(pb + lay.off_items);
  p.sep_count = reinterpret_cast<const int*>(pb + lay.off_sep_count);
  p.sep_bits = reinterpret_cast<const unsigned long long*>(pb + lay.off_sep_bits);
  p.kind = m.kind;
  p.B = a.batch;
  p.h_q = a.h_q;
  p.h_kv = a.h_kv;
  p.n_q = m.n_q;
  p.n_k = m.n_k;
  p.n_tiles = lay.n_tiles;
  p.group = a.h_q / a.h_kv;
  p.a = m.a;
  p.w = m.w;
  p.n_s = m.n_starting;
  p.L = m.L_pretrain;
  p.P = m.prefix_len;
  p.n_cap = ro.n_cap;
  p.use_cap = (m.kind == SA_MASK_LAMBDA && rope && ro.n_cap > 0) ? 1 : 0;
  p.gather = (m.kind == SA_MASK_SEPLLM && m.sep != nullptr) ? 1 : 0;
  p.scale_log2 = a.scale * LOG2E;
  const unsigned grid = (unsigned)((int64_t)a.batch * a.h_q * lay.n_tiles);
  if (a.dtype == SA_BF16) {
    hipLaunchKernelGGL(fwd_bf16_d128, dim3(grid), dim3(256), 0, s, p);
  } else if (a.d == 64) {
    hipLaunchKernelGGL(fwd_f32<64>, dim3(grid), dim3(128), 0, s, p);
  } else {
    hipLaunchKernelGGL(fwd_f32<128>, dim3(grid), dim3(128), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace sa
