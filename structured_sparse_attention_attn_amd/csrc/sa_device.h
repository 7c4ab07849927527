// Device helpers shared by the forward and backward kernels: MFMA fragment
// types, the LDS swizzle, plan-unit decoding and the key-set predicates.
// Templates over the kernel argument struct, which must carry the plan
// pointers and mask scalars under the names used here.
#pragma once

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

// Slope of query head h in base-2 logit units, m_h * log2(e), evaluated in
// double and rounded once.
template <class A>
__device__ inline float alibi_slope_log2(const A& p, int hq) {
  return (float)(exp2(-(double)p.alibi_e * (hq + 1) / p.h_q) * 1.4426950408889634);
}

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

template <class A>
__device__ inline bool visible(const A& p, const Unit& u, int i, int kk) {
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

// Iterate the units of tile t in order; F(unit, use_raw_q) is called for each.
// row_bytes: bytes of one row of the compact arrays (d * element size).
template <class A, class F>
__device__ inline void for_each_unit(const A& p, int b, int kvh, int t, int esz,
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

// Work-group id -> (batch, kv head, tile, query head in group).  Work groups
// are dealt to the 8 XCDs round-robin; each XCD gets one contiguous range of
// units so the tiles sharing K/V rows (same kv head, neighbouring tiles, the
// query heads of a group) meet in that XCD's L2.  Within a range, tiles run
// from the last (most keys) to the first.
template <class A>
__device__ inline void map_unit(const A& p, int& b, int& kvh, int& t, int& hq) {
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

constexpr int D128 = 128;
constexpr int BLK_BYTES = BK * 256;        // one 64 x 128 bf16 block

// 16-byte chunk c of row r sits at chunk c ^ f(r & 15), f swapping the two
// 2-bit halves of its argument.  Any 16 consecutive rows then spread one
// logical chunk over all 16 positions (conflict-free K fragment reads), and
// the 8 rows x 64 bytes of one V^T transpose read cover every bank twice.
__device__ inline int swzf(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// The swizzle of a block with D-element bf16 rows: 256-byte rows (D = 128)
// use swzf; 128-byte rows (D = 64, 8 chunks) use chunk c ^ ((r >> 1) & 7),
// so 16 consecutive rows (two per 256-byte bank line) put one logical chunk
// in 16 distinct bank groups.
template <int D>
__device__ inline int swz(int r) {
  if constexpr (D == 128) return swzf(r);
  else return (r >> 1) & 7;
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ inline uint4 ld16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

// A 16-byte load of data read once (queries): non-temporal, so it does not
// push out of L2 the key and value rows that other work groups read again.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint4 ld16_once(const char* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Loads of plan data that no kernel of this launch writes, through the scalar
// data cache (uniform addresses, results in scalar registers).
template <class T>
__device__ inline T ld_uniform(const T* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(reinterpret_cast<uintptr_t>(p));
}

__device__ inline float swap_halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float swap_halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Packs the 32 weights of one lane (two 32-key halves) into the four bf16x8
// B operands of the PV product: k-step ks takes registers 8 (ks % 2) .. +7 of
// half ks / 2.
__device__ inline void pack_p(const f32x16 (&s)[2], bf16x8 (&pb)[4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const f32x2 two = {s[ks >> 1][8 * (ks & 1) + e], s[ks >> 1][8 * (ks & 1) + e + 1]};
      const bf16x2 c2 = __builtin_convertvector(two, bf16x2);
      pb[ks][e] = c2[0];
      pb[ks][e + 1] = c2[1];
    }
  }
}

// Sum of the packed (rounded) weights: O is normalised by the same bf16
// weights it accumulates.
__device__ inline float sum_p(const bf16x8 (&pb)[4]) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks], pb[ks], 0, 1), one, a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks], pb[ks], 2, 3), one, a1, false);
    a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks], pb[ks], 4, 5), one, a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks], pb[ks], 6, 7), one, a1, false);
  }
  return a0 + a1;
}

// Per-tile unit list: [capped items] [gathered separator chunks] [items].
struct TileUnits {
  int it0, n_items, n_capu, n_ch, nsep;
  int cap0;            // index of the first capped item (the ordinary pass starts at it0)
  int rot;             // the ordinary items are visited from item rot on, wrapping (0: in order)
  int chrev;           // the separator chunks are visited last to first
  const char* kb;      // dense keys of this (batch, kv head)
  const char* vb;
  int64_t kst, vst;
  const char* capb;    // capped keys
  const char* ksb;     // gathered separator keys / values
  const char* vsb;
};

// The tile's capped items (LM-Infinite: leading blocks holding starting
// tokens seen from farther than L) and its ordinary items.  A capped block
// whose last key is farther than L from the tile's first query holds no pair
// of the ordinary pass (every pair of it is a capped one), so that pass skips
// it; such blocks form a prefix of the capped items.  CAP false: a kernel
// that never has capped passes (the ALiBi bias).
template <bool CAP, class A>
__device__ inline void tile_items(const A& p, int t, TileUnits& tu) {
  tu.it0 = ld_uniform(p.tile_ptr + t);
  tu.n_items = ld_uniform(p.tile_ptr + t + 1) - tu.it0;
  tu.cap0 = tu.it0;
  tu.n_capu = 0;
  tu.rot = 0;
  tu.chrev = 0;
  if (CAP && p.use_cap) {
    while (tu.n_capu < tu.n_items && ((ld_uniform(p.items + tu.it0 + tu.n_capu) >> 24) & SA_ITEM_CAPPED)) ++tu.n_capu;
    int n_skip = 0;
    while (n_skip < tu.n_capu && (ld_uniform(p.items + tu.it0 + n_skip) & 0xffffff) * BK + BK - 1 < t * TQ - p.L)
      ++n_skip;
    tu.it0 += n_skip;
    tu.n_items -= n_skip;
  }
}

// REV visits the plan's blocks last to first (the diagonal block first);
// otherwise from item tu.rot on, wrapping around.
// ROWB: bytes per row of the compact arrays (capped keys, gathered rows).
template <bool REV, int ROWB = D128 * 2, class A>
__device__ inline Unit unit_at(const A& p, const TileUnits& tu, int u) {
  Unit x;
  x.count = 0;
  x.sbits = 0;
  if (u < tu.n_capu) {
    const int blk = ld_uniform(p.items + tu.cap0 + u) & 0xffffff;
    x.kbase = tu.capb + (int64_t)blk * BK * ROWB;
    x.kstride = ROWB;
    x.kvalid = min(BK, p.n_cap - blk * BK);
    x.vbase = tu.vb + (int64_t)blk * BK * tu.vst;
    x.vstride = tu.vst;
    x.vvalid = min(BK, p.n_k - blk * BK);
    x.key0 = blk * BK;
    x.mk = MK_LCAP;
    return x;
  }
  u -= tu.n_capu;
  if (u < tu.n_ch) {
    const int c0 = (tu.chrev ? tu.n_ch - 1 - u : u) * BK;
    x.kbase = tu.ksb + (int64_t)c0 * ROWB;
    x.kstride = ROWB;
    x.vbase = tu.vsb + (int64_t)c0 * ROWB;
    x.vstride = ROWB;
    x.kvalid = x.vvalid = min(BK, tu.nsep - c0);
    x.key0 = 0;
    x.count = x.kvalid;
    x.mk = x.kvalid == BK ? MK_NONE : MK_COUNT;
    return x;
  }
  u -= tu.n_ch;
  int k = u + tu.rot;
  if (k >= tu.n_items) k -= tu.n_items;
  const int item = ld_uniform(p.items + tu.it0 + (REV ? tu.n_items - 1 - u : k));
  const int blk = item & 0xffffff;
  const int fl = item >> 24;
  x.kbase = tu.kb + (int64_t)blk * BK * tu.kst;
  x.kstride = tu.kst;
  x.vbase = tu.vb + (int64_t)blk * BK * tu.vst;
  x.vstride = tu.vst;
  x.kvalid = x.vvalid = min(BK, p.n_k - blk * BK);
  x.key0 = blk * BK;
  if (p.use_cap && (fl & SA_ITEM_CAPPED)) {
    x.mk = MK_LNORM;
  } else if (fl & SA_ITEM_FULL) {
    x.mk = MK_NONE;
  } else if (p.kind == SA_MASK_SEPLLM) {
    x.mk = MK_SEPLLM;
    x.sbits = ld_uniform(p.sep_bits + blk);
  } else if (p.kind == SA_MASK_LAMBDA) {
    x.mk = MK_LALL;
  } else {
    x.mk = MK_SEG;
  }
  return x;
}

// Masks the raw logits of one unit.  Register r of half mb holds key slot
// kk = 32 mb + 8 (r / 4) + 4 hl + r % 4; everything lane-dependent is folded
// into one base so the per-element tests use compile-time offsets, and the
// conditions use non-short-circuit operators (no branches).
template <int MK, class A>
__device__ inline void apply_mask(const A& p, const Unit& u, int qi, int hl, f32x16 (&s)[2]) {
  const int jb = u.key0 + 4 * hl;                    // key index of slot offset 0
  const unsigned long long sb = u.sbits >> (4 * hl);  // separator bits from slot offset 0
  const int cb = u.count - 4 * hl;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 32 * mb + 8 * (r >> 2) + (r & 3);  // compile-time slot offset
      const int j = jb + c;
      bool vis;
      if (MK == MK_COUNT) {
        vis = c < cb;
      } else if (MK == MK_SEPLLM) {
        const bool sepb = (sb >> c) & 1ull;
        vis = (j <= qi) & (j < p.n_k) & ((j < p.a) | (qi - j < p.w) | sepb);
      } else if (MK == MK_LALL) {
        vis = (j <= qi) & (j < p.n_k) & ((j < p.n_s) | (qi - j <= p.L));
      } else if (MK == MK_LNORM) {
        vis = (j <= qi) & (j < p.n_k) & (qi - j <= p.L);
      } else if (MK == MK_LCAP) {
        vis = (j < p.n_s) & (j < p.n_k) & (qi - j > p.L);
      } else {
        vis = (j <= p.P + qi) & (j < p.n_k);
      }
      s[mb][r] = vis ? s[mb][r] : NEG_INF;
    }
  }
}

// Adds the ALiBi-style bias -m2 * min(i - j, L) to one unit's logits (same
// register layout as apply_mask).  Masked logits stay -inf.
__device__ inline void add_alibi(const Unit& u, int qi, int hl, float m2, float Lf, f32x16 (&s)[2]) {
  const float dist0 = (float)(qi - u.key0 - 4 * hl);  // i - j at slot offset 0 (exact)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 32 * mb + 8 * (r >> 2) + (r & 3);
      s[mb][r] = fmaf(-m2, fminf(dist0 - (float)c, Lf), s[mb][r]);
    }
  }
}

// Direct global -> LDS load of BYTES per lane (4 or 16) from the wave-uniform
// address base + voff (voff per lane, bytes), written lane after lane from
// the wave-uniform LDS address lds.  It is issued in the buffer (MUBUF) form
// with a raw resource over base, not in the global (FLAT) form: while a FLAT
// instruction that writes LDS is in flight, the compiler cannot count LDS
// reads one by one and makes every later LDS read wait for all earlier ones
// (lgkmcnt(0)), which defeats reading MFMA operands ahead.  voff + BYTES must
// stay below 2^32 (callers keep row strides at most 64 MiB).
template <int BYTES>
__device__ __attribute__((always_inline)) inline void lds_dma(const void* base, uint32_t voff, void* lds) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
  static_assert(BYTES == 4 || BYTES == 16, "4 or 16 bytes per lane");
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, 0, 0, 0);
}

// Direct global -> LDS loads of a 64-row x 256-byte block into the swizzled
// layout (16-byte chunk c of row r at chunk c ^ swzf(r & 15)): wave w moves
// rows 16w .. 16w+15, four rows per instruction, each lane fetching the
// logical chunk that lands in its slot.  Rows at or past `valid` repeat row
// valid-1 (finite values, masked later).
__device__ __attribute__((always_inline)) inline void dma_block(const char* base, int64_t stride, int valid,
                                                                char* lds, int wid, int lane) {
  const int lrow = lane >> 4;
  const int lchunk = (lane & 15) ^ (lrow << 2);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = wid * 4 + j;
    const int r = min(4 * i + lrow, valid - 1);
    lds_dma<16>(base, (uint32_t)(r * (uint32_t)stride) + (uint32_t)((lchunk ^ j) << 4), lds + i * 1024);
  }
}

}  // namespace
}  // namespace sa

