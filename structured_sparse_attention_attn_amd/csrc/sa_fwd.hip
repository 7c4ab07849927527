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
// scale times log2(e) applied to the logits).  The bf16 kernel visits:
//   1. SepLLM gathered separator chunks of 64 rows (no mask but the count);
//   2. the plan's blocks: unmasked when FULL, otherwise the key-set predicate
//      (LM-Infinite CAPPED blocks exclude their capped pairs here);
//   3. LM-Infinite CAPPED blocks, capped pairs only: raw Q against R(-L) K.
// (The fp32 kernel visits the capped blocks first.)
#include <cmath>
#include <type_traits>

#include "sa_common.h"
#include "sa_device.h"

namespace sa {
namespace {

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
  const int* n_sep;   // the plan header's separator count (j >= g0)
  int cap_sep;        // separators the plan lists at most
  int kind, B, h_q, h_kv, n_q, n_k, n_tiles, group;
  int a, w, n_s, L, P, n_cap;
  int use_cap, gather;
  float scale_log2;
  int alibi;          // ALiBi-style bias -m_h * min(i-j, L) instead of RoPE (Lambda only)
  float alibi_e;      // slope exponent E: m_h = 2^(-E (h+1) / h_q)
  // bf16: q is the caller's raw query; the kernel rotates it at q_pos0 + i
  // (when rot_q) and multiplies it by q_scale itself
  int rot_q, q_pos0;
  float q_scale;
  double th1, th8, th16;  // base^(-2/d) and its 8th and 16th powers: theta_{c+1} = theta_c * th1
};

// A plan whose mask held more separators than its sep_idx section lists:
// every count it hands out is clamped, so the kernels stay in bounds, and the
// outputs are poisoned (NaN) instead of silently missing keys.
__device__ inline bool plan_overflowed(const FwdArgs& p) {
  return p.gather && ld_uniform(p.n_sep) > p.cap_sep;
}

// ===========================================================================
// bf16, d = 128 or 64: MFMA 32x32x16.  4 waves x 32 queries = one 128-query tile.
// S^T = K Q^T (keys as rows) so every lane owns one query's logits and the
// row max / row sum stay in the lane (plus one swap between the two 32-lane
// halves); then O^T += V^T P^T, the key order inside each 16-key step permuted
// to match the registers the logits already sit in.  K blocks are double- and
// V blocks triple-buffered in LDS (row-major, 16-byte chunks XOR-swizzled by
// row), filled by direct global-to-LDS loads; the next unit's loads are in
// flight while the current one computes.  V^T operands come straight from the
// row-major V block through the LDS transpose read (ds_read_b64_tr_b16).  The
// PV product runs one unit behind, before the next loads are issued: the
// compiler orders a transpose read after every LDS-bound load in flight, so
// issuing them afterwards keeps those reads from waiting on HBM.
// ===========================================================================

// ALIBI: the bias is added to every unit's logits and the blocks are visited
// from the diagonal down, so a row's first reference already includes its
// largest bias (0 at j = i): every later logit is at most the query-key spread
// above it, and the reference stays the size of a query-key logit.
template <int D, bool ALIBI>
__global__ __launch_bounds__(256, D == 64 ? 3 : 2) void fwd_bf16(FwdArgs p) {
  static_assert(D == 64 || D == 128, "head dimension");
  constexpr int ROWB = D * 2;         // bytes per row
  constexpr int BLKB = BK * ROWB;     // one 64-row block
  constexpr int NKS = D / 16;         // k-steps of the QK product
  constexpr int NDM = D / 32;         // 32-row d blocks of O^T
  constexpr int LPR = ROWB / 16;      // lanes per row of one global->LDS load (16-byte pieces)
  constexpr int RPI = 64 / LPR;       // rows per load instruction (1 KB)
  constexpr int NJ = BLKB / 4096;     // load instructions per block and wave
  constexpr int XSH = D == 128 ? 4 : 6;  // byte shift of instruction j's swizzle change
  // K blocks double-buffered, V blocks triple-buffered: [K0 K1 V0 V1 V2]
  __shared__ __attribute__((aligned(16))) char smem[5 * BLKB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hl = lane >> 5;
  int b, kvh, t, hq;
  map_unit(p, b, kvh, t, hq);
  const int q0 = t * TQ;
  const int qi = q0 + wid * 32 + l32;  // this lane's query
  const bool qok = qi < p.n_q;

  TileUnits tu;
  tile_items<!ALIBI>(p, t, tu);
  tu.nsep = p.gather ? ld_uniform(p.sep_count + t) : 0;
  tu.n_ch = (tu.nsep + BK - 1) / BK;
  tu.kb = static_cast<const char*>(p.k) + (b * p.ksB + kvh * p.ksH) * 2;
  tu.vb = static_cast<const char*>(p.v) + (b * p.vsB + kvh * p.vsH) * 2;
  tu.kst = p.ksT * 2;
  tu.vst = p.vsT * 2;
  tu.capb = static_cast<const char*>(p.kcap) + ((int64_t)b * p.h_kv + kvh) * p.cap_rows * ROWB;
  const int64_t sep_off = ((int64_t)b * p.h_kv + kvh) * p.sep_rows * ROWB;
  tu.ksb = static_cast<const char*>(p.ksep) + sep_off;
  tu.vsb = static_cast<const char*>(p.vsep) + sep_off;
  const int n_units = tu.n_capu + tu.n_ch + tu.n_items;
  // Phase-aligned walk over the plan's blocks (not for ALiBi, which needs the
  // diagonal first): the run of consecutive window blocks that ends at the
  // tile's last item is entered so that the block visited at step s of the
  // work group has index = s (mod n_items).  Neighbouring tiles of a head hold
  // the same number of items and run at the same time on one XCD, so they read
  // each window block within a few steps of one another, while it is in that
  // XCD's L2, instead of two steps later per tile (which cycles a working set
  // larger than the L2).
  if (!ALIBI && tu.n_items > 1) {
    const int b_last = ld_uniform(p.items + tu.it0 + tu.n_items - 1) & 0xffffff;
    const int m = tu.n_items;
    tu.rot = (2 * m - 1 - b_last % m + tu.n_ch % m) % m;  // block of step n_ch + u = n_ch + u (mod m)
  }
  // Gathered separator chunks: every tile of a head reads the same rows, up
  // to its own count.  The work groups an XCD runs at one time (about 64 of
  // them: its 32 CUs, two each) read them together; the next such group of
  // work groups walks them the other way, starting on the rows the previous
  // one read last, which are the ones still in the XCD's L2.
  tu.chrev = ((blockIdx.x >> 3) >> 6) & 1;
  const float m2 = ALIBI ? alibi_slope_log2(p, hq) : 0.f;
  const float Lf = (float)p.L;

  bf16x8 qf[NKS];
  auto load_q = [&](const void* base, int64_t sB, int64_t sH, int64_t sT) {
    const char* row = static_cast<const char*>(base) + (b * sB + hq * sH + (int64_t)qi * sT) * 2;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (qok) x = ld16_once(row + (16 * s + 8 * hl) * 2);
      qf[s] = __builtin_bit_cast(bf16x8, x);
    }
  };
  load_q(p.q, p.qsB, p.qsH, p.qsT);

  // Every unit but the capped ones reads R(pos) q * scale * log2(e), made
  // here in registers; the capped units (visited last) pair the raw query,
  // loaded again before them, with R(-L) k.  Lane (l32, hl) holds dims 16 s + 8 hl + e of
  // its query, so the rotate-half partner of dim c (s < D/32) is c + D/2 in
  // qf[s + D/32], same lane.  theta_c / (2 pi) comes from products of powers of
  // base^(-2/d) in fp64 (a few ulp from the direct power); the angle is
  // reduced in fp64 to a fraction of a turn, and the hardware sine and cosine
  // take turns.
  auto prep_q = [&]() {
    const float qs = p.q_scale;
    if (p.rot_q) {
      const double pos = (double)(p.q_pos0 + qi);
      double th_s = (hl ? p.th8 : 1.0) * 0.15915494309189535;  // theta_{8 hl} / (2 pi)
#pragma unroll
      for (int s = 0; s < NKS / 2; ++s) {
        double th = th_s;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double rev = pos * th;
          th *= p.th1;
          const float f = (float)(rev - rint(rev));
          const float cs = __builtin_amdgcn_cosf(f), sn = __builtin_amdgcn_sinf(f);
          const float x1 = (float)qf[s][e], x2 = (float)qf[s + NKS / 2][e];
          qf[s][e] = (__bf16)((x1 * cs - x2 * sn) * qs);
          qf[s + NKS / 2][e] = (__bf16)((x2 * cs + x1 * sn) * qs);
        }
        th_s *= p.th16;
      }
    } else {
#pragma unroll
      for (int s = 0; s < NKS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[s][e] = (__bf16)((float)qf[s][e] * qs);
    }
  };

  // Online softmax against a reference max m_ref per query (base-2 logits:
  // the queries and capped keys carry scale * log2(e)).  -m_ref enters the
  // QK^T MFMA as its initial accumulator, so the logits leave the MFMA
  // already shifted; the reference is raised only when a row's running sum
  // of one unit passes 2^10 (or while some row has no finite reference yet),
  // which keeps every p <= ~2^10 and the shift exact in the final O and LSE.
  // A unit whose logits exceed the reference by 64 base-2 units or more is
  // computed again and taken with its exact row maximum, so no weight
  // overflows whatever the logit range (any finite input).
  bool has_ref = false;
  float m_ref = 0.f, l_run = 0.f;
  f32x16 negm = f32x16{};
  f32x16 acc[NDM];
#pragma unroll
  for (int i = 0; i < NDM; ++i) acc[i] = f32x16{};

  // global -> LDS without register staging: one instruction moves RPI rows
  // (lane l -> row RPI i + l / LPR, stored chunk l % LPR); the lane fetches
  // the logical chunk that the row's swizzle puts in that slot, lchunk for the
  // wave's first instruction and lchunk ^ (j << (XSH - 4)) for its j-th (the
  // rows of instruction j differ from those of the first only in the swizzle
  // bits that j sets).  Rows past the unit's valid count repeat its last valid
  // row: finite values whose logits are masked out.
  const int lrow = lane / LPR;
  const int lchunk = (lane % LPR) ^ swz<D>(16 * wid + lrow);
  // this lane's row and logical chunk (bits 4+) for j = 0; the j-th
  // instruction's offset is lofs ^ (j << XSH) + j * 1024.  The offsets are
  // recomputed from lofs at each use (a 32-bit offset next to a uniform base
  // address, so each load is one instruction with no address arithmetic).
  const uint32_t lofs = (uint32_t)((16 * wid + lrow) * ROWB + (lchunk << 4));
  auto issue_loads = [&](const Unit& u, int kslot, int vslot) {
    char* Kb = smem + kslot * BLKB;
    char* Vb = smem + (2 + vslot) * BLKB;
    uint32_t lo = lofs;
    __asm__ volatile("" : "+v"(lo));
    if (u.kvalid == BK && u.vvalid == BK && u.kstride == ROWB && u.vstride == ROWB) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int i = wid * NJ + j;
        const uint32_t o = lo ^ (uint32_t)(j << XSH);
        lds_dma<16>(u.kbase, o + (uint32_t)(j * 1024), Kb + i * 1024);
        lds_dma<16>(u.vbase, o + (uint32_t)(j * 1024), Vb + i * 1024);
      }
      return;
    }
    const int r0 = (int)(lo / ROWB);
    const uint32_t c0 = lo & (uint32_t)(ROWB - 16);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int i = wid * NJ + j;  // rows RPI i .. RPI i + RPI - 1
      const uint32_t ch = c0 ^ (uint32_t)(j << XSH);
      const int kr = min(r0 + RPI * j, u.kvalid - 1);
      const int vr = min(r0 + RPI * j, u.vvalid - 1);
      lds_dma<16>(u.kbase, (uint32_t)kr * (uint32_t)u.kstride + ch, Kb + i * 1024);
      lds_dma<16>(u.vbase, (uint32_t)vr * (uint32_t)u.vstride + ch, Vb + i * 1024);
    }
  };

  // Per-lane LDS read bases.  K fragment (half mb, k-step ks): row 32 mb + l32,
  // logical chunk 2 ks + hl; rows l32 and 32 + l32 share row & 15, so the
  // swizzle is one per-lane XOR.  V^T fragment (k-step kst, d block dm) by
  // transpose reads: lane (16-lane group g, index i) points at key
  // kA + i/4 (+8 for the upper half of the k-step), columns
  // 32 dm + 16 (g & 1) + 4 (i & 3) .. +3, with kA = 32 (kst/2) + 16 (kst%2) + 4 hl,
  // so row & 15 is 4 hl + i/4 (+8).
  const int kf = swz<D>(l32) ^ hl;
  const int vrow = 4 * hl + ((lane & 15) >> 2);
  const int vf0 = swz<D>(vrow), vf1 = swz<D>(vrow + 8);
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int vcb = vcol >> 3;  // chunk of the column within its 32-column group

  // O^T += V^T P^T for the unit whose weights are in pb and whose V block is
  // in slot vslot: V^T fragments two MFMAs ahead
  auto pv = [&](const bf16x8 (&pb)[4], int vslot) {
    const char* vl = smem + (2 + vslot) * BLKB + vrow * ROWB + ((vcol & 7) << 1);
    auto vfrag = [&](int kst, int dm) {
      const char* a0 = vl + (32 * (kst >> 1) + 16 * (kst & 1)) * ROWB + (((4 * dm + vcb) ^ vf0) << 4);
      const char* a1 = vl + (32 * (kst >> 1) + 16 * (kst & 1) + 8) * ROWB + (((4 * dm + vcb) ^ vf1) << 4);
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a1));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 va[3];
    va[0] = vfrag(0, 0);
    va[1] = vfrag(1 / NDM, 1 % NDM);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 4 * NDM; ++i) {
      const int kst = i / NDM, dm = i % NDM;
      if (i + 2 < 4 * NDM) va[(i + 2) % 3] = vfrag((i + 2) / NDM, (i + 2) % NDM);
      acc[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % 3], pb[kst], acc[dm], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // One unit per step, the PV product one unit behind: step u accumulates
  // P(u-1) V(u-1) first (no block load is in flight then), issues the loads
  // of unit u+1, and computes S(u) and P(u).  K(u+1) goes to the K slot that
  // S(u-1) read, V(u+1) to the V slot that P(u-2) V(u-2) read, both finished
  // before this step's barrier.  The exact-max softmax (full_path) runs while
  // some row of the wave has no finite reference yet, the fast path
  // afterwards.  Every wave runs exactly one barrier per unit, whichever loop
  // it is in.
  // unit order: separator chunks, the plan's blocks, then the capped units
  const int u_cap = n_units - tu.n_capu;
  auto unit = [&](int u) { return unit_at<ALIBI, ROWB>(p, tu, u < u_cap ? u + tu.n_capu : u - u_cap); };
  Unit cur;
  if (n_units > 0) {
    cur = unit(0);
    issue_loads(cur, 0, 0);
  }
  if (u_cap > 0) prep_q();
  bf16x8 pb[4];  // P(u-1), carried into step u
  int vs_prev = 2, vs_next = 1;  // V slots of units u-1 and u+1 (u % 3 = 0 at u = 0)
  auto step = [&](int u, auto full_path) {
    const int buf = u & 1;
    // this wave's loads of unit u have landed; the barrier makes every wave's
    // visible and ends every read of the slots the next loads overwrite
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (u > 0) pv(pb, vs_prev);
    const char* Kb = smem + buf * BLKB;
    // the first three k-steps' K fragments of S(u) are requested before the
    // next unit's loads are issued (K(u) is visible since this step's
    // barrier), so their LDS latency passes while those loads go out
    const char* kl = Kb + l32 * ROWB;
    auto kfrag = [&](int mb, int ks) {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kl + mb * 32 * ROWB + (((2 * ks) ^ kf) << 4)));
    };
    bf16x8 a0[3], a1[3];
    a0[0] = kfrag(0, 0);
    a1[0] = kfrag(1, 0);
    a0[1] = kfrag(0, 1);
    a1[1] = kfrag(1, 1);
    a0[2] = kfrag(0, 2);
    a1[2] = kfrag(1, 2);
    Unit nxt;
    if (u + 1 < n_units) {
      nxt = unit(u + 1);
      issue_loads(nxt, buf ^ 1, vs_next);
    }
    vs_prev = vs_prev == 2 ? 0 : vs_prev + 1;
    vs_next = vs_next == 2 ? 0 : vs_next + 1;

    // --- S^T = K Q^T - m_ref: both 32-key halves interleaved, K fragments
    //     read two k-steps ahead of their MFMAs ---
    f32x16 s[2];
    {
      // the first k-step reads -m_ref as C and writes fresh accumulators
      __builtin_amdgcn_s_setprio(1);
      f32x16 c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[0], qf[0], negm, 0, 0, 0);
      f32x16 c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[0], qf[0], negm, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 1; ks < NKS; ++ks) {
        if (ks + 2 < NKS) {
          a0[(ks + 2) % 3] = kfrag(0, ks + 2);
          a1[(ks + 2) % 3] = kfrag(1, ks + 2);
        }
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[ks % 3], qf[ks], c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[ks % 3], qf[ks], c1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      s[0] = c0;
      s[1] = c1;
    }

    // --- mask, then the online softmax ---
    switch (cur.mk) {
      case MK_NONE: break;
      case MK_COUNT: apply_mask<MK_COUNT>(p, cur, qi, hl, s); break;
      case MK_SEPLLM: apply_mask<MK_SEPLLM>(p, cur, qi, hl, s); break;
      case MK_LALL: apply_mask<MK_LALL>(p, cur, qi, hl, s); break;
      case MK_LNORM: apply_mask<MK_LNORM>(p, cur, qi, hl, s); break;
      case MK_LCAP: apply_mask<MK_LCAP>(p, cur, qi, hl, s); break;
      default: apply_mask<MK_SEG>(p, cur, qi, hl, s); break;
    }
    if constexpr (ALIBI) add_alibi(cur, qi, hl, m2, Lf, s);
    if constexpr (!decltype(full_path)::value) {
      // common path: p = 2^(s - m_ref) straight from the MFMA output
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mb][r] = __builtin_amdgcn_exp2f(s[mb][r]);
      pack_p(s, pb);
      float psum = sum_p(pb);
      if (__any(psum > 1024.f)) {
        // rare: raise the reference of the rows whose values grew
        float pm = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) pm = fmaxf(pm, s[mb][r]);
        pm = swap_halves_max(pm);
        if (__any(!(pm < 0x1p64f))) {
          // Some logit lies 64 or more base-2 units above its row's
          // reference: its weight may have overflowed to +inf (from 128 units
          // up) and 1/pm would leave the normal range.  The unit's logits are
          // computed again from its K block, still in LDS (the slot is
          // refilled only after the next step's barrier), and the unit takes
          // the exact-max update: the reference rises to the unit's row
          // maximum and every weight is <= 1.
          {
            const char* kl = Kb + l32 * ROWB;
            f32x16 c0 = negm, c1 = negm;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
              const bf16x8 a0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kl + (((2 * ks) ^ kf) << 4)));
              const bf16x8 a1 =
                  __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kl + 32 * ROWB + (((2 * ks) ^ kf) << 4)));
              c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], c0, 0, 0, 0);
              c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], c1, 0, 0, 0);
            }
            s[0] = c0;
            s[1] = c1;
          }
          switch (cur.mk) {
            case MK_NONE: break;
            case MK_COUNT: apply_mask<MK_COUNT>(p, cur, qi, hl, s); break;
            case MK_SEPLLM: apply_mask<MK_SEPLLM>(p, cur, qi, hl, s); break;
            case MK_LALL: apply_mask<MK_LALL>(p, cur, qi, hl, s); break;
            case MK_LNORM: apply_mask<MK_LNORM>(p, cur, qi, hl, s); break;
            case MK_LCAP: apply_mask<MK_LCAP>(p, cur, qi, hl, s); break;
            default: apply_mask<MK_SEG>(p, cur, qi, hl, s); break;
          }
          if constexpr (ALIBI) add_alibi(cur, qi, hl, m2, Lf, s);
          float mx = NEG_INF;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
          mx = fmaxf(swap_halves_max(mx), 0.f);  // relative to m_ref; every row has a reference here
          const float alpha = __builtin_amdgcn_exp2f(-mx);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[mb][r] = __builtin_amdgcn_exp2f(s[mb][r] - mx);
#pragma unroll
          for (int dm = 0; dm < NDM; ++dm) acc[dm] *= alpha;
          l_run *= alpha;
          m_ref += mx;
          negm = f32x16{} - m_ref;
          pm = 1.f;  // the division below is not needed
        }
        if (pm > 1.f) {
          const float f = 1.f / pm;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) s[mb] *= f;
#pragma unroll
          for (int dm = 0; dm < NDM; ++dm) acc[dm] *= f;
          l_run *= f;
          m_ref += __log2f(pm);
          negm = f32x16{} - m_ref;
        }
        pack_p(s, pb);
        psum = sum_p(pb);
      }
      l_run += psum;
    } else {
      // some row has no finite reference yet: exact max of this unit
      float mx = NEG_INF;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
      mx = swap_halves_max(mx);  // relative to m_ref
      float delta = 0.f;
      if (mx != NEG_INF) delta = has_ref ? fmaxf(mx, 0.f) : mx;
      const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mb][r] = __builtin_amdgcn_exp2f(s[mb][r] - delta);
      pack_p(s, pb);
#pragma unroll
      for (int dm = 0; dm < NDM; ++dm) acc[dm] *= alpha;
      l_run = l_run * alpha + sum_p(pb);
      m_ref += delta;
      has_ref = has_ref || mx != NEG_INF;
      negm = f32x16{} - m_ref;
    }

    // the raw queries for the capped units: loaded once Q is no longer read
    // by this step, and waited for with the next unit's K/V at the top of the
    // next step
    if (u + 1 == u_cap && tu.n_capu > 0) load_q(p.q, p.qsB, p.qsH, p.qsT);
    cur = nxt;
  };
  int u = 0;
  for (; u < n_units && !__all(has_ref); ++u) step(u, std::true_type{});
  for (; u < n_units; ++u) step(u, std::false_type{});
  if (n_units > 0) pv(pb, vs_prev);  // the last unit (its V landed before the last barrier)

  // --- epilogue ---
  const float l_tot = swap_halves_sum(l_run);
  if (qok) {
    const bool bad = plan_overflowed(p);
    const float inv = bad ? __builtin_nanf("") : (l_tot > 0.f ? 1.f / l_tot : 0.f);
    char* orow = static_cast<char*>(p.o) + (b * p.osB + hq * p.osH + (int64_t)qi * p.osT) * 2;
#pragma unroll
    for (int dm = 0; dm < NDM; ++dm) {
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
      p.lse[((int64_t)b * p.h_q + hq) * p.n_q + qi] = bad ? __builtin_nanf("") : (m_ref + __log2f(l_tot)) * LN2;
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
  const float m2 = p.alibi ? alibi_slope_log2(p, hq) : 0.f;
  const float Lf = (float)p.L;
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
      if (p.alibi) x = fmaf(-m2, fminf((float)(qi - u.key0 - r), Lf), x);
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
    const bool bad = plan_overflowed(p);
    const float inv = bad ? __builtin_nanf("") : (l_run > 0.f ? 1.f / l_run : 0.f);
    float* orow = static_cast<float*>(p.o) + (b * p.osB + hq * p.osH + (int64_t)qi * p.osT);
#pragma unroll
    for (int c = 0; c < D; c += 4)
      *reinterpret_cast<float4*>(orow + c) =
          make_float4(acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv);
    if (p.lse != nullptr)
      p.lse[((int64_t)b * p.h_q + hq) * p.n_q + qi] = bad ? __builtin_nanf("") : (m_run + log2f(l_run)) * LN2;
  }
}

}  // namespace

hipError_t launch_fwd(const sa_mask_t& m, const sa_plan_header_t& lay, const void* plan,
                      const sa_fwd_args_t& a, const RopeOut& ro, hipStream_t s) {
  const char* pb = static_cast<const char*>(plan);
  FwdArgs p;
  memset(&p, 0, sizeof(p));
  const bool rope = a.rope == SA_ROPE_HALF;
  if (ro.qrot != nullptr) {  // fp32: the rotated query copy
    p.q = ro.qrot;
    p.qsT = a.d; p.qsH = (int64_t)m.n_q * a.d; p.qsB = p.qsH * a.h_q;
  } else {
    p.q = a.q;
    p.qsB = a.q_stride[0]; p.qsH = a.q_stride[1]; p.qsT = a.q_stride[2];
  }
  if (rope) {
    p.k = ro.krot;
    p.ksT = a.d; p.ksH = (int64_t)m.n_k * a.d; p.ksB = p.ksH * a.h_kv;
  } else {
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
  p.n_sep = reinterpret_cast<const int*>(pb + offsetof(sa_plan_header_t, n_sep));
  p.cap_sep = lay.cap_sep;
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
  p.alibi = a.rope == SA_ALIBI ? 1 : 0;
  p.alibi_e = p.alibi ? a.alibi_exp : 0.f;
  if (a.dtype == SA_BF16) {
    p.rot_q = rope ? 1 : 0;
    p.q_pos0 = m.kind == SA_MASK_SEGMENT ? m.prefix_len : 0;
    p.q_scale = p.scale_log2;
    if (rope) {
      p.th1 = std::pow((double)a.rope_base, -2.0 / a.d);
      p.th8 = std::pow((double)a.rope_base, -16.0 / a.d);
      p.th16 = std::pow((double)a.rope_base, -32.0 / a.d);
    }
  }
  const unsigned grid = (unsigned)((int64_t)a.batch * a.h_q * lay.n_tiles);
  if (a.dtype == SA_BF16 && a.d == 128) {
    if (p.alibi)
      hipLaunchKernelGGL((fwd_bf16<128, true>), dim3(grid), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((fwd_bf16<128, false>), dim3(grid), dim3(256), 0, s, p);
  } else if (a.dtype == SA_BF16) {
    if (p.alibi)
      hipLaunchKernelGGL((fwd_bf16<64, true>), dim3(grid), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((fwd_bf16<64, false>), dim3(grid), dim3(256), 0, s, p);
  } else if (a.d == 64) {
    hipLaunchKernelGGL(fwd_f32<64>, dim3(grid), dim3(128), 0, s, p);
  } else {
    hipLaunchKernelGGL(fwd_f32<128>, dim3(grid), dim3(128), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace sa
