// Backward of the sparse attention forward: dQ, dK and dV over the same plan.
//
// What is computed (the forward's logits and softmax as in sa_fwd.hip; the
// gradient is the textbook one of a masked softmax): with P_ij =
// exp(s_ij - LSE_i) over the visible pairs, D_i = <dO_i, O_i>,
// dP_ij = <dO_i, v_j> and dS_ij = P_ij (dP_ij - D_i):
//   dq~_i = scale sum_j dS_ij k~_j        dk~_j = scale sum_i dS_ij q~_i
//   dv_j  = sum_i P_ij dO_i
// in the rotated frame (q~ = R(pos_q) q, k~ = R(pos_k) k); the raw gradients
// are dq = R(-pos_q) dq~ and dk = R(-pos_k) dk~.  LM-Infinite capped pairs
// (logit scale <q_i, R(-L) k_j>) add scale R(-L) k_j dS_ij to dq_i and
// scale R(L) q_i dS_ij to dk_j.  SepLLM pairs read from the gathered
// separator rows add to those rows' gradients, which are added back to the
// separator positions.  Every sum runs in a fixed order: no atomics, the
// result is the same bit for bit from run to run.
//
// Kernels:
//   bwd_rowdot     D_i = <dO_i, O_i> (fp32).
//   bwd_dq_bf16    query-major, the forward's work units per 128-query tile:
//                  S^T = K Q^T, P = 2^(S - LSE log2 e), dP^T = V dO^T,
//                  dS, then dQ^T += K^T dS^T (K^T by LDS transpose reads).
//   bwd_dkdv_bf16  key-major: one 8-wave work group per (batch, kv head,
//                  128-key group), the group being two dense key blocks, two
//                  chunks of 64 gathered separator rows or two blocks of
//                  capped keys.  It visits every (tile, query head) that
//                  reads the group, 64 queries at a time, the next chunk's
//                  loads in flight while the current one computes: S = Q K^T,
//                  P, dP = dO V^T, dS, then dV^T += dO^T P and
//                  dK^T += Q^T dS (transpose reads of the query-side tiles).
//   bwd_dq_valu, bwd_dkdv_valu
//                  fp32, and bf16 with d = 64: the same two sums on the
//                  vector ALU in fp32 (query-major per tile; key-major per
//                  64-key unit), a thread per 32-element slice of a row.
//   bwd_finish     per row: the inverse rotations, the separator and capped
//                  contributions, the output dtype.  After the MFMA kernels
//                  only the dk, dv rows with a separator or capped
//                  contribution are left to it: those kernels write every
//                  other row in its final form (inverse rotation and bf16 in
//                  their epilogues), so the fp32 sums of those rows never go
//                  through memory.
#include <type_traits>

#include "sa_common.h"
#include "sa_device.h"

namespace sa {
namespace {

struct BwdArgs {
  const void* q;      // rotated queries, scaled by scale * log2(e) (the forward's copy)
  int64_t qsB, qsH, qsT;
  const void* qraw;   // raw queries (capped pairs)
  int64_t qrB, qrH, qrT;
  const void* k;      // rotated keys (raw when rope is off)
  int64_t ksB, ksH, ksT;
  const void* v;
  int64_t vsB, vsH, vsT;
  const void* ksep;   // [B, h_kv, sep_rows, d] gathered separator keys (rotated) / values
  const void* vsep;
  int64_t sep_rows;
  const void* kcap;   // [B, h_kv, cap_rows, d] R(-L) k * scale * log2(e)
  int64_t cap_rows;
  const void* dout;
  int64_t dsB, dsH, dsT;
  const float* lse;   // [B, h_q, n_q]
  const float* Dv;    // [B, h_q, n_q]
  float* dq_acc;      // [B, h_q, n_q, d]: scale * sum dS k~ (rotated frame)
  float* dq_cap;      // [B, h_q, n_q, d]: scale * sum dS R(-L) k (capped pairs), or null
  float* dk_acc;      // [B, h_kv, n_k, d]: sum dS q~s over the dense blocks
  float* dv_acc;      // [B, h_kv, n_k, d]
  float* dksep;       // [B, h_kv, sep_rows, d]
  float* dvsep;
  float* dkcap;       // [B, h_kv, cap_rows, d]: sum dS q (raw) over the capped pairs
  float* dvcap;       // [B, h_kv, cap_rows, d]: sum P dO over the capped pairs
  const int* tile_ptr;
  const int* items;
  const int* sep_count;
  const unsigned long long* sep_bits;
  const int* n_sep;   // the plan header's separator count
  int kind, B, h_q, h_kv, n_q, n_k, n_tiles, n_blocks, group;
  int a, w, n_s, L, P, n_cap;
  int use_cap, gather;
  float scale;
  int alibi;
  float alibi_e;
  int n_sep_chunks, n_cap_blocks;  // group counts of the key-major kernel
};

// The bf16 MFMA kernels' outputs: the final gradients are written in place by
// the kernel that owns the row (every dq row; every dk, dv row that takes no
// separator or capped contribution), and the finishing pass handles only the
// rows that do.  (A separate argument: the vector-ALU kernels keep BwdArgs
// alone, whose size steers their register allocation.)
struct BwdOut {
  int rot;             // rotary frame on (inverse rotations in the epilogues)
  int q_pos0;          // position of query 0 (the prefix length of a segment)
  void* dq;
  int64_t dqB, dqH, dqT;
  void* dk;
  int64_t dkB, dkH, dkT;
  void* dv;
  int64_t dvB, dvH, dvT;
  const int* blk_sep;  // separators (j >= g0) before each key block
  int g0;
  double th1, th4, th8;  // theta_1 = base^(-2/d) and its 4th and 8th powers (theta_c = theta_1^c)
  int n_lead;          // leading dense key groups read by every tile (dispatched first)
};

// True when key row j takes a contribution from outside its dense key group:
// a gathered separator (j >= g0, marked, within the gathered rows) or an
// LM-Infinite capped key (j < n_cap, n_cap = 0 without capped pairs).  The
// key-major kernel and the finishing pass decide it with this one test.
__device__ inline bool key_row_special(const unsigned long long* sep_bits, const int* blk_sep, int g0,
                                       int64_t sep_rows, bool has_sep, int n_cap, int j) {
  if (j < n_cap) return true;
  if (has_sep && j >= g0) {
    const int blk = j / BK, r = j - blk * BK;
    const unsigned long long word = sep_bits[blk];
    if ((word >> r) & 1ull) {
      const int64_t rank = blk_sep[blk] + __popcll(word & ((r == 0) ? 0ull : (~0ull >> (64 - r))));
      return rank < sep_rows;
    }
  }
  return false;
}

// cos and sin of pos * theta with tt = theta / (2 pi): the angle reduced in
// fp64 to a fraction of a turn, the hardware cosine and sine taking turns.
__device__ inline void turn_sc(double pos, double tt, float& c, float& s) {
  const double rev = pos * tt;
  const float f = (float)(rev - rint(rev));
  c = __builtin_amdgcn_cosf(f);
  s = __builtin_amdgcn_sinf(f);
}

// Rotates a lane's d = 128 accumulator pairs (dim c, c + 64) by pos * theta_c
// and multiplies them by f.  Lane half hl holds dims 32 dm + 8 g + 4 hl + e in
// register 4 g + e of acc[dm], so the partner of dm < 2 is dm + 2 in the same
// register.  theta_c / (2 pi) comes from products of powers of theta_1 in fp64
// (a few ulp from the direct power).
__device__ inline void rotate_acc128(const BwdOut& p, int hl, double pos, float f, f32x16 (&acc)[4]) {
  double tk = (hl ? p.th4 : 1.0) * 0.15915494309189535;  // theta_{4 hl} / (2 pi)
#pragma unroll
  for (int k = 0; k < 8; ++k) {  // dims 8 k + 4 hl + e: dm = k / 4, g = k % 4
    const int dm = k >> 2, g = k & 3;
    double tt = tk;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float c, s;
      turn_sc(pos, tt, c, s);
      tt *= p.th1;
      const float x1 = acc[dm][4 * g + e], x2 = acc[dm + 2][4 * g + e];
      acc[dm][4 * g + e] = (x1 * c - x2 * s) * f;
      acc[dm + 2][4 * g + e] = (x2 * c + x1 * s) * f;
    }
    tk *= p.th8;
    __builtin_amdgcn_sched_barrier(0);  // one group at a time: few live temporaries
  }
}

// Writes a lane's d = 128 row (layout as in rotate_acc128) as bf16, rounded
// to nearest even.
__device__ inline void store_row_bf16(char* row, int hl, const f32x16 (&acc)[4]) {
#pragma unroll
  for (int dm = 0; dm < 4; ++dm)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * dm + 8 * g + 4 * hl;
      const f32x2 x01 = {acc[dm][4 * g], acc[dm][4 * g + 1]};
      const f32x2 x23 = {acc[dm][4 * g + 2], acc[dm][4 * g + 3]};
      uint2 w;
      w.x = __builtin_bit_cast(unsigned, __builtin_convertvector(x01, bf16x2));
      w.y = __builtin_bit_cast(unsigned, __builtin_convertvector(x23, bf16x2));
      *reinterpret_cast<uint2*>(row + d0 * 2) = w;
    }
}

// ---------------------------------------------------------------------------
// D_i = <dO_i, O_i>: d * esz / 16 consecutive lanes per row (16 for bf16
// d = 128, 32 for fp32), one 16-byte piece each, then a butterfly sum over
// those lanes.
// ---------------------------------------------------------------------------

struct RowDotArgs {
  const char* dout;
  int64_t dsB, dsH, dsT;
  const char* o;
  int64_t osB, osH, osT;
  float* D;
  int B, h, n, d, esz;
};

__device__ inline float bf_lo(unsigned x) { return __uint_as_float(x << 16); }
__device__ inline float bf_hi(unsigned x) { return __uint_as_float(x & 0xffff0000u); }

__global__ __launch_bounds__(256) void bwd_rowdot(RowDotArgs p) {
  const int pieces = p.d * p.esz / 16;  // 16 for bf16 d = 128, 32 for fp32
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = g / pieces;
  const int pc = (int)(g % pieces);
  const int64_t rows = (int64_t)p.B * p.h * p.n;
  float acc = 0.f;
  if (row < rows) {
    const int i = (int)(row % p.n);
    const int64_t bh = row / p.n;
    const int h = (int)(bh % p.h), b = (int)(bh / p.h);
    const uint4 x = *reinterpret_cast<const uint4*>(p.dout + (b * p.dsB + h * p.dsH + (int64_t)i * p.dsT) * p.esz + pc * 16);
    const uint4 y = *reinterpret_cast<const uint4*>(p.o + (b * p.osB + h * p.osH + (int64_t)i * p.osT) * p.esz + pc * 16);
    const unsigned xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
    if (p.esz == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(bf_lo(xs[e]), bf_lo(ys[e]), acc);
        acc = fmaf(bf_hi(xs[e]), bf_hi(ys[e]), acc);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(__uint_as_float(xs[e]), __uint_as_float(ys[e]), acc);
    }
  }
  for (int m = 1; m < pieces; m <<= 1) acc += __shfl_xor(acc, m, pieces);  // a row's pieces: aligned lanes
  if (row < rows && pc == 0) p.D[row] = acc;
}

// Packs one 32-row C tile (rows = the MFMA contraction index) into the two
// bf16x8 B operands: k-step ks takes registers 8 ks .. 8 ks + 7.
__device__ inline void pack_tile(const f32x16& s, bf16x8 (&pb)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const f32x2 two = {s[8 * ks + e], s[8 * ks + e + 1]};
      const bf16x2 c2 = __builtin_convertvector(two, bf16x2);
      pb[ks][e] = c2[0];
      pb[ks][e + 1] = c2[1];
    }
  }
}

// ===========================================================================
// dQ: query-major, 4 waves x 32 queries per 128-query tile (the forward's
// layout: S^T = K Q^T, one query per lane).
// ===========================================================================

template <bool ALIBI>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16(BwdArgs p, BwdOut fo) {
  // K and V of the current unit and of the next one (separate arrays, so a
  // read of one slot never waits for the loads into the other)
  __shared__ __attribute__((aligned(16))) char K0[BLK_BYTES];
  __shared__ __attribute__((aligned(16))) char V0[BLK_BYTES];
  __shared__ __attribute__((aligned(16))) char K1[BLK_BYTES];
  __shared__ __attribute__((aligned(16))) char V1[BLK_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  int b, kvh, t, hq;
  map_unit(p, b, kvh, t, hq);
  const int qi = t * TQ + wid * 32 + l32;
  const bool qok = qi < p.n_q;

  TileUnits tu;
  tile_items<!ALIBI>(p, t, tu);
  tu.nsep = p.gather ? ld_uniform(p.sep_count + t) : 0;
  tu.n_ch = (tu.nsep + BK - 1) / BK;
  tu.kb = static_cast<const char*>(p.k) + (b * p.ksB + kvh * p.ksH) * 2;
  tu.vb = static_cast<const char*>(p.v) + (b * p.vsB + kvh * p.vsH) * 2;
  tu.kst = p.ksT * 2;
  tu.vst = p.vsT * 2;
  tu.capb = static_cast<const char*>(p.kcap) + ((int64_t)b * p.h_kv + kvh) * p.cap_rows * (D128 * 2);
  const int64_t sep_off = ((int64_t)b * p.h_kv + kvh) * p.sep_rows * (D128 * 2);
  tu.ksb = static_cast<const char*>(p.ksep) + sep_off;
  tu.vsb = static_cast<const char*>(p.vsep) + sep_off;
  const int n_units = tu.n_capu + tu.n_ch + tu.n_items;
  // the forward's phase-aligned walk over the window blocks (this kernel
  // visits the capped units first): neighbouring tiles read a block together
  if (!ALIBI && tu.n_items > 1) {
    const int b_last = ld_uniform(p.items + tu.it0 + tu.n_items - 1) & 0xffffff;
    const int m = tu.n_items;
    tu.rot = (2 * m - 1 - b_last % m + (tu.n_capu + tu.n_ch) % m) % m;
  }
  const float m2 = ALIBI ? alibi_slope_log2(p, hq) : 0.f;
  const float Lf = (float)p.L;

  bf16x8 qf[8], df[8];
  auto load_rows = [&](bf16x8 (&f)[8], const void* base, int64_t sB, int64_t sH, int64_t sT) {
    const char* row = static_cast<const char*>(base) + (b * sB + hq * sH + (int64_t)qi * sT) * 2;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (qok) x = ld16_once(row + (16 * s + 8 * hl) * 2);  // read once per tile
      f[s] = __builtin_bit_cast(bf16x8, x);
    }
  };
  if (tu.n_capu > 0) load_rows(qf, p.qraw, p.qrB, p.qrH, p.qrT);
  else load_rows(qf, p.q, p.qsB, p.qsH, p.qsT);
  load_rows(df, p.dout, p.dsB, p.dsH, p.dsT);
  const int64_t rowi = ((int64_t)b * p.h_q + hq) * p.n_q + (qok ? qi : 0);
  const float lse2 = qok ? p.lse[rowi] * LOG2E : 0.f;
  const float Dq = qok ? p.Dv[rowi] : 0.f;

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};

  const int kf = swzf(l32) ^ hl;
  const int vrow = 4 * hl + ((lane & 15) >> 2);
  const int vf0 = swzf(vrow), vf1 = swzf(vrow + 8);
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int vcb = vcol >> 3;

  auto store_acc = [&](float* dst, float f) {
    if (!qok) return;
    float* row = dst + rowi * D128;
#pragma unroll
    for (int dm = 0; dm < 4; ++dm)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dm + 8 * g + 4 * hl;
        *reinterpret_cast<float4*>(row + d0) =
            make_float4(acc[dm][4 * g] * f, acc[dm][4 * g + 1] * f, acc[dm][4 * g + 2] * f, acc[dm][4 * g + 3] * f);
      }
  };

  // C = A B over the 8 k-steps of d for the 32-key half mb of an LDS block
  // (A rows 32 mb + l32), fragments one k-step ahead
  auto half_product = [&](const char* blk, const bf16x8 (&bop)[8], int mb) __attribute__((always_inline)) {
    const char* kl = blk + (32 * mb + l32) * 256;
    auto frag = [&](int ks) {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kl + (((2 * ks) ^ kf) << 4)));
    };
    bf16x8 a[2];
    a[0] = frag(0);
    f32x16 c = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks + 1 < 8) a[(ks + 1) % 2] = frag(ks + 1);
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks % 2], bop[ks], c, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    return c;
  };

  auto step = [&](int u, char* Kc, char* Vc, char* Kn, char* Vn) __attribute__((always_inline)) {
    // this wave's loads of unit u have landed; the barrier makes every wave's
    // visible and ends the reads of the slot the next loads overwrite
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (u == tu.n_capu && u > 0) {
      // capped units done: their dq (raw frame) goes to dq_cap, the rest is rotated-frame
      store_acc(p.dq_cap, LN2);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
      load_rows(qf, p.q, p.qsB, p.qsH, p.qsT);
    }
    const Unit cur = unit_at<ALIBI>(p, tu, u);
    if (u + 1 < n_units) {
      const Unit nx = unit_at<ALIBI>(p, tu, u + 1);
      dma_block(nx.kbase, nx.kstride, nx.kvalid, Kn, wid, lane);
      dma_block(nx.vbase, nx.vstride, nx.vvalid, Vn, wid, lane);
    }
    // S^T = K Q^T - lse2 (base 2), masked, exponentiated
    f32x16 s[2];
    s[0] = half_product(Kc, qf, 0);
    s[1] = half_product(Kc, qf, 1);
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
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mb][r] = __builtin_amdgcn_exp2f(s[mb][r] - lse2);
    // dP^T = V dO^T; dS = P (dP - D), masked pairs exactly 0
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const f32x16 dp = half_product(Vc, df, mb);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mb][r] = s[mb][r] * (dp[r] - Dq);
    }
    bf16x8 dsb[4];
    pack_p(s, dsb);
    // dQ^T += K^T dS^T, K^T fragments by transpose reads two MFMAs ahead
    const char* tl = Kc + vrow * 256 + ((vcol & 7) << 1);
    auto tfrag = [&](int kst, int dm) {
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4*)(tl + (16 * kst) * 256 + (((4 * dm + vcb) ^ vf0) << 4)));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4*)(tl + (16 * kst + 8) * 256 + (((4 * dm + vcb) ^ vf1) << 4)));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 ta[3];
    ta[0] = tfrag(0, 0);
    ta[1] = tfrag(0, 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kst = i >> 2, dm = i & 3;
      if (i + 2 < 16) ta[(i + 2) % 3] = tfrag((i + 2) >> 2, (i + 2) & 3);
      acc[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[i % 3], dsb[kst], acc[dm], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (n_units > 0) {
    const Unit u0 = unit_at<ALIBI>(p, tu, 0);
    dma_block(u0.kbase, u0.kstride, u0.kvalid, K0, wid, lane);
    dma_block(u0.vbase, u0.vstride, u0.vvalid, V0, wid, lane);
  }
  int u = 0;
  for (; u + 1 < n_units; u += 2) {
    step(u, K0, V0, K1, V1);
    step(u + 1, K1, V1, K0, V0);
  }
  if (u < n_units) step(u, K0, V0, K1, V1);

  {
    // the final row: dq = scale R(-pos) sum + the capped part, which this
    // lane stored to dq_cap (raw frame, times ln 2) when the capped units
    // ended (only capped units: that part is still in acc), bf16
    if (!qok) return;
    if (p.use_cap && tu.n_capu == n_units && n_units > 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= LN2;
    } else {
      if (fo.rot) {
        rotate_acc128(fo, hl, -(double)(fo.q_pos0 + qi), p.scale, acc);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= p.scale;
      }
      if (p.use_cap && tu.n_capu > 0) {
        const float* cr = p.dq_cap + rowi * D128;
#pragma unroll
        for (int dm = 0; dm < 4; ++dm)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 x = *reinterpret_cast<const float4*>(cr + 32 * dm + 8 * g + 4 * hl);
            acc[dm][4 * g] += x.x;
            acc[dm][4 * g + 1] += x.y;
            acc[dm][4 * g + 2] += x.z;
            acc[dm][4 * g + 3] += x.w;
          }
      }
    }
    store_row_bf16(static_cast<char*>(fo.dq) + (b * fo.dqB + hq * fo.dqH + (int64_t)qi * fo.dqT) * 2, hl, acc);
  }
}

// ===========================================================================
// dK, dV: key-major.  Work group = (batch, kv head, key group); 4 waves, wave
// w owns keys 32 (w & 1) .. +31 of the group and queries 32 (w >> 1) .. +31 of
// each 64-query chunk; S = Q K^T has queries as rows and one key per lane, so
// the gradient accumulators dK^T, dV^T (d x 32 keys) stay in the lane.
// ===========================================================================

enum GroupKind : int { G_DENSE = 0, G_SEP = 1, G_CAP = 2 };

// Key-on-lane masks: register r of the tile holds query i0 + 8 (r / 4) + r % 4
// (i0 = the tile's first query + 4 hl), the lane's key is j.
template <int MK>
__device__ inline void mask_keys(const BwdArgs& p, int i0, int j, bool jsep, int count_ok, f32x16& s) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = i0 + 8 * (r >> 2) + (r & 3);
    bool vis = i < p.n_q;
    if (MK == MK_COUNT) {
      vis = vis & (count_ok != 0);
    } else if (MK == MK_NONE) {
    } else if (MK == MK_SEPLLM) {
      vis = vis & (j <= i) & (j < p.n_k) & ((j < p.a) | (i - j < p.w) | jsep);
    } else if (MK == MK_LALL) {
      vis = vis & (j <= i) & (j < p.n_k) & ((j < p.n_s) | (i - j <= p.L));
    } else if (MK == MK_LNORM) {
      vis = vis & (j <= i) & (j < p.n_k) & (i - j <= p.L);
    } else if (MK == MK_LCAP) {
      vis = vis & (j < p.n_s) & (j < p.n_k) & (i - j > p.L);
    } else {
      vis = vis & (j <= p.P + i) & (j < p.n_k);
    }
    s[r] = vis ? s[r] : NEG_INF;
  }
}

// First tile t in [lo, n_tiles) with sep_count[t] > c0 (sep_count is
// nondecreasing in t); n_tiles if none.
__device__ inline int first_gathering_tile(const BwdArgs& p, int c0) {
  int lo = 0, hi = p.n_tiles;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (ld_uniform(p.sep_count + mid) > c0) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// The item of block blk in tile t, or -1.  The plan lists a tile's leading
// blocks 0 .. lo_end-1 and then one run of consecutive blocks ending at the
// tile's last item, so blk can only sit at index lo + blk or at
// (hi - 1) - (last block - blk): two probes instead of a search (each search
// step is a dependent scalar load).
__device__ inline int find_item(const BwdArgs& p, int t, int blk) {
  const int lo = ld_uniform(p.tile_ptr + t), hi = ld_uniform(p.tile_ptr + t + 1);
  if (hi <= lo) return -1;
  const int last = ld_uniform(p.items + hi - 1) & 0xffffff;
  const int iw = hi - 1 - (last - blk);
  if (blk <= last && iw >= lo) {
    const int it = ld_uniform(p.items + iw);
    if ((it & 0xffffff) == blk) return it;
  }
  if (blk < hi - lo) {
    const int it = ld_uniform(p.items + lo + blk);
    if ((it & 0xffffff) == blk) return it;
  }
  return -1;
}

// find_item for a per-lane tile (plain loads).
__device__ inline int find_item_lane(const BwdArgs& p, int t, int blk) {
  const int lo = p.tile_ptr[t], hi = p.tile_ptr[t + 1];
  if (hi <= lo) return -1;
  const int last = p.items[hi - 1] & 0xffffff;
  const int iw = hi - 1 - (last - blk);
  if (blk <= last && iw >= lo) {
    const int it = p.items[iw];
    if ((it & 0xffffff) == blk) return it;
  }
  if (blk < hi - lo) {
    const int it = p.items[lo + blk];
    if ((it & 0xffffff) == blk) return it;
  }
  return -1;
}

constexpr int TINFO_CAP = 2048;  // tiles the key-major kernel tabulates per group

// One 64-row unit of a 128-key group (dense block, separator chunk or capped block).
struct KeyUnit {
  const char* kbase;
  const char* vbase;
  int64_t kstr, vstr;
  int valid;       // rows held (0: the unit does not exist)
  int key0;        // key index of row 0 (dense and capped units)
  int idx;         // block / chunk index
  float* dk_out;
  float* dv_out;
};

template <bool ALIBI>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_bf16(BwdArgs p, BwdOut fo) {
  // the group's 128 keys and values; two buffers of (64 queries, their dO rows,
  // their lse * log2(e) and D), one filled while the other is read
  __shared__ __attribute__((aligned(16))) char Kg[2 * BLK_BYTES];
  __shared__ __attribute__((aligned(16))) char Vg[2 * BLK_BYTES];
  __shared__ __attribute__((aligned(16))) char Qb0[BLK_BYTES];
  __shared__ __attribute__((aligned(16))) char Db0[BLK_BYTES];
  __shared__ __attribute__((aligned(16))) char Qb1[BLK_BYTES];
  __shared__ __attribute__((aligned(16))) char Db1[BLK_BYTES];
  __shared__ __attribute__((aligned(16))) float LD0[2][64];
  __shared__ __attribute__((aligned(16))) float LD1[2][64];
  // how each tile from t0 on reads the group (see unit_mk; built once below)
  __shared__ int tinfo[TINFO_CAP];
  __shared__ int tinfo_end;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int kw = wid & 3, qw = wid >> 2;  // keys 32 kw .. of the group; query half of a chunk
  const int hu = kw >> 1;                 // this wave's unit
  const int BH = p.B * p.h_kv;
  const int bh = blockIdx.x % BH;
  const int gi = blockIdx.x / BH;
  const int b = bh / p.h_kv, kvh = bh % p.h_kv;
  const int n_sep_pairs = (p.n_sep_chunks + 1) / 2, n_cap_pairs = (p.n_cap_blocks + 1) / 2;

  // Grid order, longest walks first: the dense groups that every tile reads
  // (SepLLM's initial tokens; LM-Infinite's starting tokens when no pass caps
  // them), the gathered-separator chunks, the capped blocks, the other dense
  // groups.
  int kind, pi;
  if (gi < fo.n_lead) { kind = G_DENSE; pi = gi; }
  else if (gi - fo.n_lead < n_sep_pairs) { kind = G_SEP; pi = gi - fo.n_lead; }
  else if (gi - fo.n_lead < n_sep_pairs + n_cap_pairs) { kind = G_CAP; pi = gi - fo.n_lead - n_sep_pairs; }
  else { kind = G_DENSE; pi = gi - n_sep_pairs - n_cap_pairs; }

  // (clamped to the gathered rows: a mask past the plan's sep_max bound)
  const int n_sep_all = kind == G_SEP ? min(ld_uniform(p.n_sep), (int)p.sep_rows) : 0;
  if (kind == G_SEP && pi * 2 * BK >= n_sep_all) return;
  KeyUnit U0, U1;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    KeyUnit& u = x ? U1 : U0;
    u.idx = 2 * pi + x;
    u.key0 = u.idx * BK;
    if (kind == G_SEP) {
      const int64_t ho = ((int64_t)b * p.h_kv + kvh) * p.sep_rows + (int64_t)u.idx * BK;
      u.kbase = static_cast<const char*>(p.ksep) + ho * (D128 * 2);
      u.vbase = static_cast<const char*>(p.vsep) + ho * (D128 * 2);
      u.kstr = u.vstr = D128 * 2;
      u.valid = max(0, min(BK, n_sep_all - u.idx * BK));
      u.dk_out = p.dksep + ho * D128;
      u.dv_out = p.dvsep + ho * D128;
      u.key0 = 0;
    } else if (kind == G_CAP) {
      const int64_t ho = ((int64_t)b * p.h_kv + kvh) * p.cap_rows + (int64_t)u.idx * BK;
      u.kbase = static_cast<const char*>(p.kcap) + ho * (D128 * 2);
      u.kstr = D128 * 2;
      u.vbase = static_cast<const char*>(p.v) + (b * p.vsB + kvh * p.vsH + (int64_t)u.idx * BK * p.vsT) * 2;
      u.vstr = p.vsT * 2;
      u.valid = max(0, min(BK, p.n_cap - u.idx * BK));
      u.dk_out = p.dkcap + ho * D128;
      u.dv_out = p.dvcap + ho * D128;
    } else {
      u.kbase = static_cast<const char*>(p.k) + (b * p.ksB + kvh * p.ksH + (int64_t)u.idx * BK * p.ksT) * 2;
      u.vbase = static_cast<const char*>(p.v) + (b * p.vsB + kvh * p.vsH + (int64_t)u.idx * BK * p.vsT) * 2;
      u.kstr = p.ksT * 2;
      u.vstr = p.vsT * 2;
      u.valid = max(0, min(BK, p.n_k - u.idx * BK));
      const int64_t ho = ((int64_t)b * p.h_kv + kvh) * p.n_k + (int64_t)u.idx * BK;
      u.dk_out = p.dk_acc + ho * D128;
      u.dv_out = p.dv_acc + ho * D128;
    }
  }
  // keys of unit x by waves 4x .. 4x+3 (dma_block moves rows 16 w' .. 16 w' + 15)
  {
    const KeyUnit u = (wid >> 2) ? U1 : U0;
    if (u.valid > 0) {
      dma_block(u.kbase, u.kstr, u.valid, Kg + (wid >> 2) * BLK_BYTES, wid & 3, lane);
      dma_block(u.vbase, u.vstr, u.valid, Vg + (wid >> 2) * BLK_BYTES, wid & 3, lane);
    }
  }

  const KeyUnit mu = hu ? U1 : U0;
  const int kslot64 = 32 * (kw & 1) + l32;  // row within this wave's unit
  const int kslot = 32 * kw + l32;          // row within the group
  const int j = mu.key0 + kslot64;
  bool jsep = false;
  if (kind == G_DENSE && p.kind == SA_MASK_SEPLLM && j < p.n_k && mu.valid > 0)
    jsep = (p.sep_bits[mu.idx] >> kslot64) & 1ull;

  f32x16 dka[4], dva[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { dka[i] = f32x16{}; dva[i] = f32x16{}; }

  const int kf = swzf(l32) ^ hl;
  const int vrow = 4 * hl + ((lane & 15) >> 2);
  const int vf0 = swzf(vrow), vf1 = swzf(vrow + 8);
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int vcb = vcol >> 3;

  const bool q_raw = kind == G_CAP;
  const void* qsrc = q_raw ? p.qraw : p.q;
  const int64_t qB = q_raw ? p.qrB : p.qsB, qH = q_raw ? p.qrH : p.qsH, qT = q_raw ? p.qrT : p.qsT;

  // mask kind of unit x in tile t (-1: not read by the tile)
  auto unit_mk = [&](int x, int t, int& count) -> int {
    const int valid = x ? U1.valid : U0.valid;
    const int uidx = x ? U1.idx : U0.idx;
    count = 0;
    if (valid <= 0) return -1;
    if (kind == G_SEP) {
      count = ld_uniform(p.sep_count + t) - uidx * BK;
      return count > 0 ? MK_COUNT : -1;
    }
    const int it = find_item(p, t, uidx);
    if (it < 0) return -1;
    const int fl = it >> 24;
    if (kind == G_CAP) return (fl & SA_ITEM_CAPPED) ? MK_LCAP : -1;
    if (p.use_cap && (fl & SA_ITEM_CAPPED)) {
      // no pair of the ordinary pass when the block is farther than L from the whole tile
      if (uidx * BK + BK - 1 < t * TQ - p.L) return -1;
      return MK_LNORM;
    }
    if (fl & SA_ITEM_FULL) return MK_NONE;
    if (p.kind == SA_MASK_SEPLLM) return MK_SEPLLM;
    if (p.kind == SA_MASK_LAMBDA) return MK_LALL;
    return MK_SEG;
  };
  // chunk cursor: (tile, query head of the group, 64-query half) and the
  // tile's mask kind and separator count per unit
  struct Cur {
    int t, gq, ch;
    int mk0, mk1, cnt0, cnt1;
  };

  int t0;
  if (kind == G_SEP) t0 = first_gathering_tile(p, pi * 2 * BK);
  else t0 = max(0, U0.key0 - (p.kind == SA_MASK_SEGMENT ? p.P : 0)) / TQ;

  // The tiles from t0 on, evaluated once by all threads (each a few tiles,
  // every plan read a plain per-lane load) into tinfo: the walk below then
  // reads LDS instead of a chain of dependent scalar loads per tile.  A dense
  // block's readers are consecutive: the first tile that reads neither unit
  // ends the walk.  More than TINFO_CAP tiles: the scalar walk.
  const bool use_tab = p.n_tiles - t0 <= TINFO_CAP;
  if (use_tab) {
    if (tid == 0) tinfo_end = p.n_tiles;
    __syncthreads();
    for (int t = t0 + tid; t < p.n_tiles; t += 512) {
      int mk[2], cnt[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const KeyUnit& u = x ? U1 : U0;
        mk[x] = -1;
        cnt[x] = 0;
        if (u.valid <= 0) continue;
        if (kind == G_SEP) {
          cnt[x] = max(0, min(BK, p.sep_count[t] - u.idx * BK));
          mk[x] = cnt[x] > 0 ? MK_COUNT : -1;
          continue;
        }
        const int it = find_item_lane(p, t, u.idx);
        if (it < 0) continue;
        const int fl = it >> 24;
        if (kind == G_CAP) {
          mk[x] = (fl & SA_ITEM_CAPPED) ? MK_LCAP : -1;
        } else if (p.use_cap && (fl & SA_ITEM_CAPPED)) {
          mk[x] = (u.idx * BK + BK - 1 < t * TQ - p.L) ? -1 : MK_LNORM;
        } else if (fl & SA_ITEM_FULL) {
          mk[x] = MK_NONE;
        } else {
          mk[x] = p.kind == SA_MASK_SEPLLM ? MK_SEPLLM : (p.kind == SA_MASK_LAMBDA ? MK_LALL : MK_SEG);
        }
      }
      tinfo[t - t0] = (mk[0] & 0xF) | ((mk[1] & 0xF) << 4) | (cnt[0] << 8) | (cnt[1] << 16);
      if (kind == G_DENSE && mk[0] < 0 && mk[1] < 0) atomicMin(&tinfo_end, t);
    }
    __syncthreads();
  }
  const int t_end = use_tab ? tinfo_end : p.n_tiles;

  // first tile at or after t that reads the group (t = n_tiles when none)
  auto tile_from = [&](int t) -> Cur {
    Cur c{p.n_tiles, 0, 0, -1, -1, 0, 0};
    if (use_tab) {
      for (; t < t_end; ++t) {
        const int v = __builtin_amdgcn_readfirstlane(tinfo[t - t0]);
        const int m0 = (v & 0xF) == 0xF ? -1 : (v & 0xF), m1 = ((v >> 4) & 0xF) == 0xF ? -1 : ((v >> 4) & 0xF);
        if (m0 >= 0 || m1 >= 0) {
          c.t = t;
          c.mk0 = m0;
          c.mk1 = m1;
          c.cnt0 = (v >> 8) & 0xFF;
          c.cnt1 = (v >> 16) & 0xFF;
          return c;
        }
      }
      return c;
    }
    for (; t < p.n_tiles; ++t) {
      int c0, c1;
      const int m0 = unit_mk(0, t, c0), m1 = unit_mk(1, t, c1);
      if (m0 >= 0 || m1 >= 0) {
        c.t = t;
        c.mk0 = m0;
        c.mk1 = m1;
        c.cnt0 = c0;
        c.cnt1 = c1;
        return c;
      }
      if (kind == G_DENSE) return c;  // the tiles reading a dense block are consecutive
    }
    return c;
  };

  // A gathered separator chunk is read by every tile from t0 on, a leading
  // dense group by every tile.  With separator groups present, those groups
  // walk their tiles last to first: the ones of a kv head that run together
  // on one XCD all start at the last tile, so they read each tile's Q and dO
  // rows at about the same time, while the rows are in that XCD's L2
  // (walking first to last, each would stream its own range).  Without them
  // a leading group walks first to last, in step with the dense groups that
  // follow it, which read the first tiles too.
  const bool back = kind == G_SEP || (kind == G_DENSE && pi < fo.n_lead && p.gather);
  // last tile at or before t that reads the group (t = n_tiles when none)
  auto tile_back = [&](int t) -> Cur {
    Cur c{p.n_tiles, 0, 0, -1, -1, 0, 0};
    for (; t >= t0; --t) {
      int m0, m1, c0, c1;
      if (use_tab) {
        const int v = __builtin_amdgcn_readfirstlane(tinfo[t - t0]);
        m0 = (v & 0xF) == 0xF ? -1 : (v & 0xF);
        m1 = ((v >> 4) & 0xF) == 0xF ? -1 : ((v >> 4) & 0xF);
        c0 = (v >> 8) & 0xFF;
        c1 = (v >> 16) & 0xFF;
      } else {
        m0 = unit_mk(0, t, c0);
        m1 = unit_mk(1, t, c1);
      }
      if (m0 >= 0 || m1 >= 0) {
        c.t = t;
        c.mk0 = m0;
        c.mk1 = m1;
        c.cnt0 = c0;
        c.cnt1 = c1;
        return c;
      }
    }
    return c;
  };

  auto advance = [&](Cur c) -> Cur {
    ++c.ch;
    if (c.ch == 2 || c.t * TQ + 64 * c.ch >= p.n_q) {
      c.ch = 0;
      if (++c.gq == p.group) return back ? tile_back(c.t - 1) : tile_from(c.t + 1);
    }
    return c;
  };
  auto issue = [&](const Cur& c, char* Qd, char* Dd, float (*LDd)[64]) __attribute__((always_inline)) {
    const int hq = kvh * p.group + c.gq;
    const int qc0 = c.t * TQ + 64 * c.ch;
    const int qvalid = min(64, p.n_q - qc0);
    if (wid < 4)
      dma_block(static_cast<const char*>(qsrc) + (b * qB + hq * qH + (int64_t)qc0 * qT) * 2, qT * 2, qvalid, Qd,
                wid, lane);
    else
      dma_block(static_cast<const char*>(p.dout) + (b * p.dsB + hq * p.dsH + (int64_t)qc0 * p.dsT) * 2, p.dsT * 2,
                qvalid, Dd, wid & 3, lane);
    if (wid == 0 || wid == 4) {
      const int64_t r0 = ((int64_t)b * p.h_q + hq) * p.n_q + qc0;
      const float* src = wid == 0 ? p.lse + r0 : p.Dv + r0;
      lds_dma<4>(src, (uint32_t)min(lane, qvalid - 1) * 4u, LDd[wid >> 2]);
    }
  };

  auto compute = [&](const Cur& c, const char* Qc, const char* Dc, const float (*LDc)[64]) __attribute__((always_inline)) {
    const int mk = hu ? c.mk1 : c.mk0;
    const int count = hu ? c.cnt1 : c.cnt0;
    if (mk < 0) return;
    const int hq = kvh * p.group + c.gq;
    const float m2 = ALIBI ? alibi_slope_log2(p, hq) : 0.f;
    const int qc0 = c.t * TQ + 64 * c.ch;
    const int count_ok = kslot64 < count;
    f32x16 s = f32x16{}, dp = f32x16{};
    {
      const char* ql = Qc + (32 * qw + l32) * 256;
      const char* dl = Dc + (32 * qw + l32) * 256;
      const char* kl = Kg + kslot * 256;
      const char* vl = Vg + kslot * 256;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int off = ((2 * ks) ^ kf) << 4;
        const bf16x8 qa = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ql + off));
        const bf16x8 kb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kl + off));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kb, s, 0, 0, 0);
        const bf16x8 da = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(dl + off));
        const bf16x8 vb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(vl + off));
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vb, dp, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const int i0 = qc0 + 32 * qw + 4 * hl;
    switch (mk) {
      case MK_NONE: mask_keys<MK_NONE>(p, i0, j, jsep, count_ok, s); break;
      case MK_COUNT: mask_keys<MK_COUNT>(p, i0, j, jsep, count_ok, s); break;
      case MK_SEPLLM: mask_keys<MK_SEPLLM>(p, i0, j, jsep, count_ok, s); break;
      case MK_LALL: mask_keys<MK_LALL>(p, i0, j, jsep, count_ok, s); break;
      case MK_LNORM: mask_keys<MK_LNORM>(p, i0, j, jsep, count_ok, s); break;
      case MK_LCAP: mask_keys<MK_LCAP>(p, i0, j, jsep, count_ok, s); break;
      default: mask_keys<MK_SEG>(p, i0, j, jsep, count_ok, s); break;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 l4 = *reinterpret_cast<const float4*>(&LDc[0][32 * qw + 8 * g + 4 * hl]);
      const float4 d4 = *reinterpret_cast<const float4*>(&LDc[1][32 * qw + 8 * g + 4 * hl]);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        float x = s[r];
        if constexpr (ALIBI) x = fmaf(-m2, fminf((float)(i0 + 8 * g + e - j), (float)p.L), x);
        const float pe = __builtin_amdgcn_exp2f(x - lv[e] * LOG2E);
        s[r] = pe;
        dp[r] = pe * (dp[r] - dv4[e]);
      }
    }
    bf16x8 pb[2], db[2];
    pack_tile(s, pb);
    pack_tile(dp, db);
    const char* dt = Dc + (32 * qw + vrow) * 256 + ((vcol & 7) << 1);
    const char* qt = Qc + (32 * qw + vrow) * 256 + ((vcol & 7) << 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ks = i >> 2, dm = i & 3;
      const int o0 = (16 * ks) * 256 + (((4 * dm + vcb) ^ vf0) << 4);
      const int o1 = (16 * ks + 8) * 256 + (((4 * dm + vcb) ^ vf1) << 4);
      const bf16x4 dlo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(dt + o0));
      const bf16x4 dhi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(dt + o1));
      dva[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(dlo, dhi, 0, 1, 2, 3, 4, 5, 6, 7),
                                                       pb[ks], dva[dm], 0, 0, 0);
      const bf16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(qt + o0));
      const bf16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(qt + o1));
      dka[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7),
                                                       db[ks], dka[dm], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The two waves on a SIMD (wave w and w + 4: the same keys, the two query
  // halves) would run the same phases at the same time; the first half's
  // wave issues first, so it runs ahead and its softmax meets the other's
  // products.
  if (qw == 0) __builtin_amdgcn_s_setprio(2);
  // chunk loop: wait for chunk c and for every read of the other buffers, start
  // chunk c+1 into them, compute chunk c
  Cur cur = back ? tile_back(p.n_tiles - 1) : tile_from(t0);
  if (cur.t < p.n_tiles) issue(cur, Qb0, Db0, LD0);
  while (cur.t < p.n_tiles) {
    {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      const Cur nx = advance(cur);
      if (nx.t < p.n_tiles) issue(nx, Qb1, Db1, LD1);
      compute(cur, Qb0, Db0, LD0);
      cur = nx;
    }
    if (cur.t >= p.n_tiles) break;
    {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      const Cur nx = advance(cur);
      if (nx.t < p.n_tiles) issue(nx, Qb0, Db0, LD0);
      compute(cur, Qb1, Db1, LD1);
      cur = nx;
    }
  }

  // waves qw = 1 hand their sums to waves qw = 0 through LDS (32 KB per key
  // quarter: Kg, Vg, Qb0 + Db0, Qb1 + Db1), which add them and store
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  float* redk = reinterpret_cast<float*>(kw == 0 ? Kg : kw == 1 ? Vg : kw == 2 ? Qb0 : Qb1);
  float* redv = kw < 2 ? redk + 4096 : reinterpret_cast<float*>(kw == 2 ? Db0 : Db1);
  if (qw == 1) {
#pragma unroll
    for (int dm = 0; dm < 4; ++dm)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        redk[(dm * 16 + r) * 64 + lane] = dka[dm][r];
        redv[(dm * 16 + r) * 64 + lane] = dva[dm][r];
      }
  }
  __syncthreads();
  if (qw == 0 && kslot64 < mu.valid) {
#pragma unroll
    for (int dm = 0; dm < 4; ++dm)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dka[dm][r] += redk[(dm * 16 + r) * 64 + lane];
        dva[dm][r] += redv[(dm * 16 + r) * 64 + lane];
      }
    if (kind == G_DENSE &&
        !key_row_special(p.sep_bits, fo.blk_sep, fo.g0, p.sep_rows, p.gather != 0, p.use_cap ? p.n_cap : 0, j)) {
      // no contribution from another group: the final rows, dv = sum and
      // dk = R(-j) ln 2 sum (the queries carry scale * log2(e)), bf16
      store_row_bf16(static_cast<char*>(fo.dv) + (b * fo.dvB + kvh * fo.dvH + (int64_t)j * fo.dvT) * 2, hl, dva);
      if (fo.rot) {
        rotate_acc128(fo, hl, -(double)j, LN2, dka);
      } else {
#pragma unroll
        for (int dm = 0; dm < 4; ++dm) dka[dm] *= LN2;
      }
      store_row_bf16(static_cast<char*>(fo.dk) + (b * fo.dkB + kvh * fo.dkH + (int64_t)j * fo.dkT) * 2, hl, dka);
    } else {
      float* krow = mu.dk_out + (int64_t)kslot64 * D128;
      float* vrow_o = mu.dv_out + (int64_t)kslot64 * D128;
#pragma unroll
      for (int dm = 0; dm < 4; ++dm)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * dm + 8 * g + 4 * hl;
          *reinterpret_cast<float4*>(krow + d0) =
              make_float4(dka[dm][4 * g], dka[dm][4 * g + 1], dka[dm][4 * g + 2], dka[dm][4 * g + 3]);
          *reinterpret_cast<float4*>(vrow_o + d0) =
              make_float4(dva[dm][4 * g], dva[dm][4 * g + 1], dva[dm][4 * g + 2], dva[dm][4 * g + 3]);
        }
    }
  }
}

// ===========================================================================
// Vector-ALU backward: fp32 (no bf16 rounding anywhere), and bf16 with
// d = 64 (bf16 rows read and widened, every product and sum in fp32).  The
// same sums as above, the same accumulator sections and the same finishing
// kernel.  The query copy and the capped keys carry scale * log2(e) for bf16
// (the RoPE stage's convention) and nothing for fp32, which decides the
// factor of the logits (1 or scale * log2(e)), of dq_cap (ln 2 or scale) and
// of dk_acc in the finish (ln 2 or scale).  A thread owns a 32-element slice
// of its row; a dot product is the slice's fma chain plus a butterfly over
// the row's D/32 lanes (adjacent lanes, so every lane gets the same sum).
// ===========================================================================

constexpr int F32_SLICE = 32;

template <int TPR>
__device__ inline float row_sum(float x) {
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// One 16-byte piece of a row (4 fp32 or 8 bf16 elements) widened to fp32.
template <class T>
__device__ inline void load_piece(const T* src, float* x) {
  const uint4 v = *reinterpret_cast<const uint4*>(src);
  const unsigned w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(w[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf_lo(w[e]);
      x[2 * e + 1] = bf_hi(w[e]);
    }
  }
}

// Loads a 32-element slice (zeros when !ok).
template <class T>
__device__ inline void load_slice(const T* src, bool ok, float (&x)[F32_SLICE]) {
  constexpr int EP = 16 / (int)sizeof(T);
#pragma unroll
  for (int c = 0; c < F32_SLICE; c += EP) {
    if (ok) load_piece(src + c, x + c);
    else
#pragma unroll
      for (int e = 0; e < EP; ++e) x[c + e] = 0.f;
  }
}

// Stages `rows` rows (row r at base + r * stride bytes) of a D-element T row
// into an fp32 LDS array [nrows][D], zeros past `valid`.
template <class T, int D, int NT>
__device__ inline void stage_rows(float (*dst)[D], int nrows, const char* base, int64_t stride, int valid, int tid) {
  constexpr int EP = 16 / (int)sizeof(T), CH = D / EP;
  for (int x = tid; x < nrows * CH; x += NT) {
    const int r = x / CH, ch = x % CH;
    float v[EP];
    if (r < valid) load_piece(reinterpret_cast<const T*>(base + r * stride) + ch * EP, v);
    else
#pragma unroll
      for (int e = 0; e < EP; ++e) v[e] = 0.f;
#pragma unroll
    for (int e = 0; e < EP; ++e) dst[r][ch * EP + e] = v[e];
  }
}

// dQ: one work group per (batch, query head, 128-query tile), the forward's
// units in the forward's order; thread = (query, slice).
//   dq_acc_i = scale sum dS_ij k~_j        dq_cap_i = scale sum dS_ij R(-L) k_j
template <class T, int D>
__global__ __launch_bounds__(TQ * D / F32_SLICE) void bwd_dq_valu(BwdArgs p) {
  constexpr int ESZ = (int)sizeof(T);
  constexpr bool F32 = ESZ == 4;
  constexpr int TPR = D / F32_SLICE, NT = TQ * TPR;
  __shared__ __attribute__((aligned(16))) float Ks[BK][D];
  __shared__ __attribute__((aligned(16))) float Vs[BK][D];
  const int tid = threadIdx.x;
  const int c0 = (tid % TPR) * F32_SLICE;
  int b, kvh, t, hq;
  map_unit(p, b, kvh, t, hq);
  const int qi = t * TQ + tid / TPR;
  const bool qok = qi < p.n_q;
  const int64_t row = ((int64_t)b * p.h_q + hq) * p.n_q + (qok ? qi : 0);
  float q[F32_SLICE], g[F32_SLICE], dq[F32_SLICE], dqc[F32_SLICE];
  load_slice(static_cast<const T*>(p.dout) + b * p.dsB + hq * p.dsH + (int64_t)qi * p.dsT + c0, qok, g);
  auto load_q = [&](bool raw) {
    const T* src = raw ? static_cast<const T*>(p.qraw) + b * p.qrB + hq * p.qrH + (int64_t)qi * p.qrT
                       : static_cast<const T*>(p.q) + b * p.qsB + hq * p.qsH + (int64_t)qi * p.qsT;
    load_slice(src + c0, qok, q);
  };
  load_q(false);
  bool q_is_raw = false;
#pragma unroll
  for (int c = 0; c < F32_SLICE; ++c) { dq[c] = 0.f; dqc[c] = 0.f; }
  const float lse2 = qok ? p.lse[row] * LOG2E : 0.f;
  const float Di = qok ? p.Dv[row] : 0.f;
  const float sl2 = F32 ? p.scale * LOG2E : 1.f;
  const float m2 = p.alibi ? alibi_slope_log2(p, hq) : 0.f;
  const float Lf = (float)p.L;

  auto unit = [&](const Unit& u, bool raw_q) {
    if (raw_q != q_is_raw) {
      load_q(raw_q);
      q_is_raw = raw_q;
    }
    stage_rows<T, D, NT>(Ks, BK, u.kbase, u.kstride, u.kvalid, tid);
    stage_rows<T, D, NT>(Vs, BK, u.vbase, u.vstride, u.vvalid, tid);
    __syncthreads();
    for (int r = 0; r < BK; ++r) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < F32_SLICE; ++c) {
        s = fmaf(q[c], Ks[r][c0 + c], s);
        dp = fmaf(g[c], Vs[r][c0 + c], dp);
      }
      s = row_sum<TPR>(s);
      dp = row_sum<TPR>(dp);
      float x = s * sl2;
      if (p.alibi) x = fmaf(-m2, fminf((float)(qi - u.key0 - r), Lf), x);
      const bool vis = qok && r < u.kvalid && (u.mk == MK_NONE || visible(p, u, qi, r));
      const float pr = vis ? exp2f(x - lse2) : 0.f;
      const float ds = pr * (dp - Di);
      if (raw_q) {
#pragma unroll
        for (int c = 0; c < F32_SLICE; ++c) dqc[c] = fmaf(ds, Ks[r][c0 + c], dqc[c]);
      } else {
#pragma unroll
        for (int c = 0; c < F32_SLICE; ++c) dq[c] = fmaf(ds, Ks[r][c0 + c], dq[c]);
      }
    }
    __syncthreads();
  };
  for_each_unit(p, b, kvh, t, ESZ, (int64_t)D * ESZ, unit);
  // dq_cap = scale sum dS R(-L) k: the capped keys carry scale * log2(e) for bf16
  const float cap_mul = F32 ? p.scale : LN2;
  if (qok) {
    float* o = p.dq_acc + row * D + c0;
#pragma unroll
    for (int c = 0; c < F32_SLICE; c += 4)
      *reinterpret_cast<float4*>(o + c) =
          make_float4(dq[c] * p.scale, dq[c + 1] * p.scale, dq[c + 2] * p.scale, dq[c + 3] * p.scale);
    if (p.use_cap) {
      float* oc = p.dq_cap + row * D + c0;
#pragma unroll
      for (int c = 0; c < F32_SLICE; c += 4)
        *reinterpret_cast<float4*>(oc + c) =
            make_float4(dqc[c] * cap_mul, dqc[c + 1] * cap_mul, dqc[c + 2] * cap_mul, dqc[c + 3] * cap_mul);
    }
  }
}

// dK, dV: key-major, one work group per (batch, kv head, 64-key unit: a
// gathered separator chunk, a capped block or a dense block); thread =
// (key, slice).  It walks the tiles that read the unit in order, every query
// head of the group, 32 queries at a time staged in LDS:
//   dk_j += dS_ij q_i (q~, or the raw q for capped pairs)   dv_j += P_ij dO_i
template <class T, int D>
__global__ __launch_bounds__(BK * D / F32_SLICE) void bwd_dkdv_valu(BwdArgs p) {
  constexpr int ESZ = (int)sizeof(T);
  constexpr bool F32 = ESZ == 4;
  constexpr int TPR = D / F32_SLICE, NT = BK * TPR, QC = 32;
  __shared__ __attribute__((aligned(16))) float Qs[QC][D];
  __shared__ __attribute__((aligned(16))) float Gs[QC][D];
  __shared__ float Ls[QC], Ds[QC];
  const int tid = threadIdx.x;
  const int kk = tid / TPR, c0 = (tid % TPR) * F32_SLICE;
  const int BH = p.B * p.h_kv;
  const int bh = blockIdx.x % BH;
  const int gi = blockIdx.x / BH;
  const int b = bh / p.h_kv, kvh = bh % p.h_kv;
  int kind, idx;
  if (gi < p.n_sep_chunks) { kind = G_SEP; idx = gi; }
  else if (gi < p.n_sep_chunks + p.n_cap_blocks) { kind = G_CAP; idx = gi - p.n_sep_chunks; }
  else { kind = G_DENSE; idx = gi - p.n_sep_chunks - p.n_cap_blocks; }
  // (clamped to the gathered rows: a mask past the plan's sep_max bound)
  const int n_sep_all = kind == G_SEP ? min(ld_uniform(p.n_sep), (int)p.sep_rows) : 0;
  if (kind == G_SEP && idx * BK >= n_sep_all) return;

  const int64_t rowb = (int64_t)D * ESZ;
  const char* kbase;
  const char* vbase;
  int64_t kstr, vstr;
  int valid, key0 = idx * BK;
  float *dk_out, *dv_out;
  if (kind == G_SEP) {
    const int64_t ho = ((int64_t)b * p.h_kv + kvh) * p.sep_rows + (int64_t)idx * BK;
    kbase = static_cast<const char*>(p.ksep) + ho * rowb;
    vbase = static_cast<const char*>(p.vsep) + ho * rowb;
    kstr = vstr = rowb;
    valid = min(BK, n_sep_all - idx * BK);
    dk_out = p.dksep + ho * D;
    dv_out = p.dvsep + ho * D;
    key0 = 0;
  } else if (kind == G_CAP) {
    const int64_t ho = ((int64_t)b * p.h_kv + kvh) * p.cap_rows + (int64_t)idx * BK;
    kbase = static_cast<const char*>(p.kcap) + ho * rowb;
    kstr = rowb;
    vbase = static_cast<const char*>(p.v) + (b * p.vsB + kvh * p.vsH + (int64_t)key0 * p.vsT) * ESZ;
    vstr = p.vsT * ESZ;
    valid = min(BK, p.n_cap - key0);
    dk_out = p.dkcap + ho * D;
    dv_out = p.dvcap + ho * D;
  } else {
    kbase = static_cast<const char*>(p.k) + (b * p.ksB + kvh * p.ksH + (int64_t)key0 * p.ksT) * ESZ;
    vbase = static_cast<const char*>(p.v) + (b * p.vsB + kvh * p.vsH + (int64_t)key0 * p.vsT) * ESZ;
    kstr = p.ksT * ESZ;
    vstr = p.vsT * ESZ;
    valid = min(BK, p.n_k - key0);
    const int64_t ho = ((int64_t)b * p.h_kv + kvh) * p.n_k + key0;
    dk_out = p.dk_acc + ho * D;
    dv_out = p.dv_acc + ho * D;
  }
  const bool kok = kk < valid;
  float kx[F32_SLICE], vx[F32_SLICE], dk[F32_SLICE], dv[F32_SLICE];
  load_slice(reinterpret_cast<const T*>(kbase + kk * kstr) + c0, kok, kx);
  load_slice(reinterpret_cast<const T*>(vbase + kk * vstr) + c0, kok, vx);
#pragma unroll
  for (int c = 0; c < F32_SLICE; ++c) { dk[c] = 0.f; dv[c] = 0.f; }
  const int j = key0 + kk;
  const bool q_raw = kind == G_CAP;
  const char* qsrc = static_cast<const char*>(q_raw ? p.qraw : p.q);
  const int64_t qB = q_raw ? p.qrB : p.qsB, qH = q_raw ? p.qrH : p.qsH, qT = q_raw ? p.qrT : p.qsT;
  const float sl2 = F32 ? p.scale * LOG2E : 1.f;
  const float Lf = (float)p.L;

  // the unit as one tile reads it (mk < 0: not read)
  auto unit_of = [&](int t) -> Unit {
    Unit u;
    u.key0 = key0;
    u.count = 0;
    u.sbits = 0;
    u.mk = -1;
    if (kind == G_SEP) {
      u.count = ld_uniform(p.sep_count + t) - idx * BK;
      if (u.count > 0) u.mk = MK_COUNT;
      return u;
    }
    const int it = find_item(p, t, idx);
    if (it < 0) return u;
    const int fl = it >> 24;
    if (kind == G_CAP) {
      if (fl & SA_ITEM_CAPPED) u.mk = MK_LCAP;
    } else if (p.use_cap && (fl & SA_ITEM_CAPPED)) {
      u.mk = MK_LNORM;
    } else if (fl & SA_ITEM_FULL) {
      u.mk = MK_NONE;
    } else if (p.kind == SA_MASK_SEPLLM) {
      u.mk = MK_SEPLLM;
      u.sbits = ld_uniform(p.sep_bits + idx);
    } else if (p.kind == SA_MASK_LAMBDA) {
      u.mk = MK_LALL;
    } else {
      u.mk = MK_SEG;
    }
    return u;
  };
  // Tiles reading the unit: separator chunk c from the first tile gathering
  // more than 64 c rows to the last (the counts never decrease); a dense
  // block from the tile holding its first key while the tiles list it
  // (consecutive); a capped block: every tile, each checked.
  int t = 0;
  if (kind == G_SEP) t = first_gathering_tile(p, idx * BK);
  else if (kind == G_DENSE) t = max(0, key0 - (p.kind == SA_MASK_SEGMENT ? p.P : 0)) / TQ;
  for (; t < p.n_tiles; ++t) {
    const Unit u = unit_of(t);
    if (u.mk < 0) {
      if (kind == G_DENSE) break;
      continue;
    }
    for (int gq = 0; gq < p.group; ++gq) {
      const int hq = kvh * p.group + gq;
      const float m2 = p.alibi ? alibi_slope_log2(p, hq) : 0.f;
      const int q_end = min(p.n_q, (t + 1) * TQ);
      for (int qc0 = t * TQ; qc0 < q_end; qc0 += QC) {
        const int qv = q_end - qc0;
        stage_rows<T, D, NT>(Qs, QC, qsrc + (b * qB + hq * qH + (int64_t)qc0 * qT) * ESZ, qT * ESZ, qv, tid);
        stage_rows<T, D, NT>(Gs, QC,
                             static_cast<const char*>(p.dout) + (b * p.dsB + hq * p.dsH + (int64_t)qc0 * p.dsT) * ESZ,
                             p.dsT * ESZ, qv, tid);
        if (tid < QC) {
          const int i = qc0 + tid;
          const int64_t ri = ((int64_t)b * p.h_q + hq) * p.n_q + i;
          Ls[tid] = i < q_end ? p.lse[ri] * LOG2E : 0.f;
          Ds[tid] = i < q_end ? p.Dv[ri] : 0.f;
        }
        __syncthreads();
        for (int r = 0; r < QC; ++r) {
          const int i = qc0 + r;
          float s = 0.f, dp = 0.f;
#pragma unroll
          for (int c = 0; c < F32_SLICE; ++c) {
            s = fmaf(kx[c], Qs[r][c0 + c], s);
            dp = fmaf(vx[c], Gs[r][c0 + c], dp);
          }
          s = row_sum<TPR>(s);
          dp = row_sum<TPR>(dp);
          float x = s * sl2;
          if (p.alibi) x = fmaf(-m2, fminf((float)(i - j), Lf), x);
          const bool vis = kok && i < q_end && (u.mk == MK_NONE || visible(p, u, i, kk));
          const float pr = vis ? exp2f(x - Ls[r]) : 0.f;
          const float ds = pr * (dp - Ds[r]);
#pragma unroll
          for (int c = 0; c < F32_SLICE; ++c) {
            dk[c] = fmaf(ds, Qs[r][c0 + c], dk[c]);
            dv[c] = fmaf(pr, Gs[r][c0 + c], dv[c]);
          }
        }
        __syncthreads();
      }
    }
  }
  if (kok) {
    float* ko = dk_out + (int64_t)kk * D + c0;
    float* vo = dv_out + (int64_t)kk * D + c0;
#pragma unroll
    for (int c = 0; c < F32_SLICE; c += 4) {
      *reinterpret_cast<float4*>(ko + c) = make_float4(dk[c], dk[c + 1], dk[c + 2], dk[c + 3]);
      *reinterpret_cast<float4*>(vo + c) = make_float4(dv[c], dv[c + 1], dv[c + 2], dv[c + 3]);
    }
  }
}

// ===========================================================================
// Finish: per row, the inverse rotation of the rotated-frame sums, the
// separator and capped contributions, the output dtype.
//   dq_i = R(-pos_q(i)) dq_acc_i + dq_cap_i
//   dk_j = R(-j) ln2 (dk_acc_j + dksep_rank(j)) + scale R(L) dkcap_j
//   dv_j = dv_acc_j + dvsep_rank(j) + dvcap_j
// Thread = (row, 8 rotation pairs), as in the RoPE stage.
// ===========================================================================

struct FinishArgs {
  int which;             // 0: dq, 1: dk, 2: dv
  const float* acc;      // [B, h, n, d]
  const float* sep;      // [B, h, sep_rows, d] or null
  int64_t sep_rows;
  const float* cap;      // dq: [B, h, n, d]; dk, dv: [B, h, cap_rows, d]; or null
  int64_t cap_rows;
  int n_cap;
  char* out;
  int64_t osB, osH, osT;
  int B, h, n, d, esz;
  int rotate, pos0, L;
  float acc_scale, cap_scale;
  const unsigned long long* sep_bits;
  const int* blk_sep;
  int g0;
  int special_only;      // dk, dv: only rows with a separator or capped contribution
  int scan_n;            // rows visited per head: n, or the leading n_cap
  ThetaTable theta;
};

__device__ inline void angle_sc(double pos, double th, float* c, float* s) {
  const double TWO_PI_HI = 6.283185307179586232;
  const double TWO_PI_LO = 2.4492935982947064e-16;
  const double INV_TWO_PI = 0.15915494309189535;
  const double ang = pos * th;
  const double kq = rint(ang * INV_TWO_PI);
  double r = fma(-kq, TWO_PI_HI, ang);
  r = fma(-kq, TWO_PI_LO, r);
  sincosf((float)r, s, c);
}

__device__ inline unsigned short to_bf16(float f) {  // round to nearest even (finite inputs)
  const unsigned u = __float_as_uint(f);
  return (unsigned short)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__global__ __launch_bounds__(256) void bwd_finish(FinishArgs p) {
  const int tpr = p.d / 16;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t vis = gid / tpr;
  if (vis >= (int64_t)p.B * p.h * p.scan_n) return;
  const int c0 = (int)(gid % tpr) * 8;
  const int half = p.d / 2;
  const int i = (int)(vis % p.scan_n);
  const int64_t bh = vis / p.scan_n;
  const int64_t row = bh * p.n + i;
  const int h = (int)(bh % p.h), b = (int)(bh / p.h);
  if (p.special_only &&
      !key_row_special(p.sep_bits, p.blk_sep, p.g0, p.sep_rows, p.sep != nullptr, p.cap != nullptr ? p.n_cap : 0, i))
    return;
  const float* a = p.acc + row * p.d;
  float x1[8], x2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x1[e] = a[c0 + e];
    x2[e] = a[c0 + half + e];
  }
  if (p.sep != nullptr && i >= p.g0) {
    const int blk = i / BK, r = i - blk * BK;
    const unsigned long long word = p.sep_bits[blk];
    const int64_t rank = p.blk_sep[blk] + __popcll(word & ((r == 0) ? 0ull : (~0ull >> (64 - r))));
    if (((word >> r) & 1ull) && rank < p.sep_rows) {  // rows past a broken sep_max bound: none
      const float* sr = p.sep + (bh * p.sep_rows + rank) * p.d;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x1[e] += sr[c0 + e];
        x2[e] += sr[c0 + half + e];
      }
    }
  }
  float y1[8], y2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x1[e] *= p.acc_scale;
    x2[e] *= p.acc_scale;
  }
  if (p.rotate) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float c, s;
      angle_sc(-(double)(p.pos0 + i), p.theta.th[c0 + e], &c, &s);
      y1[e] = x1[e] * c - x2[e] * s;
      y2[e] = x2[e] * c + x1[e] * s;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) { y1[e] = x1[e]; y2[e] = x2[e]; }
  }
  if (p.cap != nullptr) {
    const float* cr = nullptr;
    if (p.which == 0) cr = p.cap + row * p.d;
    else if (i < p.n_cap) cr = p.cap + (bh * p.cap_rows + i) * p.d;
    if (cr != nullptr) {
      if (p.which == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float c, s;
          angle_sc((double)p.L, p.theta.th[c0 + e], &c, &s);
          const float z1 = cr[c0 + e], z2 = cr[c0 + half + e];
          y1[e] += p.cap_scale * (z1 * c - z2 * s);
          y2[e] += p.cap_scale * (z2 * c + z1 * s);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          y1[e] += p.cap_scale * cr[c0 + e];
          y2[e] += p.cap_scale * cr[c0 + half + e];
        }
      }
    }
  }
  char* o = p.out + (b * p.osB + h * p.osH + (int64_t)i * p.osT) * p.esz;
  if (p.esz == 2) {
    unsigned short* o16 = reinterpret_cast<unsigned short*>(o);
    uint4 w1, w2;
    w1.x = to_bf16(y1[0]) | ((unsigned)to_bf16(y1[1]) << 16);
    w1.y = to_bf16(y1[2]) | ((unsigned)to_bf16(y1[3]) << 16);
    w1.z = to_bf16(y1[4]) | ((unsigned)to_bf16(y1[5]) << 16);
    w1.w = to_bf16(y1[6]) | ((unsigned)to_bf16(y1[7]) << 16);
    w2.x = to_bf16(y2[0]) | ((unsigned)to_bf16(y2[1]) << 16);
    w2.y = to_bf16(y2[2]) | ((unsigned)to_bf16(y2[3]) << 16);
    w2.z = to_bf16(y2[4]) | ((unsigned)to_bf16(y2[5]) << 16);
    w2.w = to_bf16(y2[6]) | ((unsigned)to_bf16(y2[7]) << 16);
    *reinterpret_cast<uint4*>(o16 + c0) = w1;
    *reinterpret_cast<uint4*>(o16 + c0 + half) = w2;
  } else {
    float* of = reinterpret_cast<float*>(o);
    *reinterpret_cast<float4*>(of + c0) = make_float4(y1[0], y1[1], y1[2], y1[3]);
    *reinterpret_cast<float4*>(of + c0 + 4) = make_float4(y1[4], y1[5], y1[6], y1[7]);
    *reinterpret_cast<float4*>(of + c0 + half) = make_float4(y2[0], y2[1], y2[2], y2[3]);
    *reinterpret_cast<float4*>(of + c0 + half + 4) = make_float4(y2[4], y2[5], y2[6], y2[7]);
  }
}

}  // namespace

hipError_t launch_bwd(const sa_mask_t& m, const sa_plan_header_t& lay, const void* plan,
                      const sa_fwd_args_t& a, const sa_bwd_args_t& g, const RopeOut& ro,
                      const BwdWs& w, const ThetaTable& theta, hipStream_t s) {
  const char* pb = static_cast<const char*>(plan);
  const bool rope = a.rope == SA_ROPE_HALF;
  const bool alibi = a.rope == SA_ALIBI;
  const int64_t rows_q = (int64_t)a.batch * a.h_q * m.n_q;
  const bool f32 = a.dtype == SA_F32;
  const int esz = f32 ? 4 : 2;
  // 1. D = rowsum(dO * O)
  {
    RowDotArgs r;
    r.dout = static_cast<const char*>(g.dout);
    r.dsB = g.dout_stride[0]; r.dsH = g.dout_stride[1]; r.dsT = g.dout_stride[2];
    r.o = static_cast<const char*>(a.o);
    r.osB = a.o_stride[0]; r.osH = a.o_stride[1]; r.osT = a.o_stride[2];
    r.D = w.D;
    r.B = a.batch; r.h = a.h_q; r.n = m.n_q; r.d = a.d; r.esz = esz;
    const int64_t threads = rows_q * (a.d * esz / 16);
    hipLaunchKernelGGL(bwd_rowdot, dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, s, r);
  }
  BwdArgs p;
  memset(&p, 0, sizeof(p));
  if (ro.qrot != nullptr) {  // the rotated (bf16: and pre-scaled) query copy
    p.q = ro.qrot;
    p.qsT = a.d; p.qsH = (int64_t)m.n_q * a.d; p.qsB = p.qsH * a.h_q;
  } else {                   // fp32 without rotation: the caller's queries
    p.q = a.q;
    p.qsB = a.q_stride[0]; p.qsH = a.q_stride[1]; p.qsT = a.q_stride[2];
  }
  p.qraw = a.q;
  p.qrB = a.q_stride[0]; p.qrH = a.q_stride[1]; p.qrT = a.q_stride[2];
  if (rope) {
    p.k = ro.krot;
    p.ksT = a.d; p.ksH = (int64_t)m.n_k * a.d; p.ksB = p.ksH * a.h_kv;
  } else {
    p.k = a.k;
    p.ksB = a.k_stride[0]; p.ksH = a.k_stride[1]; p.ksT = a.k_stride[2];
  }
  p.v = a.v;
  p.vsB = a.v_stride[0]; p.vsH = a.v_stride[1]; p.vsT = a.v_stride[2];
  p.ksep = ro.ksep; p.vsep = ro.vsep; p.sep_rows = ro.sep_rows;
  p.kcap = ro.kcap; p.cap_rows = ro.cap_rows;
  p.dout = g.dout;
  p.dsB = g.dout_stride[0]; p.dsH = g.dout_stride[1]; p.dsT = g.dout_stride[2];
  p.lse = a.lse;
  p.Dv = w.D;
  p.dq_acc = w.dq_acc; p.dq_cap = w.dq_cap;
  p.dk_acc = w.dk_acc; p.dv_acc = w.dv_acc;
  p.dksep = w.dksep; p.dvsep = w.dvsep;
  p.dkcap = w.dkcap; p.dvcap = w.dvcap;
  p.tile_ptr = reinterpret_cast<const int*>(pb + lay.off_tile_ptr);
  p.items = reinterpret_cast<const int*>(pb + lay.off_items);
  p.sep_count = reinterpret_cast<const int*>(pb + lay.off_sep_count);
  p.sep_bits = reinterpret_cast<const unsigned long long*>(pb + lay.off_sep_bits);
  p.n_sep = reinterpret_cast<const int*>(pb + offsetof(sa_plan_header_t, n_sep));
  p.kind = m.kind; p.B = a.batch; p.h_q = a.h_q; p.h_kv = a.h_kv;
  p.n_q = m.n_q; p.n_k = m.n_k; p.n_tiles = lay.n_tiles; p.n_blocks = lay.n_blocks;
  p.group = a.h_q / a.h_kv;
  p.a = m.a; p.w = m.w; p.n_s = m.n_starting; p.L = m.L_pretrain; p.P = m.prefix_len;
  p.n_cap = ro.n_cap;
  p.use_cap = (m.kind == SA_MASK_LAMBDA && rope && ro.n_cap > 0) ? 1 : 0;
  p.gather = (m.kind == SA_MASK_SEPLLM && m.sep != nullptr) ? 1 : 0;
  p.scale = a.scale;
  p.alibi = alibi ? 1 : 0;
  p.alibi_e = alibi ? a.alibi_exp : 0.f;
  p.n_sep_chunks = p.gather ? (int)(ro.sep_rows / BK) : 0;
  p.n_cap_blocks = p.use_cap ? (int)ceil_div(ro.n_cap, BK) : 0;
  const bool valu = f32 || a.d != 128;  // the MFMA kernels are bf16 with d = 128
  // the MFMA kernels write the final rows themselves (see BwdOut)
  const bool fuse = !valu;
  BwdOut fo;
  memset(&fo, 0, sizeof(fo));
  fo.rot = rope ? 1 : 0;
  fo.q_pos0 = m.kind == SA_MASK_SEGMENT ? m.prefix_len : 0;
  fo.dq = g.dq;
  fo.dqB = g.dq_stride[0]; fo.dqH = g.dq_stride[1]; fo.dqT = g.dq_stride[2];
  fo.dk = g.dk;
  fo.dkB = g.dk_stride[0]; fo.dkH = g.dk_stride[1]; fo.dkT = g.dk_stride[2];
  fo.dv = g.dv;
  fo.dvB = g.dv_stride[0]; fo.dvH = g.dv_stride[1]; fo.dvT = g.dv_stride[2];
  fo.blk_sep = reinterpret_cast<const int*>(pb + lay.off_blk_sep);
  fo.g0 = lay.g0;
  if (rope) {
    fo.th1 = theta.th[1];
    fo.th4 = theta.th[4];
    fo.th8 = theta.th[8];
  }
  {
    // dense key groups (128 keys) that every tile reads: SepLLM's initial
    // tokens, LM-Infinite's starting tokens when no capped pass takes them
    int lead_keys = 0;
    if (m.kind == SA_MASK_SEPLLM) lead_keys = m.a;
    else if (m.kind == SA_MASK_LAMBDA && !p.use_cap) lead_keys = m.n_starting;
    const int n_groups = (int)((lay.n_blocks + 1) / 2);
    fo.n_lead = std::min(n_groups, (int)ceil_div(std::min(lead_keys, m.n_k), 2 * BK));
  }
  if (valu) {
    const unsigned gq = (unsigned)((int64_t)a.batch * a.h_q * lay.n_tiles);
    const int64_t units = (int64_t)p.n_sep_chunks + p.n_cap_blocks + lay.n_blocks;
    const unsigned gk = (unsigned)(units * a.batch * a.h_kv);
    if (f32 && a.d == 64) {
      hipLaunchKernelGGL((bwd_dq_valu<float, 64>), dim3(gq), dim3(TQ * 64 / F32_SLICE), 0, s, p);
      hipLaunchKernelGGL((bwd_dkdv_valu<float, 64>), dim3(gk), dim3(BK * 64 / F32_SLICE), 0, s, p);
    } else if (f32) {
      hipLaunchKernelGGL((bwd_dq_valu<float, 128>), dim3(gq), dim3(TQ * 128 / F32_SLICE), 0, s, p);
      hipLaunchKernelGGL((bwd_dkdv_valu<float, 128>), dim3(gk), dim3(BK * 128 / F32_SLICE), 0, s, p);
    } else {
      hipLaunchKernelGGL((bwd_dq_valu<__bf16, 64>), dim3(gq), dim3(TQ * 64 / F32_SLICE), 0, s, p);
      hipLaunchKernelGGL((bwd_dkdv_valu<__bf16, 64>), dim3(gk), dim3(BK * 64 / F32_SLICE), 0, s, p);
    }
  }
  // 2. dQ (query-major)
  if (!valu) {
    const unsigned grid = (unsigned)((int64_t)a.batch * a.h_q * lay.n_tiles);
    if (alibi) hipLaunchKernelGGL(bwd_dq_bf16<true>, dim3(grid), dim3(256), 0, s, p, fo);
    else hipLaunchKernelGGL(bwd_dq_bf16<false>, dim3(grid), dim3(256), 0, s, p, fo);
  }
  // 3. dK, dV (key-major): separator chunks, then capped blocks, then dense blocks
  if (!valu) {
    const int64_t groups = (int64_t)(p.n_sep_chunks + 1) / 2 + (p.n_cap_blocks + 1) / 2 + (lay.n_blocks + 1) / 2;
    const unsigned grid = (unsigned)(groups * a.batch * a.h_kv);
    if (alibi) hipLaunchKernelGGL(bwd_dkdv_bf16<true>, dim3(grid), dim3(512), 0, s, p, fo);
    else hipLaunchKernelGGL(bwd_dkdv_bf16<false>, dim3(grid), dim3(512), 0, s, p, fo);
  }
  // 4. finish: dq, dk, dv (after the MFMA kernels: only the dk, dv rows with
  // a separator or capped contribution)
  for (int which = 0; which < 3; ++which) {
    if (fuse && (which == 0 || (!p.gather && !p.use_cap))) continue;
    FinishArgs f;
    memset(&f, 0, sizeof(f));
    f.which = which;
    f.d = a.d;
    f.esz = esz;
    f.L = m.L_pretrain;
    f.theta = theta;
    f.sep_bits = p.sep_bits;
    f.blk_sep = reinterpret_cast<const int*>(pb + lay.off_blk_sep);
    f.g0 = lay.g0;
    f.B = a.batch;
    if (which == 0) {
      f.acc = w.dq_acc;
      f.cap = p.use_cap ? w.dq_cap : nullptr;
      f.h = a.h_q; f.n = m.n_q;
      f.out = static_cast<char*>(g.dq);
      f.osB = g.dq_stride[0]; f.osH = g.dq_stride[1]; f.osT = g.dq_stride[2];
      f.rotate = rope;
      f.pos0 = m.kind == SA_MASK_SEGMENT ? m.prefix_len : 0;
      f.acc_scale = 1.f;
      f.cap_scale = 1.f;
      f.g0 = 0x7fffffff;  // no separator rows on the query side
    } else {
      f.acc = which == 1 ? w.dk_acc : w.dv_acc;
      f.sep = p.gather ? (which == 1 ? w.dksep : w.dvsep) : nullptr;
      f.sep_rows = ro.sep_rows;
      f.cap = p.use_cap ? (which == 1 ? w.dkcap : w.dvcap) : nullptr;
      f.cap_rows = ro.cap_rows;
      f.n_cap = ro.n_cap;
      f.h = a.h_kv; f.n = m.n_k;
      char* dst = static_cast<char*>(which == 1 ? g.dk : g.dv);
      const int64_t* st = which == 1 ? g.dk_stride : g.dv_stride;
      f.out = dst;
      f.osB = st[0]; f.osH = st[1]; f.osT = st[2];
      f.rotate = which == 1 && rope;
      f.pos0 = 0;
      // dk_acc: sum dS q~ pre-scaled by scale * log2(e) (bf16), unscaled (fp32)
      f.acc_scale = which == 1 ? (f32 ? a.scale : LN2) : 1.f;
      f.cap_scale = which == 1 ? a.scale : 1.f;
    }
    f.special_only = fuse ? 1 : 0;
    f.scan_n = f.n;
    if (fuse && !p.gather) f.scan_n = (int)std::min<int64_t>(ro.n_cap, f.n);  // only capped rows
    const int64_t threads = (int64_t)f.B * f.h * f.scan_n * (a.d / 16);
    if (threads == 0) continue;
    hipLaunchKernelGGL(bwd_finish, dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, s, f);
  }
  return hipGetLastError();
}

}  // namespace sa
