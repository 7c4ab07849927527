// LM-Infinite's optional top-k middle tokens (LM-Infinite page, section
// "method"): for every head and query i, the k middle tokens
// (n_starting <= j < i - L) with the largest logits join the query's key set.
// A middle token lies beyond the window, so its logit is the capped one,
// scale <R(L) q_i, k_j>, which both ranks and weights it.
//
// mid_select: per 128-query tile (4 waves x 32 queries, the forward's
//   layout: S^T = K Q^T, one query per lane) every middle key block is
//   scored on MFMA against R(L) q scaled by scale * log2(e), split into a
//   bf16 high part and a bf16 low part (two products, about 16 bits of the
//   query), and each lane keeps its query's best k (score, index) pairs in
//   registers, larger score first and the lower index on ties.
// mid_merge: the selected keys' values are folded into the forward's output
//   through its log-sum-exp: O' = (O 2^(LSE2 - m) + sum_t 2^(s_t - m) v_t) /
//   (2^(LSE2 - m) + sum_t 2^(s_t - m)), m the largest exponent.
#include "sa_common.h"
#include "sa_device.h"

namespace sa {
namespace {

// Per-lane selection lists hold up to KMAX (score, index) pairs; the launch
// picks the smallest KMAX in {8, 16, 32, 64} that holds k.  Lists of 32 and
// 64 pairs run one wave per SIMD (their registers).
constexpr int KMID_LIMIT = 64;

struct MidArgs {
  const char* q;   // raw queries [B, h_q, n_q, d]
  int64_t qsB, qsH, qsT;
  const char* k;   // raw keys [B, h_kv, n_k, d]
  int64_t ksB, ksH, ksT;
  const char* v;
  int64_t vsB, vsH, vsT;
  char* o;         // forward output, rewritten
  int64_t osB, osH, osT;
  float* lse;      // [B, h_q, n_q], rewritten
  int* sel;        // [B, h_q, n_q, kmid] selected key indices (-1: none)
  float* score;    // [B, h_q, n_q, kmid] their logits, base 2
  int B, h_q, h_kv, n_q, n_k, n_tiles, group, n_s, L, kmid;
  float scale_log2;
  float cosL[64], sinL[64];  // cos, sin of L * theta_c (rotate-half pairs); identity without RoPE
};

__device__ inline bool better(float x, int j, float y, int jy) { return (x > y) | ((x == y) & (j < jy)); }

template <int KMID_MAX>
__global__ __launch_bounds__(256, KMID_MAX <= 16 ? 2 : 1) void mid_select(MidArgs p) {
  __shared__ __attribute__((aligned(16))) char K0[BLK_BYTES];
  __shared__ __attribute__((aligned(16))) char K1[BLK_BYTES];
  __shared__ float scr[32 * 256];  // a block's scores, thread t's in column t
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  // work group -> (batch, query head, tile): tiles from the last (most middle
  // keys) over all heads at once, so the longest tiles of every head start
  // first and the shortest ones fill the end of the launch
  const int BH = p.B * p.h_q;
  const int g = blockIdx.x;
  const int t = p.n_tiles - 1 - g / BH;
  const int bh = g % BH;
  const int hq = bh % p.h_q, b = bh / p.h_q;
  const int kvh = hq / p.group;
  const int q0 = t * TQ;
  const int qi = q0 + wid * 32 + l32;
  const bool qok = qi < p.n_q;

  // R(L) q * scale * log2(e), as bf16 high + low parts (B operands: this lane's
  // query, d = 16 s + 8 hl + e)
  bf16x8 qh[8], qlo[8];
  {
    const char* row = p.q + (b * p.qsB + hq * p.qsH + (int64_t)(qok ? qi : 0) * p.qsT) * 2;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      // columns c = 16 s + 8 hl + e and their rotation partners c +- 64
      const int c0 = 16 * s + 8 * hl;
      const int pc0 = c0 < 64 ? c0 + 64 : c0 - 64;
      uint4 xa = make_uint4(0, 0, 0, 0), xb = xa;
      if (qok) {
        xa = *reinterpret_cast<const uint4*>(row + c0 * 2);
        xb = *reinterpret_cast<const uint4*>(row + pc0 * 2);
      }
      const unsigned as[4] = {xa.x, xa.y, xa.z, xa.w}, bs[4] = {xb.x, xb.y, xb.z, xb.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = __uint_as_float(e & 1 ? as[e >> 1] & 0xffff0000u : as[e >> 1] << 16);
        const float xp = __uint_as_float(e & 1 ? bs[e >> 1] & 0xffff0000u : bs[e >> 1] << 16);
        const int pr = (c0 + e) & 63;  // rotation pair
        const float y = (c0 < 64 ? x * p.cosL[pr] - xp * p.sinL[pr] : x * p.cosL[pr] + xp * p.sinL[pr]) * p.scale_log2;
        const __bf16 hi = (__bf16)y;
        qh[s][e] = hi;
        qlo[s][e] = (__bf16)(y - (float)hi);
      }
    }
  }

  // middle key blocks of the tile: keys n_s .. q_last - L - 1
  const int q_last = min(q0 + TQ, p.n_q) - 1;
  const int j_hi = min(q_last - p.L - 1, p.n_k - 1);
  const int blk_lo = p.n_s / BK;
  const int blk_hi = j_hi >= p.n_s ? j_hi / BK : blk_lo - 1;
  const int n_blk = blk_hi - blk_lo + 1;

  // The lane's list, best first: its last kk slots hold the selection; the
  // KMID_MAX - kk slots before them hold sentinels (+inf, index -1) that
  // nothing displaces, so the kk-th best is always the last slot.
  const int kk = p.kmid;
  const int pad = KMID_MAX - kk;
  float bv[KMID_MAX];
  int bi[KMID_MAX];
#pragma unroll
  for (int e = 0; e < KMID_MAX; ++e) {
    bv[e] = e < pad ? __builtin_huge_valf() : -__builtin_huge_valf();
    bi[e] = e < pad ? -1 : 0x7fffffff;
  }
  float thr_v = -__builtin_huge_valf();  // the kk-th best so far (the last slot)
  int thr_i = 0x7fffffff;
  const char* kb = p.k + (b * p.ksB + kvh * p.ksH) * 2;
  const int64_t kst = p.ksT * 2;
  const int kf = swzf(l32) ^ hl;
  const int jmax = qi - p.L - 1;  // this query's last middle key
  const int wave_q0 = q0 + wid * 32;
  const int wave_jmin = wave_q0 - p.L - 1;      // the wave's smallest last middle key
  const bool wave_full = wave_q0 + 31 < p.n_q;  // every lane holds a query

  auto step = [&](int u, char* Kc, char* Kn) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    const int blk = blk_lo + u;
    if (u + 1 < n_blk)
      dma_block(kb + (int64_t)(blk + 1) * BK * kst, kst, min(BK, p.n_k - (blk + 1) * BK), Kn, wid, lane);
    // S^T = K q_hi^T + K q_lo^T: both parts accumulate into one chain per
    // 32-key half, the two halves interleaved
    f32x16 s[2];
    {
      const char* kl = Kc + l32 * 256;
      f32x16 h0 = f32x16{}, h1 = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int off = ((2 * ks) ^ kf) << 4;
        const bf16x8 a0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kl + off));
        const bf16x8 a1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kl + 32 * 256 + off));
        h0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qh[ks], h0, 0, 0, 0);
        h1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qh[ks], h1, 0, 0, 0);
        h0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qlo[ks], h0, 0, 0, 0);
        h1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qlo[ks], h1, 0, 0, 0);
      }
      s[0] = h0;
      s[1] = h1;
    }
    // candidates: register r of half mb is key j0 + 32 mb + 8 (r / 4) + r % 4,
    // so register order is ascending key order.  Keys that are not middle keys
    // of the lane's query are set to -inf (only blocks at the edges of the
    // wave's middle range have any).  The scores go to the lane's column of
    // LDS and the lane marks those at or above its k-th best (bit 16 mb + r);
    // the marked ones are then taken in ascending key order, each read back
    // from LDS and inserted while it still beats the (rising) k-th best.  A
    // score below the k-th best at the block's start can never enter, so the
    // lists end as if every key had been offered in turn.
    const int j0 = blk * BK + 4 * hl;
    if (!(blk * BK >= p.n_s && blk * BK + BK - 1 <= wave_jmin && blk * BK + BK <= p.n_k && wave_full)) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * mb + 8 * (r >> 2) + (r & 3);
          const bool ok = qok & (j >= p.n_s) & (j <= jmax) & (j < p.n_k);
          s[mb][r] = ok ? s[mb][r] : -__builtin_huge_valf();
        }
    }
    unsigned hitm = 0u;
    const float lo = fmaxf(thr_v, -__FLT_MAX__);  // (excludes -inf while the list is not full)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = s[mb][r];
        scr[(16 * mb + r) * 256 + tid] = x;
        hitm |= x >= lo ? (1u << (16 * mb + r)) : 0u;
      }
    while (__any(hitm != 0u)) {
      if (hitm != 0u) {
        const int bit = __ffs(hitm) - 1;
        hitm &= hitm - 1u;
        float x = scr[bit * 256 + tid];
        int j = j0 + 32 * (bit >> 4) + 8 * ((bit & 15) >> 2) + (bit & 3);
        if (better(x, j, thr_v, thr_i)) {
#pragma unroll
          for (int e = 0; e < KMID_MAX; ++e) {
            const bool sw = better(x, j, bv[e], bi[e]);
            const float tv = bv[e];
            const int ti = bi[e];
            bv[e] = sw ? x : tv;
            bi[e] = sw ? j : ti;
            x = sw ? tv : x;
            j = sw ? ti : j;
          }
          thr_v = bv[KMID_MAX - 1];
          thr_i = bi[KMID_MAX - 1];
        }
      }
    }
  };
  if (n_blk > 0) dma_block(kb + (int64_t)blk_lo * BK * kst, kst, min(BK, p.n_k - blk_lo * BK), K0, wid, lane);
  int u = 0;
  for (; u + 1 < n_blk; u += 2) {
    step(u, K0, K1);
    step(u + 1, K1, K0);
  }
  if (u < n_blk) step(u, K0, K1);

  // each query's keys are split between lanes l32 and l32 + 32 (4-key groups of
  // alternate halves): merge the two sorted lists
#pragma unroll
  for (int e2 = 0; e2 < KMID_MAX; ++e2) {
    float x = __shfl_xor(bv[e2], 32);
    int j = __shfl_xor(bi[e2], 32);
    if (hl == 0 && e2 >= pad && x != -__builtin_huge_valf()) {
#pragma unroll
      for (int e = 0; e < KMID_MAX; ++e) {
        if (better(x, j, bv[e], bi[e])) {
          const float tv = bv[e];
          const int ti = bi[e];
          bv[e] = x;
          bi[e] = j;
          x = tv;
          j = ti;
        }
      }
    }
  }
  if (qok && hl == 0) {
    const int64_t rowi = ((int64_t)b * p.h_q + hq) * p.n_q + qi;
#pragma unroll
    for (int e = 0; e < KMID_MAX; ++e) {
      if (e >= pad) {
        const bool has = bv[e] != -__builtin_huge_valf();
        p.sel[rowi * kk + e - pad] = has ? bi[e] : -1;
        p.score[rowi * kk + e - pad] = bv[e];
      }
    }
  }
}

// Thread = (row, 8 output columns): 16 threads per row.
__global__ __launch_bounds__(256) void mid_merge(MidArgs p) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid >> 4;
  const int cc = (int)(gid & 15);
  if (row >= (int64_t)p.B * p.h_q * p.n_q) return;
  const int i = (int)(row % p.n_q);
  const int64_t bhq = row / p.n_q;
  const int hq = (int)(bhq % p.h_q), b = (int)(bhq / p.h_q);
  const int kvh = hq / p.group;
  const float lse2 = p.lse[row] * 1.4426950408889634f;
  float m = lse2;
  for (int e = 0; e < p.kmid; ++e) {
    const int j = p.sel[row * p.kmid + e];
    if (j >= 0) m = fmaxf(m, p.score[row * p.kmid + e]);
  }
  const float f0 = __builtin_amdgcn_exp2f(lse2 - m);
  float den = f0;
  unsigned short* orow = reinterpret_cast<unsigned short*>(p.o + (b * p.osB + hq * p.osH + (int64_t)i * p.osT) * 2);
  const uint4 ox = *reinterpret_cast<const uint4*>(orow + cc * 8);
  const unsigned os[4] = {ox.x, ox.y, ox.z, ox.w};
  float acc[8];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    acc[2 * f] = __uint_as_float(os[f] << 16) * f0;
    acc[2 * f + 1] = __uint_as_float(os[f] & 0xffff0000u) * f0;
  }
  for (int e = 0; e < p.kmid; ++e) {
    const int j = p.sel[row * p.kmid + e];
    if (j < 0) continue;
    const float w = __builtin_amdgcn_exp2f(p.score[row * p.kmid + e] - m);
    den += w;
    const uint4 vx = *reinterpret_cast<const uint4*>(p.v + (b * p.vsB + kvh * p.vsH + (int64_t)j * p.vsT) * 2 + cc * 16);
    const unsigned vs[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      acc[2 * f] = fmaf(w, __uint_as_float(vs[f] << 16), acc[2 * f]);
      acc[2 * f + 1] = fmaf(w, __uint_as_float(vs[f] & 0xffff0000u), acc[2 * f + 1]);
    }
  }
  const float inv = 1.f / den;
  uint4 w4;
  unsigned ws[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const f32x2 two = {acc[2 * f] * inv, acc[2 * f + 1] * inv};
    const bf16x2 c2 = __builtin_convertvector(two, bf16x2);
    ws[f] = __builtin_bit_cast(unsigned, c2);
  }
  w4.x = ws[0];
  w4.y = ws[1];
  w4.z = ws[2];
  w4.w = ws[3];
  *reinterpret_cast<uint4*>(orow + cc * 8) = w4;
  if (cc == 0) p.lse[row] = (m + __log2f(den)) * 0.6931471805599453f;
}

}  // namespace

hipError_t launch_topk_middle(const sa_mask_t& m, const sa_fwd_args_t& a, int kmid, int32_t* sel, float* score,
                              hipStream_t s) {
  MidArgs p;
  memset(&p, 0, sizeof(p));
  p.q = static_cast<const char*>(a.q);
  p.qsB = a.q_stride[0]; p.qsH = a.q_stride[1]; p.qsT = a.q_stride[2];
  p.k = static_cast<const char*>(a.k);
  p.ksB = a.k_stride[0]; p.ksH = a.k_stride[1]; p.ksT = a.k_stride[2];
  p.v = static_cast<const char*>(a.v);
  p.vsB = a.v_stride[0]; p.vsH = a.v_stride[1]; p.vsT = a.v_stride[2];
  p.o = static_cast<char*>(a.o);
  p.osB = a.o_stride[0]; p.osH = a.o_stride[1]; p.osT = a.o_stride[2];
  p.lse = a.lse;
  p.sel = sel;
  p.score = score;
  p.B = a.batch;
  p.h_q = a.h_q;
  p.h_kv = a.h_kv;
  p.n_q = m.n_q;
  p.n_k = m.n_k;
  p.n_tiles = (int)ceil_div(m.n_q, TQ);
  p.group = a.h_q / a.h_kv;
  p.n_s = m.n_starting;
  p.L = m.L_pretrain;
  p.kmid = kmid;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  for (int c = 0; c < 64; ++c) {
    if (a.rope == SA_ROPE_HALF) {
      const double ang = (double)m.L_pretrain * std::pow((double)a.rope_base, -2.0 * c / a.d);
      p.cosL[c] = (float)std::cos(ang);
      p.sinL[c] = (float)std::sin(ang);
    } else {
      p.cosL[c] = 1.f;
      p.sinL[c] = 0.f;
    }
  }
  const unsigned grid = (unsigned)((int64_t)a.batch * a.h_q * p.n_tiles);
  if (kmid <= 8)
    hipLaunchKernelGGL(mid_select<8>, dim3(grid), dim3(256), 0, s, p);
  else if (kmid <= 16)
    hipLaunchKernelGGL(mid_select<16>, dim3(grid), dim3(256), 0, s, p);
  else if (kmid <= 32)
    hipLaunchKernelGGL(mid_select<32>, dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(mid_select<KMID_LIMIT>, dim3(grid), dim3(256), 0, s, p);
  const int64_t threads = (int64_t)a.batch * a.h_q * m.n_q * 16;
  hipLaunchKernelGGL(mid_merge, dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace sa
