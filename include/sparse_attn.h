/*
 * sparse_attn.h -- C ABI of libsparse_attn.so: causal attention restricted to a
 * structured sparse key set, for AMD Instinct MI355X (gfx950).
 *
 * For each query i the visible keys A_i are
 *   SepLLM      j <= i and (j < a  or  0 <= i-j < w  or  sep[j] = 1)
 *               (SepLLM page, part 5 item 2: initial a, separators before i,
 *               n neighbouring tokens; masked logits are -inf, part 6.1);
 *   LM-Infinite j <= i and (j < n_starting  or  i-j <= L_pretrain)
 *               (LM-Infinite page, section "method", Lambda-shaped mask), with
 *               the logit taken at the capped distance min(i-j, L_pretrain);
 *   segment     keys are [prefix P | segment]; query i sees j <= P + i, RoPE
 *               positions 0..P-1 for the prefix and P+i for query i
 *               (segmented-execution page, method / overall framework).
 * Logits are scale * <R(pos_q) q_i, R(pos_k) k_j> with rotate-half RoPE,
 * theta_c = base^(-2c/d); output O_i = softmax over A_i of the logits times V.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or keeps a pointer after the call returns.
 *  - Work is enqueued on the given stream (0 = the null stream) and is
 *    asynchronous; results are ready after the caller synchronises the stream.
 *  - Every argument is checked on the host before anything is launched.  On a
 *    bad argument the call returns SA_EINVAL / SA_EUNSUPPORTED / SA_ENOSPACE,
 *    launches nothing and sets a message readable with sa_last_error().
 *    A failed launch returns SA_EHIP.  Device faults surface at the caller's
 *    next synchronisation.
 *  - Calls are thread-safe; the only global state is the per-thread message.
 *  - Code objects are built for gfx950 only; on another device the calls that
 *    launch work return SA_EUNSUPPORTED.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { SA_OK = 0, SA_EINVAL = -1, SA_EUNSUPPORTED = -2, SA_ENOSPACE = -3, SA_EHIP = -4 };
enum { SA_MASK_SEPLLM = 0, SA_MASK_LAMBDA = 1, SA_MASK_SEGMENT = 2 };
enum { SA_F32 = 0, SA_BF16 = 1 };
enum { SA_ROPE_NONE = 0, SA_ROPE_HALF = 1, SA_ALIBI = 2 };

/* Plan geometry: 128-query tiles, 64-key blocks. */
enum { SA_TQ = 128, SA_BK = 64 };
/* Item flags (bits 24..31 of an item; bits 0..23 hold the block index). */
enum { SA_ITEM_FULL = 1, SA_ITEM_CAPPED = 2 };

/*
 * The pages' mask parameters for one sequence; shared by every head, layer
 * and batch row that uses the same plan.
 *   kind        SA_MASK_*.
 *   n_q, n_k    query and key counts.  SEPLLM / LAMBDA: n_q == n_k (= m).
 *               SEGMENT: n_k == prefix_len + n_q.  1 <= n_q, n_k < 2^24 * 64.
 *   a, w        SEPLLM: initial tokens a >= 0, neighbours w >= 1 (the query
 *               itself counts as a neighbour).
 *   sep         SEPLLM: device uint8 [n_k], nonzero = separator; NULL = none.
 *   n_starting  LAMBDA: starting span >= 0.
 *   L_pretrain  LAMBDA: window i-j <= L_pretrain and distance cap, >= 0.
 *   prefix_len  SEGMENT: P >= 0.
 *   sep_max     SEPLLM: 0, or the caller's upper bound on the separators the
 *               plan lists (the nonzero entries of sep at positions
 *               j >= g0 = 64*ceil(a/64); a bound on all nonzero entries of
 *               sep serves).  It sizes the plan's sep_idx section and the
 *               gathered separator rows of the workspaces (sep_rows =
 *               64*ceil(min(sep_max, n_k)/64)) instead of n_k.  A mask that
 *               breaks the bound is detected on the device: the plan keeps
 *               the first sep_max separators and records the true count,
 *               sa_plan_status reports SA_ENOSPACE, and the forward writes
 *               NaN to every output row and log-sum-exp of such a plan.
 *               0 = no bound.  Must be >= 0.
 * Fields that do not belong to `kind` are ignored.
 */
typedef struct {
  int32_t kind;
  int32_t n_q, n_k;
  int32_t a, w;
  const uint8_t *sep;
  int32_t n_starting, L_pretrain;
  int32_t prefix_len;
  int32_t sep_max;
} sa_mask_t;

/*
 * Plan buffer layout (a POD byte buffer built on the device by
 * sparse_attn_plan; it holds offsets, never pointers).  The section offsets
 * are a function of the mask scalars only and are reported by
 * sa_plan_layout(); the header at offset 0 repeats them and adds the
 * data-dependent counts.
 *   tile_ptr  int32 [n_tiles+1]   CSR offsets of each tile's items
 *   items     int32 [cap_items]   block | flags << 24, ascending per tile
 *   sep_count int32 [n_tiles]     separators gathered by tile t: those in
 *                                 [g0, 64*floor(max(0,q0-w+1)/64)), g0 = 64*ceil(a/64)
 *   sep_idx   int32 [cap_sep]     ascending positions j >= g0 with sep[j] != 0
 *                                 (cap_sep = n_k, or min(sep_max, n_k); the first
 *                                 cap_sep of them when n_sep exceeds it)
 *   sep_bits  uint64 [n_blocks]   bit r of word b = (sep[64b+r] != 0)
 *   blk_sep   int32 [n_blocks+1]  separators (j >= g0) before block b
 * LAMBDA and SEGMENT plans have sep_count, sep_bits and blk_sep all zero.
 */
typedef struct {
  uint32_t magic;        /* 0x31504153 'SAP1' */
  int32_t version;       /* 1 */
  int32_t kind, tq, bk, n_q, n_k, n_tiles, n_blocks;
  int32_t n_items;       /* written by the device */
  int32_t n_sep;         /* written by the device: separators at j >= g0 */
  int32_t g0, cap_items, cap_sep, max_items_per_tile, reserved;
  int64_t off_tile_ptr, off_items, off_sep_count, off_sep_idx, off_sep_bits, off_blk_sep;
  int64_t total_bytes;
} sa_plan_header_t;

/*
 * Forward arguments.  Tensors are [batch, heads, tokens, d] with the last
 * dimension contiguous; *_stride give the element strides of the batch, head
 * and token dimensions (the token stride at most 64 MiB in bytes, else
 * SA_EUNSUPPORTED: the kernels address the rows of a 64-row block with 32-bit
 * offsets).
 *   dtype       SA_F32 or SA_BF16 for q, k, v and o.
 *   d           head dimension: 64 or 128 (bf16 and f32).
 *   h_q, h_kv   h_q % h_kv == 0; query head h reads kv head h / (h_q/h_kv).
 *   rope        position encoding: SA_ROPE_NONE; SA_ROPE_HALF (rotate-half RoPE,
 *               theta_c = rope_base^(-2c/d)); or SA_ALIBI (LAMBDA masks only,
 *               else SA_EUNSUPPORTED): no rotation, and the logit of query
 *               head h gains the ALiBi-style bias -m_h * min(i-j, L_pretrain)
 *               with m_h = 2^(-E (h+1) / h_q), E = alibi_exp -- the
 *               LM-Infinite page, section "method": the bias matrix of
 *               ALiBi-style models clipped at the same cap.
 *   rope_base   SA_ROPE_HALF: the RoPE base (> 1); ignored otherwise.
 *   scale       logit scale, normally 1/sqrt(d).
 *   alibi_exp   SA_ALIBI: the slope exponent E > 0 (8 is the usual value);
 *               ignored otherwise.
 *   q           [batch, h_q, n_q, d] raw (unrotated) queries.
 *   k, v        [batch, h_kv, n_k, d] raw keys and values.
 *   o           [batch, h_q, n_q, d] output (written).
 *   lse         optional fp32 [batch, h_q, n_q] contiguous natural-log
 *               log-sum-exp of the scaled logits; NULL = not written.
 */
typedef struct {
  int32_t dtype;
  int32_t batch, h_q, h_kv, d;
  int32_t rope;
  float rope_base;
  float scale;
  float alibi_exp;
  const void *q; int64_t q_stride[3];
  const void *k; int64_t k_stride[3];
  const void *v; int64_t v_stride[3];
  void *o; int64_t o_stride[3];
  float *lse;
} sa_fwd_args_t;

/* Message of the last failed call on this thread ("" if none); never NULL. */
const char *sa_last_error(void);

/* Host only: section offsets and capacities of the plan for mask m. */
int sa_plan_layout(const sa_mask_t *m, sa_plan_header_t *layout);

/* Host only: bytes a plan buffer for mask m needs. */
int sa_plan_bytes(const sa_mask_t *m, size_t *bytes);

/*
 * Build the plan for mask m into the device buffer `plan` (plan_bytes >=
 * sa_plan_bytes).  Per 128-query tile it lists the 64-key blocks holding a
 * visible pair (sink blocks and window blocks for SepLLM; every such block
 * for LAMBDA and SEGMENT) with FULL / CAPPED flags, and for SepLLM the
 * compacted separator list each tile gathers instead of visiting the blocks
 * between its sinks and its window (SepLLM page, part 5 item 2 and part 6.2:
 * only the kept entries of Q K^T are computed).  The plan depends on the mask
 * only and serves every head and layer.  Errors: SA_EINVAL (bad mask, NULL
 * plan), SA_ENOSPACE (plan_bytes too small), SA_EHIP.
 */
int sparse_attn_plan(const sa_mask_t *m, void *plan, size_t plan_bytes, hipStream_t stream);

/*
 * Waits for `stream` (the plan must have been built on it) and copies the
 * plan's header to *out (may be NULL).  Returns SA_ENOSPACE when the mask
 * held more separators than the plan could list (n_sep > cap_sep: the
 * caller's sep_max was too small; rebuild with a larger bound), SA_EINVAL
 * for a NULL or short plan or a header that is not a plan's, SA_EHIP on a
 * HIP error, else SA_OK.
 */
int sa_plan_status(const void *plan, size_t plan_bytes, hipStream_t stream, sa_plan_header_t *out);

/* Host only: bytes of device workspace sparse_attn_fwd needs for (m, args). */
int sa_fwd_workspace_bytes(const sa_mask_t *m, const sa_fwd_args_t *args, size_t *bytes);

/*
 * Host only: where the RoPE stage (sparse_attn_rope / the first stage of
 * sparse_attn_fwd) puts its results in the workspace: byte offsets from the
 * workspace base, -1 for a section the call does not use.  Element type is
 * args->dtype; rows are d elements, contiguous.
 *   krot  [batch, h_kv, n_k, d]      R(pos_k(j)) k_j, rounded once (SA_ROPE_HALF)
 *   ksep  [batch, h_kv, sep_rows, d] row r = krot row SEP[r] (SepLLM with
 *   vsep  [batch, h_kv, sep_rows, d]   separators; vsep holds raw v), for the
 *                                      rows some tile gathers
 *   kcap  [batch, h_kv, cap_rows, d] row j < min(n_starting, n_k):
 *                                    R(-L_pretrain) k_j times scale*log2(e) for
 *                                    bf16 (times 1 for f32) (LAMBDA with RoPE)
 *   qrot  [batch, h_q, n_q, d]       rotated queries (f32 with RoPE only)
 * (LM-Infinite page, section "method": <R(L) q, k> = <q, R(-L) k>; SepLLM
 * page, part 6.2: only kept keys take part.)
 */
typedef struct {
  int64_t krot, ksep, vsep, kcap, qrot;
  int64_t sep_rows, cap_rows;
  int64_t total;
} sa_fwd_ws_layout_t;
int sa_fwd_workspace_layout(const sa_mask_t *m, const sa_fwd_args_t *args, sa_fwd_ws_layout_t *layout);

/*
 * Sparse attention forward for every batch row and head: a RoPE stage
 * (queries at pos_q, keys at pos_k, the LM-Infinite capped keys R(-L) k_j for
 * j < n_starting, and the SepLLM separator rows gathered), then the fused
 * forward over the plan's live blocks only (online softmax in fp32).  `plan`
 * must have been built for the same mask on this stream (or be complete).
 * ws: device workspace of ws_bytes >= sa_fwd_workspace_bytes; its contents
 * are scratch.  Errors: SA_EINVAL, SA_EUNSUPPORTED (dtype/d/device),
 * SA_ENOSPACE (plan or workspace too small), SA_EHIP.
 */
int sparse_attn_fwd(const sa_mask_t *m, const void *plan, size_t plan_bytes,
                    const sa_fwd_args_t *args, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * The two stages of sparse_attn_fwd as separate calls (same arguments, same
 * workspace), so a caller can time or schedule them apart.  sparse_attn_rope
 * writes the rotated keys, the gathered separator rows and the capped keys
 * into ws (and, for f32, the rotated queries; bf16 queries are rotated and
 * scaled inside sparse_attn_attend); sparse_attn_attend then reads them.  Calling
 * sparse_attn_rope then sparse_attn_attend on one stream equals
 * sparse_attn_fwd.  Errors as for sparse_attn_fwd.
 */
int sparse_attn_rope(const sa_mask_t *m, const void *plan, size_t plan_bytes,
                     const sa_fwd_args_t *args, void *ws, size_t ws_bytes, hipStream_t stream);
int sparse_attn_attend(const sa_mask_t *m, const void *plan, size_t plan_bytes,
                       const sa_fwd_args_t *args, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Backward of sparse_attn_fwd: the gradients of O with respect to the raw q,
 * k and v, given the upstream gradient dO (the textbook gradient of a masked
 * softmax, over the same key sets: SepLLM page, part 6.2, which trains with
 * the mask; LM-Infinite's capped distance and the segment prefix enter the
 * same way as in the forward, the rotations being undone at the end).
 *   dout  [batch, h_q, n_q, d] upstream gradient (dtype of the forward).
 *   dq    [batch, h_q, n_q, d], dk, dv [batch, h_kv, n_k, d]: written (not
 *         accumulated); GQA heads sum into their kv head's dk, dv.
 * Strides in elements, last dimension contiguous, 16-byte aligned.
 */
typedef struct {
  const void *dout; int64_t dout_stride[3];
  void *dq; int64_t dq_stride[3];
  void *dk; int64_t dk_stride[3];
  void *dv; int64_t dv_stride[3];
} sa_bwd_args_t;

/* Host only: bytes of device workspace sparse_attn_bwd needs for (m, args). */
int sa_bwd_workspace_bytes(const sa_mask_t *m, const sa_fwd_args_t *args, size_t *bytes);

/*
 * Computes dq, dk, dv for the forward described by (m, plan, args): args is
 * the forward's argument block with o and lse as that forward wrote them
 * (lse is required here).  It reruns the RoPE stage into ws, then a row-sum
 * kernel (D = rowsum(dO * O)), a query-major dQ kernel over the plan's units,
 * a key-major dK/dV kernel (one work group per 64-key group: dense block,
 * gathered separator chunk or capped block; every sum in a fixed order, no
 * atomics) and a per-row finishing kernel (inverse rotations, separator and
 * capped contributions).  bf16 with d = 128 runs on MFMA kernels; f32 with
 * d = 64 or 128 and bf16 with d = 64 on vector-ALU kernels (bf16 rows
 * widened, every product and sum in fp32; same sections, same order of the
 * key-major sums).
 * ws: ws_bytes >= sa_bwd_workspace_bytes; scratch.  Errors: SA_EINVAL,
 * SA_EUNSUPPORTED, SA_ENOSPACE, SA_EHIP.
 */
int sparse_attn_bwd(const sa_mask_t *m, const void *plan, size_t plan_bytes,
                    const sa_fwd_args_t *args, const sa_bwd_args_t *grads, void *ws,
                    size_t ws_bytes, hipStream_t stream);

/*
 * Streaming decode, one new token per sequence per step, keys stored rotated
 * at their original positions.
 * kind SA_MASK_SEPLLM: the generation-time cache of the SepLLM page (part
 *   6.2, generation): Initial (the first a tokens), Separator (at most s
 *   separators, the most recent), Local window (the last w tokens, the newest
 *   included) and Past (tokens that left the local window since the last
 *   compression).  When a + s + w + |Past| reaches c, Past's separators join
 *   the Separator part in order (the oldest beyond s dropped) and Past is
 *   emptied; then the new query attends to every held token.
 * kind SA_MASK_LAMBDA: LM-Infinite's Lambda set for the new query t (LM-Infinite
 *   page, section "method"): the first a = n_starting tokens and the window
 *   t - L_pretrain .. t (w = L_pretrain + 1 slots; s and c are ignored).  A
 *   starting token farther than L_pretrain takes the capped logit
 *   scale <R(L) q_t, k_j>.
 *   batch, h_q, h_kv, d   sizes (bf16, d = 128; h_q % h_kv == 0, at most 8
 *                         query heads per kv head).
 *   a, s, w, c            SEPLLM: a >= 0, s >= 1, w >= 1, c > a + s + w,
 *                         c <= 4096.  LAMBDA: a = n_starting >= 0.
 *   rope, rope_base       SA_ROPE_NONE or SA_ROPE_HALF.
 *   scale                 logit scale.
 *   kind                  SA_MASK_SEPLLM or SA_MASK_LAMBDA.
 *   L_pretrain            LAMBDA: the window and cap, a + L_pretrain + 1 <= 65536.
 */
typedef struct {
  int32_t batch, h_q, h_kv, d;
  int32_t a, s, w, c;
  int32_t rope;
  float rope_base;
  float scale;
  int32_t kind;
  int32_t L_pretrain;
} sa_stream_cfg_t;

/*
 * Host only: bytes of the cache state (caller-owned device memory, one buffer:
 * the K and V rows [batch, h_kv, c, d], per-slot token index and separator
 * flag, per-sequence counters) and of the per-step workspace.
 */
int sa_stream_state_bytes(const sa_stream_cfg_t *cfg, size_t *bytes);
int sa_decode_workspace_bytes(const sa_stream_cfg_t *cfg, size_t *bytes);

/* Empties every sequence's cache (a fill kernel on the stream). */
int sparse_attn_stream_reset(const sa_stream_cfg_t *cfg, void *state, size_t state_bytes,
                             hipStream_t stream);

/*
 * One decode step for every sequence: q [batch, h_q, d], k, v [batch, h_kv, d]
 * (raw projections of the new token, contiguous), is_sep uint8 [batch] (the
 * new token is a separator), o [batch, h_q, d] written, lse fp32 [batch, h_q]
 * or NULL.  The new token takes position t = the number of tokens the
 * sequence has seen.  Steps on one state must be stream-ordered.  Errors:
 * SA_EINVAL, SA_EUNSUPPORTED, SA_ENOSPACE, SA_EHIP.
 */
int sparse_attn_decode_step(const sa_stream_cfg_t *cfg, void *state, size_t state_bytes,
                            const void *q, const void *k, const void *v, const uint8_t *is_sep,
                            void *o, float *lse, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * The same decode step with no workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The per-step scratch (rotated queries,
 * capped logits, per-split partial sums: sa_decode_workspace_bytes) lives in a
 * static array of SA_DECODE_STATIC_SCRATCH_BYTES in each GPU's memory, held by
 * the library until the process ends; the call allocates nothing.  A
 * configuration needing more scratch than that returns SA_ENOSPACE.  Every
 * call on one GPU shares that GPU's array: calls that overlap in time on one
 * GPU (other streams, other threads) race and must be ordered by the caller.
 * Arguments, results and errors are those of sparse_attn_decode_step.
 */
enum { SA_DECODE_STATIC_SCRATCH_BYTES = 32 << 20 };
int sparse_attn_decode_step_static(const sa_stream_cfg_t *cfg, void *state, size_t state_bytes,
                                   const void *q, const void *k, const void *v, const uint8_t *is_sep,
                                   void *o, float *lse, hipStream_t stream);

/*
 * Host only: the state layout (byte offsets of the K rows, V rows, per-slot
 * token index int32 [batch, c], per-slot flag uint8 [batch, c] and the
 * per-sequence counters int32 [batch, 8]: t, n_init, n_sep, sep_head, n_past,
 * n_local, local_head, reserved).
 */
int sa_stream_layout(const sa_stream_cfg_t *cfg, int64_t offsets[5]);

/*
 * LM-Infinite's optional top-k middle tokens (LM-Infinite page, section
 * "method"), applied to the output of sparse_attn_fwd for a LAMBDA mask
 * (bf16, d = 128, SA_ROPE_HALF or SA_ROPE_NONE): for every head and query i,
 * the k_mid middle tokens n_starting <= j < i - L_pretrain with the largest
 * logits scale <R(L) q_i, k_j> (ties to the lower j) join the key set, with
 * that same logit.  args must be the forward's (raw q, k, v; its o and lse,
 * which are rewritten in place to the extended attention).  sel int32 and
 * score fp32 [batch, h_q, n_q, k_mid] receive the chosen j (ascending score
 * order, -1 when a query has fewer middle tokens) and their base-2 logits.
 * 1 <= k_mid <= SA_TOPK_MIDDLE_MAX.  Errors: SA_EINVAL, SA_EUNSUPPORTED, SA_EHIP.
 */
enum { SA_TOPK_MIDDLE_MAX = 64 };
int sparse_attn_topk_middle(const sa_mask_t *m, const sa_fwd_args_t *args, int32_t k_mid,
                            int32_t *sel, float *score, hipStream_t stream);

/* Host only: bytes of device workspace topk_retrieve needs. */
int sa_topk_workspace_bytes(int32_t n_heads, int32_t pool_len, size_t *bytes);

/*
 * Forward-only top-k retrieval of the prefix (segmented-execution page, key
 * design 3: the segment-end query picks R keys of a detached read-only pool
 * for the long-range heads).  For each head h < n_heads:
 *   s_j = ((0 + q_0 k_j0) + q_1 k_j1) + ... + q_{d-1} k_{j,d-1}  in fp64 (every
 *   product of bf16/fp32 inputs is exact), j < pool_len;
 *   idx[h, 0..k-1] = the k largest s_j, ties to the smaller j, in ascending j.
 * Arguments:
 *   dtype        SA_F32 or SA_BF16 for q_score, pool_k, pool_v, pref_k, pref_v.
 *   q_score      row h at q_score + h*q_head_stride elements, d contiguous (raw).
 *   pool_k       row j of head h at pool_k + h*pool_head_stride + j*pool_row_stride;
 *                16-byte aligned, strides (in elements) multiples of 16 bytes.
 *   pool_v       same strides; NULL = no gather.
 *   idx          out int32 [n_heads, k] contiguous.
 *   score        out fp64 [n_heads, k] contiguous (s at idx), or NULL.
 *   pref_k/v     if pool_v != NULL: pool rows idx[h, r] are copied to row r of
 *                head h at pref_* + h*pref_head_stride + r*pref_row_stride.
 *   ws           device workspace of ws_bytes >= sa_topk_workspace_bytes.
 * Limits: 1 <= k <= pool_len, d in {64, 128}.  Errors as above.
 */
int topk_retrieve(int32_t dtype, int32_t n_heads, int32_t pool_len, int32_t d, int32_t k,
                  const void *q_score, int64_t q_head_stride,
                  const void *pool_k, const void *pool_v,
                  int64_t pool_head_stride, int64_t pool_row_stride,
                  int32_t *idx, double *score,
                  void *pref_k, void *pref_v, int64_t pref_head_stride, int64_t pref_row_stride,
                  void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Segment carry (segmented-execution page, overall framework and key designs
 * 2-3: (C_i, o_i) = F(x_i, C_{i-1}, R_{i-1})): the state one segment hands to
 * the next, taken after the segment's forward.
 *   k, v      [n_heads, prefix_len + seg_len, d] raw keys and values the
 *             segment attended to ([prefix | segment] per head), strides in
 *             elements; heads 0..n_local-1 are local, the rest long-range.
 *   tail_k/_v [n_local, >= keep, d] receive the local heads' latest
 *             keep = min(tail_len, prefix_len + seg_len) rows, in order (the
 *             carried tail C_i; the next segment reads it as its prefix).
 *   pool_k/_v [n_heads - n_local, pool_cap, d] receive the long-range heads'
 *             segment rows (k, v rows prefix_len .. prefix_len+seg_len-1) at
 *             pool rows pool_len .. pool_len+seg_len-1 (the detached pool the
 *             next prefix is retrieved from with topk_retrieve).
 * dtype SA_BF16 or SA_F32; d * element size a multiple of 16 bytes; every
 * pointer 16-byte aligned and every stride a multiple of 16 bytes; row
 * strides of the destinations >= d.  Tail pointers may be NULL when
 * n_local == 0, pool pointers when n_local == n_heads.  No destination row
 * may overlap a source row or another destination row (checked on the host
 * per head over the span from its first to its last row; use separate or
 * alternating buffers).  Errors: SA_EINVAL, SA_ENOSPACE (pool_len + seg_len >
 * pool_cap), SA_EUNSUPPORTED (device), SA_EHIP.
 */
int sparse_attn_segment_carry(int32_t dtype, int32_t n_heads, int32_t n_local, int32_t d,
                              int32_t prefix_len, int32_t seg_len, int32_t tail_len,
                              const void *k, const void *v, int64_t kv_head_stride,
                              int64_t kv_row_stride, void *tail_k, void *tail_v,
                              int64_t tail_head_stride, int64_t tail_row_stride, void *pool_k,
                              void *pool_v, int64_t pool_head_stride, int64_t pool_row_stride,
                              int64_t pool_len, int64_t pool_cap, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_ATTN_H */
