/*
 * bwa.h -- C ABI of the MI355X (gfx950) blockwise / ring exact-attention library.
 *
 * What it computes.  Exact attention O = softmax(scale * Q K^T) V, one query
 * block against one key/value block at a time.  Each block pair yields a
 * partial output and its row log-sum-exp; partials of successive KV blocks
 * (the rounds of a ring) are combined by FlashAttention-style rescaling, so
 * the merged result equals unblocked attention up to rounding.
 *   - "LV-XAttn: Distributed Cross-Attention for Long Visual Inputs in
 *     Multimodal Large Language Models" (Pith review), "What carries the
 *     argument": KV blocks stay on their worker; the query block Q_i, the
 *     partial output O_i and the softmax statistics L_i rotate; partial
 *     outputs are rescaled as in FlashAttention.  Figure 3 caption
 *     (Algorithm 1): inputs Q_i, K_i, V_i, state O_i, L_i, n rounds.
 *   - "Ring Attention with Blockwise Transformers for Near-Infinite Context",
 *     abstract: query blocks stay, key/value blocks travel the ring,
 *     blockwise attention with no approximation.
 * On one GPU the n ring workers are n shards of the sequence on one device;
 * a round is a stream-ordered kernel launch and no data moves between GPUs.
 *
 * Conventions shared by every entry point.
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or keeps caller memory; scratch memory
 *     is passed in as `workspace` (size from the *_workspace query).
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL is the default stream).  Arguments are validated on the host
 *     before anything is enqueued: a non-OK status means nothing was enqueued
 *     (except BWA_ERR_HIP, which reports a failed launch).
 *   - Errors are return codes only: no exceptions, no abort.  The last
 *     failing call's detail is kept per host thread (bwa_last_error()).
 *   - Layout: a bwa_tensor is [B, H, S, D] with element strides sB, sH, sS
 *     and unit stride along D (so [B, S, H, D] storage works by strides).
 *     The base pointer must be 16-byte aligned and sB, sH, sS multiples of
 *     16 bytes; a row (sS) spans less than 16 MiB.  D must be 64 or 128.
 *   - Sizes: B*H and S below 2^31, B*H*S at most 2^33 rows per tensor, and
 *     B*H*n times the 16-row tiles of a shard at most 2^30 (the largest
 *     launch grid); larger calls (reachable only with broadcast zero
 *     strides) return BWA_ERR_UNSUPPORTED.
 *   - scale is the softmax scale (callers pass 1/sqrt(D)); it must be finite
 *     and positive.  LSE values are fp32, natural log, scale included.
 *     An empty set of visible keys gives (O = 0, LSE = -inf).
 *   - causal is self-attention masking by position and requires S_Q == S_KV:
 *       0: none;
 *       1: rows are in sequence order, key j visible to query i iff j <= i;
 *       2: rows are in the striped order over the n shards (bwa_ring_fwd
 *          and bwa_ring_bwd, n must divide S): shard w = rows
 *          [w*S/n, (w+1)*S/n) holds sequence positions w, w+n, w+2n, ... in
 *          order, and key j is
 *          visible to query i iff its position is not after i's.  Every block
 *          pair is then about half visible, which balances a causal ring
 *          (Striped Attention's token assignment, named in the LV-XAttn
 *          review's references).
 *   - Shards: a length-S sequence split n ways has shard k =
 *     [floor(k*S/n), floor((k+1)*S/n)).  Query blocks and KV shards use the
 *     same split.  Round r pairs for virtual worker w:
 *       BWA_SCHED_KV_STATIONARY (LV-XAttn): Q block (w - r) mod n, KV shard w;
 *       BWA_SCHED_Q_STATIONARY  (Ring):     Q block w, KV shard (w - r) mod n.
 *     Every round is a perfect matching and the n rounds cover all n^2
 *     pairs.  Query block j therefore merges KV shards in the order
 *     j, j+1, ... (KV-stationary) or j, j-1, ... (Q-stationary), mod n.
 *   - Thread safety: calls on different streams may run concurrently if
 *     their output buffers are disjoint.  The only mutable global state is
 *     the per-device address of the scratch array of
 *     bwa_ring_bwd_noalloc, looked up once under a lock.
 */
#ifndef BWA_H_
#define BWA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BWA_VERSION 1

typedef enum {
  BWA_OK = 0,
  BWA_ERR_INVALID_ARG = 1, /* null pointer, bad shape, mismatched operands */
  BWA_ERR_UNSUPPORTED = 2, /* valid but not implemented (dtype, D, alignment) */
  BWA_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or too small */
  BWA_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  BWA_ERR_INTERNAL = 5
} bwa_status;

typedef enum { BWA_F32 = 0, BWA_BF16 = 1 } bwa_dtype;

typedef enum {
  BWA_SCHED_KV_STATIONARY = 0, /* LV-XAttn: KV stays, Q/O/L rotate */
  BWA_SCHED_Q_STATIONARY = 1   /* Ring Attention: Q stays, K/V rotate */
} bwa_schedule;

/*
 * How the n rounds run on the one GPU.  All three compute the same n^2 block
 * pairs and merge each query block's partials in its schedule's order; they
 * differ only in fp32 rounding.
 *   ROUNDS: n launches, one per round, each the round's n pairs; the running
 *           (O, L) of every query block lives in fp32 between rounds.
 *   FUSED:  one launch; each workgroup walks its query block's KV shards in
 *           schedule order, carrying the softmax state in registers.
 *   SPLIT:  one launch computes every pair's partial into the workspace,
 *           then one merge launch combines them in schedule order.
 *   ROUNDS_TRANSFER: ROUNDS, plus the exchange made real: after every round
 *           but the last, each worker's outgoing blocks are copied on the
 *           device into the receive buffers the next round computes from
 *           (KV-stationary: Q_i in its dtype, O_i and L_i in fp32; Q-stationary:
 *           K_i and V_i), so the per-round message bytes are HBM traffic.
 *           Results are bitwise equal to ROUNDS.  (LV-XAttn review, "What
 *           carries the argument": the blocks each schedule sends per round.)
 */
typedef enum {
  BWA_MODE_ROUNDS = 0,
  BWA_MODE_FUSED = 1,
  BWA_MODE_SPLIT = 2,
  BWA_MODE_ROUNDS_TRANSFER = 3
} bwa_mode;

typedef struct bwa_tensor {
  void* ptr;       /* device pointer, 16-byte aligned */
  int32_t dtype;   /* bwa_dtype */
  int32_t reserved;
  int64_t B, H, S, D;
  int64_t sB, sH, sS; /* element strides; stride along D is 1 */
} bwa_tensor;

/*
 * One block pair: query rows [q0, q0+nq) attend to key/value rows
 * [k0, k0+nk) of every (batch, head).  (LV-XAttn review, "What carries the
 * argument": the block attention of the query block a worker holds against
 * its local KV block, rescaled as in FlashAttention.)
 *   o_acc   fp32 [B, H, S_Q, D] contiguous: running normalised output.
 *   lse_acc fp32 [B, H, S_Q]: running log-sum-exp.
 *   accumulate = 0: rows [q0, q0+nq) are overwritten with this pair's
 *                   partial (O_p, L_p);
 *   accumulate = 1: the partial is rescale-merged into the rows' running
 *                   (O, L) (the identity is O = 0, L = -inf).
 * Other rows are not touched.  causal masks by global position
 * (key k0+j visible to query q0+i iff k0+j <= q0+i).
 * q, k, v share one dtype (fp32 or bf16).
 */
bwa_status bwa_partial_fwd(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                           int64_t q0, int64_t nq, int64_t k0, int64_t nk, float scale,
                           int causal, float* o_acc, float* lse_acc, int accumulate,
                           void* stream);

/*
 * Rescale-merge of two partials over disjoint key sets, row by row
 * (LV-XAttn review, "What carries the argument" and "Assumptions": the
 * online-softmax rescaling of partial O and L is exact):
 *   M = max(L_a, L_b),  L = M + ln(e^(L_a - M) + e^(L_b - M)),
 *   O = e^(L_a - L) O_a + e^(L_b - L) O_b;   (0, -inf) is the identity.
 * o_* fp32 [rows, D] contiguous, lse_* fp32 [rows].  Outputs may alias
 * either input exactly (same pointer), not partially.
 */
bwa_status bwa_merge(int64_t rows, int64_t D, const float* o_a, const float* lse_a,
                     const float* o_b, const float* lse_b, float* o_out, float* lse_out,
                     void* stream);

/*
 * n-way merge of per-shard partials in each query block's ring order (the
 * running (O, L) of the LV-XAttn review's "What carries the argument",
 * combined shard by shard): for a row of query block j the partials of KV
 * shards j, j+1, ... (KV-stationary) or j, j-1, ... (Q-stationary), mod n,
 * are rescale-merged into the identity (0, -inf) in that order.
 *   o_parts   fp32 [n][B, H, S_Q, D] contiguous, partial k from KV shard k.
 *   lse_parts fp32 [n][B, H, S_Q] contiguous.
 *   o         [B, H, S_Q, D] output tensor (fp32 or bf16, any strides).
 *   lse       fp32 [B, H, S_Q] output.
 * Query blocks use the n-way split of S_Q (conventions above).  This is the
 * second launch of bwa_ring_fwd's SPLIT mode, whose workspace holds o_parts
 * then lse_parts (each region 256-byte aligned).
 */
bwa_status bwa_merge_partials(int n, bwa_schedule sched, const float* o_parts,
                              const float* lse_parts, const bwa_tensor* o, float* lse,
                              void* stream);

/* Bytes of workspace bwa_ring_fwd needs (0 if none); 0 also for invalid arguments. */
size_t bwa_ring_fwd_workspace(const bwa_tensor* q, const bwa_tensor* k, int n, bwa_mode mode);

/*
 * The whole ring forward on one GPU: n KV shards and n query blocks, n
 * rounds of the chosen schedule, every query block's partials merged in its
 * schedule's order (LV-XAttn review, Figure 3 / Algorithm 1 and "What
 * carries the argument"; Ring Attention abstract).
 *   q [B, H, S_Q, D], k and v [B, H, S_KV, D], one dtype.
 *   o   [B, H, S_Q, D] in q's dtype (any strides per the conventions).
 *   lse fp32 [B, H, S_Q] contiguous.
 *   1 <= n <= S_KV.  causal requires S_Q == S_KV.
 *   workspace: device memory of at least bwa_ring_fwd_workspace() bytes,
 *   256-byte aligned (may be NULL when that is 0).
 */
bwa_status bwa_ring_fwd(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v, int n,
                        bwa_schedule sched, bwa_mode mode, int causal, float scale,
                        const bwa_tensor* o, float* lse, void* workspace, size_t ws_bytes,
                        void* stream);

/* Bytes of workspace bwa_ring_bwd needs; 0 also for invalid arguments. */
size_t bwa_ring_bwd_workspace(const bwa_tensor* q, const bwa_tensor* k, int n, bwa_mode mode);

/*
 * Exact gradient of the ring forward (LV-XAttn review, referee report major
 * comment 1: the distributed backward must reproduce the gradient of the
 * exact attention formula).  With P = exp(scale Q K^T - LSE):
 *   dV = P^T dO,  dP = dO V^T,  Delta = rowsum(dO * O),
 *   dS = P * (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q.
 * Each block pair contributes additively, using the global LSE and Delta.
 * KV-stationary: dK, dV stay with their shard while (Q, dO, LSE, Delta, dQ)
 * rotate; Q-stationary: the reverse.  Modes as in bwa_ring_fwd (SPLIT is
 * treated as FUSED): ROUNDS runs the rounds as launches in the schedule's
 * order; FUSED accumulates dQ over the KV shards in the schedule's order and,
 * for rows in sequence order (causal 0 or 1), dK and dV over all query rows
 * in sequence order (the same sums; only fp32 rounding differs).
 *   o, dout [B, H, S_Q, D] and lse fp32 [B, H, S_Q] from the forward.
 *   dq [B, H, S_Q, D], dk and dv [B, H, S_KV, D] in q's dtype (overwritten).
 *   causal: 0, 1 or 2 as in the conventions above (the forward's value).
 * bf16 only, D = 64 or 128 (fp32 inputs give BWA_ERR_UNSUPPORTED).
 * workspace: at least bwa_ring_bwd_workspace() bytes, 256-byte aligned:
 * Delta fp32 [B, H, S_Q] (every mode) and, for ROUNDS, fp32 dQ, dK, dV
 * accumulators carried between the round launches.
 */
bwa_status bwa_ring_bwd(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                        const bwa_tensor* o, const float* lse, const bwa_tensor* dout, int n,
                        bwa_schedule sched, bwa_mode mode, int causal, float scale,
                        const bwa_tensor* dq, const bwa_tensor* dk, const bwa_tensor* dv,
                        void* workspace, size_t ws_bytes, void* stream);

/*
 * bwa_ring_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and arguments without a workspace.  Its scratch
 * (Delta, fp32 [B, H, S_Q]) lives in a library-owned device array of
 * BWA_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library runs on holds
 * until the process ends.  Nothing is allocated or freed by the call.
 *   - mode FUSED or SPLIT (the same for the backward); ROUNDS gives
 *     BWA_ERR_UNSUPPORTED (its fp32 accumulators do not fit the array).
 *   - B * H * S_Q * 4 bytes (rounded up to 256) above the array's size give
 *     BWA_ERR_WORKSPACE: at most 4,194,304 query rows over all heads.
 *   - Every call on one GPU uses that GPU's one array, and Delta is rewritten
 *     in full by each call before it is read: calls that overlap on one GPU
 *     (different streams without ordering) race.
 * Results are bitwise those of bwa_ring_bwd in FUSED mode.
 */
#define BWA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
bwa_status bwa_ring_bwd_noalloc(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                                const bwa_tensor* o, const float* lse, const bwa_tensor* dout,
                                int n, bwa_schedule sched, bwa_mode mode, int causal, float scale,
                                const bwa_tensor* dq, const bwa_tensor* dk, const bwa_tensor* dv,
                                void* stream);

/*
 * Recompute of keys and values from the one shared copy of the visual
 * features (LV-XAttn review, "What carries the argument": all
 * cross-attention layers read the same y, so only y is kept and K = y W_k,
 * V = y W_v are recomputed when needed):
 *   k[b, h, s, d] = sum_e y[b, s, e] * W_k[e, h*D + d], likewise v with W_v.
 *   y     bf16 [B, S_KV, E] contiguous.
 *   wk_t, wv_t bf16 [H*D, E] contiguous: W_k, W_v transposed (row n holds
 *         column n of W), the [out, in] layout of a linear layer's weight.
 *         A caller holding W row-major as [E, H*D] passes its transpose
 *         (one copy per weight update): both GEMM operands then have the
 *         contraction index E contiguous, which the 16-byte operand loads
 *         need.
 *   k, v  bf16 [B, H, S_KV, D] tensors (any strides per the conventions).
 * bf16 only; E must be a multiple of 64 and H*D a multiple of 128.
 */
bwa_status bwa_kv_recompute(const void* y, const void* wk_t, const void* wv_t, int64_t B,
                            int64_t S_KV, int64_t E, int64_t H, int64_t D, int32_t dtype,
                            const bwa_tensor* k, const bwa_tensor* v, void* stream);

/*
 * Gradients through the K/V recompute (same passage as bwa_kv_recompute: the
 * backward of K = y W_k, V = y W_v from the one shared y):
 *   dwk_t[n, e] = sum_{b,s} dk[b, h, s, d] * y[b, s, e]    (n = h*D + d),
 *   dwv_t likewise with dv,
 *   dy[b, s, e] = sum_n dk[b, h, s, d] * wk_t[n, e] + dv[b, h, s, d] * wv_t[n, e].
 *   y, wk_t, wv_t as in bwa_kv_recompute (bf16, contiguous).
 *   dk, dv  bf16 [B, H, S_KV, D] tensors sharing one set of strides.
 *   dwk_t, dwv_t  fp32 [H*D, E] contiguous (gradients of wk_t, wv_t);
 *   dy      fp32 [B, S_KV, E] contiguous.  Any output may be NULL (skipped),
 *           not all three.
 *   accumulate = 0 overwrites the outputs, 1 adds to them (for cross-attention
 *   layers that share y).
 * E and H*D must be multiples of 256, S_KV a multiple of 64.  fp32
 * accumulation of bf16 products; no other rounding.
 */
bwa_status bwa_kv_recompute_bwd(const void* y, const void* wk_t, const void* wv_t,
                                const bwa_tensor* dk, const bwa_tensor* dv, int64_t B,
                                int64_t S_KV, int64_t E, int64_t H, int64_t D, float* dwk_t,
                                float* dwv_t, float* dy, int32_t accumulate, void* stream);

/*
 * Per-round cost model of the two ring schedules and the choice between them
 * (LV-XAttn review, "What carries the argument": the per-round runtime
 * identity).  With d = H*D the model width, a round of either schedule
 * computes one block pair, f = 4 * (S_Q/n) * (S_KV/n) * d FLOP (two
 * contractions, a multiply-add counted as 2), and sends one message that the
 * model takes to overlap the compute, so a round lasts max(compute, comm):
 *   KV-stationary (LV-XAttn): 2*S_Q*d/n + S_Q/n elements (Q_i, O_i, L_i);
 *   Q-stationary (Ring):      2*S_KV*d/n elements (K_i, V_i).
 * Times: compute = f / flops_per_s, comm = elements * elem_bytes / bytes_per_s.
 * *choice receives the schedule with the shorter round (KV-stationary on a
 * tie); *model, if not NULL, receives the five times in seconds.
 * All sizes and rates must be positive (BWA_ERR_INVALID_ARG otherwise).
 * Host-only: enqueues nothing and needs no GPU.
 */
typedef struct {
  double t_compute;                /* f / flops_per_s */
  double t_comm_kv_stationary;     /* LV-XAttn message */
  double t_comm_q_stationary;      /* Ring message */
  double t_round_kv_stationary;    /* max(t_compute, t_comm_kv_stationary) */
  double t_round_q_stationary;     /* max(t_compute, t_comm_q_stationary) */
} bwa_schedule_model;

bwa_status bwa_choose_schedule(int64_t S_Q, int64_t S_KV, int64_t d_model, int32_t n,
                               double flops_per_s, double bytes_per_s, int32_t elem_bytes,
                               int32_t* choice, bwa_schedule_model* model);

/* Static string naming a status code. */
const char* bwa_status_string(bwa_status s);
/* Detail of the calling thread's last failing call ("" if none). */
const char* bwa_last_error(void);
/* BWA_VERSION of the built library. */
int bwa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BWA_H_ */
