/*
 * moe.h -- C ABI of libmoe.so, one GPU's share of a fused Mixture-of-Experts
 * layer on AMD Instinct MI355X (gfx950).
 *
 * The method is the one described on the news page "Cursor's MoK achieves
 * 2.37x performance boost on NVIDIA GB300 NVL72" (KuCoin news flash; cited
 * below as "MoK flash" with its article section):
 *   section 01 (the communication tax of MoE): route tokens, count how many
 *     tokens each expert has, decide where each lands with one expert's rows
 *     kept together for the grouped GEMM, wait until data is complete, send
 *     results back to each token's original position (dispatch / combine);
 *     training adds the two exchanges in the reverse direction.
 *   section 02 (how to compute while sending tokens): pull dispatch (the
 *     receiver reads each token given only where it lives), push combine,
 *     pull reverse-combine and push reverse-dispatch in the backward; one
 *     megakernel whose communication side tells the compute side through
 *     GPU-local counters when a batch of tokens is complete; the batch size
 *     handed to the experts as a tunable; GPU-resident control with no CPU
 *     step per round; MXFP8 quantisation folded into the dispatch, grouped
 *     GEMM and SwiGLU datapath.
 *   section 03: the measured unit is the whole layer -- schedule, dispatch,
 *     expert FFN, combine and the final weighted merge.
 * On one GPU the source of every token is local, so dispatch is an on-device
 * row gather and combine a weighted row merge.
 *
 * Conventions for every entry point
 *   - All tensor arguments are DEVICE pointers to caller-owned, contiguous,
 *     row-major buffers; struct arguments (moe_desc, moe_weights, moe_saved)
 *     are HOST pointers read during the call only.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without synchronising.  No call reads device data
 *     back to the host, allocates device memory, or keeps state between calls.
 *   - Host-side validation failures return a negative moe_status and enqueue
 *     nothing.  A failed launch returns MOE_ERR_HIP.  Failures found on the
 *     device (an expert index out of range, a wait that exceeded its bound)
 *     are written to the optional device status word (moe_saved.status, an
 *     int32 the caller zeroes); outputs are then undefined.
 *   - Calls sharing one workspace must not overlap in time.
 *
 * Shapes: T tokens, d hidden size, E experts on this GPU, k experts per token,
 * I expert intermediate size, R = T*k routed rows.  An assignment is numbered
 * a = t*k + j (token t, slot j).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef MOE_API
#define MOE_API __attribute__((visibility("default")))
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,   /* null pointer, bad shape, k > E, ...           */
  MOE_ERR_UNSUPPORTED = -2,   /* valid but not implemented (e.g. d % 64 != 0) */
  MOE_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required    */
  MOE_ERR_HIP = -4,           /* a HIP launch failed                           */
  MOE_ERR_TIMEOUT = -5,       /* device: a bounded wait expired                */
  MOE_ERR_INVALID_ROUTE = -6  /* device: an expert index outside [0, E)        */
} moe_status;

typedef enum moe_dtype {
  MOE_F32 = 0,    /* IEEE binary32                                           */
  MOE_BF16 = 1,   /* bfloat16                                                */
  MOE_MXFP8 = 2   /* OCP MX: E4M3 codes (uint8) + one E8M0 scale (uint8) per
                     32 consecutive elements along the contraction axis      */
} moe_dtype;

typedef enum moe_score {
  MOE_SCORE_SOFTMAX = 0,
  MOE_SCORE_SIGMOID = 1
} moe_score;

/* Layer description.  Read on the host during each call. */
typedef struct moe_desc {
  int32_t T, d, E, k, I;
  int32_t act_dtype;     /* MOE_F32 or MOE_BF16: X, Wr, Y, dY, dX          */
  int32_t expert_dtype;  /* MOE_F32 (needs act F32), MOE_BF16 or MOE_MXFP8 */
  int32_t score;         /* moe_score                                       */
  int32_t renorm;        /* 1: gates renormalised over the chosen k          */
  int32_t fused;         /* 1: persistent launches driven by device-side
                            ready counters; 0: one launch per step          */
  int32_t stage_rows;    /* rows per ready counter (the minibatch handed to
                            the expert GEMM): 0 = auto (bf16 experts: 256
                            when T k >= 256 E, else 128; MXFP8: 128), else
                            64, 128 or 256 (MXFP8 experts: 0 or 128); any
                            value gives the same results                   */
  int32_t n_workgroups;  /* persistent grid size; 0 = auto: as many as
                          * fit on the CUs at once, but no more than the
                          * most tasks any phase of the launch can have
                          * (and at least 8); any size gives the same
                          * results                                        */
  uint32_t flags;        /* MOE_FLAG_* below                                */
  /* DeepSeek-V3-style routing options (0 = off):
   * n_group, topk_group: group-limited selection.  The E experts form
   *   n_group groups of E / n_group consecutive ids (E % n_group == 0,
   *   n_group <= 64); a group's score is the sum of its two largest keys;
   *   the topk_group best groups are kept (ties to the lower group) and the
   *   k experts are chosen among them (k <= topk_group * E / n_group).
   * routed_scale: factor on every gate (0 means 1).
   * With n_group > 1 or MOE_FLAG_BIAS_SELECT_ONLY the experts are ranked
   * by the key sigmoid(z) (+ bias with MOE_FLAG_BIAS_SELECT_ONLY), z the
   * gate logits; both need score MOE_SCORE_SIGMOID.  Without them the
   * (biased) logits themselves are ranked. */
  int32_t n_group;
  int32_t topk_group;
  float routed_scale;
  /* macro_tokens > 0 (and < T): moe_forward walks the tokens in macrobatches
   * of this many tokens (the last one ragged) through a ring of two
   * workspace slots, each sized for one macrobatch (moe_workspace_size
   * returns both): the staging rows are a fixed pool reused batch after
   * batch, so memory stays bounded for any T (MoK flash §02, the ring token
   * buffer).  With fused = 1 the merge of macrobatch i runs inside the
   * launch of macrobatch i+1, beside its routing and dispatch.  Outputs are
   * identical to one call over all T.
   * The saved layout (counts, offsets, perm, inv) and activations (a, b, h)
   * describe one layout over all T and must be NULL; logits, topk_idx, gate
   * and status are written.  The other calls return MOE_ERR_UNSUPPORTED
   * for such a descriptor. */
  int32_t macro_tokens;
  /* n_producer_cus > 0: CU partition of the fused forward (MoK flash §02:
   * compute units split between moving tokens and the expert FFN).  The
   * first n_producer_cus x (workgroups per CU) workgroups of the persistent
   * grid run only the routing, layout, gather and combine tasks, the others
   * only the expert GEMM tiles.  0 = no partition: every workgroup claims
   * every phase.  With a partition both sides must be resident at once, so
   * n_workgroups may not exceed the resident limit (else
   * MOE_ERR_INVALID_ARG), and at least one GEMM workgroup must remain. */
  int32_t n_producer_cus;
} moe_desc;

/* Flags. */
#define MOE_FLAG_DIRECT_PULL 0x1u  /* fused bf16 forward: the up-projection
                                      reads token rows from X through the
                                      layout instead of a staged copy       */
#define MOE_FLAG_PERSISTENT_SPLIT 0x2u /* fused forward: one persistent
                                      launch per phase group (routing and
                                      gather | up projection | down
                                      projection | combine)              */
#define MOE_FLAG_PERSISTENT_WGRAD_APART 0x4u /* fused backward: two
                                      persistent launches, the weight
                                      gradients after the rest           */
#define MOE_FLAG_PERSISTENT_SINGLE 0x8u /* fused forward and backward: every
                                      phase in one persistent launch     */
#define MOE_FLAG_PERSISTENT_GEMM_APART 0x800u /* fused forward: the down
                                      projection in a persistent launch of
                                      its own (routing .. up projection |
                                      down projection | combine)         */
#define MOE_FLAG_MXFP8_WGRAD 0x1000u /* backward with MXFP8 experts: the
                                      weight gradients in MXFP8 too (their
                                      operands quantised along the expert's
                                      rows); without it they take bf16
                                      operands                             */
#define MOE_FLAG_BIAS_SELECT_ONLY 0x10u /* the router bias steers the
                                      selection only: experts ranked by
                                      sigmoid(logit) + bias, gates from the
                                      unbiased logits, no bias gradient    */
#define MOE_FLAG_SPIN_LIMIT_TINY 0x100u /* test only: bounded waits give up
                                      after a few polls (exercises the
                                      MOE_ERR_TIMEOUT path)                 */
#define MOE_FLAG_TEST_DROP_READY 0x200u /* test only, fused forward: the
                                      gather of row tile 0 does not raise
                                      its ready counter, so the waits on it
                                      expire: the call records
                                      MOE_ERR_TIMEOUT, every workgroup
                                      drains its queues and exits, and y is
                                      undefined                            */
#define MOE_FLAG_TEST_SHUFFLE_CLAIMS 0x400u /* test only, fused calls:
                                      workgroups start claiming on a
                                      sub-queue hashed from their id instead
                                      of their XCD's (another claim order;
                                      results are unchanged)               */

/* Expert weights, in output-major order (row n of a matrix is output
 * feature n, contiguous along the contraction axis):
 *   w1, w3: [E, I, d]   gate and up projections
 *   w2    : [E, d, I]   down projection
 * Element type desc->expert_dtype.  For MOE_MXFP8 the arrays hold E4M3 codes
 * and the *_scale arrays hold E8M0 codes: w1_scale/w3_scale [E, I, d/32],
 * w2_scale [E, d, I/32]; NULL otherwise. */
typedef struct moe_weights {
  const void* w1;
  const void* w3;
  const void* w2;
  const uint8_t* w1_scale;
  const uint8_t* w3_scale;
  const uint8_t* w2_scale;
} moe_weights;

/* Optional device buffers.  moe_forward writes each non-NULL one;
 * moe_backward reads gate, offsets, perm, inv, a, b and h
 * (all required there).
 *   logits   float [T, E]   router logits (bias not included)
 *   topk_idx int32 [T, k]   chosen experts, largest logit first
 *   gate     float [T, k]   gates of the chosen experts
 *   counts   int32 [E]      rows per expert
 *   offsets  int32 [E+1]    exclusive prefix sum of counts
 *   perm     int32 [R]      perm[r] = assignment on row r (rows grouped by
 *                           expert, increasing assignment inside a group)
 *   inv      int32 [R]      inv[a]  = row of assignment a
 *   a, b     act   [R, I]   pre-activations x W1^T and x W3^T (bf16 only)
 *   h        act   [R, I]   silu(a) * b
 *   status   int32 [1]      device status word (see conventions)       */
typedef struct moe_saved {
  float* logits;
  int32_t* topk_idx;
  float* gate;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  void* a;
  void* b;
  void* h;
  int32_t* status;
} moe_saved;

/* Bytes of workspace the calls below need for `desc` (covers moe_forward,
 * moe_backward, moe_router_backward, moe_layout and moe_gather).  Returns MOE_ERR_INVALID_ARG for
 * an invalid descriptor.  Host only. */
MOE_API int moe_workspace_size(const moe_desc* desc, size_t* bytes);

/* Router top-k and gates (MoK flash §01: the router re-decides every step
 * which experts each token goes to; the score function and normalisation
 * follow desc->score / desc->renorm).
 *   logits   float [T, E]  input
 *   bias     float [E] or NULL, added to the logits (in fp32) before both
 *            selection and gates
 *   topk_idx int32 [T, k]  output: the k largest biased logits, largest
 *            first, exact ties to the lower expert index
 *   gate     float [T, k]  output
 * No workspace.  Needs 1 <= k <= min(E, 16), E <= 1024. */
MOE_API int moe_route(const moe_desc* desc, const float* logits, const float* bias,
              int32_t* topk_idx, float* gate, void* stream);

/* Per-expert counting and layout (MoK flash §01: count each expert's tokens
 * first, then place them so one expert's rows are contiguous).
 *   topk_idx int32 [T, k]  input, distinct experts per token
 *   counts   int32 [E], offsets int32 [E+1], perm int32 [R], inv int32 [R]:
 *            outputs as in moe_saved (a stable counting sort by expert)
 * An index outside [0, E) sets MOE_ERR_INVALID_ROUTE in `status` (may be
 * NULL) and leaves the outputs undefined. */
MOE_API int moe_layout(const moe_desc* desc, const int32_t* topk_idx, int32_t* counts,
               int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* status,
               void* workspace, size_t workspace_bytes, void* stream);

/* Dispatch as a row gather (MoK flash §02: tokens are laid out in expert
 * order so each expert's rows are contiguous for its GEMM).
 *   x    act [T, d] input
 *   perm int32 [R] from moe_layout, or NULL
 *   inv  int32 [R] from moe_layout, or NULL (at least one of the two)
 *   xp   act [R, d] output, xp[r] = x[perm[r] / k], i.e. xp[inv[t k + j]] = x[t]
 * With inv the gather runs token-major: each token row is read once and
 * written to its k rows.  With only perm it is the pull of MoK flash §02:
 * each destination row reads its token given only the source position.
 * Both write the same bytes.  Row indices outside [0, R) in inv are
 * skipped; perm entries must lie in [0, R).
 * For desc->expert_dtype == MOE_MXFP8 the gather also quantises (MoK flash
 * §02, quantisation folded into the dispatch): xp receives E4M3 codes
 * uint8 [R, d] and xp_scale E8M0 codes uint8 [R, d/32]; else xp_scale is
 * ignored. */
MOE_API int moe_gather(const moe_desc* desc, const void* x, const int32_t* perm, const int32_t* inv,
               void* xp, uint8_t* xp_scale, void* stream);

/* MXFP8 quantisation of a [rows, K] bf16 matrix along K in blocks of 32
 * (the standalone quantise step that the fused path folds away; also used
 * to prepare MXFP8 weights).  codes uint8 [rows, K], scales uint8
 * [rows, K/32].  K % 32 == 0. */
MOE_API int moe_quantize_mxfp8(const void* src, int64_t rows, int64_t K,
                       uint8_t* codes, uint8_t* scales, void* stream);

/* MXFP8 quantisation of the transpose of each bf16 matrix of a batch (the
 * backward's weights, MoK flash §03: the data gradients contract W1, W3
 * over I and W2 over d, the axes their forward does not block along).
 *   src    bf16  [batch, rows, cols]
 *   codes  uint8 [batch, cols, rows]      E4M3 codes of src^T
 *   scales uint8 [batch, cols, rows/32]   E8M0 codes, blocks of 32 along rows
 * rows % 32 == 0 (else MOE_ERR_INVALID_ARG); batch <= 65535, rows <=
 * 128 * 65535 and cols <= 2^30 (else MOE_ERR_UNSUPPORTED).  The same encoding as
 * moe_quantize_mxfp8. */
MOE_API int moe_quantize_mxfp8_t(const void* src, int64_t batch, int64_t rows, int64_t cols,
                                 uint8_t* codes, uint8_t* scales, void* stream);

/* The whole forward layer (MoK flash §03: schedule, dispatch, expert FFN,
 * combine and the final weighted merge).
 *   x     act [T, d];  wr act [E, d] (row e scores expert e);
 *   bias  float [E] or NULL (added to the logits);
 *   w     expert weights (see moe_weights);
 *   y     act [T, d] output: y[t] = sum_j gate[t,j] * FFN_{idx[t,j]}(x[t]),
 *         FFN_e(v) = (silu(v W1_e^T) * (v W3_e^T)) W2_e^T;
 *   saved optional outputs (may be NULL).
 * With desc->fused = 1 the layer runs as tasks claimed from device-side
 * queues phase by phase (after a small clearing launch): one persistent
 * launch runs routing, counting, layout, gather and both projections, an
 * up-projection tile starting as soon as the ready counter of its rows
 * shows them staged and a down-projection tile as soon as every
 * up-projection tile of its rows has stored H (MoK flash §02: GPU-local
 * counters); the combine follows as a plain launch.  MXFP8 experts run
 * routing through the gather, the up projection and the down projection as
 * three persistent launches by default.
 * MOE_FLAG_PERSISTENT_SINGLE puts the combine in the persistent launch too,
 * MOE_FLAG_PERSISTENT_GEMM_APART gives the down projection its own launch,
 * MOE_FLAG_PERSISTENT_SPLIT gives each phase group its own. */
MOE_API int moe_forward(const moe_desc* desc, const void* x, const void* wr,
                const float* bias, const moe_weights* w, void* y,
                const moe_saved* saved, void* workspace,
                size_t workspace_bytes, void* stream);

/* Bytes of the static device scratch array moe_forward_noalloc works in. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same layer and the same results bit for bit, with the
 * workspace in a static device array of MOE_NOALLOC_SCRATCH_BYTES (256 MiB)
 * inside the library instead of a caller buffer.  Each GPU the library runs
 * on holds its own array until the process ends; the call allocates nothing
 * (no hipMalloc, no allocating library routine).
 *   Arguments as in moe_forward, without workspace and workspace_bytes.
 *   When the forward's workspace for all T tokens fits the array, one call
 *   runs and every saved output may be asked for.  Otherwise the tokens
 *   run in consecutive macrobatches of the most tokens whose two ring slots
 *   fit (at most desc->macro_tokens when that is set), as moe_forward does for
 *   desc->macro_tokens: y and the per-token saved outputs (logits, topk_idx,
 *   gate, status) are written, and asking for the layout (counts, offsets,
 *   perm, inv) or the activations (a, b, h), which describe one batch over
 *   all T, returns MOE_ERR_WORKSPACE.  MOE_ERR_WORKSPACE is also returned
 *   when not one token's workspace fits the array (d, E or I too large).
 * Every call on a GPU uses that GPU's one array, which keeps the previous
 * call's contents (the call clears what must start at zero): calls that
 * overlap in time on one GPU, on any streams, race and give undefined
 * results.  Thread-safe to call from several host threads as long as their
 * calls do not overlap on the device. */
MOE_API int moe_forward_noalloc(const moe_desc* desc, const void* x, const void* wr,
                                const float* bias, const moe_weights* w, void* y,
                                const moe_saved* saved, void* stream);

/* The weighted merge on its own (MoK flash §01: each expert's result
 * returns to its token's position, weighted by the token's gates) -- the
 * forward's last step, for callers that run the expert GEMMs themselves.
 *   yp   act [R, d] input, the expert outputs in expert order (the layout
 *        of moe_layout)
 *   gate float [T, k], inv int32 [R]: the routing's gates and moe_layout's
 *        inverse permutation
 *   y    act [T, d] output, y[t] = sum_j gate[t, j] yp[inv[t k + j]],
 *        accumulated in fp32 in slot order j = 0 .. k-1: the forward's own
 *        combine, bit for bit
 * Entries of inv outside [0, R) read row 0.  No workspace; T = 0 is a
 * no-op.  Activation type desc->act_dtype (bf16 or f32). */
MOE_API int moe_combine(const moe_desc* desc, const void* yp, const float* gate, const int32_t* inv,
                        void* y, void* stream);

/* Backward of the expert path with the routing frozen (MoK flash §01/§02:
 * pull reverse-combine, expert dgrad and wgrad, push reverse-dispatch).
 * bf16 activations; bf16 or MXFP8 experts (below).
 *   dy    act [T, d] upstream gradient;  x act [T, d] the forward input;
 *   saved the forward's gate, offsets, perm, inv, a, b, h;
 *   dx    act [T, d] output, gradient through the experts only;
 *   dw1, dw3 act [E, I, d], dw2 act [E, d, I] outputs (overwritten; zero
 *         for experts without rows);
 *   dgate float [T, k] output, dL/dgate.
 * With desc->fused = 1 the phases (setup, rowprep and pulls, dH, dW2, dXp,
 * dW1/dW3, dX) run as: setup and pulls in one plain launch, dH, dXp, dW2
 * and dW1/dW3 in a persistent launch each, dX a plain launch
 * (MOE_FLAG_PERSISTENT_SINGLE: one persistent launch for every phase;
 * MOE_FLAG_PERSISTENT_WGRAD_APART: the data gradients in one, the weight
 * gradients in another);
 * with fused = 0 each phase is an ordinary grid.  Needs bf16 activations
 * with d % 128 == 0 and I % 128 == 0 (else MOE_ERR_UNSUPPORTED).
 * With desc->expert_dtype == MOE_MXFP8 the data gradients dHu = G W2 and
 * dXp = dA W1 + dB W3 run in MXFP8 (MoK flash §03), each operand blocked
 * along that product's contraction axis, and w holds the transposed weights
 * from moe_quantize_mxfp8_t: w1, w3 the codes of W1^T, W3^T uint8 [E, d, I]
 * with w1_scale, w3_scale [E, d, I/32]; w2 the codes of W2^T [E, I, d] with
 * w2_scale [E, I, d/32] (all required).  dY and [dA | dB] are quantised
 * along their rows inside the call.  The weight gradients take bf16
 * operands as in the bf16 backward, or with MOE_FLAG_MXFP8_WGRAD run in
 * MXFP8 too: dW2 = (g G)^T H, dW1 = dA^T x, dW3 = dB^T x with g G, H, dA,
 * dB and the x rows quantised along the expert's rows (blocks of 32 from
 * its first row) inside the call, into a larger workspace
 * (moe_workspace_size with the same flags).  dX's gather-sum and dgate
 * take bf16 operands.  With desc->fused = 1 this variant runs one
 * persistent launch per phase (the MOE_FLAG_PERSISTENT_SINGLE and
 * _WGRAD_APART flags do not apply to it), with the quantisations as plain
 * launches between them. */
MOE_API int moe_backward(const moe_desc* desc, const void* dy, const void* x,
                 const moe_weights* w, const moe_saved* saved, void* dx,
                 void* dw1, void* dw3, void* dw2, float* dgate,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Router backward through the gates (the router step of MoK flash §01 run
 * backwards; the selection is piecewise constant and passes no gradient).
 * With the chosen experts frozen, dgate flows to the biased logits
 * z = x Wr^T + bias of the chosen experts:
 *   softmax, renorm: dz_j = g_j (dg_j - sum_i g_i dg_i)
 *   sigmoid, renorm: dz_j = (dg_j - sum_i g_i dg_i) / S * s_j (1 - s_j),
 *                    s = sigmoid(z), S = sum of the chosen s
 *   sigmoid, plain : dz_j = dg_j s_j (1 - s_j)
 * (softmax without renorm makes every logit's gradient nonzero:
 * MOE_ERR_UNSUPPORTED), zero for the other logits, and then
 *   dwr = dz^T x, dbias = sum over tokens of dz, dx += dz Wr.
 *   x       act [T, d]   the forward's input
 *   wr      act [E, d]   router weight (as in moe_forward)
 *   bias    float [E] or NULL, the router bias of the forward
 *   saved   the forward's logits, topk_idx, gate, offsets and perm (all
 *           required); other fields ignored
 *   dgate   float [T, k] gradient of the gates (moe_backward's output)
 *   dlogits float [T, E] output or NULL: dL/dz
 *   dwr     act [E, d]   output (fp32 accumulation, overwritten)
 *   dbias   float [E] output or NULL
 *   dx      act [T, d]   in/out: dz Wr is ADDED to it (pass the expert
 *           path's dx from moe_backward to get the layer's full dx)
 * Gates scaled by desc->routed_scale c: the unscaled gate g / c receives
 * c dgate.  With MOE_FLAG_BIAS_SELECT_ONLY the gate logits exclude the bias
 * and dbias is written as zeros (the bias steers the selection only).
 * Every sum runs in a fixed order: results are deterministic.  Uses the
 * workspace of moe_workspace_size. */
MOE_API int moe_router_backward(const moe_desc* desc, const void* x, const void* wr, const float* bias,
                        const moe_saved* saved, const float* dgate, float* dlogits, void* dwr,
                        float* dbias, void* dx, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Static description of a status code. */
MOE_API const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
