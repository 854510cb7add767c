/*
 * smoe.h -- C ABI of libsmoe.so: the routed-expert MoE FFN path of a
 * speculative MoE decoder (INT4 self-draft, FP16 verification), hand-written
 * HIP for gfx950 (MI355X).
 *
 * Sources, cited by page title and section:
 *   [S1] "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step
 *        Speculative Offloading" (AI summary), Key Contributions 1-4 and
 *        Methodology in Plain English.
 *   [S2] "Specter previews expert routing with an INT4 copy of the model
 *        itself", What shipped.
 *
 * Conventions shared by every entry point
 *   - fp16 tensors are passed as raw IEEE binary16 bit patterns (uint16_t).
 *   - All tensors are row-major and dense (no strides).
 *   - Every pointer is device memory unless a parameter says "host".  The
 *     caller owns every buffer; the library never allocates or frees.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work; results are valid once the stream reaches that point.
 *   - Shapes: H % 128 == 0, I % 128 == 0, 1 <= k <= E <= 256, T >= 0.
 *     T == 0 (or rows == 0) is a no-op that returns SMOE_OK.
 *   - Arguments are checked on the host before anything is enqueued; a bad
 *     argument returns a nonzero status and sets smoe_last_error() (thread
 *     local, valid until the next call on that thread).  The library never
 *     aborts.  Launch failures return SMOE_ERR_HIP with HIP's message.
 *   - Data errors only visible on the device (an expert id outside [0, E),
 *     a null weight pointer for a touched expert) are reported by OR-ing a
 *     SMOE_DERR_* bit into the optional `err_word` (int32 device memory);
 *     the offending work is skipped, nothing is read or written out of
 *     bounds.  The caller reads err_word after synchronising.
 *   - The first call on a device checks that it is a gfx950 GPU and returns
 *     SMOE_ERR_UNSUPPORTED otherwise.
 */
#ifndef SMOE_H
#define SMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMOE_ABI_VERSION 7

typedef enum {
    SMOE_OK = 0,
    SMOE_ERR_NULL = 1,         /* a required pointer is NULL                 */
    SMOE_ERR_SHAPE = 2,        /* a size or shape constraint is violated     */
    SMOE_ERR_UNSUPPORTED = 3,  /* device is not gfx950, or option not built  */
    SMOE_ERR_HIP = 4,          /* a HIP runtime call or launch failed        */
    SMOE_ERR_NOT_PINNED = 5,   /* host source of a stage is not page-locked  */
    SMOE_ERR_WORKSPACE = 6     /* workspace NULL or smaller than required    */
} smoe_status;

/* device-side data error bits (OR-ed into err_word) */
#define SMOE_DERR_BAD_ID      1   /* an expert id outside [0, E)            */
#define SMOE_DERR_NULL_EXPERT 2   /* a touched expert has a NULL weight     */
#define SMOE_DERR_SYNC        4   /* moe_draft_layer: a grid barrier timed out */

/* Version of this header's ABI; the binding refuses a mismatched library. */
int smoe_abi_version(void);

/* Message of the last failed call on this thread ("" after a success). */
const char* smoe_last_error(void);

/* ------------------------------------------------------------------------
 * Expert weight descriptors (device arrays of E entries, uploaded by the
 * caller; entries may point anywhere in device memory, e.g. at resident or
 * staging slots).
 *
 * smoe_w4_mat: one GPTQ INT4 matrix W[K, N] with group size 128, in the usual
 * GPTQ checkpoint layout ([S2] the draft's routed experts are GPTQ INT4,
 * group 128):
 *   qweight int32 [K/8, N]    nibble i (bits 4i..4i+3) of word [r, n] is the
 *                             4-bit code of row 8r+i, column n;
 *   scales  fp16  [K/128, N]  scale of (group, column);
 *   qzeros  int32 [K/128, N/8] nibble i of word [g, c] is the 4-bit zero of
 *                             column 8c+i in group g (no offset).
 *   W[kk, n] = (q[kk, n] - z[kk/128, n]) * s[kk/128, n].
 * A draft expert holds w13 (K = H, N = 2I; columns 0..I-1 are the gate
 * projection, I..2I-1 the up projection) and w2 (K = I, N = H).
 *
 * smoe_f16_expert: the FP16 target expert in nn.Linear layout (y = x W^T):
 *   w13 fp16 [2I, H] (rows 0..I-1 gate, I..2I-1 up), w2 fp16 [H, I].
 * ---------------------------------------------------------------------- */
typedef struct {
    const int32_t* qweight;
    const uint16_t* scales;
    const int32_t* qzeros;
} smoe_w4_mat;

typedef struct {
    smoe_w4_mat w13;
    smoe_w4_mat w2;
} smoe_w4_expert;

typedef struct {
    const uint16_t* w13;
    const uint16_t* w2;
} smoe_f16_expert;

/* ------------------------------------------------------------------------
 * moe_route_topk -- top-k routing by the FP16 router ([S1] Key Contributions
 * 3: the target router's decisions are authoritative; [S2] the draft reuses
 * the target's router and shared-expert tensors).
 *
 *   x             fp16 [T, H]   token activations
 *   w_router      fp16 [E, H]   router weight
 *   w_shared_gate fp16 [H]      optional (NULL = none) shared-expert gate
 *   renormalize   0: weights are the softmax over all E at the chosen ids;
 *                 1: those weights divided by their sum
 *   topk_ids      int32 [T, k]  out: experts by decreasing logit, equal
 *                               logits lower index first
 *   topk_w        fp32  [T, k]  out: routing weights
 *   shared_gate   fp32  [T]     out (required iff w_shared_gate is given):
 *                               sigmoid(x . w_shared_gate)
 * Logits are fp32 sums of exact fp16 products taken in one fixed order, so
 * the chosen ids are reproducible bit for bit: hidden chunks of 8 elements,
 * chunk c owned by lane c mod 64, each lane adding its products in
 * increasing index; then six pairwise rounds s_p += s_(p xor d), d = 32..1.
 * ---------------------------------------------------------------------- */
smoe_status moe_route_topk(const uint16_t* x, const uint16_t* w_router,
                           const uint16_t* w_shared_gate, int T, int H, int E, int k,
                           int renormalize, int32_t* topk_ids, float* topk_w,
                           float* shared_gate, void* stream);

/* ------------------------------------------------------------------------
 * elb_count -- Expert Lookahead Buffer update ([S1] Key Contributions 3 and
 * Methodology in Plain English: a per-layer table of expert counts kept in
 * device memory and bumped by each draft step's routing; copies of it taken
 * at chunk boundaries decide what to prefetch).
 *
 *   topk_ids  int32 [T, k]
 *   counters  int32 [L, E]  in/out: counters[layer, e] += number of (t, j)
 *                           with topk_ids[t, j] == e.  Accumulates across
 *                           calls; the caller clears or snapshots it at
 *                           chunk boundaries (plain copies / memsets).
 *   err_word  optional; ids outside [0, E) are skipped and flagged.
 * Integer atomics: the result does not depend on execution order.
 * ---------------------------------------------------------------------- */
smoe_status elb_count(const int32_t* topk_ids, int T, int k, int E, int layer, int L,
                      int32_t* counters, int32_t* err_word, void* stream);

/* ------------------------------------------------------------------------
 * moe_gather -- group the T*k (token, slot) pairs by expert ([S1] Key
 * Contributions 4 and Methodology: both the draft and the verification FFN
 * process each expert's rows as one block).  Pair p = t*k + j.
 * Stable: inside one expert, rows follow increasing p.
 *
 *   expert_offsets int32 [E+1]  out: rows of expert e are [off[e], off[e+1])
 *   sorted_pair    int32 [T*k]  out: pair held by each sorted row (-1 past
 *                               the last valid row)
 *   sorted_token   int32 [T*k]  out: sorted_pair / k (-1 past the end)
 *   pair_pos       int32 [T*k]  out: sorted row of pair p (-1 if dropped)
 *   active         int32 [E]    out: touched experts in increasing id, then -1
 *   n_active       int32 [1]    out: number of touched experts
 *   err_word       optional; ids outside [0, E) are dropped and flagged.
 * T*k must not exceed 1<<20.
 * ---------------------------------------------------------------------- */
smoe_status moe_gather(const int32_t* topk_ids, int T, int k, int E, int32_t* expert_offsets,
                       int32_t* sorted_token, int32_t* sorted_pair, int32_t* pair_pos,
                       int32_t* active, int32_t* n_active, int32_t* err_word, void* stream);

/* ------------------------------------------------------------------------
 * moe_route_plan -- moe_route_topk, elb_count and moe_gather of one step in a
 * single launch, for decode-sized T ([S1] Key Contributions 3-4: the drafted
 * tokens' expert choices come from the target router, are tallied in GPU
 * counters and gathered by expert inside one fused launch).  One workgroup
 * evaluates every router dot product of a small step.  Larger steps
 * (T*(E+1)*H above 2^16) run as two launches when a workspace is given: the
 * router dot products one per wave across the chip into the workspace, then
 * one workgroup for the top k, the ELB update and the maps.  Without one,
 * steps with more than one token and T*(E+1)*H above 2^18 run the routing
 * kernel, then the ELB update and the maps in one workgroup.
 *
 * Arguments and outputs are those of the three calls (same meaning, layout
 * and bit-identical values, whichever form runs).  counters may be NULL (no
 * ELB update; layer and L are then ignored).
 *   workspace        device, NULL or >= 4*T*(E+1) bytes (E+1 with a shared
 *                    gate, else E), 16-byte aligned; caller-owned, holds the
 *                    step's fp32 logits until the call's kernels end; a
 *                    smaller workspace_bytes or a misaligned workspace is
 *                    SMOE_ERR_WORKSPACE.
 * Limits: T*k <= 1024 and T*(E+1) <= 4096 (one workgroup holds the pairs and
 * logits); beyond them SMOE_ERR_SHAPE -- use the separate calls.  T == 0
 * writes empty maps.
 * ---------------------------------------------------------------------- */
smoe_status moe_route_plan(const uint16_t* x, const uint16_t* w_router,
                           const uint16_t* w_shared_gate, int T, int H, int E, int k,
                           int renormalize, int layer, int L, int32_t* counters,
                           int32_t* topk_ids, float* topk_w, float* shared_gate,
                           int32_t* expert_offsets, int32_t* sorted_token, int32_t* sorted_pair,
                           int32_t* pair_pos, int32_t* active, int32_t* n_active,
                           void* workspace, size_t workspace_bytes, int32_t* err_word,
                           void* stream);

/* ------------------------------------------------------------------------
 * w4a16_grouped_ffn -- draft routed-expert SwiGLU FFN over GPTQ INT4 weights
 * for every touched expert, one launch per projection across all experts
 * ([S1] Key Contributions 4: fused multi-expert INT4 draft kernel, one GPU
 * launch; [S2] W4A16: INT4 tiles dequantised while the products are formed
 * in higher precision).
 *
 * For every sorted row r of expert e (rows from moe_gather):
 *   h = silu(x[sorted_token[r]] . Wg_e) * (x[sorted_token[r]] . Wu_e)   (fp16)
 *   y_sorted[r] = h . Wd_e                                              (fp16)
 * with W dequantised per group; products accumulate in fp32.
 *
 *   x              fp16 [T, H]
 *   sorted_token, expert_offsets, active, n_active: from moe_gather
 *   experts        device array of E smoe_w4_expert
 *   k              top-k (rows = T*k bounds the sorted rows)
 *   group_size     must be 128
 *   y_sorted       fp16 [T*k, H] out (rows past off[E] untouched)
 *   workspace      device, >= smoe_workspace_bytes(0, T, k, H, I, E) bytes,
 *                  256-byte aligned: holds h (fp16 [T*k, I]) between the two
 *                  projections; no initialisation needed.
 *   H, I           at most 16384 each (activations are staged in LDS).
 * The maps must be moe_gather's for these ids: with T == 1 the kernels use
 * its ordering (the i-th touched expert by increasing id owns sorted row i)
 * to request activation rows before reading the maps.
 * ---------------------------------------------------------------------- */
smoe_status w4a16_grouped_ffn(const uint16_t* x, const int32_t* sorted_token,
                              const int32_t* expert_offsets, const int32_t* active,
                              const int32_t* n_active, const smoe_w4_expert* experts, int T,
                              int k, int H, int I, int E, int group_size, uint16_t* y_sorted,
                              void* workspace, size_t workspace_bytes, int32_t* err_word,
                              void* stream);

/* ------------------------------------------------------------------------
 * w4a16_grouped_ffn_shared -- w4a16_grouped_ffn plus the layer's dense FP16
 * shared expert over all T rows of x ([S1] Key Contributions 2: the draft
 * keeps the shared experts at FP16 beside the INT4 routed experts; Key
 * Contributions 4: the draft step's sub-computations batched into few
 * launches).  Its columns run as extra workgroups of the two multi-row INT4
 * launches: with 2..4 rows through the matrix-vector routine where its
 * registers fit them (H in 1544-2048 or 3592-4096, shared_I in 2568-3072 or
 * 3592-4096), with 5..16 rows as 16-column MFMA items (H and shared_I of at
 * least 1024); otherwise in launches of their own after them.
 *
 *   x .. workspace, err_word, stream: as w4a16_grouped_ffn (y_sorted is
 *                  bit-identical to that call's)
 *   shared_w13     fp16 [2*shared_I, H]: gate rows, then up rows (nn.Linear)
 *   shared_w2      fp16 [H, shared_I]
 *   shared_I       positive multiple of 128
 *   shared_h       fp16 [T, shared_I] out: silu(x . gate) * (x . up), fp16
 *   shared_out     fp16 [T, H] out: shared_h . w2^T (unscaled: a sigmoid gate
 *                  is the combine's shared_scale)
 * shared_h and shared_out are bit-identical to verify_grouped_gemm's outputs
 * for the shared expert as its only expert with all T rows in order: up to
 * 4 rows (both take the matrix-vector routine), and for 5..63 rows when H and
 * shared_I are at least 1024 (both take the one-expert ring arithmetic);
 * other shapes agree within the FP16 tolerance of the reference.  All four
 * shared pointers are required (SMOE_ERR_NULL), 16-byte aligned
 * (SMOE_ERR_SHAPE).
 * ---------------------------------------------------------------------- */
smoe_status w4a16_grouped_ffn_shared(const uint16_t* x, const int32_t* sorted_token,
                                     const int32_t* expert_offsets, const int32_t* active,
                                     const int32_t* n_active, const smoe_w4_expert* experts,
                                     int T, int k, int H, int I, int E, int group_size,
                                     uint16_t* y_sorted, const uint16_t* shared_w13,
                                     const uint16_t* shared_w2, int shared_I,
                                     uint16_t* shared_h, uint16_t* shared_out, void* workspace,
                                     size_t workspace_bytes, int32_t* err_word, void* stream);

/* ------------------------------------------------------------------------
 * w4a16_grouped_ffn_noalloc -- w4a16_grouped_ffn without a workspace
 * argument, for callers that cannot allocate device memory around the call
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The workspace lives in a scratch array that the library
 * holds in device memory, SMOE_NOALLOC_SCRATCH_BYTES on each GPU it runs on,
 * from the library's load until the process ends.  The call allocates and
 * frees nothing.
 *
 * Arguments, outputs and errors are those of w4a16_grouped_ffn (same kernels,
 * bit-identical results), without workspace / workspace_bytes.  A request
 * whose workspace, smoe_workspace_bytes(0, T, k, H, I, E), exceeds
 * SMOE_NOALLOC_SCRATCH_BYTES returns SMOE_ERR_SHAPE before anything is
 * enqueued (h takes T*k*I*2 bytes: e.g. T*k <= 256 rows at I = 6400).
 * Every call on one GPU shares that GPU's scratch: calls whose executions
 * overlap on one GPU (on different streams, or from different threads)
 * race; calls on one stream are ordered and safe.  The scratch keeps the
 * last call's contents; the kernels need no initialised scratch.
 * ---------------------------------------------------------------------- */
#define SMOE_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)

smoe_status w4a16_grouped_ffn_noalloc(const uint16_t* x, const int32_t* sorted_token,
                                      const int32_t* expert_offsets, const int32_t* active,
                                      const int32_t* n_active, const smoe_w4_expert* experts,
                                      int T, int k, int H, int I, int E, int group_size,
                                      uint16_t* y_sorted, int32_t* err_word, void* stream);

/* ------------------------------------------------------------------------
 * awq_grouped_ffn -- w4a16_grouped_ffn for AWQ-style draft experts ([S1]
 * Main Findings: the draft's routing fidelity is compared across GGUF, GPTQ
 * and AWQ 4-bit copies).  An AWQ-style expert was quantised after each input
 * channel c of a projection had been multiplied by a positive factor a[c]
 * (chosen from activation statistics), so the product takes the activation
 * divided by the same factor:
 *   h = silu((x / a13) . Wg) * ((x / a13) . Wu),   y = (h / a2) . Wd,
 * with W dequantised from the GPTQ layout of w4a16_grouped_ffn (same
 * group 128, codes, scales and zeros).  Each quotient is rounded to fp16, as
 * the activations are.
 *
 *   act_scales     device array of 2*E pointers: act_scales[2e] is expert
 *                  e's fp16 [H] divisors of the gate/up input, act_scales[2e
 *                  + 1] its fp16 [I] divisors of the down input (16-byte
 *                  aligned, positive, finite; a touched expert with a NULL
 *                  entry is skipped and flagged SMOE_DERR_NULL_EXPERT)
 * Every other argument, output and limit is that of w4a16_grouped_ffn.
 * Multi-row steps run the VALU kernels (the divisors are applied where those
 * stage their rows), not the MFMA kernel of w4a16_grouped_ffn.
 * ---------------------------------------------------------------------- */
smoe_status awq_grouped_ffn(const uint16_t* x, const int32_t* sorted_token,
                            const int32_t* expert_offsets, const int32_t* active,
                            const int32_t* n_active, const smoe_w4_expert* experts,
                            const uint16_t* const* act_scales, int T, int k, int H, int I, int E,
                            int group_size, uint16_t* y_sorted, void* workspace,
                            size_t workspace_bytes, int32_t* err_word, void* stream);

/* ------------------------------------------------------------------------
 * wq_grouped_ffn -- w4a16_grouped_ffn for other draft code widths ([S1] Main
 * Findings and Future Directions: the draft's fidelity is compared across
 * quantisation precisions, 2-, 4- and 8-bit, and the precision is a design
 * lever).  The experts are in the GPTQ layout of the same group size (128)
 * with `bits`-bit codes:
 *   qweight int32 [K*bits/32, N]  code i (bits bits*i .. bits*i+bits-1) of
 *                                 word [r, n] is row (32/bits)*r + i of
 *                                 column n;
 *   scales  fp16  [K/128, N];
 *   qzeros  int32 [K/128, N*bits/32]  code i of word [g, c] is the zero of
 *                                 column (32/bits)*c + i in group g;
 *   W[kk, n] = (q[kk, n] - z[kk/128, n]) * s[kk/128, n].
 * smoe_w4_expert/smoe_w4_mat hold the three pointers whatever the width.
 * Arguments, outputs and workspace are those of w4a16_grouped_ffn; bits is
 * 2, 4 or 8 (else SMOE_ERR_UNSUPPORTED), and bits == 4 is w4a16_grouped_ffn.
 * ---------------------------------------------------------------------- */
smoe_status wq_grouped_ffn(const uint16_t* x, const int32_t* sorted_token,
                           const int32_t* expert_offsets, const int32_t* active,
                           const int32_t* n_active, const smoe_w4_expert* experts, int T, int k,
                           int H, int I, int E, int bits, int group_size, uint16_t* y_sorted,
                           void* workspace, size_t workspace_bytes, int32_t* err_word,
                           void* stream);

/* ------------------------------------------------------------------------
 * moe_draft_route_ffn -- one-token (T = 1) draft step of a layer: the work
 * of moe_route_plan followed by w4a16_grouped_ffn ([S1] Key Contributions 4:
 * routing, gathering and the experts' FFN of a draft step inside one fused
 * launch).  Three launches: the router logits (one wave per router row),
 * then the gate/up projection, whose every workgroup takes the top k of
 * those logits itself (one extra workgroup writes the routing outputs, the
 * ELB increments and the maps), then the down projection.
 *
 * Arguments keep the meaning and layout of those two calls with T = 1:
 *   x              fp16 [1, H]
 *   w_router, w_shared_gate, renormalize, layer, L, counters: moe_route_plan
 *                  (counters may be NULL: no ELB update)
 *   experts, group_size (128), I: w4a16_grouped_ffn
 *   topk_ids [k], topk_w [k], shared_gate [1], expert_offsets [E+1],
 *   sorted_token [k], sorted_pair [k], pair_pos [k], active [E],
 *   n_active [1]   out: bit-identical to moe_route_plan's
 *   y_sorted       fp16 [k, H] out: bit-identical to w4a16_grouped_ffn's
 *   shared_w13, shared_w2, shared_I, shared_h, shared_out: an optional dense
 *                  FP16 shared expert ([S2] What shipped: the draft reuses
 *                  the target's shared experts in FP16) computed inside the
 *                  same gate/up and down launches: shared_w13 fp16 [2*shared_I,
 *                  H] (gate rows, then up rows), shared_w2 fp16 [H, shared_I],
 *                  shared_h fp16 [shared_I] (caller-owned scratch between the
 *                  projections), shared_out fp16 [1, H] out, bit-identical to
 *                  verify_grouped_gemm on the same row as one always-on group.
 *                  shared_w13 NULL = no shared expert (the other four are then
 *                  ignored).  Several shared experts of one layer pass as one
 *                  of their summed intermediate.
 *   logits         fp32 [E] (+1 with w_shared_gate: the gate's logit last),
 *                  optional: the router logits of x in the pinned order, as
 *                  moe_combine_route_logits writes them; when given the call
 *                  takes them instead of computing them (two launches) and
 *                  every output is the same as without.  NULL: computed here.
 *   workspace      >= smoe_workspace_bytes(0, 1, k, H, I, E) bytes,
 *                  256-byte aligned
 * Limits: k <= 32, E <= 256, H and I at most 16384; with a shared expert,
 * shared_I a positive multiple of 128 and H, shared_I at most 8192
 * (SMOE_ERR_SHAPE beyond); shared_w13, shared_w2, shared_h 16-byte aligned.
 * The caller owns every buffer; nothing is allocated.
 * ---------------------------------------------------------------------- */
smoe_status moe_draft_route_ffn(const uint16_t* x, const uint16_t* w_router,
                                const uint16_t* w_shared_gate, int H, int I, int E, int k,
                                int renormalize, int layer, int L, int32_t* counters,
                                const smoe_w4_expert* experts, int group_size,
                                int32_t* topk_ids, float* topk_w, float* shared_gate,
                                int32_t* expert_offsets, int32_t* sorted_token,
                                int32_t* sorted_pair, int32_t* pair_pos, int32_t* active,
                                int32_t* n_active, uint16_t* y_sorted,
                                const uint16_t* shared_w13, const uint16_t* shared_w2,
                                int shared_I, uint16_t* shared_h, uint16_t* shared_out,
                                const float* logits, void* workspace, size_t workspace_bytes,
                                int32_t* err_word, void* stream);

/* ------------------------------------------------------------------------
 * moe_draft_layer -- one-token (T = 1) draft step of a whole MoE layer in a
 * single launch ([S1] Key Contributions 4 and Methodology in Plain English:
 * the draft's routing and expert sub-computations are dispatched inside one
 * fused GPU launch): the router logits (unless given), the top-k routing
 * with the ELB update and the maps, the routed INT4 experts' FFN, the
 * optional FP16 shared expert, and the combine with residual, norm epilogue
 * and the next layer's router logits.  One workgroup per CU, all resident;
 * phases are separated by grid barriers inside the launch.
 *
 * Arguments keep the meaning and layout of moe_draft_route_ffn (x,
 * w_router, w_shared_gate, logits, H, I, E, k, renormalize, layer, L,
 * counters, experts, group_size, the routing outputs, y_sorted, the shared
 * expert and shared_h) followed by those of moe_combine_route_logits
 * (residual, out, norm_out, norm_eps, next_w_router, next_w_shared_gate,
 * next_E, next_logits), all for this one token:
 *   logits         fp32 [E (+1)] of x from the launch before, or NULL: the
 *                  call computes them itself (one more grid barrier)
 *   y_sorted       fp16 [k, H] out, shared_out fp16 [1, H] out, shared_h
 *                  fp16 [shared_I] scratch: written inside the launch
 *   residual       fp16 [1, H] or NULL; out fp16 [1, H] out (required)
 *   norm_out       fp16 [1, H] out or NULL (no norm epilogue)
 *   next_w_router  fp16 [next_E, H] or NULL; with it norm_out and
 *                  next_logits (fp32 [next_E (+1)]) are required
 *   workspace      >= smoe_workspace_bytes(2, 1, k, H, I, E) bytes,
 *                  256-byte aligned; its first 8 bytes are the barrier
 *                  counters and must be zero before the first call (every
 *                  completed call leaves them zero; new workspaces from the
 *                  binding are zero-filled).
 * Every output is bit-identical to moe_draft_route_ffn followed by
 * moe_combine (or moe_combine_route_logits): same kernels' arithmetic and
 * summation orders.
 * Limits: E <= 64, k <= 32, H and I multiples of 128 with H <= 8192; the
 * instantiated geometries are those of the Phi-3.5-MoE (H 4096, I 6400, no
 * shared expert), DeepSeek-V2-Lite (H 2048, I 1408, shared I 2816) and
 * Qwen1.5-MoE (H 2048, I 1408, shared I 5632) layers, and H 2048, I 1408
 * without a shared expert.  Any other shape returns SMOE_ERR_UNSUPPORTED
 * before anything is enqueued (use moe_draft_route_ffn and
 * moe_combine_route_logits instead).  smoe_draft_layer_supported tells.
 * Device errors: SMOE_DERR_SYNC when a grid barrier waited longer than
 * 100 ms (a workgroup was not resident: another kernel held its CU); the
 * outputs are then undefined and the workspace's counters must be zeroed
 * before the next call.  Calls sharing a workspace must not overlap.
 * ---------------------------------------------------------------------- */
smoe_status moe_draft_layer(const uint16_t* x, const uint16_t* w_router,
                            const uint16_t* w_shared_gate, const float* logits, int H, int I,
                            int E, int k, int renormalize, int layer, int L, int32_t* counters,
                            const smoe_w4_expert* experts, int group_size, int32_t* topk_ids,
                            float* topk_w, float* shared_gate, int32_t* expert_offsets,
                            int32_t* sorted_token, int32_t* sorted_pair, int32_t* pair_pos,
                            int32_t* active, int32_t* n_active, uint16_t* y_sorted,
                            const uint16_t* shared_w13, const uint16_t* shared_w2, int shared_I,
                            uint16_t* shared_h, uint16_t* shared_out, const uint16_t* residual,
                            uint16_t* out, uint16_t* norm_out, float norm_eps,
                            const uint16_t* next_w_router, const uint16_t* next_w_shared_gate,
                            int next_E, float* next_logits, void* workspace,
                            size_t workspace_bytes, int32_t* err_word, void* stream);

/* 1 when moe_draft_layer has an instantiation for this shape (shared_I = 0:
 * no shared expert) on the current device, else 0. */
int smoe_draft_layer_supported(int H, int I, int E, int k, int shared_I);

/* ------------------------------------------------------------------------
 * moe_combine_route_logits -- one token (T = 1): moe_combine of a layer's
 * expert outputs with its norm epilogue, and in the same launch the next
 * layer's router logits of the normalised row ([S1] Key Contributions 4:
 * fewer launches per draft step; in a chain of pre-norm layers the combine
 * of layer l and the routing of layer l+1 read the same row).
 *
 *   y_sorted, pair_pos, topk_w, shared_out, shared_scale, residual, k, H,
 *   out, norm_out, norm_eps: moe_combine with T = 1 (norm_out required);
 *                  out and norm_out are bit-identical to moe_combine's
 *   w_router       fp16 [E, H] router of the next layer
 *   w_shared_gate  fp16 [H] optional shared-expert gate row of that layer
 *   logits         fp32 [E] (+1 with w_shared_gate) out: the pinned-order
 *                  logits of norm_out, bit-identical to those
 *                  moe_draft_route_ffn computes from norm_out (pass them to
 *                  it as its logits argument)
 * Limits: H a multiple of 128, at most 8192; 1 <= k, E <= 256.
 * ---------------------------------------------------------------------- */
smoe_status moe_combine_route_logits(const uint16_t* y_sorted, const int32_t* pair_pos,
                                     const float* topk_w, const uint16_t* shared_out,
                                     const float* shared_scale, const uint16_t* residual, int k,
                                     int H, uint16_t* out, uint16_t* norm_out, float norm_eps,
                                     const uint16_t* w_router, const uint16_t* w_shared_gate,
                                     int E, float* logits, void* stream);

/* ------------------------------------------------------------------------
 * verify_grouped_gemm -- FP16 SwiGLU FFN of the target experts over the
 * rows grouped by expert: expert-wise verification regrouping ([S1] Key
 * Contributions 4 and Methodology: the tokens routed to one expert are packed
 * so per-token matrix-vector products become one matrix-matrix product per
 * expert; results equal the per-token ordering).  Runs on MFMA with fp32
 * accumulation; h is rounded to fp16 between the projections.
 *
 *   x              fp16 [T, H]
 *   sorted_token   int32 [rows]  token of each sorted row
 *   expert_offsets int32 [E+1]
 *   active/n_active  optional pair (both NULL = scan all E experts)
 *   experts        device array of E smoe_f16_expert (may point at resident
 *                  or staging slots)
 *   expert_mask    optional uint8 [E]; experts with mask 0 are skipped, so
 *                  cache hits can run before misses arrive ([S1] Key
 *                  Contributions 3 and Methodology: on-device experts run
 *                  while the weights of the others are still being copied)
 *   rows           number of sorted rows (T*k for routed experts; T for a
 *                  shared expert run as one group with offsets {0, T})
 *   y_sorted       fp16 [rows, H] out
 *   workspace      >= smoe_workspace_bytes(1, T, k, H, I, E) with k = rows/T
 *                  (rounded up); no zeroing needed.
 * ---------------------------------------------------------------------- */
smoe_status verify_grouped_gemm(const uint16_t* x, const int32_t* sorted_token,
                                const int32_t* expert_offsets, const int32_t* active,
                                const int32_t* n_active, const smoe_f16_expert* experts,
                                const uint8_t* expert_mask, int T, int rows, int H, int I,
                                int E, uint16_t* y_sorted, void* workspace,
                                size_t workspace_bytes, int32_t* err_word, void* stream);

/* ------------------------------------------------------------------------
 * verify_grouped_gemm_shared -- verify_grouped_gemm over the routed experts
 * and, in the same two launches, the FFN of a dense FP16 shared expert over
 * all T tokens ([S1] Key Contributions 2: shared experts stay FP16 and run
 * for every token; the verification step covers the whole layer).  The
 * shared expert's work items lead each launch, so its short, latency-bound
 * items overlap the routed experts' stream instead of running as launches of
 * their own afterwards.  Shapes whose routed launches do not run the ring
 * kernels (very few tokens, the tiled many-row regime, short reductions)
 * take the routed call followed by launches of the shared expert alone;
 * the outputs have the same meaning either way.
 *
 * Arguments: those of verify_grouped_gemm, then
 *   shared_w13     fp16 [2*shared_I, H] (gate rows, then up rows)
 *   shared_w2      fp16 [H, shared_I]
 *   shared_I       multiple of 128
 *   shared_h       fp16 [T, shared_I] caller-owned scratch
 *   shared_out     fp16 [T, H] out: the shared expert's output, rounded to
 *                  fp16 (fp32 accumulation; h rounded between projections),
 *                  to pass to moe_combine as shared_out
 * All shared pointers are required and 16-byte aligned.
 * ---------------------------------------------------------------------- */
smoe_status verify_grouped_gemm_shared(const uint16_t* x, const int32_t* sorted_token,
                                       const int32_t* expert_offsets, const int32_t* active,
                                       const int32_t* n_active, const smoe_f16_expert* experts,
                                       const uint8_t* expert_mask, int T, int rows, int H, int I,
                                       int E, uint16_t* y_sorted, const uint16_t* shared_w13,
                                       const uint16_t* shared_w2, int shared_I,
                                       uint16_t* shared_h, uint16_t* shared_out, void* workspace,
                                       size_t workspace_bytes, int32_t* err_word, void* stream);

/* ------------------------------------------------------------------------
 * moe_combine -- weighted sum of the chosen experts' outputs plus the shared
 * expert (the pages leave this step implicit; it is the usual routed-MoE
 * combine):
 *   out[t] = fp16( sum_j topk_w[t,j] * y_sorted[pair_pos[t*k+j]]
 *                  + c_t * shared_out[t] + residual[t] )
 * summed in fp32 in that order (j increasing), one rounding to fp16.
 *   y_sorted     fp16 [T*k, H]
 *   pair_pos     int32 [T, k], rows of y_sorted
 *   shared_out   fp16 [T, H] optional (NULL = no shared term)
 *   shared_scale fp32 [T]    optional (NULL = 1), c_t
 *   residual     fp16 [T, H] optional (NULL = none)
 *   pairs with pair_pos == -1 contribute nothing.
 *   out          fp16 [T, H]; may alias residual.
 *   norm_out     fp16 [T, H] optional (NULL = none): the next pre-norm
 *                layer's input, out[t] / sqrt(mean(out[t]^2) + norm_eps)
 *                computed from the rounded out (the pages say draft and
 *                target share the normalisation without defining it; this
 *                is a unit-weight RMS norm).  Must not alias out.
 * ---------------------------------------------------------------------- */
smoe_status moe_combine(const uint16_t* y_sorted, const int32_t* pair_pos, const float* topk_w,
                        const uint16_t* shared_out, const float* shared_scale,
                        const uint16_t* residual, int T, int k, int H, uint16_t* out,
                        uint16_t* norm_out, float norm_eps, void* stream);

/* ------------------------------------------------------------------------
 * expert_stage_async -- copy one non-resident expert from page-locked host
 * memory into a device slot on a side stream and record an event after it
 * ([S1] Key Contributions 3-4: cache-miss expert loads overlap the compute of
 * cache hits, using dedicated streams, events and pinned non-blocking copies).
 *
 *   dst_device       device destination (bytes long)
 *   src_pinned_host  host source; must be page-locked (hipHostMalloc or
 *                    torch pin_memory), else SMOE_ERR_NOT_PINNED
 *   side_stream      hipStream_t the copy is queued on
 *   done_event       hipEvent_t recorded on side_stream after the copy
 *                    (NULL = none); the compute stream waits on it before
 *                    touching dst.
 * ---------------------------------------------------------------------- */
smoe_status expert_stage_async(void* dst_device, const void* src_pinned_host, size_t bytes,
                               void* side_stream, void* done_event);

/* ------------------------------------------------------------------------
 * smoe_stream_read -- measurement aid, not a step of the path: reads `bytes`
 * of device memory at `src` once, grid-stride over `blocks` workgroups of
 * 256 threads, with the 16-byte non-temporal loads the weight-streaming
 * kernels use, and writes the XOR of the 32-bit words each workgroup read to
 * sink[workgroup] (uint32 [blocks]).  Its duration is the memory-bound
 * ceiling for streaming that many bytes in one launch; the throughput of the
 * draft FFN is reported against a sequence of such reads of the same byte
 * counts.  bytes must be a multiple of 16, src 16-byte aligned, 1 <= blocks
 * <= 65535.
 * ---------------------------------------------------------------------- */
smoe_status smoe_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks,
                             void* stream);

/* Workspace size in bytes for which = 0 (w4a16_grouped_ffn), 1
 * (verify_grouped_gemm) or 2 (moe_draft_layer, T = 1); 0 for an invalid
 * request. */
size_t smoe_workspace_bytes(int which, int T, int k, int H, int I, int E);

#ifdef __cplusplus
}
#endif

#endif /* SMOE_H */
