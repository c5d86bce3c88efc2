/*
 * moe_verify.h — C ABI of the MoE expert operation inside a speculative-decoding
 * verification pass, for AMD Instinct MI355X (gfx950).
 *
 * The operation (one MoE layer, one verify pass of n drafted tokens):
 *   1. route:   each token's K largest router logits and their softmax gates
 *               ("Making Every Verified Token Count: Adaptive Verification for
 *               MoE Speculative Decoding", Sec. 2.2, Eq. (4));
 *   2. union:   the distinct experts over all n*K token-slots, with the slots
 *               grouped by expert ("Less Experts, Faster Decoding", Sec. 3,
 *               Eq. (1); adaptive-verification page, Eq. (5));
 *   3. experts: SwiGLU y = (silu(x W_gate) * (x W_up)) W_down for every slot,
 *               either deduplicating (each union expert streamed from HBM once
 *               per pass) or per-slot (each expert read once per token-slot)
 *               ("Speculative Decoding for Mixture-of-Experts Models: Expert
 *               Bytes, Kernel Bandwidth and the Best Draft Length", abstract and
 *               Table 5 / Table 6);
 *   4. combine: gate-weighted sum of the K slot outputs plus the shared experts
 *               (adaptive-verification page, Sec. 2.2).
 *
 * Conventions for every entry point
 *   - Pointers marked (device) are device pointers; the caller allocates and
 *     owns all memory.  The library allocates nothing and keeps no state
 *     between calls; calls on different streams with disjoint buffers may run
 *     concurrently, except the one-launch passes (moe_verify_layer*), which
 *     need the whole device (see there).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  Outputs are valid once the stream has reached the call.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns an error code and enqueues nothing.
 *   - Faults only the device can see (an expert id outside [0, E) in ids given
 *     by the caller) are recorded: moe_build_union writes U = -1, and the FFN
 *     entry points set a bit in the error word at the start of their
 *     workspace, which moe_get_error reads back.  Outputs of a call that
 *     recorded a fault are unspecified.
 *   - Token-slot s = t*K + k names the k-th expert of token t.
 *
 * Storage layouts (row-major, one row per output feature, as in a Linear
 * weight):
 *   x         [n][d]          f32 or bf16
 *   w_gate    [E][f][d]       row j holds column j of the d x f matrix W_gate
 *   w_up      [E][f][d]
 *   w_down    [E][d][f]       row c holds column c of the f x d matrix W_down
 *   fp8 scales (w_dtype = MOE_FP8_E4M3, OCP E4M3FN codes): one fp32 per
 *             128 x 128 block of each stored matrix, indexed
 *             [E][rows/128][cols/128]; weight = decode(code) * scale.
 *   shared experts use the same layouts with S in place of E.
 * Supported (w_dtype, x_dtype): (F32, F32), (BF16, BF16), (FP8_E4M3, BF16).
 * Limits: 1 <= n <= 32, 1 <= K <= 8, K <= E <= 256, 0 <= S <= 4;
 *         d and f multiples of 8 (bf16), 4 (f32) or 128 (fp8), at most 65536.
 * Every device pointer must be 16-byte aligned; workspaces 256-byte aligned.
 */
#ifndef MOE_VERIFY_H
#define MOE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef void* moe_stream_t; /* hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,          /* null/misaligned pointer or size out of range */
  MOE_ERR_UNSUPPORTED = 2,  /* dtype combination or shape not supported */
  MOE_ERR_WORKSPACE = 3,    /* workspace too small or misaligned */
  MOE_ERR_HIP = 4,          /* the HIP runtime refused a launch or copy */
  MOE_ERR_BAD_IDS = 5,      /* (device) an expert id outside [0, E) was seen */
  MOE_ERR_TIMEOUT = 6,      /* (device) a bounded wait gave up */
  MOE_ERR_BAD_TREE = 7,     /* (device) a draft tree or its probabilities out of range */
  MOE_ERR_TOO_LARGE = 8     /* the pass needs more than moe_verify_layer_noalloc's scratch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;
typedef enum { MOE_MODE_DEDUP = 0, MOE_MODE_PERSLOT = 1 } moe_mode;

/* Layer geometry: routed experts E, experts per token K, hidden d, expert
 * intermediate f, shared experts S, storage types of weights and tokens. */
typedef struct {
  int32_t E, K, d, f, S;
  int32_t w_dtype, x_dtype; /* moe_dtype */
} moe_shape;

/* Expert weights (device).  s_* / sh_s_* are read only for fp8 weights;
 * sh_* are read only when S > 0. */
typedef struct {
  const void *w_gate, *w_up, *w_down;
  const float *s_gate, *s_up, *s_down;
  const void *sh_gate, *sh_up, *sh_down;
  const float *sh_s_gate, *sh_s_up, *sh_s_down;
} moe_weights;

/* Router top-K (adaptive-verification page, Sec. 2.2, Eq. (4)).
 *   logits (device) f32 [n][E]
 *   ids    (device) int32 [n][K]: the K experts with the largest logits, in
 *          descending-logit order; equal logits go to the lower id, NaN ranks
 *          below every number, -0.0 equals +0.0.
 *   gates  (device) f32 [n][K]: softmax over the K selected logits.
 * Errors: MOE_ERR_ARG for n, E or K out of range or null pointers. */
moe_status moe_route_topk(const float* logits, int32_t n, int32_t E, int32_t K,
                          int32_t* ids, float* gates, moe_stream_t stream);

/* Expert union of a verify pass ("Less Experts, Faster Decoding", Sec. 3,
 * Eq. (1)) and the slots grouped by expert (the expert-bytes page, Table 6:
 * rows sorted by expert before the tiled product).  cap = min(n*K, E).
 *   ids        (device) int32 [n*K]
 *   U          (device) int32 [1]: distinct ids, or -1 if an id is outside [0, E)
 *   union_ids  (device) int32 [cap]: ascending distinct ids; -1 beyond U
 *   offsets    (device) int32 [cap+1]: slots of union_ids[u] are
 *              perm[offsets[u] .. offsets[u+1]); entries from U on equal n*K
 *   perm       (device) int32 [n*K]: slots ordered by (id, slot)
 *   slot_rank  (device) int32 [n*K]: position of ids[s] in union_ids
 * Bit-exact and deterministic.  Errors: MOE_ERR_ARG. */
moe_status moe_build_union(const int32_t* ids, int32_t n, int32_t K, int32_t E,
                           int32_t* U, int32_t* union_ids, int32_t* offsets,
                           int32_t* perm, int32_t* slot_rank, moe_stream_t stream);

/* Route and union in one launch: the same outputs as moe_route_topk followed
 * by moe_build_union on its ids (one workgroup routes every token into LDS and
 * builds the union from there).  Errors: MOE_ERR_ARG. */
moe_status moe_route_union(const float* logits, int32_t n, int32_t E, int32_t K,
                           int32_t* ids, float* gates, int32_t* U, int32_t* union_ids,
                           int32_t* offsets, int32_t* perm, int32_t* slot_rank,
                           moe_stream_t stream);

/* Per-layer expert budget on a union ("MoE-Spec: Expert Budgeting for
 * Efficient Speculative Decoding", abstract: a layer of the verify pass loads
 * at most C experts, those contributing most to the verified tokens).  The
 * page gives no formula; here an expert's contribution is the float32 sum of
 * the gates of its slots (ascending slot order), the C largest are kept
 * (equal contributions: the lower id; NaN below every number), and a dropped
 * slot adds nothing to the layer output.
 *   gates      (device) f32 [n][K]: the pass's gates
 *   U, union_ids, offsets, perm, slot_rank (device, in/out): the union of
 *              moe_build_union / moe_route_union for the same slots, rewritten
 *              in place when C < U: U = C; union_ids the kept experts
 *              ascending (-1 beyond); offsets over the kept groups, entries
 *              from U on = the number of kept slots; perm the kept slots
 *              grouped by expert as before, then the dropped slots in
 *              ascending order; slot_rank -1 for a dropped slot.  Unchanged
 *              when C >= U or U < 0.
 *   gates_out  (device) f32 [n][K] (may be gates): 0 for a dropped slot; with
 *              renorm = 1 the kept gates of a token that lost a slot are
 *              divided by their float32 sum (k ascending; 0 if that sum is 0).
 * moe_expert_ffn_dedup on the rewritten union streams the kept experts only
 * and writes zero output rows for the dropped slots; moe_combine with
 * gates_out then gives the budgeted layer output.
 * 1 <= C; renorm 0 or 1.  Bit-exact and deterministic.  Errors: MOE_ERR_ARG. */
moe_status moe_expert_budget(const float* gates, int32_t n, int32_t K, int32_t E, int32_t C,
                             int32_t renorm, int32_t* U, int32_t* union_ids, int32_t* offsets,
                             int32_t* perm, int32_t* slot_rank, float* gates_out,
                             moe_stream_t stream);

/* Deduplicating expert FFN: each expert of the union (and each shared expert)
 * is streamed from HBM once and applied to every slot routed to it (the
 * expert-bytes page, abstract).  The union arrays are those of
 * moe_build_union for the same ids.
 *   x         (device) [n][d] in shape->x_dtype
 *   y_slots   (device) f32 [n][K][d]: SwiGLU output of slot (t, k)
 *   y_shared  (device) f32 [n][S][d] (may be NULL when S == 0)
 *   bytes     (device) uint64 [2] or NULL: [0] = (U + S) * b, the bytes this
 *             call streams; [1] = n * (K + S) * b, what per-slot requests;
 *             b = bytes of one expert (3*d*f*elem, plus fp8 scales)
 *   ws        (device) workspace of at least moe_workspace_size(shape, n, DEDUP)
 *             bytes, zero-filled before its first use (moe_workspace_init).
 * Slots that belong to no group (perm entries from offsets[U] on: those an
 * expert budget dropped) get zero output rows.
 * Errors: MOE_ERR_ARG / _UNSUPPORTED / _WORKSPACE on the host; a device-side
 * U < 0 records MOE_ERR_BAD_IDS in the workspace. */
moe_status moe_expert_ffn_dedup(const moe_shape* shape, const moe_weights* w,
                                const void* x, int32_t n, const int32_t* U,
                                const int32_t* union_ids, const int32_t* offsets,
                                const int32_t* perm, float* y_slots, float* y_shared,
                                uint64_t* bytes, void* ws, size_t ws_bytes,
                                moe_stream_t stream);

/* Per-slot expert FFN: the expert of every slot (t, k), and every shared
 * expert for every token, is read once for that slot (the expert-bytes page,
 * abstract; Table 5, one grid slice per token-slot pair).  Same outputs as the
 * deduplicating call.
 *   ids    (device) int32 [n][K]; a slot with an id outside [0, E) gets a zero
 *          output row and records MOE_ERR_BAD_IDS in the workspace.
 *   bytes  (device) uint64 [2] or NULL: both entries n * (K + S) * b. */
moe_status moe_expert_ffn_perslot(const moe_shape* shape, const moe_weights* w,
                                  const void* x, int32_t n, const int32_t* ids,
                                  float* y_slots, float* y_shared, uint64_t* bytes,
                                  void* ws, size_t ws_bytes, moe_stream_t stream);

/* Combine (adaptive-verification page, Sec. 2.2: the layer output is the
 * weighted sum of the selected experts):
 *   out[t] = sum_{k ascending} gates[t][k] * y_slots[t][k] + sum_s y_shared[t][s]
 * out (device) [n][d] of out_dtype (MOE_F32 or MOE_BF16, round to nearest even).
 * y_shared may be NULL when S == 0.  d must be a multiple of 4; y_slots,
 * y_shared and out 16-byte aligned, gates 4-byte aligned.
 * Errors: MOE_ERR_ARG (pointers, sizes) / _UNSUPPORTED (out_dtype, d). */
moe_status moe_combine(const float* y_slots, const float* gates, const float* y_shared,
                       int32_t n, int32_t K, int32_t S, int32_t d, void* out,
                       int32_t out_dtype, moe_stream_t stream);

/* One MoE layer of a verify pass in one launch: the route of moe_route_topk,
 * the union of moe_build_union (deduplicating mode), the expert FFN of
 * moe_expert_ffn_dedup or moe_expert_ffn_perslot (mode) and the combine of
 * moe_combine, with the same results bit for bit (the pages of each step are
 * cited at those calls).  Every workgroup routes the pass itself and streams
 * a fixed share of the UP and DOWN work; intermediate results are exchanged
 * between workgroups through device-coherent stores, with bounded waits.
 *   logits    (device) f32 [n][E];  x (device) [n][d] in shape->x_dtype
 *   out       (device) [n][d] of out_dtype (MOE_F32 or MOE_BF16)
 *   ids, gates (device, optional) [n][K] routing outputs
 *   U, union_ids, offsets, perm, slot_rank (device, optional: all or none)
 *             the union outputs of moe_build_union; written in dedup mode only
 *   y_slots [n][K][d], y_shared [n][S][d] (device f32, optional, 16-byte
 *             aligned): slot outputs; NULL keeps them in the workspace
 *   bytes     (device, optional) uint64 [2] as in the FFN calls
 *   ws        workspace of at least moe_workspace_size(shape, n, mode) bytes,
 *             zero-filled before its first use; the call leaves its counters
 *             zero.  Calls sharing a workspace must not overlap in time.
 * The launch fills the CUs its stream may use (one workgroup per CU; a
 * stream created with a CU mask gets one workgroup per CU of its mask) and
 * its workgroups wait for one another, so all of them must be resident at
 * once: do not run it beside other kernels that hold CUs (another stream's
 * one-launch pass, or collective kernels on another stream); the chain of
 * entry points above has no such waits and gives the same results.  If a
 * workgroup cannot start, the others' bounded waits give up and record
 * MOE_ERR_TIMEOUT instead of hanging; the outputs are then unspecified.  A
 * wait gives up after 2^21 polls (about a second), or after the number of
 * polls in the 32-bit workspace word at byte 192 when that word is nonzero
 * and smaller (moe_workspace_init leaves it zero).
 * Errors: MOE_ERR_ARG / _UNSUPPORTED / _WORKSPACE on the host; a bounded
 * device wait that gives up records MOE_ERR_TIMEOUT (moe_get_error). */
moe_status moe_verify_layer(const moe_shape* shape, const moe_weights* w, const float* logits,
                            const void* x, int32_t n, int32_t mode, void* out, int32_t out_dtype,
                            int32_t* ids, float* gates, int32_t* U, int32_t* union_ids,
                            int32_t* offsets, int32_t* perm, int32_t* slot_rank, float* y_slots,
                            float* y_shared, uint64_t* bytes, void* ws, size_t ws_bytes,
                            moe_stream_t stream);

/* moe_verify_layer without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The control block, hand-over flags,
 * intermediate activations and any slot outputs the caller does not keep
 * live in a static device array of 16 MiB that every GPU the library runs on
 * holds until the process ends; the call itself allocates nothing.
 *   Arguments, outputs and results as moe_verify_layer (same kernels, the
 *   same results bit for bit), less ws and ws_bytes.
 *   Limit: passes whose moe_verify_layer workspace need (control block and
 *   flags 33,024 B, H n(K+S)f*4 B, plus n*K*d*4 B when y_slots is NULL and
 *   n*S*d*4 B when y_shared is NULL, each rounded up to 256 B) exceeds
 *   16 MiB return MOE_ERR_TOO_LARGE before anything is enqueued.
 *   Set-up: the first call on a device looks up that device's copy of the
 *   array and clears its control block and flags with a kernel enqueued on
 *   `stream` ahead of the pass.
 *   Sharing: every call on one GPU uses the same array, which keeps the last
 *   call's contents; calls that overlap in time on one GPU (different
 *   streams, or graphs replayed concurrently) race and give unspecified
 *   results.  Device faults are recorded in the array's error word, which
 *   moe_get_error(NULL, stream) reads and clears.
 * Errors: as moe_verify_layer, plus MOE_ERR_TOO_LARGE. */
moe_status moe_verify_layer_noalloc(const moe_shape* shape, const moe_weights* w,
                                    const float* logits, const void* x, int32_t n, int32_t mode,
                                    void* out, int32_t out_dtype, int32_t* ids, float* gates,
                                    int32_t* U, int32_t* union_ids, int32_t* offsets,
                                    int32_t* perm, int32_t* slot_rank, float* y_slots,
                                    float* y_shared, uint64_t* bytes, moe_stream_t stream);

/* moe_verify_layer in deduplicating mode with a per-layer expert budget:
 * the route and union, then moe_expert_budget(C, renorm) on them, the
 * deduplicating FFN over the kept experts and the combine with the budgeted
 * gates, with the same results bit for bit as that chain of calls.  gates
 * (when given) receives the budgeted gates, the union outputs the budgeted
 * union, y_slots zero rows for the dropped slots, bytes[0] (min(U, C) + S) b.
 * Other arguments as moe_verify_layer.  Errors: MOE_ERR_ARG for C < 1 or
 * renorm not 0 or 1, otherwise as moe_verify_layer. */
moe_status moe_verify_layer_budget(const moe_shape* shape, const moe_weights* w,
                                   const float* logits, const void* x, int32_t n, int32_t C,
                                   int32_t renorm, void* out, int32_t out_dtype, int32_t* ids,
                                   float* gates, int32_t* U, int32_t* union_ids, int32_t* offsets,
                                   int32_t* perm, int32_t* slot_rank, float* y_slots,
                                   float* y_shared, uint64_t* bytes, void* ws, size_t ws_bytes,
                                   moe_stream_t stream);

/* moe_verify_layer with the mode chosen on the device for each pass: the
 * pass deduplicates iff its byte share (U + S) / (n (K + S)) is below r, the
 * ratio beta_dedup / beta_slot of the two kernels' effective bandwidths
 * measured at this n (the expert-bytes page, Eq. (7) and Table 1: r and u as
 * ratios of sums).  U is the pass's own union, counted on the device, so no
 * host round trip decides the mode.  r = 0 always runs per-slot, r > 1 always
 * deduplicates (u <= 1).
 *   mode_out  (device, optional) int32 [1]: the moe_mode the pass ran
 *   bytes     (device, optional) uint64 [2]: [0] bytes the chosen mode
 *             streamed, [1] n (K + S) b
 * Other arguments as moe_verify_layer (no routing or union outputs; the slot
 * outputs stay in the workspace).  Errors: MOE_ERR_ARG for r negative or not
 * finite, otherwise as moe_verify_layer. */
moe_status moe_verify_layer_auto(const moe_shape* shape, const moe_weights* w,
                                 const float* logits, const void* x, int32_t n, float r,
                                 void* out, int32_t out_dtype, int32_t* mode_out,
                                 uint64_t* bytes, void* ws, size_t ws_bytes,
                                 moe_stream_t stream);

/* EVICT utility-guided truncation of a draft tree, ahead of its verify pass
 * ("Making Every Verified Token Count: Adaptive Verification for MoE
 * Speculative Decoding", Sec. 3.1-3.2, Eqs. (7)-(10)).
 *   parent   (device) int32 [N]: parent node of v, parent[v] < v (breadth-first
 *            order); -1 for a child of the root token
 *   q        (device) f32 [N]: draft probability of v given its parent, in [0, 1]
 *   cost     (device) f32 [N]: cost[k-1] = C(k), the profiled latency of a step
 *            that verifies k nodes, > 0
 *   order    (device) int32 [N]: nodes by path score, descending (equal scores:
 *            lower index first); T_k = order[0..k) is ancestor-closed
 *   scores   (device, optional) f64 [N]: Score(v), the float64 product of q over
 *            the path, taken from the root outward
 *   expected (device, optional) f64 [N]: expected[k-1] = E_hat(T_k), prefix sums
 *            of the sorted scores
 *   k_best   (device) int32 [1]: k* = argmax_k E_hat(T_k) / C(k), the smallest k
 *            on equal utility; 0 when the tree is invalid
 *   ws       workspace (>= 256 bytes, 256-aligned) for the error word.
 * 1 <= N <= 1024.  Errors: MOE_ERR_ARG on the host; a parent outside [-1, v),
 * q outside [0, 1] or cost <= 0 records MOE_ERR_BAD_TREE (moe_get_error). */
moe_status moe_evict_select(const int32_t* parent, const float* q, const float* cost, int32_t N,
                            int32_t* order, double* scores, double* expected, int32_t* k_best,
                            void* ws, size_t ws_bytes, moe_stream_t stream);

/* EcoSpec cost-aware draft selection ("Less Experts, Faster Decoding:
 * Cost-Aware Speculative Decoding for Mixture-of-Experts", Sec. 4.2, Eqs.
 * (7)-(9), Algorithm 1): gamma times, score every unselected node by
 * P / (|path footprint \ B| + eps), select the best and add its path
 * footprint to the buffer B.
 *   parent, q  (device) as moe_evict_select (P = float64 product of q over the
 *              path, from the root out; q in [0, 1])
 *   pred       (device) uint64 [N][W]: predicted (layer, expert) set of each
 *              node as a bitset, bit l*E + e in word (l*E + e) / 64
 *   buffer0    (device, optional) uint64 [W]: experts already resident; NULL =
 *              empty
 *   selected   (device) int32 [gamma]: nodes in selection order (equal scores:
 *              the lower index, so every prefix is ancestor-closed)
 *   buffer_out (device, optional) uint64 [W]: the final buffer
 *   ws         workspace (>= 256 bytes, 256-aligned) for the error word.
 * 1 <= gamma <= N <= 1024, 1 <= W <= 256, N * W <= 8192, eps > 0.
 * Errors: MOE_ERR_ARG / _UNSUPPORTED (N * W) on the host; an invalid tree or
 * probability records MOE_ERR_BAD_TREE. */
moe_status moe_ecospec_select(const int32_t* parent, const float* q, const uint64_t* pred,
                              const uint64_t* buffer0, int32_t N, int32_t W, int32_t gamma,
                              double eps, int32_t* selected, uint64_t* buffer_out, void* ws,
                              size_t ws_bytes, moe_stream_t stream);

/* Offline Bellman policy of draft lengths over a reference sequence ("The
 * Limits of Speculation: Bounding Speculative Decoding in MoE", Sec. 4.1-4.3,
 * Eqs. (7)-(8)): from position i a step drafts k tokens (1 <= k <= L),
 * accepts a of them with P(a | k) = (prod_{j<a} p_j)(1 - p_a) (a < k) or
 * prod_{j<k} p_j (a = k), costs Cost(i, k, a) and moves to min(i + a + 1, N);
 *   dp[i] = min_k sum_{a=0..k} P(a | k) (Cost(i, k, a) + dp[min(i + a + 1, N)]),
 * dp[N] = 0, by backward induction.
 *   q      (device) f64 [N]: q[m] = the draft model's probability of reference
 *          token m + 1 given the prefix up to m, in [0, 1]; p_j at position i
 *          is q[i + j], and 0 past the end of the sequence
 *   cost   (device) f64 [N][L][L+1]: cost[i][k-1][a] = Cost(i, k, a), finite
 *   dp     (device) f64 [N+1]: minimum expected remaining cost from each position
 *   k_best (device) int32 [N]: the minimising draft length (equal expected
 *          costs: the shorter draft)
 *   ws     workspace (>= 256 bytes, 256-aligned) for the error word.
 * Each product and sum is one float64 operation, in the equations' order (j
 * and a ascending), so results are deterministic.  1 <= N <= 2^22,
 * 1 <= L <= 32.  Errors: MOE_ERR_ARG on the host; q outside [0, 1] or a
 * non-finite cost records MOE_ERR_BAD_TREE (moe_get_error). */
moe_status moe_bellman_policy(const double* q, const double* cost, int32_t N, int32_t L,
                              double* dp, int32_t* k_best, void* ws, size_t ws_bytes,
                              moe_stream_t stream);

/* One-time layout transform of expert weights into the layouts above
 * (untimed set-up, not part of a verify pass).  The source layout is the
 * d x f / f x d matrices of the SwiGLU expert stored row by row (input
 * feature first), as a caller holding W_gate, W_up [E][d][f] and W_down
 * [E][f][d] has them:
 *   src_gate, src_up (device) [count][d][f];  src_down (device) [count][f][d]
 *   src_s_gate, src_s_up (device, fp8 only) f32 [count][d/128][f/128];
 *   src_s_down (device, fp8 only) f32 [count][f/128][d/128]
 * and the outputs are the library's layouts (one row per output feature):
 *   dst_gate, dst_up [count][f][d];  dst_down [count][d][f];  fp8 scales
 *   dst_s_gate, dst_s_up [count][f/128][d/128], dst_s_down [count][d/128][f/128]
 * Every element (and every block scale) is copied bit for bit.  count is E
 * for the routed experts or S for the shared ones (1 <= count <= 256);
 * elements are of shape->w_dtype; the caller allocates every buffer and
 * sources and destinations must not overlap.  The scale arguments are read
 * only for fp8 weights.
 * Errors: MOE_ERR_ARG (pointers, count, a destination equal to its source),
 * MOE_ERR_UNSUPPORTED (dtype, d or f), MOE_ERR_HIP. */
moe_status moe_pack_weights(const moe_shape* shape, int32_t count, const void* src_gate,
                            const void* src_up, const void* src_down, const float* src_s_gate,
                            const float* src_s_up, const float* src_s_down, void* dst_gate,
                            void* dst_up, void* dst_down, float* dst_s_gate, float* dst_s_up,
                            float* dst_s_down, moe_stream_t stream);

/* Bytes of workspace any FFN or layer call needs for passes of up to n_max
 * tokens (0 for an invalid shape). */
size_t moe_workspace_size(const moe_shape* shape, int32_t n_max, int32_t mode);

/* Zero-fill a workspace on `stream` (with a kernel, never a memset node). */
moe_status moe_workspace_init(void* ws, size_t ws_bytes, moe_stream_t stream);

/* Host-only: b = bytes of one expert; union = (U + S) * b, requested =
 * n * (K + S) * b (the expert-bytes page, Fig. 2 and Table 1).  Either output
 * pointer (host) may be NULL.  Errors: MOE_ERR_ARG / _UNSUPPORTED. */
moe_status moe_byte_counts(const moe_shape* shape, int32_t n, int32_t U,
                           uint64_t* union_bytes, uint64_t* requested_bytes);

/* Synchronizes `stream`, then returns and clears the device error word kept
 * at the start of `ws`: MOE_OK, MOE_ERR_BAD_IDS, MOE_ERR_BAD_TREE or
 * MOE_ERR_TIMEOUT.  ws = NULL reads the error word of the current device's
 * moe_verify_layer_noalloc scratch (MOE_OK if no such call ran there). */
moe_status moe_get_error(void* ws, moe_stream_t stream);

/* Diagnostic, host-only: the unit partition the one-launch pass uses for one
 * phase, computed with the same code on the host.  counts[ng] (host) are the
 * tokens of each group (0..32); tile = 0 splits the ng * upg units evenly
 * over `grid` workgroups, tile = 8, 16 or 32 splits them by the cost a unit
 * of a group of that many tokens has with that token tile (up != 0: the UP
 * phase, else DOWN), as deduplicating passes of more than 8 tokens do.
 * Outputs (host): first_unit[grid + 1], workgroup c owning units
 * [first_unit[c], first_unit[c + 1]); optionally owner_lo[ng], owner_hi[ng],
 * the first and last workgroup owning a unit of each group, as the DOWN
 * phase's waits compute them (both NULL or both set).  upg = units per
 * group, 1..16384; grid 1..4096; ng 1..264.  Errors: MOE_ERR_ARG. */
moe_status moe_unit_partition(const int32_t* counts, int32_t ng, int32_t tile, int32_t up,
                              int32_t upg, int32_t grid, int64_t* first_unit, int32_t* owner_lo,
                              int32_t* owner_hi);

/* Diagnostic: decode `count` E4M3FN codes (device) to f32 (device) with the
 * same conversion the fp8 FFN kernels use. */
moe_status moe_decode_fp8(const uint8_t* codes, float* out, int64_t count,
                          moe_stream_t stream);

/* The hipError_t behind this thread's most recent MOE_ERR_HIP, and its text. */
int32_t moe_last_hip_error(void);
const char* moe_hip_error_string(void);

const char* moe_status_str(int32_t status);
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_VERIFY_H */
