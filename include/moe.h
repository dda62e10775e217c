/*
 * moe.h — C ABI of the batch-invariant MoE layer forward pass for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer: router scoring + top-k (or fixed hash routing), dispatch
 * (token permutation by expert), a grouped SwiGLU expert FFN over the routed
 * (token, expert) rows plus one always-on shared expert, and a weighted
 * combine.  Sources (web pages, cited by title and section):
 *   [DS] "6 基建与训练稳定性优化" — DeepSeek-V4 infrastructure walkthrough
 *        (liyongzhi.xyz, deepseek_v4 sections/06-infra): 6.1 dispatch ->
 *        compute -> combine; 6.2 FP4 (E2M1) expert weights with block scales;
 *        6.3 learned routing (scores = W h, top-k) and hash routing
 *        (expert = hash(token id) mod E); 6.5 SwiGLU = SiLU(W_g x) * (W_v x).
 *   [FW] "MoE 模型中的訓練與推論一致性：數值漂移發生之處" — Fireworks AI post
 *        on MoE train/inference parity: floating-point addition is not
 *        associative; the MoE finalize is a per-token weighted sum of the
 *        top-k expert outputs, followed by += shared expert (trap 3); keep the
 *        k contributions in fp32 and cast once (Qwen3.5-MoE case study);
 *        per-fusion control flags (lessons).
 *   [MT] "美团把训练和推理的概率做到逐位相同:分歧藏在一个加法顺序里" — bitwise
 *        parity needs every GEMM to see its full K (no split sums).
 *   [LD] feedbbs.com/linuxdo/72580 — shared experts see every token and are
 *        added to the weighted routed sum (section 共享专家); GLU gate/up
 *        branches (section on GLU); token dropping makes outputs depend on the
 *        batch (section on output determinism) — this library never drops.
 *   [V4] nxmr.cn/news/146660 section 2.2 — the router is a small linear layer
 *        producing E logits, softmax weights, top-k.
 *
 * Determinism contract: for fixed inputs every output row is bitwise
 * identical for any batch size T, any batch composition or order, any stream
 * and any repeat.  Routing keys use a fixed fp32 accumulation order and a
 * library-defined exp (below); the expert GEMMs use one MFMA instruction shape
 * and one K order for every T, K is never split across workgroups, and no
 * floating-point atomics are used anywhere.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers owned by the caller (plain device memory,
 *     16-byte aligned).  The library never allocates or frees memory and keeps
 *     no state except a thread-local error message.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *     call only enqueues kernels on that stream: no host synchronisation and
 *     no host<->device copies.
 *   - All arguments are validated on the host before anything is enqueued.  On
 *     error nothing is launched, outputs are untouched, and a negative
 *     moe_status is returned; moe_last_error() describes it.  Launch failures
 *     map to MOE_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Activations/outputs are row-major [rows, cols]; weights are [out, in]
 *     with the reduction dimension contiguous (as nn.Linear).
 *   - Unchecked preconditions: inputs are finite (non-finite values give
 *     unspecified but deterministic results); E8M0 scale bytes are <= 252
 *     (dequantised values stay finite in bf16); topk_idx values handed to
 *     moe_permute / moe_combine are in [0, E) and distinct per token.
 *   - Limits: 1 <= k <= 32, k <= E <= 1024, T >= 0 (T = 0 is a no-op),
 *     D, I, I_shared multiples of 32 and >= 32.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32

/* flags of moe_grouped_swiglu and moe_layer_forward: the gated activation of
 * every expert FFN the call runs (routed and shared experts alike).  0 is
 * SwiGLU, SiLU(g) * u with g = W_g x, u = W_u x.  At most one of:
 *   MOE_FLAG_GLU_CLAMP  the clamped SwiGLU of [DS] 6.5: g is capped from above
 *                       at 10 and u clamped to [-10, 10], then SiLU(g) * u;
 *   MOE_FLAG_GLU_SITU   SiTU-GLU ([LD], section SiTU-GLU):
 *                       [4 tanh(g / 4) * sigmoid(g)] * [25 tanh(u / 25)].
 * Both act on the fp32 GEMM results before the one rounding of h, per element
 * and the same for every T, so the determinism contract below is unchanged.
 * Both bits together, or any other bit, give MOE_ERR_UNSUPPORTED. */
#define MOE_FLAG_GLU_CLAMP 0x1u
#define MOE_FLAG_GLU_SITU 0x2u
/* moe_layer_forward only: the routed experts (MXFP4 weights) run FP4 x FP8,
 * as moe_grouped_swiglu_w4a8 describes (x quantised to MXFP8 once per token,
 * h per routed row); a shared expert must then be bf16 and keeps its bf16
 * path.  Needs bf16 activations and D, I multiples of 128.
 * moe_layer_workspace_bytes with w = MOE_MXFP4 covers this flag. */
#define MOE_FLAG_W4A8 0x4u

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  MOE_ERR_DTYPE = -3,       /* unsupported dtype combination */
  MOE_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required */
  MOE_ERR_UNSUPPORTED = -6, /* valid request that the library does not implement */
  MOE_ERR_HIP = -7          /* a HIP launch failed */
} moe_status;

/* MOE_MXFP4 is a weight format only: E2M1 codes packed two per byte (element
 * 2i in the low nibble) [rows, cols/2] plus one E8M0 scale byte per 32
 * consecutive elements along the reduction axis [rows, cols/32]; value =
 * e2m1(code) * 2^(scale - 127) (OCP Microscaling v1.0; [DS] 6.2). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP4 = 2 } moe_dtype;

typedef enum { MOE_ROUTE_SOFTMAX = 0, MOE_ROUTE_SIGMOID = 1, MOE_ROUTE_HASH = 2 } moe_route;

/* Expert weights of G experts (G = E routed, or 1 shared), each row-major:
 *   gate, up: [G, I, D]   down: [G, D, I]
 * MOE_MXFP4: gate/up/down hold packed codes ([G, I, D/2], [G, D, I/2]) and
 * gate_scale/up_scale [G, I, D/32], down_scale [G, D, I/32] hold E8M0 bytes;
 * the scale pointers must be NULL for other dtypes.
 * dtype must equal the activation dtype, except that MOE_MXFP4 weights go
 * with MOE_BF16 activations. */
typedef struct {
  const void* gate;
  const void* up;
  const void* down;
  const uint8_t* gate_scale;
  const uint8_t* up_scale;
  const uint8_t* down_scale;
  moe_dtype dtype;
} moe_expert_weights;

/* ---------------------------------------------------------------------------
 * moe_router_topk — routing ([DS] 6.3 learned routing and hash routing; [V4]
 * 2.2 linear router + softmax + top-k).
 *
 *  x [T, D] (act = MOE_F32 or MOE_BF16), w_router [E, D] (same dtype),
 *  bias [E] fp32 or NULL (= 0).  Outputs topk_idx [T, k] int32 in rank order
 *  and topk_w [T, k] fp32.
 *
 *  Logits: L[t,e] = sum_d x[t,d] w[e,d] in fp32 with this fixed order: 64
 *  partial sums start at +0; element d is added with fmaf to partial
 *  (d/8) mod 64, d increasing; then partial[j] += partial[j+m] for
 *  m = 32, 16, 8, 4, 2, 1 (a pairwise tree); L = partial[0].
 *  exp is this library's routing exp: n = rint(x*fp32(log2 e)),
 *  r = fma(-n, fp32(ln2), x), r = fma(-n, fp32(ln2 - fp32(ln2)), r),
 *  p = degree-7 Taylor polynomial with fp32(1/j!) coefficients by Horner with
 *  fma, result p * 2^n (two exact scalings outside the normal range);
 *  x > 89 -> +inf, x < -104 -> +0.
 *   MOE_ROUTE_SOFTMAX: key = L (+ bias); w_j = exp(L_j - L_max) / Z, L_max the
 *                      largest logit among the k selected experts.
 *   MOE_ROUTE_SIGMOID: s = 1/(1 + exp(-L)) (IEEE division), key = s (+ bias);
 *                      w_j = s_j / Z.  The bias only decides selection.
 *   Z sums the selected terms in ascending expert id, in fp32, from +0.
 *  Selection: the k largest keys, ties to the lower expert id (+0 == -0).
 *   MOE_ROUTE_HASH: x, w_router, bias unused (may be NULL); token_ids [T]
 *                   int32 required.  Slot j takes
 *                   fmix32(tid + j*0x9E3779B9 mod 2^32) mod E (MurmurHash3
 *                   finaliser), stepping to (c+1) mod E past experts already
 *                   taken; w = 1/k; topk_idx is in slot order.
 *  workspace: moe_router_workspace_bytes(T, E) bytes (logits); may be NULL
 *  when that is 0 (hash routing).
 * ------------------------------------------------------------------------- */
size_t moe_router_workspace_bytes(int64_t T, int E, moe_route mode);
int moe_router_topk(const void* x, moe_dtype act, const void* w_router, const float* bias,
                    const int32_t* token_ids, int64_t T, int D, int E, int k, moe_route mode,
                    int32_t* topk_idx, float* topk_w, void* workspace, size_t workspace_bytes,
                    void* stream);

/* moe_routing_scores — the routing scores of the selection step, element by
 * element, bit-identical to what moe_router_topk uses: MOE_ROUTE_SIGMOID gives
 * 1/(1 + exp(-l)), MOE_ROUTE_SOFTMAX gives exp(l) (the routing exp above).
 * logits, out: [n] fp32.  For callers that log or reuse router probabilities. */
int moe_routing_scores(const float* logits, int64_t n, moe_route mode, float* out, void* stream);

/* ---------------------------------------------------------------------------
 * moe_permute — dispatch ([DS] 6.1: tokens go to their experts): the stable
 * counting sort of the T*k (token, slot) pairs by expert id.
 *
 *  expert_counts [E]: rows per expert; expert_offsets [E+1]: exclusive prefix
 *  sum (expert_offsets[E] = T*k); row_token [T*k]: token of each permuted row
 *  (rows of one expert in ascending token order); pair_row [T*k]: permuted row
 *  of pair (t, j), index t*k + j.  No capacity limit, no dropping.
 *  If x is not NULL, also gathers x_perm[r] = x[row_token[r]] ([T*k, D], act).
 *  workspace: moe_permute_workspace_bytes(T, E) bytes.
 * ------------------------------------------------------------------------- */
size_t moe_permute_workspace_bytes(int64_t T, int E);
int moe_permute(const int32_t* topk_idx, int64_t T, int k, int E, int32_t* expert_counts,
                int32_t* expert_offsets, int32_t* row_token, int32_t* pair_row, const void* x,
                moe_dtype act, int D, void* x_perm, void* workspace, size_t workspace_bytes,
                void* stream);

/* ---------------------------------------------------------------------------
 * moe_grouped_swiglu — expert compute ([DS] 6.5 SwiGLU; [LD] GLU branches):
 * for every row r of expert e (expert_offsets[e] <= r < expert_offsets[e+1]),
 *   g = W_gate[e] a_r, u = W_up[e] a_r        (fp32 accumulation, full K = D)
 *   h = round(silu(g) * u),  silu(g) = g / (1 + e^-g)
 *       (or the activation that flags select: MOE_FLAG_GLU_CLAMP / _SITU)
 *   out[r] = round(W_down[e] h)               (fp32 accumulation, full K = I)
 * where a_r = x_rows[row_index[r]] if row_index is not NULL, else x_rows[r],
 * and round() is bf16 round-to-nearest-even (bf16/MXFP4 weights) or the fp32
 * value itself (fp32).  MXFP4 weights are decoded exactly to bf16 first, so
 * their result equals the bf16 path on the decoded weights bit for bit.
 * Rows of one expert never interact: each row's output is independent of the
 * other rows and of their number.
 *  R: number of rows (= expert_offsets[E]); for a shared expert pass E = 1 and
 *  expert_offsets = {0, T}.  flags: 0, MOE_FLAG_GLU_CLAMP or MOE_FLAG_GLU_SITU.
 *  row_index entries must be valid rows of x_rows (they are not checked).
 *  workspace: moe_grouped_swiglu_workspace_bytes(R, E, D, I, act) bytes
 *  (h rows, and the tile tables that the call writes from expert_offsets).
 * ------------------------------------------------------------------------- */
size_t moe_grouped_swiglu_workspace_bytes(int64_t R, int E, int D, int I, moe_dtype act);
int moe_grouped_swiglu(const void* x_rows, const int32_t* row_index,
                       const int32_t* expert_offsets, int64_t R, int E, int D, int I,
                       const moe_expert_weights* w, moe_dtype act, uint32_t flags, void* out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * FP4 x FP8 expert compute (W4A8; [DS] 6.2: FP4 expert weights run in an FP8
 * GEMM).  The page does not say how activations become FP8; the reading here
 * is OCP MX: E4M3 elements (OCP FP8, bias 7, no infinities, largest 448) with
 * one E8M0 scale per 32 consecutive values along K:
 *   X = floor(log2(max |v| over the block's finite values)) - 8, scale byte
 *   X + 127 clamped to [0, 254] (byte 0 when the block has no finite nonzero
 *   value); element = the E4M3 code nearest to v / 2^X, ties to the even
 *   code, magnitudes past 448 clamped to 448 with their sign, NaN -> 0x7F.
 *
 * moe_mx_e4m3_quantize: R bf16 rows of K (K % 32 == 0) -> codes [R, K] u8 and
 *   scales [R, K/32] u8; row r reads x[row_index[r]] (row_index NULL: x[r]).
 *   x 16-byte aligned, codes 8-byte aligned.
 *
 * moe_grouped_swiglu_w4a8: moe_grouped_swiglu with MXFP4 weights and MXFP8
 *   activations.  The rows x_rows[row_index[r]] are quantised per 32 along D,
 *   the gate/up GEMM runs on gfx950's scaled FP4 x FP8 MFMA (both block scales
 *   applied in the instruction, fp32 accumulation, K stepped by 128 in
 *   increasing order from 0 for every row), h = round_bf16(glu(g, u)) is
 *   quantised per 32 along I, and the down GEMM gives out = round_bf16(W_down h).
 *   Every output row depends only on its own input row, whatever R or E.
 *   w: MXFP4 (codes + scales); x_rows, out bf16.  D and I multiples of 128.
 *   flags: 0, MOE_FLAG_GLU_CLAMP or MOE_FLAG_GLU_SITU.
 *   workspace: moe_grouped_swiglu_w4a8_workspace_bytes(R, E, D, I) bytes.
 * ------------------------------------------------------------------------- */
int moe_mx_e4m3_quantize(const void* x, const int32_t* row_index, int64_t R, int K,
                         uint8_t* codes, uint8_t* scales, void* stream);
size_t moe_grouped_swiglu_w4a8_workspace_bytes(int64_t R, int E, int D, int I);
int moe_grouped_swiglu_w4a8(const void* x_rows, const int32_t* row_index,
                            const int32_t* expert_offsets, int64_t R, int E, int D, int I,
                            const moe_expert_weights* w, uint32_t flags, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_combine — the MoE finalize ([FW] trap 3 and case study):
 *   acc = +0; for each of token t's experts in ascending expert id:
 *       acc = fmaf(topk_w[t,j], float(expert_out[pair_row[t*k+j]]), acc)
 *   if shared_out: acc = acc + float(shared_out[t])
 *   y[t] = round(acc)       (bf16 RNE, or fp32 as is)
 *  expert_out [T*k, D], shared_out [T, D] or NULL, y [T, D], all act dtype.
 * ------------------------------------------------------------------------- */
int moe_combine(const void* expert_out, const int32_t* topk_idx, const float* topk_w,
                const int32_t* pair_row, const void* shared_out, int64_t T, int k, int D,
                moe_dtype act, void* y, void* stream);

/* ---------------------------------------------------------------------------
 * moe_residual_rmsnorm — the residual add and RMSNorm of the next block's
 * input, the last kernel of the unfused MoE tail ([FW] trap 3:
 * rmsnorm(out + residual)); RMSNorm as [LD] defines it (section "RMSNorm
 * before up-projection"), g * h / sqrt(mean(h^2) + eps):
 *   h[t] = round(x[t] + residual[t])                  -> residual_out[t]
 *   ss = sum over d of h[t,d]^2                        (fp32, order below)
 *   normed[t,d] = round(gamma[d] * (h[t,d] * (1 / sqrt(ss / D + eps))))
 * round() is bf16 RNE (bf16) or the fp32 value itself; the norm sees the
 * rounded residual.  Order of ss, the same for every T and for both entry
 * points ([FW] trap 2: the norm's reduction tree must not follow the launch
 * layout): 1024 partials, partial p sums h[d]^2 with fmaf from +0 over the
 * 8-feature chunks c = d/8 with c % 1024 == p, in increasing d; then
 * p += p + m for m = 512, 256, ..., 1; the division, square root and
 * reciprocal are IEEE fp32.
 *  x, residual, residual_out, normed [T, D]; gamma [D]; all act dtype.
 *  residual_out may be residual itself (in place); no other overlap.
 *  D: a positive multiple of 32.  eps: finite and >= 0 (else
 *  MOE_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------- */
int moe_residual_rmsnorm(const void* x, const void* residual, const void* gamma, float eps,
                         int64_t T, int D, moe_dtype act, void* residual_out, void* normed,
                         void* stream);

/* ---------------------------------------------------------------------------
 * moe_combine_rmsnorm — moe_combine fused with moe_residual_rmsnorm of its
 * output (the finalize + next-RMSNorm fusion of [FW] trap 3, without the
 * all-reduce): the bits of moe_combine into y followed by
 * moe_residual_rmsnorm(y, residual, ...), without writing or reading y.
 * Arguments as in those two calls.
 * ------------------------------------------------------------------------- */
int moe_combine_rmsnorm(const void* expert_out, const int32_t* topk_idx, const float* topk_w,
                        const int32_t* pair_row, const void* shared_out, const void* residual,
                        const void* gamma, float eps, int64_t T, int k, int D, moe_dtype act,
                        void* residual_out, void* normed, void* stream);

/* ---------------------------------------------------------------------------
 * moe_layer_forward — the whole layer: route, permute, grouped SwiGLU over the
 * routed rows and the shared expert (one launch for both), combine.  y [T, D].
 * The residual connection is not part of the layer.
 *  routed: E experts; shared: NULL (no shared expert, I_shared ignored) or one
 *  expert with inter dim I_shared (bf16 when routed weights are MXFP4).
 *  flags: 0, MOE_FLAG_GLU_CLAMP or MOE_FLAG_GLU_SITU (the gated activation of
 *  the routed and the shared experts), optionally | MOE_FLAG_W4A8.
 *  workspace: moe_layer_workspace_bytes(...) bytes.
 * ------------------------------------------------------------------------- */
size_t moe_layer_workspace_bytes(int64_t T, int D, int E, int k, int I, int I_shared,
                                 moe_dtype act, moe_dtype w);
int moe_layer_forward(const void* x, const int32_t* token_ids, const void* w_router,
                      const float* bias, const moe_expert_weights* routed,
                      const moe_expert_weights* shared, int64_t T, int D, int E, int k, int I,
                      int I_shared, moe_route mode, moe_dtype act, uint32_t flags, void* y,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_layer_forward_fused — the whole layer in ONE kernel launch ([DS] 6.1:
 * dispatch, expert compute and combine fused into one kernel whose experts
 * are processed in waves).  Same arguments, results and bits as
 * moe_layer_forward: every step runs the same fixed chains (router order,
 * top-k, counting sort, one MFMA chain per GEMM output, fixed-order combine);
 * only the GEMM tile shapes may differ, which changes no bit.
 *  The launch's workgroups draw the layer's steps as tasks from one ordered
 *  queue (router logits, shared-expert gate/up, top-k, permutation, routed
 *  gate/up, shared down, routed down, combine); a task waits only for whole
 *  earlier phases, so the shared expert's gate/up overlaps the routing and no
 *  kernel boundary separates the steps.
 *  Limits: act = MOE_BF16; routed weights MOE_BF16 or MOE_MXFP4; the shared
 *  expert (if any) MOE_BF16; flags 0, MOE_FLAG_GLU_CLAMP or MOE_FLAG_GLU_SITU
 *  (MOE_FLAG_W4A8 gives MOE_ERR_UNSUPPORTED).
 *  workspace: moe_layer_fused_workspace_bytes(...) bytes, 256-byte aligned.
 *  Its first 256 bytes hold the task queue's state: they must be zero before
 *  the first call on that workspace (e.g. the workspace allocated zeroed),
 *  and every call leaves them zero again.  The 32-bit word at byte offset 8 is
 *  a sticky error flag: nonzero if a wait inside a call gave up (a bounded
 *  spin; the outputs of that call are then undefined).  Calls that share a
 *  workspace must be ordered (one stream).
 * ------------------------------------------------------------------------- */
size_t moe_layer_fused_workspace_bytes(int64_t T, int D, int E, int k, int I, int I_shared);
int moe_layer_forward_fused(const void* x, const int32_t* token_ids, const void* w_router,
                            const float* bias, const moe_expert_weights* routed,
                            const moe_expert_weights* shared, int64_t T, int D, int E, int k,
                            int I, int I_shared, moe_route mode, moe_dtype act, uint32_t flags,
                            void* y, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_layer_forward_noalloc — moe_layer_forward for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The caller passes inputs and outputs only;
 * the workspace is a scratch array of MOE_NOALLOC_SCRATCH_BYTES that the
 * library holds in device memory, one copy per GPU, kept until the process
 * ends.  Arguments, results and bits are those of moe_layer_forward (the
 * same kernels).  The call allocates nothing and calls no allocating library
 * routine; its first call on a device looks up that device's scratch address.
 *  Limit: moe_layer_workspace_bytes(T, D, E, k, I, I_shared, act, routed
 *  dtype) must not exceed MOE_NOALLOC_SCRATCH_BYTES (64 MiB: decode batches of
 *  a D = 7168, E = 256, k = 8, I = 2048 layer up to a few hundred tokens);
 *  larger layers get MOE_ERR_WORKSPACE before anything is launched.
 *  Every call on one GPU uses the same scratch, which keeps the last call's
 *  contents (each call writes what it reads first).  Calls that overlap on
 *  one GPU (two streams, or two host threads without ordering) race on it:
 *  order them on one stream.
 * ------------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_layer_forward_noalloc(const void* x, const int32_t* token_ids, const void* w_router,
                              const float* bias, const moe_expert_weights* routed,
                              const moe_expert_weights* shared, int64_t T, int D, int E, int k,
                              int I, int I_shared, moe_route mode, moe_dtype act,
                              uint32_t flags, void* y, void* stream);

/* ---------------------------------------------------------------------------
 * Stage timing (measurement only).  When set, the next moe_layer_forward
 * calls on this host thread record events[0] before the first kernel and
 * events[i+1] after stage i on the call's stream; stages: 0 routing,
 * 1 permutation, 2 gate/up SwiGLU GEMM, 3 down GEMM, 4 combine
 * (MOE_STAGE_EVENTS events).  With MOE_STAGE_EVENTS + MOE_KERNEL_EVENTS events,
 * events[6] / events[7] also mark the start / end of the gate/up GEMM kernel
 * itself and events[8] / events[9] those of the down GEMM kernel (kernel time
 * without the launch gaps the stage events include; hipExtLaunchKernel).
 * The events are hipEvent_t handles created by the caller; pass NULL / 0 to
 * stop recording.
 * ------------------------------------------------------------------------- */
#define MOE_STAGE_EVENTS 6
#define MOE_KERNEL_EVENTS 4
int moe_set_stage_events(void* const* events, int n_events);

const char* moe_status_string(int status);
const char* moe_last_error(void); /* thread-local message of the last non-OK return */
int moe_abi_version(void);
/* Identifier of the sources this binary was built from (16 hex digits of a
 * hash over the kernel and host sources, this header and the build flags),
 * so that a caller can refuse a binary built from other sources. */
const char* moe_build_id(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
