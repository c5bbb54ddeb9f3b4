/*
 * moe_experts.h — C ABI of the MI355X (gfx950) MoE experts library.
 *
 * The library runs the experts step of a mixture-of-experts layer on one GPU
 * (and, optionally, the router step before it, moe_route):
 * group the router's top-k slots by expert (histogram, prefix sum to segment
 * end offsets, stable permutation), a grouped GEMM for the gate and up
 * projections with the activation and route weight applied in its epilogue,
 * a grouped GEMM for the down projection, and a fixed-order combine back to
 * token order.
 *
 * Sources (vLLM API pages):
 *   - "vllm.model_executor.layers.fused_moe.experts.moonep_experts": module
 *     docstring (the three grouped GEMMs, route weight on the activation,
 *     empty segments skipped), MoonEPExperts.apply (cu_seqlens as int32
 *     cumulative end offsets, one per weight row; rows past the last end
 *     zero-filled), moonep_grouped_gemm ([G, N, K] weights, K contiguous).
 *   - "vllm.model_executor.layers.fused_moe.experts.flashinfer_moe_ep":
 *     module docstring (route on the top-k output, compute and combine in the
 *     experts step), FlashInferMoeEpExperts.apply (int32 ids, output written
 *     in place, not accumulated).
 *   - "vllm.model_executor.layers.fused_moe.experts.trtllm_mxfp4_moe":
 *     TrtLlmMxfp4ExpertsBase (MXFP4 weights with bf16 activations, SwiGLU-OAI
 *     with alpha / beta / clamp limit), workspace_shapes (output keeps the
 *     unpadded hidden size).
 *   - "vllm.models.deepseek_v4.nvidia.fi_moe": DeepseekV4MegaMoEExpertsFI
 *     (workspace allocated before the first forward so warm-up and capture
 *     never allocate; token capacity checked against a fixed maximum).
 *
 * Conventions for every entry point:
 *   - Pointers marked (device) are HIP device pointers; (host) are host.
 *   - bf16 tensors are raw 16-bit bfloat16 words, row-major, last dim contiguous.
 *   - Weights use the [E, N, K] layout: w_gate, w_up [E, I, H]; w_down [E, H, I].
 *     MXFP4 weights are packed e2m1 codes [E, N, K/2] (element 2i in the low
 *     nibble of byte i) with e8m0 scale bytes [E, N, K/32], one per 32
 *     consecutive K elements (OCP Microscaling v1.0).
 *   - The caller owns every buffer, including the workspace. The library never
 *     allocates, frees or synchronises inside a forward call: it only enqueues
 *     kernels on `stream` (a hipStream_t; NULL = the default stream). One
 *     exception to "on `stream`": the forwards of bf16 prefill problems run
 *     the kernels of their segments of at most 32 rows on a second stream
 *     that the library creates once per device (non-blocking, default
 *     priority), forked from `stream` and joined back into it with events
 *     inside the call, so that to the caller the work is ordered as if all
 *     of it ran on `stream`, and capturing `stream` into a HIP graph
 *     captures both. That stream is shared by all such calls on a device:
 *     it is correct across host threads but serialises their cold-segment
 *     kernels, and a capture on one thread must not overlap a bf16 prefill
 *     forward on another thread of the same device.
 *     moe_experts_forward_noalloc keeps everything on `stream`.
 *   - Inputs are read-only; outputs are overwritten.
 *   - Calls with distinct workspaces may run concurrently. Two calls in flight
 *     on one workspace race.
 *   - Return 0 on success or a negative moe_status. Host-side validation is
 *     O(1) and reads no device memory; a failing call enqueues nothing.
 *     Problems found on the device (bad expert ids, malformed cu_seqlens) are
 *     written to a status word in the workspace: read it with
 *     moe_device_error() after the stream has been synchronised.
 */
#ifndef MOE_EXPERTS_H
#define MOE_EXPERTS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* a hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,  /* null pointer, non-positive size, k > E, unknown enum, non-finite parameter */
  MOE_ENOTSUP = -2, /* valid but unsupported: H or I not a multiple of 64, E > 4096, limit <= 0, ... */
  MOE_ENOSPC = -3,  /* workspace smaller than the *_workspace_bytes() figure for this problem */
  MOE_EHIP = -4,    /* a HIP launch or query failed */
  MOE_ETIMEDOUT = -5 /* moe_device_error: a bounded wait inside the single-launch decode step
                        gave up (its results are invalid) */
} moe_status;

/* Weight format. trtllm_mxfp4_moe page, TrtLlmMxfp4ExpertsBase._supports_quant_scheme
 * (MXFP4 weights with unquantized activations); moonep_experts page (bf16). */
typedef enum { MOE_W_BF16 = 0, MOE_W_MXFP4 = 1 } moe_wfmt;

/* Activation. moonep_experts page, module docstring (silu(gate) * up);
 * trtllm_mxfp4_moe page, TrtLlmMxfp4ExpertsBase (SwiGLU-OAI with alpha, beta,
 * clamp limit). SwiGLU-OAI is read as
 *   g' = min(g, limit), u' = clamp(u, -limit, limit), f = g' * sigmoid(alpha g') * (u' + beta).
 * SiTu, as the same class's constructor comment gives it:
 *   f = alpha * tanh(g / alpha) * sigmoid(g) * beta * tanh(u / beta), alpha > 0, beta > 0. */
typedef enum { MOE_ACT_SILU = 0, MOE_ACT_SWIGLU_OAI = 1, MOE_ACT_SITU = 2 } moe_act;

/* Activation format of the GEMM inputs. trtllm_mxfp4_moe page,
 * TrtLlmMxfp4ExpertsBase._supports_quant_scheme: with MXFP4 weights the
 * activations are either unquantized or dynamically quantized MXFP8.
 *   MOE_A_BF16:  bf16 rows, carried exactly into the block-scaled MFMA (MXFP4
 *                weights) as two e4m3 parts per value.
 *   MOE_A_MXFP8: each GEMM input row (the token rows for GEMM1, the activation
 *                rows for GEMM2) is quantized per 32 values along K, OCP
 *                Microscaling v1.0 reading: scale 2^(floor(log2 amax) - 8), its
 *                e8m0 code clamped to [0, 254]; elements e4m3, round to nearest
 *                even, saturated at +-448. MXFP4 weights only (else MOE_ENOTSUP). */
typedef enum { MOE_A_BF16 = 0, MOE_A_MXFP8 = 1 } moe_afmt;

typedef struct {
  int32_t T;     /* tokens: rows of x and out (NvS for the pre-grouped entry) */
  int32_t H;     /* hidden size (K of GEMM1, N of GEMM2); multiple of 64 */
  int32_t I;     /* intermediate size (N of GEMM1, K of GEMM2); multiple of 64 */
  int32_t E;     /* experts, i.e. weight rows (segments incl. redundant slots for the pre-grouped entry) */
  int32_t k;     /* slots per token (ignored by the pre-grouped entry) */
  int32_t wfmt;  /* moe_wfmt */
  int32_t act;   /* moe_act */
  float alpha;   /* SwiGLU-OAI and SiTu */
  float beta;    /* SwiGLU-OAI and SiTu */
  float limit;   /* SwiGLU-OAI only; > 0, may be +inf */
  int32_t weight_on_input; /* 0: route weight multiplies the activation (default);
                              1: it multiplies the token's input row before GEMM1 (each
                              routed row x * w rounded to bf16) and the activation is
                              not weighted (moonep_experts page, MoonEPExperts.apply,
                              input-weighted top-1 routing). Costs one more read and
                              write of the routed rows. */
  int32_t a_fmt;           /* moe_afmt; 0 (bf16) when zero-initialised */
  /* Per-expert parameters (device float32 arrays of E values, 4-byte aligned;
   * NULL, the zero-initialised default, keeps the scalar above, or a scale
   * of 1, for every expert). trtllm_mxfp4_moe page, TrtLlmMxfp4ExpertsBase
   * constructor: the activation's alpha, beta and clamp limit are kept as
   * per-expert tensors; flashinfer_moe_ep page, epilogue_from_quant_config:
   * one weight global scale per expert becomes the fc1 alpha (multiplies the
   * gate and up products of that expert's rows, before the activation) and
   * the fc2 alpha (multiplies the down product). The library reads them on
   * the device at every call and does not validate them there: check them
   * once on the host with moe_check_expert_params. For the pre-grouped entry
   * the index is the segment (E = segments). */
  const float* alpha_e;
  const float* beta_e;
  const float* limit_e;
  const float* fc1_alpha;
  const float* fc2_alpha;
  /* MXFP4 weights: the weights in the prefill kernels' own format, written
   * by moe_mx_pack_weights from the same w_gate / w_up / w_down and scales
   * (device, 16-byte aligned), or NULL (the zero-initialised default).
   * flashinfer_moe_ep page, process_weights_after_loading: the weights are
   * put into the kernel's format once, before the first forward. When set,
   * the token-major MXFP4 x MXFP8 prefill path reads the weights from here
   * and skips the per-call transpose of their scales, and the
   * weight-streaming (decode) kernels of both entries read their codes from
   * here (each 16 rows x 128 K values are then one contiguous 1 KB, already
   * in MFMA operand order; results bitwise those of the canonical codes).
   * The canonical tensors are still required (the decode kernels read the
   * scales from them, and the single-launch decode step reads the codes
   * too). The library cannot tell a stale packing
   * from a fresh one: re-pack after changing the weights. Set with bf16
   * weights: MOE_EINVAL. */
  const void* mx_packed;
  /* bf16 weights: the same weights in the operand-block layout, written by
   * moe_bf16_pack_weights (device, 16-byte aligned), or NULL (the
   * zero-initialised default). flashinfer_moe_ep page,
   * process_weights_after_loading: the weights are put into the kernel's
   * format once, before the first forward. When set, the tiled and the
   * cold-segment prefill kernels (both entries) read the weights from here:
   * each 1 KB load is then one contiguous block in MFMA operand order; the
   * results are bitwise those of the row layout. The canonical tensors are
   * still required (the weight-streaming kernels of small problems read
   * them). Re-pack after changing the weights. Set with another weight
   * format: MOE_EINVAL. */
  const void* bf16_packed;
} moe_problem;

/* Byte offsets of the intermediates inside a forward workspace (for tests and
 * tools; the forward call does not need them). Fields not used by a path are 0. */
typedef struct {
  size_t status;     /* int32[4]: [0] bad expert ids / malformed offsets, [1] valid slots M */
  size_t counts;     /* int32[E]   rows per segment */
  size_t cu_seqlens; /* int32[E]   cumulative end offsets */
  size_t perm;       /* int32[T*k] sorted row -> flat slot t*k+j (first M entries) */
  size_t inv_perm;   /* int32[T*k] flat slot -> sorted row, -1 for masked / bad ids */
  size_t w_sorted;   /* float[T*k] route weight per sorted row */
  size_t act;        /* bf16 [T*k, I] activation rows in sorted order */
  size_t y;          /* bf16 [S, T*k, H] down-projection rows in sorted order; when the
                        down projection's K is split into S ranges (S <= 4, chosen on
                        the device to fill the compute units; 1 on the decode path),
                        partial sums per range, added by the combine */
  size_t total;      /* = moe_experts_workspace_bytes() */
  /* MXFP4 weights only (0 otherwise): GEMM input rows split for the
   * block-scaled MFMA, each region R rows of K bytes of e4m3 hi parts, then R
   * rows of K bytes of lo parts (unused with MXFP8 activations), then R rows of
   * e8m0 scale codes, one per 32 values, padded to a multiple of 16 bytes. */
  size_t xq;         /* token rows, K = H: R = xq_rows */
  size_t xq_rows;    /* T when split in token order (small problems, weight on the
                        activation), else T*k in sorted row order */
  size_t aq;         /* activation rows, K = I, R = T*k, sorted row order */
  size_t single_launch; /* 1 when the forward runs the decode step as one launch after the
                           align: weight-streaming tiles, the one-workgroup align, route
                           weight on the activation, H and I <= 4096, and the environment
                           variable MOE_EXPERTS_FUSED_DECODE=1 at the call (off by default:
                           measured slower than the separate launches). GEMM1, GEMM2 and the
                           combine then share one persistent kernel (flashinfer_moe_ep page,
                           module docstring: one launch) and moe_experts_forward_timed records
                           events 2, 3 and 4 together after it; act is not written with MXFP4
                           weights (GEMM1 writes the split rows in aq). The workspace holds
                           its counters either way. */
  size_t mx_tiled;   /* 1 when MXFP4 weights with MXFP8 activations run the LDS-tiled
                        block-scaled kernels (more than 32 rows per expert on average,
                        unless MOE_EXPERTS_MX_PREFILL=0 at the call). Then xq holds the
                        token rows (xq_rows = T; T*k sorted rows with the route weight on
                        the input) in the split layout above with no lo part used, and
                        aq holds only the e4m3 activation codes, T*k rows of I bytes in
                        sorted row order, their scales in aq_sc. */
  size_t aq_sc;      /* mx_tiled: e8m0 scales of the activation rows, per 256-row tile t
                        (the align's tiles of each segment, in segment order) and
                        128-column group g: a 1 KB block at aq_sc + (t * ceil(I/128) + g)
                        * 1024, 4 bytes per tile row holding the scales of its column
                        blocks 4g, 4g+2, 4g+1, 4g+3 in that order (0 past I / 32) */
} moe_ws_layout;

/* Bytes of the packed weights (moe_problem.mx_packed) of problem p: for
 * each expert, column tile and 128-K stage of GEMM1 (ceil(I / 128) column
 * tiles of 128 gate and the same 128 up rows, ceil(H / 128) stages) and of
 * GEMM2 (ceil(H / 256) tiles of 256 down rows, ceil(I / 128) stages), one
 * 17408-byte block: 256 rows x 64 bytes of e2m1 codes (row r's 16-byte chunk
 * c at r * 64 + 16 (c ^ ((r >> 2) & 3)); codes past N or past K are 0), then
 * the rows' 1 KB e8m0 scale block (row r's four block scales of the stage at
 * r * 4 in the order 0, 2, 1, 3; blocks past K are 0, rows past N repeat row
 * N - 1's). GEMM1's blocks for all experts, then GEMM2's; within an expert
 * column tile major. 0 when p is invalid or its weights are not MXFP4 (k is
 * not looked at). flashinfer_moe_ep page, process_weights_after_loading. */
size_t moe_mx_packed_bytes(const moe_problem* p);

/* Writes the packed weights of problem p (moe_mx_packed_bytes bytes) into
 * packed (device, 16-byte aligned, caller-owned) from the canonical MXFP4
 * tensors (the moe_experts_forward arguments of the same names), on stream;
 * asynchronous like the forward. Host-side errors before any launch:
 * MOE_EINVAL (invalid p, weights not MXFP4, a NULL or misaligned pointer),
 * MOE_ENOSPC (packed_bytes below moe_mx_packed_bytes). */
int moe_mx_pack_weights(const moe_problem* p, const void* w_gate, const void* w_up, const void* w_down,
                        const uint8_t* s_gate, const uint8_t* s_up, const uint8_t* s_down, void* packed,
                        size_t packed_bytes, moe_stream_t stream);

/* Bytes of the bf16 operand-block weights (moe_problem.bf16_packed) of problem
 * p: the gate weights [E, I, H], then the up weights [E, I, H], then the down
 * weights [E, H, I], 2 E I H bytes each, each matrix [N, K] stored as 1 KB
 * blocks of 16 rows x 32 K values, block (nb, kb) at ((e N / 16 + nb) K / 32 +
 * kb) * 1024 bytes from its region's start, its 16-byte piece l (l < 64)
 * holding row 16 nb + l % 16, values 32 kb + 8 (l / 16)..+7 (the B operand of
 * v_mfma_f32_16x16x32_bf16, lane by lane). 0 when p is invalid or its weights
 * are not bf16 (k is not looked at: the layout serves both entries).
 * flashinfer_moe_ep page, process_weights_after_loading. */
size_t moe_bf16_packed_bytes(const moe_problem* p);

/* Writes the operand-block weights of problem p (moe_bf16_packed_bytes bytes)
 * into packed (device, 16-byte aligned, caller-owned) from the canonical bf16
 * tensors w_gate, w_up [E, I, H] and w_down [E, H, I] (device, 16-byte
 * aligned), on stream; asynchronous like the forward. Host-side errors before
 * any launch: MOE_EINVAL (invalid p, weights not bf16, a NULL or misaligned
 * pointer), MOE_ENOSPC (packed_bytes below moe_bf16_packed_bytes). */
int moe_bf16_pack_weights(const moe_problem* p, const void* w_gate, const void* w_up, const void* w_down,
                          void* packed, size_t packed_bytes, moe_stream_t stream);

/* Workspace bytes a moe_experts_forward call on problem *p needs (0 if *p is
 * invalid). Depends only on the sizes in *p, so a workspace sized once for the
 * largest T serves every smaller T (fi_moe page: allocate before the first
 * forward). */
size_t moe_experts_workspace_bytes(const moe_problem* p);

/* Fills *layout for problem *p; MOE_EINVAL for an invalid problem. */
int moe_experts_workspace_layout(const moe_problem* p, moe_ws_layout* layout);

/*
 * The experts step, token-major in and out.
 *   x            (device) bf16 [T, H]
 *   topk_ids     (device) int32 [T, k]; -1 = masked slot (contributes nothing);
 *                any other id outside [0, E) is skipped and counted in the
 *                workspace status word (moe_device_error)
 *   topk_weights (device) float32 [T, k], applied to the activation before the
 *                down projection
 *   w_gate, w_up (device) [E, I, H] bf16, or MXFP4 codes [E, I, H/2]
 *   w_down       (device) [E, H, I] bf16, or MXFP4 codes [E, H, I/2]
 *   s_gate, s_up, s_down (device) e8m0 scales [E, N, K/32] for MXFP4, NULL for bf16
 *                x, weights, scales and out 16-byte aligned (else MOE_EINVAL);
 *                MXFP4 needs H, I <= 16384; T*H and T*k*max(H, I) must stay below 2^31
 *                and I*H at most 2^30 (else MOE_ENOTSUP)
 *   out          (device) bf16 [T, H], overwritten:
 *                out[t] = sum over j = 0..k-1, in that order, in fp32, of
 *                W_down[e] (f(W_gate[e] x[t], W_up[e] x[t]) * w[t,j]),  e = ids[t,j]
 *   workspace    (device) at least moe_experts_workspace_bytes(p) bytes,
 *                256-byte aligned
 * Numerics: bf16 MFMA products with fp32 accumulation; the activation is
 * rounded once to bf16 before the down GEMM and each slot's down-projection
 * row once to bf16 before the fp32 combine.
 */
int moe_experts_forward(const moe_problem* p, const void* x, const int32_t* topk_ids,
                        const float* topk_weights, const void* w_gate, const void* w_up,
                        const void* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                        const uint8_t* s_down, void* out, void* workspace, size_t workspace_bytes,
                        moe_stream_t stream);

/* Same as moe_experts_forward, and additionally records the caller's
 * hipEvent_t handles stage_events[0..n_events-1] on `stream` between the
 * stages (align, GEMM1, GEMM2, combine: event i before stage i, the last
 * after the last stage) so a benchmark can time each kernel on the stream it
 * runs on. n_events must be 0 (no recording) or 5. */
int moe_experts_forward_timed(const moe_problem* p, const void* x, const int32_t* topk_ids,
                              const float* topk_weights, const void* w_gate, const void* w_up,
                              const void* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                              const uint8_t* s_down, void* out, void* workspace,
                              size_t workspace_bytes, moe_stream_t stream,
                              void* const* stage_events, int n_events);

/*
 * moe_experts_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The library's own scratch array (32 MiB,
 * one per device, held from the library's load until the process ends)
 * serves as the workspace; nothing is allocated or freed, and the call
 * enqueues the same kernels as moe_experts_forward on `stream`.
 * Arguments, layouts and results are those of moe_experts_forward.
 * Limits: problems whose moe_experts_workspace_bytes() exceeds 32 MiB get
 * MOE_ENOSPC (a decode step of T=32, H=I=2880, E=128, top-4 needs about
 * 3 MiB). Every call on a device shares that device's scratch and leaves its
 * contents behind (no kernel expects it to start zeroed): calls that overlap
 * on one device, on any streams, race. The device status word stays in the
 * scratch, so bad expert ids are skipped as by moe_experts_forward but not
 * reported (moe_device_error needs a caller-owned workspace).
 */
int moe_experts_forward_noalloc(const moe_problem* p, const void* x, const int32_t* topk_ids,
                                const float* topk_weights, const void* w_gate, const void* w_up,
                                const void* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                                const uint8_t* s_down, void* out, moe_stream_t stream);

/* Workspace bytes for moe_align on (T, k, E); 0 if invalid. */
size_t moe_align_workspace_bytes(int32_t T, int32_t k, int32_t E);

/*
 * Grouping only (the forward's first stage, exposed for bit-exact testing).
 * moonep_experts page, MoonEPExperts.apply (cumulative sum of per-row counts)
 * and module docstring (rows contiguous per weight row).
 *   topk_ids   (device) int32 [T, k]
 *   counts     (device) int32 [E]     slots per expert (valid ids only)
 *   cu_seqlens (device) int32 [E]     cumulative end offsets
 *   perm       (device) int32 [T*k]   perm[p] = t*k+j for sorted row p, ascending
 *                                     inside each segment; entries >= M are -1
 *   inv_perm   (device) int32 [T*k]   inverse, -1 for masked / bad slots
 *   workspace  (device) moe_align_workspace_bytes(T, k, E) bytes
 */
int moe_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* counts,
              int32_t* cu_seqlens, int32_t* perm, int32_t* inv_perm, void* workspace,
              size_t workspace_bytes, moe_stream_t stream);

/* Workspace bytes for moe_experts_forward_grouped on *p (p->T = NvS,
 * p->E = segments); 0 if invalid. */
size_t moe_experts_grouped_workspace_bytes(const moe_problem* p);

/*
 * Pre-grouped experts step (moonep_experts page: rows already contiguous per
 * weight row in segment order, [E+B] segments including redundant slots).
 *   x_nvs      (device) bf16 [NvS, H], NvS = p->T
 *   cu_seqlens (device) int32 [G] cumulative end offsets, G = p->E; must be
 *              non-decreasing and <= NvS, else the status word is set and
 *              the whole output is zero
 *   route_w    (device) float32 [NvS]
 *   weights / scales as in moe_experts_forward with E = G
 *   out_nvs    (device) bf16 [NvS, H], overwritten; rows >= cu_seqlens[G-1] are 0
 */
int moe_experts_forward_grouped(const moe_problem* p, const void* x_nvs, const int32_t* cu_seqlens,
                                const float* route_w, const void* w_gate, const void* w_up,
                                const void* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                                const uint8_t* s_down, void* out_nvs, void* workspace,
                                size_t workspace_bytes, moe_stream_t stream);

/*
 * Router step: per-token expert logits -> the top-k expert ids and route
 * weights that moe_experts_forward takes.
 * trtllm_mxfp4_moe page, TrtLlmMxfp4ExpertsMonolithic (router and experts in
 * one call): _supports_routing_method names Renormalize, RenormalizeNaive and
 * DeepSeekV3; apply passes the score-correction bias, the number of expert
 * groups, the groups kept (topk_group) and the routed scaling factor. The page
 * prints no formulas; the library reads them as:
 *   MOE_ROUTE_RENORMALIZE (also RenormalizeNaive, which differs only in
 *     evaluation order): w_j = exp(l_j) / sum over the k picks of exp(l_i),
 *     the picks being the k largest logits.
 *   MOE_ROUTE_DEEPSEEK_V3 (DeepSeek-V3 gating): s = sigmoid(l), selection
 *     score s + bias; with n_group > 1 the E experts form n_group contiguous
 *     groups, a group scores the sum of its two largest selection scores and
 *     only the topk_group best groups stay eligible; the k largest selection
 *     scores are picked and w_j = scale * s_j / sum of the picked s (0 if that
 *     sum is 0).
 * Ties go to the lower index; output slots are in descending selection score.
 * Logits are clamped to the finite float32 range first (NaN = most negative).
 * DeepSeekV3 scores are sigmoid evaluated in double and rounded to float,
 * selection scores float adds, so picks are reproducible bit for bit.
 *   logits       (device) float32 [T, E]
 *   bias         (device) float32 [E], finite, or NULL (DeepSeekV3 only; ignored
 *                otherwise)
 *   topk_ids     (device) int32 [T, k], overwritten
 *   topk_weights (device) float32 [T, k], overwritten
 * Limits: 1 <= E <= 1024, 1 <= k <= min(E, 32) (MOE_ENOTSUP beyond 1024 or 32,
 * MOE_EINVAL for k > E); DeepSeekV3 with n_group > 1 needs n_group <= 64,
 * E % n_group == 0, E / n_group >= 2, 1 <= topk_group <= n_group and
 * k <= topk_group * E / n_group (MOE_EINVAL otherwise). No workspace; nothing
 * is allocated.
 */
typedef enum { MOE_ROUTE_RENORMALIZE = 0, MOE_ROUTE_DEEPSEEK_V3 = 1 } moe_route_method;

typedef struct {
  int32_t T, E, k;
  moe_route_method method;
  int32_t n_group;              /* DeepSeekV3: 0 or 1 = no group limit */
  int32_t topk_group;           /* DeepSeekV3 with n_group > 1 */
  float routed_scaling_factor;  /* DeepSeekV3: weights multiplied by it (1 = none) */
} moe_route_problem;

int moe_route(const moe_route_problem* p, const float* logits, const float* bias, int32_t* topk_ids,
              float* topk_weights, moe_stream_t stream);

/* moe_experts_forward_grouped that also records caller-created hipEvents on
 * `stream` at its stage boundaries (stage_events[0] before the segment
 * tables, [1] before GEMM1, [2] before GEMM2, [3] before the zero tail, [4]
 * after it) so a benchmark can time each kernel on the stream it runs on.
 * n_events must be 0 (no recording) or 5. */
int moe_experts_forward_grouped_timed(const moe_problem* p, const void* x_nvs, const int32_t* cu_seqlens,
                                      const float* route_w, const void* w_gate, const void* w_up,
                                      const void* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                                      const uint8_t* s_down, void* out_nvs, void* workspace,
                                      size_t workspace_bytes, moe_stream_t stream,
                                      void* const* stage_events, int n_events);

/* Reads the device status words of a workspace used by moe_experts_forward,
 * moe_experts_forward_grouped or moe_align: *n_bad = number of expert ids
 * outside [0, E) other than -1 in the last call (or 1 if its cu_seqlens were
 * malformed). Returns MOE_ETIMEDOUT if a wait of the single-launch decode
 * step gave up in that call (none ever should: every wait is on work that
 * running workgroups took earlier; the bound only guarantees the kernel
 * ends). Synchronous copy: call after the stream has finished. */
int moe_device_error(const void* workspace, int32_t* n_bad);

/*
 * Host-side check of per-expert parameter arrays before they are uploaded
 * (flashinfer_moe_ep page, epilogue_from_quant_config: the scales must be
 * finite and positive, one per expert). Each pointer is a HOST array of p->E
 * float32 values, or NULL (not checked). Rules, per expert, as for the
 * scalars of moe_problem: fc1_alpha and fc2_alpha finite and > 0; for
 * SwiGLU-OAI alpha and beta finite and limit > 0 (+inf allowed, NaN not);
 * for SiTu alpha and beta finite and > 0. Returns MOE_OK, MOE_EINVAL (a
 * non-finite value, a NaN limit, a bad problem) or MOE_ENOTSUP (a limit or a
 * SiTu parameter <= 0, a scale <= 0). Reads host memory only.
 */
int moe_check_expert_params(const moe_problem* p, const float* alpha_e, const float* beta_e,
                            const float* limit_e, const float* fc1_alpha, const float* fc2_alpha);

/* Static description of a status code. */
const char* moe_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_EXPERTS_H */
