/*
 * libqgemv — dequantise-fused skinny GEMV / GEMM for MI355X (gfx950).
 *
 *   y[N x M] = x[N x K] . dequant(W)[K x M]        N = 1..8 tokens
 *
 * over low-bit packed weights, with optional fused residual add and SwiGLU
 * epilogues and a mixture-of-experts variant that runs only each token's
 * selected experts.
 *
 * The operation follows the subject pages:
 *   - NInfer article (单卡 LLM 推理引擎 NInfer 完全解析), section 2 (custom
 *     CUDA operators and mixed quantised weights): decode throughput is bound
 *     by weight reads, fewer weight bits mean fewer bytes read, and each
 *     weight format gets its own fused kernel that does the matmul, residual
 *     add and SwiGLU in one read and one write; the groupwise-int recipe mixes
 *     4-bit and 5-bit groups, the NVFP4 artefact imports 4-bit weights.
 *   - Same article, "what NInfer is" and section 3: 1 to 8 concurrent decode
 *     lanes, and a multi-token-prediction verify pass of several tokens.
 *   - Decapybara page (GitHub - giveen/Decapybara), CUDA kernel list: a
 *     blocked NVFP4 matrix-vector multiply, a top-8 softmax MoE router.
 *   - memra page (avifenesh/memra), model notes: checkpoints are repacked
 *     into the engine's own layout; unsupported combinations are rejected.
 *   - RustingStrata page, format list: a Q8_0-style symmetric int8 format;
 *     known issues: reordering floating-point work between runs changes
 *     results, so every reduction here has a fixed order.
 *
 * Formats (logical definition; 32 weights per group / 16 per NVFP4 block,
 * both along K):
 *   QGEMV_INT4   w = d*q + m, q in 0..15, d and m fp16 per group
 *   QGEMV_INT5   w = d*q + m, q in 0..31, d and m fp16 per group
 *   QGEMV_INT8   w = d*q,     q in -127..127 (two's complement), fp16 d per group
 *   QGEMV_NVFP4  w = s_t * e2m1(code) * e4m3(b), OCP FP4 E2M1 codes, one OCP
 *                FP8 E4M3 scale b per 16 weights, one fp32 tensor scale s_t
 *   QGEMV_MXFP4  w = e2m1(code) * 2^(e - 127), one OCP E8M0 scale e per 32
 *   QGEMV_MXFP8  w = e4m3(code) * 2^(e - 127), one OCP E8M0 scale e per 32
 *                (OCP microscaling; the Decapybara kernel list names an
 *                MXFP8 block-scaled GEMV). The packer picks
 *                e = 127 + clamp(floor(log2 amax) - emax, -127, 127), emax 8
 *                for E4M3 and 2 for E2M1, and rounds w / 2^(e - 127) to the
 *                nearest code (ties to even, saturating). MX weights run on
 *                qgemv_mx only; qgemv and the MoE entry points reject them
 *                with QGEMV_EFORMAT.
 * The packed device layout is the library's own; qgemv_packed_bytes gives
 * its size. Weights are logically [K x M] and stored output-row-major.
 *
 * Conventions for every entry point:
 *   - Return value: QGEMV_OK (0) or a negative qgemv_status; never an
 *     exception, never printed. qgemv_strerror gives the text.
 *   - All arguments are validated on the host before any launch; an invalid
 *     call launches nothing and returns an error.
 *   - Device entry points are asynchronous on `stream` (0 = the null stream),
 *     never synchronise, and take device pointers owned by the caller. The
 *     library allocates nothing; its only global state is a per-device cache
 *     of the compute-unit count and kernel occupancy. Concurrent calls on
 *     different streams are safe when their output buffers (and workspaces)
 *     do not overlap.
 *   - Host entry points (pack) take host pointers and need no GPU.
 *   - Pointers to packed weights, scales and activations must be 16-byte
 *     aligned (QGEMV_EALIGN otherwise); float outputs 4-byte aligned.
 *   - Limits: 1 <= N <= 32 on qgemv / qgemv_swiglu / qgemv_ex /
 *     qgemv_swiglu_ex in every format (9 to 32 tokens share one MFMA operand
 *     slot per 16: verify windows of speculative decoding, NInfer article,
 *     section 3; the plain GEMV runs 17 to 32 tokens as two launches of at
 *     most 16); N <= 8 with the RMSNorm prologue, the batch-invariant order
 *     and on the MoE entry points (QGEMV_EUNSUPPORTED otherwise);
 *     K % 32 == 0, M >= 1, packed matrix under 4 GiB.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QGEMV_INT4 = 1,
  QGEMV_INT5 = 2,
  QGEMV_INT8 = 3,
  QGEMV_NVFP4 = 4,
  QGEMV_MXFP4 = 5,
  QGEMV_MXFP8 = 6
} qgemv_format;

typedef enum {
  QGEMV_OK = 0,
  QGEMV_EINVAL = -1,       /* null pointer, bad size or non-finite weights */
  QGEMV_EFORMAT = -2,      /* unknown format value */
  QGEMV_EALIGN = -3,       /* pointer alignment or shape alignment violated */
  QGEMV_ERANGE = -4,       /* a scale field overflows its encoding */
  QGEMV_EWORKSPACE = -5,   /* workspace missing or too small */
  QGEMV_EHIP = -6,         /* the HIP runtime reported an error at launch */
  QGEMV_EUNSUPPORTED = -7  /* a size outside the supported range (e.g. N > 32) */
} qgemv_status;

/* Text for a status code (static storage). */
const char* qgemv_strerror(int status);

/* Library version: major*10000 + minor*100 + patch. */
int qgemv_version(void);

/* ---------------------------------------------------------------- host --- */

/* Bytes of the packed weight buffer `wq` and scale buffer `ws` for an
 * [M][K] matrix in format `fmt`. Rows are padded to 16 and K to 128 inside
 * the layout (padding holds weight 0). */
int qgemv_packed_bytes(int fmt, int64_t M, int64_t K, size_t* wq_bytes, size_t* ws_bytes);

/* Quantise and pack a host fp32 matrix W[M][K] (row-major) into host
 * buffers wq, ws of qgemv_packed_bytes sizes. Quantisation rules (the pages
 * name the formats only; these are the plainest readings):
 *   int4/int5: per group of 32, d = fp16((max - min) / (2^b - 1)) (fp32
 *     arithmetic), m = fp16(min), q = clamp(rint((w - m) / d)) in fp64,
 *     ties to even, q = 0 when d = 0;
 *   int8: d = fp16(amax / 127), q = clamp(rint(w / d), -127, 127);
 *   nvfp4: s_t = amax(W) / 2688 in fp32 (1 if that is 0), block scale
 *     b = E4M3_rne_saturating(amax_b / (6 * s_t)), codes
 *     E2M1_rne_saturating(w / (b * s_t)) computed in fp64, +0 when b = 0.
 * Negative zeros in W count as +0. Errors: EINVAL for null pointers,
 * non-finite weights or bad sizes, ERANGE when d or m overflows fp16. */
int qgemv_pack(int fmt, const float* W, int64_t M, int64_t K, void* wq, void* ws);

/* Pack logical codes and scale fields (host) without quantising.
 *   codes:  [M][K] uint8 (int4 0..15, int5 0..31, nvfp4 4-bit E2M1 codes)
 *           or int8 (int8 format)
 *   scales: int formats: uint16 fp16 bits of d, [M][K/32];
 *           nvfp4: uint8 E4M3 codes, [M][K/16]
 *   mins:   uint16 fp16 bits of m, [M][K/32] (int4/int5), else NULL
 *   tensor_scale: s_t (nvfp4), ignored otherwise.
 * Codes outside the format's range give EINVAL. */
int qgemv_pack_codes(int fmt, const void* codes, const void* scales, const uint16_t* mins,
                     float tensor_scale, int64_t M, int64_t K, void* wq, void* ws);

/* -------------------------------------------------------------- device --- */

/* y[n][m] = residual[n][m] + sum_k x[n][k] * W[m][k] for n < N, m < M.
 *   wq, ws:   packed weights and scales (qgemv_pack layout), device
 *   x:        bf16 activations [N][K], row-major, device
 *   residual: fp32 [N][M] or NULL; may be the same buffer as y
 *   y:        fp32 [N][M] output
 * Accumulation is fp32 in a fixed order: repeated calls give identical bits. */
int qgemv(int fmt, const void* wq, const void* ws, const void* x, const float* residual,
          float* y, int64_t M, int64_t K, int N, hipStream_t stream);

/* Fused gate/up projection with SwiGLU (NInfer article, section 2):
 *   h[n][i] = silu(g) * u,  g = x . W[i],  u = x . W[I + i],  silu(g) = g / (1 + e^-g)
 * for the [2I][K] matrix packed as one matrix (rows 0..I-1 gate, I..2I-1
 * up, one NVFP4 tensor scale for both). h is fp32 [N][I]. I % 16 == 0
 * (QGEMV_EALIGN otherwise). */
int qgemv_swiglu(int fmt, const void* wq, const void* ws, const void* x, float* h,
                 int64_t I, int64_t K, int N, hipStream_t stream);

/* Optional fusions of qgemv_ex / qgemv_swiglu_ex, for chaining layers without
 * separate normalisation or conversion kernels (NInfer article, section 2:
 * the per-format fused kernels do the normalisation, matmul, residual add and
 * SwiGLU in one read and one write):
 *   norm_src:   RMSNorm prologue. The activations become
 *                 x[n][k] = norm_src[n][k] * norm_gamma[k] / sqrt(mean_k norm_src[n][k]^2 + norm_eps)
 *               ([N][K] fp32 and [K] fp32, device, 16-byte aligned; the `x`
 *               argument is then ignored and may be NULL). The GPU multiplies
 *               bf16(norm_gamma * norm_src) and applies the per-token scale,
 *               computed in fp32, to the dot products.
 *   out_bf16:   also write the output (y, or h for SwiGLU) rounded to bf16
 *               (nearest even), [N][M] or [N][I], device; the fp32 output
 *               pointer may then be NULL.
 *   flags:      QGEMV_BATCH_INVARIANT: every token's outputs are the same
 *               bits whatever N is and wherever the token sits in the batch
 *               (the summation order then depends on K only), for
 *               byte-identical speculative decoding (NInfer article, section
 *               3: multi-token-prediction verify windows; RustingStrata page,
 *               known issues: reordered floating-point work diverges). Costs
 *               some speed at N < 8. Other bits: QGEMV_EINVAL.
 *   workspace:  device memory of qgemv_split_workspace_bytes (256-byte
 *               aligned, ZERO-FILLED BEFORE ITS FIRST USE) that lets the
 *               launch balance its last row blocks: when the row blocks do not
 *               divide evenly over the compute units, the leftover blocks'
 *               K ranges are cut into fragments (at most 8) whose partial sums
 *               meet in the workspace, added by the block's last fragment in
 *               fragment order (the workgroups wait, bounded, only on
 *               lower-numbered ones, which start first on every XCD). Results
 *               stay reproducible from call to call but their bits differ
 *               from a call without a workspace (with norm_src the fragments
 *               also add their parts of each token's sum of squares). Not
 *               used with QGEMV_BATCH_INVARIANT or N > 8. Every call leaves
 *               the flags it used at zero, so one fill serves later calls in
 *               stream order; calls that may overlap in time need separate
 *               workspaces. The first 32-bit word is a sticky flag that
 *               becomes nonzero if a wait ever timed out. The results of
 *               that call are then invalid, and so is the workspace: a late
 *               fragment may still raise its flag after the waiter gave up,
 *               so zero the whole workspace again before reusing it. The
 *               library never reads the word back (that would need a
 *               synchronisation); the caller checks it after synchronising.
 *               workspace_bytes: its size (QGEMV_EWORKSPACE if smaller).
 * Zero-initialise unused fields. */
enum { QGEMV_BATCH_INVARIANT = 1 };
typedef struct qgemv_fusion {
  const float* norm_src;
  const float* norm_gamma;
  float norm_eps;
  uint16_t* out_bf16;
  int flags;
  void* workspace;
  size_t workspace_bytes;
} qgemv_fusion;

/* Bytes of the workspace above for the current device (it depends on the
 * device's compute-unit count). */
int qgemv_split_workspace_bytes(size_t* bytes);

/* qgemv with the optional fusions above (fusion may be NULL). */
int qgemv_ex(int fmt, const void* wq, const void* ws, const void* x, const float* residual, float* y,
             int64_t M, int64_t K, int N, const qgemv_fusion* fusion, hipStream_t stream);

/* qgemv_swiglu with the optional fusions above (fusion may be NULL). */
int qgemv_swiglu_ex(int fmt, const void* wq, const void* ws, const void* x, float* h, int64_t I, int64_t K,
                    int N, const qgemv_fusion* fusion, hipStream_t stream);

/* Byte stride between consecutive experts in an expert-stacked weight or
 * scale buffer: the packed size rounded up to 256. */
int qgemv_expert_stride(int fmt, int64_t M, int64_t K, size_t* wq_stride, size_t* ws_stride);

/* Workspace bytes qgemv_moe needs for E experts, hidden H, intermediate I,
 * N tokens and top_k experts per token. */
int qgemv_moe_workspace_bytes(int E, int64_t H, int64_t I, int N, int top_k, size_t* bytes);

/* Mixture-of-experts FFN for N tokens that each selected top_k experts
 * (Decapybara page: top-8 softmax router; NInfer article, section 2: fused
 * SwiGLU):
 *   for each token t and slot j with e = ids[t][j] in [0, E):
 *     h = SwiGLU(x[t] . W_gu[e])            (fp32, [I])
 *     o = h . W_dn[e]                       (fp32, [H])
 *   y[t] = residual[t] + sum_j gates[t][j] * o_j   (j in increasing order)
 *   wq_gu, ws_gu: E experts of [2I][H] packed, stacked at qgemv_expert_stride
 *   wq_dn, ws_dn: E experts of [H][I] packed, stacked likewise
 *   ids [N][top_k] int32, gates [N][top_k] fp32 (used as given), device
 *   residual [N][H] fp32 or NULL (may equal y); y [N][H] fp32
 *   workspace: device scratch of qgemv_moe_workspace_bytes, 16-byte aligned
 * Only the experts some token selected are read. Ids outside [0, E) add
 * nothing and set the error flag that qgemv_moe_index reports. Duplicate
 * ids in a row are processed as separate slots. top_k <= 8, N <= 8,
 * H % 32 == 0 and I % 32 == 0 (QGEMV_EALIGN otherwise). */
int qgemv_moe(int fmt, const void* wq_gu, const void* ws_gu, const void* wq_dn, const void* ws_dn,
              int E, int64_t H, int64_t I, const void* x, const int32_t* ids, const float* gates,
              int top_k, const float* residual, float* y, int N, void* workspace,
              size_t workspace_bytes, hipStream_t stream);

/* qgemv_moe without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Its h / o scratch lives in a static
 * device array of qgemv_moe_noalloc_max_bytes (4 MiB) per GPU, held until the
 * process ends; the call allocates and frees nothing. Calls whose
 * qgemv_moe_workspace_bytes exceed that return QGEMV_EWORKSPACE. Every call
 * on one GPU shares that GPU's array, so calls that may overlap in time on
 * one GPU (different streams) race; calls in one stream are safe. Arguments
 * and results otherwise as qgemv_moe (same kernels, same bits). */
int qgemv_moe_noalloc(int fmt, const void* wq_gu, const void* ws_gu, const void* wq_dn, const void* ws_dn,
                      int E, int64_t H, int64_t I, const void* x, const int32_t* ids, const float* gates,
                      int top_k, const float* residual, float* y, int N, hipStream_t stream);

/* The size of qgemv_moe_noalloc's static scratch, in bytes. */
int qgemv_moe_noalloc_max_bytes(size_t* bytes);

/* Top-k softmax router (Decapybara page, CUDA kernel list: a top-8 softmax
 * router in front of the experts). For each token t < N:
 *   ids[t][j]   the j-th largest of logits[t][0..E) (j < top_k); equal
 *               logits go in increasing expert order; -0 equals +0; a NaN
 *               ranks below every number
 *   gates[t][j] exp(l_j - l_0) / sum_{i<top_k} exp(l_i - l_0) in fp32,
 *               summed in increasing i (the softmax over the selected
 *               logits, which equals the full softmax renormalised)
 *   logits [N][E] fp32, ids [N][top_k] int32, gates [N][top_k] fp32, device.
 * The ids are exact; the gates are meaningful for finite logits.
 * 1 <= top_k <= min(E, 64), E <= 16384 (QGEMV_EUNSUPPORTED otherwise). */
int qgemv_moe_route(const float* logits, int N, int E, int top_k, int32_t* ids, float* gates,
                    hipStream_t stream);

/* Workspace bytes of qgemv_moe_fused. */
int qgemv_moe_fused_workspace_bytes(int E, int64_t H, int64_t I, int N, int top_k, size_t* bytes);

/* The MoE FFN of qgemv_moe in a single launch, routed on the device from
 * router logits (the router of qgemv_moe_route, run by every workgroup):
 *   ids, gates = route(logits [N][E], top_k)
 *   y[t] = residual[t] + sum_j gates[t][j] * down_e(SwiGLU(gate_up_e(x[t])))
 * With N * top_k <= 8 routed rows (batch-1 decode at top-8) it is one
 * launch: each gate/up work item publishes its rows of h and raises its
 * own flag in the workspace to the call's number (the library numbers its
 * calls in the process 1, 2, ... in 64 bits); each output item waits
 * (bounded) until every flag of its experts holds that number, computes
 * every expert's output for 16 columns of y and sums them in fixed order in
 * LDS. With more rows it runs qgemv_moe_route and then the launches of
 * qgemv_moe, whose bits it then reproduces for the same ids and gates.
 * Either way results are bitwise reproducible from call to call.
 *   ids_out [N][top_k], gates_out [N][top_k]: receive the routing (device),
 *   or NULL.
 *   workspace: device memory of qgemv_moe_fused_workspace_bytes, 16-byte
 *   aligned, ZERO-FILLED BEFORE ITS FIRST USE. It starts with an error word
 *   and the flags, which no later call mistakes for its own (each call
 *   waits for its own number), so one fill serves every later call in
 *   stream order with the same I (the flag region's size depends on I only;
 *   N, E, H and top_k may change if the workspace is large enough). Calls
 *   that may overlap in time need separate workspaces. Byte offset 12 holds
 *   a sticky 32-bit flag that becomes nonzero if a dependency wait ever
 *   timed out: the results of that call are then invalid; the flag stays
 *   set until the caller clears it. Workgroups wait only on lower-numbered
 *   ones, which start first on every XCD, so the waits need no
 *   co-residency.
 * Other arguments and limits as qgemv_moe; 1 <= top_k <= min(E, 8). */
int qgemv_moe_fused(int fmt, const void* wq_gu, const void* ws_gu, const void* wq_dn, const void* ws_dn,
                    int E, int64_t H, int64_t I, const void* x, const float* logits, int top_k,
                    const float* residual, float* y, int N, int32_t* ids_out, float* gates_out,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* MoE routing index (the step qgemv_moe runs first; Decapybara page, CUDA
 * kernel list: the top-8 MoE path groups each token's selected experts),
 * into caller buffers (device, 4-byte aligned):
 *   counts [E]      slots routed to each expert
 *   offsets [E+1]   exclusive prefix sum of counts
 *   pairs [N*top_k] flat slot t*top_k + j, ordered by (expert, t, j); -1 after
 *                   offsets[E]
 *   active [E]      experts with a nonzero count, ascending; -1 after
 *   meta [2]        {number of active experts, 1 if any id was outside [0, E)}
 * Exact integer results, built from the same device routine that every
 * expert workgroup of qgemv_moe runs (the a-th smallest selected expert and
 * its entries, for each slot a). N <= 8, top_k <= 8, 1 <= E <= 16384
 * (QGEMV_EUNSUPPORTED / QGEMV_EINVAL otherwise). */
int qgemv_moe_index(const int32_t* ids, int N, int top_k, int E, int32_t* counts, int32_t* offsets,
                    int32_t* pairs, int32_t* active, int32_t* meta, hipStream_t stream);

/* The same index built by the routine of a chosen MoE path, so that each
 * path's routing can be compared bit for bit with its definition:
 *   routine 0: the per-slot routing of qgemv_moe (= qgemv_moe_index);
 *   routine 1: the all-slots lane ranking of qgemv_moe_fused's single launch.
 * Other values: QGEMV_EINVAL. Arguments and results as qgemv_moe_index. */
int qgemv_moe_index_by(int routine, const int32_t* ids, int N, int top_k, int E, int32_t* counts,
                       int32_t* offsets, int32_t* pairs, int32_t* active, int32_t* meta, hipStream_t stream);

/* Debug / parity: write the fp32 weights the packed buffers encode,
 * w_out[m][k] for m < M, k < K. Values are exactly:
 *   int4/int5: fp32(d*q + m) rounded once; int8: d*q;
 *   nvfp4: fp32(s_t * (e2m1 * b)) rounded once;
 *   mxfp4 / mxfp8: e2m1 or e4m3 value * 2^(e - 127) (exact in fp32). */
int qgemv_dequant(int fmt, const void* wq, const void* ws, int64_t M, int64_t K, float* w_out,
                  hipStream_t stream);

/* Dynamic MXFP8 activation quantiser (Decapybara kernel list: a dynamic
 * 32-element MXFP8 activation quantiser). For each token n < N and 32-block
 * b along K, with the bf16 values v of x[n][32b .. 32b+31]:
 *   X = floor(log2(max |v|)) - 8, clamped to [-127, 127]; -127 if all zero
 *   scales[n][b] = X + 127                                 (E8M0)
 *   codes[n][32b + i] = E4M3(v_i / 2^X): nearest, ties to even, saturating
 *                       at +-448, sign bit kept (-0 -> 0x80), NaN -> NaN
 *   x [N][K] bf16 bits, codes [N][K] bytes (both 16-byte aligned),
 *   scales [N][K/32] bytes; device. K % 32 == 0. Exact: one correct result. */
int qgemv_act_quant(const void* x, int N, int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t stream);

/* MX GEMV on gfx950's block-scaled MFMA (Decapybara kernel list: MXFP8
 * block-scaled matrix-vector multiply):
 *   y[n][m] = residual[n][m] + sum_k xq[n][k] * w[m][k]
 * with xq[n][k] = e4m3(codes[n][k]) * 2^(scales[n][k/32] - 127) (the output
 * of qgemv_act_quant) and w the MXFP8 or MXFP4 weights (QGEMV_MXFP8 /
 * QGEMV_MXFP4, packed by qgemv_pack). Every product is exact; sums are fp32
 * in a fixed order (reproducible run to run).
 *   wq, ws: packed weights; xq [N][K] codes (16-byte aligned), xs [N][K/32]
 *   E8M0 bytes; residual [N][M] fp32 or NULL (may equal y); y [N][M] fp32.
 * 1 <= N <= 32 (two blocks of 16 tokens share each weight operand). */
int qgemv_mx(int fmt, const void* wq, const void* ws, const uint8_t* xq, const uint8_t* xs,
             const float* residual, float* y, int64_t M, int64_t K, int N, hipStream_t stream);

/* qgemv_mx with the SwiGLU epilogue of qgemv_swiglu (NInfer article, section
 * 2: SwiGLU fused into the matmul): wq, ws hold [2I][K] MX weights, gate rows
 * [0, I) then up rows [I, 2I); h[n][i] = silu(g) * u with g, u the two MX
 * GEMV outputs (no residual). I % 16 == 0; other arguments as qgemv_mx. */
int qgemv_mx_swiglu(int fmt, const void* wq, const void* ws, const uint8_t* xq, const uint8_t* xs, float* h,
                    int64_t I, int64_t K, int N, hipStream_t stream);

/* qgemv_mx_swiglu with h handed on already quantised for the next MX
 * projection (NInfer article, section 2: SwiGLU fused into the matmul;
 * Decapybara page, kernel list: the dynamic 32-element MXFP8 activation
 * quantiser): writes the E4M3 codes hq [N][I] and E8M0 scales hs [N][I/32]
 * that qgemv_act_quant gives for bf16(h) (h rounded to bf16, nearest even),
 * in one launch instead of two. h [N][I] fp32 may be NULL; if given it also
 * receives the h that was quantised (within qgemv_mx_swiglu's tolerance of
 * the exact SwiGLU; its K split differs, so its bits may differ from
 * qgemv_mx_swiglu's). I % 32 == 0 (QGEMV_EALIGN); hq 4-byte aligned; all
 * device; other arguments as qgemv_mx_swiglu. */
int qgemv_mx_swiglu_quant(int fmt, const void* wq, const void* ws, const uint8_t* xq, const uint8_t* xs, float* h,
                          uint8_t* hq, uint8_t* hs, int64_t I, int64_t K, int N, hipStream_t stream);

/* Measurement aid: stream-read `bytes` (multiple of 16) from `buf` with
 * 128-bit non-temporal loads, folding them into sink[0] (a device uint32).
 * Gives the achievable read bandwidth that the GEMV kernels approach. */
int qgemv_probe_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
