/*
 * fp8w8a8.h - C ABI of the MI355X (gfx950) FP8 W8A8 linear layer.
 *
 * What it computes (HunyuanVideo1.5 BF16->FP8 retrospective, aigcage.com/blog/
 * hunyuanvideo-fp8, section 3.1): a bf16 activation is quantised per token at
 * run time to FP8 E4M3 ("float8_e4m3fn"), multiplied on the matrix cores by a
 * weight that was quantised per output channel ahead of time (section 2 of the
 * same page), and the epilogue applies the activation scale, the weight scale
 * and the bias and writes bf16.
 *
 *   s[m]      = fl32(max_k |A[m,k]| / 448)                   (0 for an all-zero row)
 *   qA[m,k]   = e4m3fn_rne_sat(fl32(A[m,k] / s[m]))          (signed zero when s[m] == 0)
 *   out[m,n]  = bf16_rne( fl32( sum_k dec(qA[m,k]) * dec(qW[n,k]) ) * s[m] * sW[n] + bias[n] )
 *
 * The product accumulates in fp32 on the MFMA units; the epilogue runs in fp32
 * and rounds once to bf16 (round to nearest even). e4m3fn is the OCP 8-bit E4M3
 * encoding: bias 7, largest finite 448, no infinity, 0x7F/0xFF NaN. Quantisation
 * saturates at +-448 and rounds to nearest, ties to even.
 *
 * Layouts. Every matrix is dense, row-major, last index fastest:
 *   A bf16 [m, k], qA u8 [m, k], W bf16 [n, k], qW u8 [n, k], out bf16 [m, n].
 *   The weight keeps nn.Linear's [n, k] layout with k contiguous (the section's
 *   "column-major B"); it is never transposed or copied into another layout.
 *   Scales are fp32: s [m], sW [n]. bias is bf16 [n] or NULL.
 *
 * Ownership. The caller allocates and frees every device buffer. The library
 * never allocates device memory at run time; the only device memory it holds is
 * the fixed scratch array of fp8_linear_run_noalloc, part of its code object on each
 * GPU it runs on. A plan is a small host object owned by the
 * library (create / destroy); it borrows the weight, weight-scale and bias
 * pointers, which must stay valid while the plan is used.
 *
 * Streams. Every launch is asynchronous on the caller's hipStream_t (NULL is
 * the default stream); the library never synchronises. A plan is immutable
 * after create, so runs on different streams may use it concurrently.
 *
 * Errors. Functions return FP8W8A8_OK (0) or a negative status. Arguments are
 * checked on the host before anything is launched; nothing is printed, nothing
 * aborts and nothing falls back to another implementation (section 3.3 of the
 * retrospective moves such decisions out of the forward call). Device faults
 * are asynchronous and surface at the caller's next synchronisation, as usual
 * in HIP. Rows m == 0 are a no-op returning FP8W8A8_OK; an empty weight
 * (n == 0 or k == 0) is FP8W8A8_ERR_BAD_SHAPE, like the empty-input error
 * that the ComfyUI FP8 quantiser page (runcomfy.com, "Quantize Model to FP8
 * Format", common errors) gives for an empty model.
 */
#ifndef FP8W8A8_H
#define FP8W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------- */
#define FP8W8A8_OK 0
#define FP8W8A8_ERR_INVALID_ARG (-1)          /* a required pointer is NULL, or an unknown enum value */
#define FP8W8A8_ERR_BAD_SHAPE (-2)            /* a size is out of range or not a multiple of 16 */
#define FP8W8A8_ERR_MISALIGNED (-3)           /* a pointer breaks the alignment stated below */
#define FP8W8A8_ERR_BAD_DEVICE (-4)           /* the device is not a gfx950 GPU */
#define FP8W8A8_ERR_WORKSPACE_TOO_SMALL (-5)  /* the workspace is smaller than fp8_linear_workspace_bytes */
#define FP8W8A8_ERR_HIP (-6)                  /* a HIP runtime call or launch failed */
#define FP8W8A8_ERR_CAPTURE (-7)              /* the call cannot be recorded into a HIP graph (fp8_quant_gemm) */
#define FP8W8A8_ERR_TOO_LARGE (-8)            /* the input exceeds fp8_linear_run_noalloc's fixed scratch */

/* ---- activation kinds for fp8_linear_run ------------------------------------ */
#define FP8W8A8_A_BF16 0  /* a is bf16 [m, k]; the run quantises it per token into the workspace */
#define FP8W8A8_A_E4M3 1  /* a is already e4m3fn codes [m, k] with per-row scales a_scale [m] */

/* Size limits checked by every entry point. */
#define FP8W8A8_MAX_ROWS ((int64_t)1 << 24) /* m (or rows) must be below this */
#define FP8W8A8_MAX_DIM ((int64_t)1 << 20)  /* n, k and cols must not exceed this */

/* Human-readable text of a status code (a static string; never NULL). */
const char* fp8w8a8_status_string(int status);

/*
 * fp8_quant_rows - dynamic per-token quantisation (HunyuanVideo1.5 retrospective,
 * section 3.1, second step of the chain; section 3.4 quantises one activation
 * once and hands it to several projections).
 *
 *   x_bf16    device, bf16 [rows, cols], 16-byte aligned
 *   rows      0 <= rows < FP8W8A8_MAX_ROWS (0 is a no-op)
 *   cols      16 <= cols <= FP8W8A8_MAX_DIM, cols % 16 == 0
 *   q_out     device, u8 e4m3fn codes [rows, cols], 16-byte aligned, written
 *   scale_out device, fp32 [rows], 4-byte aligned, written: s[r] = fl32(amax_r / 448)
 *   stream    hipStream_t or NULL
 * Inputs must be finite (NaN / Inf give unspecified codes). Codes and scales are
 * bit-identical to the definition at the top of this file.
 */
int fp8_quant_rows(const void* x_bf16, int64_t rows, int64_t cols, void* q_out, float* scale_out,
                   void* stream);

/*
 * fp8_quant_weights_per_channel - quantise an nn.Linear weight W [n, k] per output
 * channel, ahead of time (retrospective, section 2: weights are quantised per
 * channel in advance). Same arithmetic and arguments as fp8_quant_rows with
 * rows = n, cols = k; n == 0 or k == 0 is FP8W8A8_ERR_BAD_SHAPE.
 */
int fp8_quant_weights_per_channel(const void* w_bf16, int64_t n, int64_t k, void* w_fp8_out,
                                  float* w_scale_out, void* stream);

/* ---- activation producers that emit FP8 ----------------------------------------
 *
 * HunyuanVideo1.5 retrospective, section 3, item 5 (producer fusion): the GELU or
 * SiLU in front of the FFN-down linear can hand the FP8 linear its (e4m3fn codes,
 * per-token scale) pair directly, instead of writing bf16 that a separate pass
 * quantises. The result is defined as the unfused path's:
 *
 *   y[r,c]          = bf16_rne(act(x[r,c]))   (the exact function value, rounded once)
 *   (q_out, scale)  = fp8_quant_rows(y)        (bit for bit)
 *
 * The page names "GELU/SiLU" and no formula; three textbook functions are offered:
 *   FP8W8A8_ACT_GELU_ERF   x * Phi(x) = x/2 * erfc(-x / sqrt 2)
 *   FP8W8A8_ACT_GELU_TANH  x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3)))
 *   FP8W8A8_ACT_SILU       x / (1 + exp(-x))
 * A bf16 -> bf16 function is a 65536-entry table: the caller allocates it
 * (FP8W8A8_ACT_TABLE_BYTES, device memory, 16-byte aligned), builds it once per
 * device with fp8_act_table_build, keeps it alive while producers use it, and
 * passes it to every producer call. Entries for finite inputs are the correctly
 * rounded bf16 of the function; non-finite inputs are outside the contract (the
 * table maps NaN to NaN, +inf to +inf and -inf to -0, and the quantiser's codes
 * for them are unspecified).
 */
#define FP8W8A8_ACT_GELU_ERF 1
#define FP8W8A8_ACT_GELU_TANH 2
#define FP8W8A8_ACT_SILU 3
#define FP8W8A8_ACT_TABLE_BYTES 131072 /* 65536 bf16 entries, indexed by the input's bit pattern */

/*
 * fp8_act_table_build - fill `table` (device, FP8W8A8_ACT_TABLE_BYTES, 16-byte
 * aligned, written) with bf16_rne(act(x)) for every bf16 bit pattern x, on the
 * current device, asynchronously on `stream`. An unknown act is
 * FP8W8A8_ERR_INVALID_ARG.
 */
int fp8_act_table_build(int act, void* table, void* stream);

/*
 * fp8_act_rows - the unfused producer: y_bf16[r, c] = table[x_bf16[r, c]].
 *
 *   x_bf16   device, bf16 [rows, cols], 16-byte aligned
 *   rows     0 <= rows < FP8W8A8_MAX_ROWS (0 is a no-op)
 *   cols     16 <= cols <= FP8W8A8_MAX_DIM, cols % 16 == 0
 *   table    device, built by fp8_act_table_build, 16-byte aligned (read)
 *   y_bf16   device, bf16 [rows, cols], 16-byte aligned, written (must not overlap x)
 */
int fp8_act_rows(const void* x_bf16, int64_t rows, int64_t cols, const void* table, void* y_bf16,
                 void* stream);

/*
 * fp8_act_quant_rows - the fused producer: the codes and scales fp8_quant_rows
 * would give for fp8_act_rows' output, from one read of x and no bf16 output.
 * Arguments as fp8_quant_rows, plus `table` (device, built by
 * fp8_act_table_build, 16-byte aligned, read). Feed q_out / scale_out to
 * fp8_linear_run with FP8W8A8_A_E4M3.
 */
int fp8_act_quant_rows(const void* x_bf16, int64_t rows, int64_t cols, const void* table, void* q_out,
                       float* scale_out, void* stream);

/*
 * A constructed linear: validated shapes, borrowed weight pointers and the GEMM
 * kernel configuration chosen for each activation-row bucket. The choice is made
 * once here from (n, k, compute-unit count), as the retrospective's
 * section 3.3 asks (bind the backend at construction, keep the forward narrow),
 * and per call only one integer compare on m picks the bucket (section 3.2: FFN-up
 * and FFN-down shapes want different tiles).
 */
typedef struct fp8_linear_plan fp8_linear_plan;

/*
 * fp8_linear_create - build a plan for out[m, n] = A[m, k] x W[n, k]^T.
 *
 *   device     HIP device ordinal; must be a gfx950 GPU (else FP8W8A8_ERR_BAD_DEVICE)
 *   n, k       16 <= n, k <= FP8W8A8_MAX_DIM, both multiples of 16
 *   w_fp8      device, e4m3fn codes [n, k], 16-byte aligned (borrowed)
 *   w_scale    device, fp32 [n], 16-byte aligned (borrowed)
 *   bias_bf16  device, bf16 [n], 16-byte aligned, or NULL for no bias (borrowed)
 *   out        receives the plan; unchanged on error
 * Shape, pointer and alignment checks run before the device is queried.
 */
int fp8_linear_create(int device, int64_t n, int64_t k, const void* w_fp8, const float* w_scale,
                      const void* bias_bf16, fp8_linear_plan** out);

/*
 * Workspace a FP8W8A8_A_BF16 run with m rows needs: the per-token codes [m, k]
 * then the scales [m], each rounded up to 256 bytes. 0 for m <= 0 and for a NULL plan.
 * FP8W8A8_A_E4M3 runs need no workspace.
 */
size_t fp8_linear_workspace_bytes(const fp8_linear_plan* plan, int64_t m);

/*
 * fp8_linear_run - one forward of the linear (retrospective, section 3.3: a plain
 * tensor is quantised and multiplied; an FP8 tensor goes straight to the GEMM;
 * section 3.5: an input that is already e4m3fn comes with its per-token scale).
 * The plan's device must be the current HIP device (FP8W8A8_ERR_BAD_DEVICE
 * otherwise, checked when m > 0), and a non-NULL stream must belong to it.
 *
 *   plan        from fp8_linear_create
 *   m           0 <= m < FP8W8A8_MAX_ROWS (0 is a no-op)
 *   a           device; bf16 [m, k] (a_kind FP8W8A8_A_BF16) or e4m3fn codes [m, k]
 *               (FP8W8A8_A_E4M3); 16-byte aligned
 *   a_kind      FP8W8A8_A_BF16 or FP8W8A8_A_E4M3
 *   a_scale     device fp32 [m], 4-byte aligned: required for FP8W8A8_A_E4M3, ignored
 *               (may be NULL) for FP8W8A8_A_BF16
 *   out_bf16    device, bf16 [m, n], 16-byte aligned, written
 *   workspace   device, 256-byte aligned, at least fp8_linear_workspace_bytes(plan, m)
 *               bytes for FP8W8A8_A_BF16 (after the call it holds qA then s);
 *               ignored for FP8W8A8_A_E4M3
 *   stream      hipStream_t or NULL; the quantisation and the GEMM are two launches
 *               on this stream, in order, with no synchronisation
 */
int fp8_linear_run(const fp8_linear_plan* plan, int64_t m, const void* a, int a_kind,
                   const float* a_scale, void* out_bf16, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * fp8_linear_run_group - several linears on one activation: the same results as
 * nplans calls of fp8_linear_run(plans[i], m, a, a_kind, a_scale, outs_bf16[i], ...),
 * with the activation quantised once (FP8W8A8_A_BF16). The retrospective (section 3.4)
 * has the hidden states feed the Q, K and V projections (three weights, one input);
 * quantising them once per token serves all three. When every plan would run the
 * 256 x 256 tiles (configuration 0 or 6) at a k of 2048..4096 and one launch needs fewer
 * rounds of tiles over the CUs than the separate ones (or as many, all full), the GEMMs go
 * out as ONE persistent launch whose workgroups walk the tiles of all the problems (one
 * first prologue and one final output drain instead of nplans of each); when every plan
 * would run a skinny
 * configuration (5 or 7, a few tokens), as ONE launch over all the problems' channel blocks
 * (enough workgroups to fill the device, where one problem alone leaves it half idle; in
 * configuration 7, 32 channels per workgroup, when their 16-channel blocks together
 * outnumber the CUs);
 * otherwise each plan's GEMM runs as in fp8_linear_run. Outputs are bit-identical to the
 * separate calls either way.
 *
 *   plans       1 <= nplans <= FP8W8A8_MAX_GROUP plans, all with the same k and device
 *   outs_bf16   nplans device pointers, bf16 [m, n_i] each, 16-byte aligned
 *   workspace   as fp8_linear_run, sized by fp8_linear_workspace_bytes(plans[0], m)
 *   m, a, a_kind, a_scale, stream   as fp8_linear_run
 * Returns FP8W8A8_ERR_INVALID_ARG for a NULL array or element or an nplans outside
 * the range, FP8W8A8_ERR_BAD_SHAPE for plans whose k differ, FP8W8A8_ERR_BAD_DEVICE
 * for plans on different devices; nothing is launched then.
 */
#define FP8W8A8_MAX_GROUP 4
int fp8_linear_run_group(const fp8_linear_plan* const* plans, int nplans, int64_t m, const void* a, int a_kind,
                         const float* a_scale, void* const* outs_bf16, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * fp8_linear_run_noalloc - fp8_linear_run without a workspace argument, for callers
 * that cannot allocate device memory at all (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). A FP8W8A8_A_BF16 run quantises the
 * activation into a fixed scratch array that the library holds in device memory, one
 * per GPU, from the first call on that GPU until the process ends; nothing is
 * allocated or freed by any call (the first call on a GPU only looks the array's
 * address up). Same kernels, hence bit-identical output, as fp8_linear_run with a
 * workspace.
 *
 *   plan, m, a, a_kind, a_scale, out_bf16, stream   as fp8_linear_run
 * The codes and scales of m rows take fp8_linear_workspace_bytes(plan, m) bytes of the
 * scratch; above FP8W8A8_NOALLOC_SCRATCH_BYTES the call returns FP8W8A8_ERR_TOO_LARGE
 * and launches nothing (80 MiB holds, e.g., 4096 tokens of k = 8192 or 32760 tokens of
 * k = 2048). FP8W8A8_A_E4M3 runs use no scratch and have no size limit beyond
 * fp8_linear_run's. The scratch keeps the last call's codes; every BF16 run rewrites
 * all the codes and scales its GEMM reads, so nothing needs clearing. All calls on
 * one GPU share its scratch: two BF16 runs that overlap in time on the same GPU (for
 * example on two streams) race, and the caller must order them. The scratch's address is
 * looked up (hipGetSymbolAddress) at the first BF16 call with m > 0 on each GPU; a caller
 * that records the call into a HIP graph makes one such call outside the capture first
 * (a lookup refused during capture returns FP8W8A8_ERR_HIP and launches nothing).
 */
#define FP8W8A8_NOALLOC_SCRATCH_BYTES ((size_t)80 << 20)
int fp8_linear_run_noalloc(const fp8_linear_plan* plan, int64_t m, const void* a, int a_kind,
                           const float* a_scale, void* out_bf16, void* stream);

/* Free a plan (NULL is ignored). Does not touch the borrowed device buffers. */
void fp8_linear_destroy(fp8_linear_plan* plan);

/*
 * fp8_linear - one-shot create + run + destroy with the same arguments and rules
 * as those calls (device = the current HIP device). Convenience for tests and
 * scripts; a model keeps a plan instead, so the forward does no set-up work.
 */
int fp8_linear(const void* a, int a_kind, const float* a_scale, int64_t m, int64_t n, int64_t k,
               const void* w_fp8, const float* w_scale, const void* bias_bf16, void* out_bf16,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Introspection of the construction-time choice (for tests and reports).
 * fp8_linear_plan_config writes, for an activation with m rows, the id of the GEMM
 * kernel configuration the plan launches and its tile (block rows in m, block
 * columns in n), and the number of output tiles: one workgroup each, except in the
 * persistent configuration (6), which launches one workgroup per compute unit (the
 * count rounded down to a multiple of 8, at most the tile count) that walks them.
 * Returns FP8W8A8_ERR_INVALID_ARG for a NULL plan or output pointer.
 */
int fp8_linear_plan_config(const fp8_linear_plan* plan, int64_t m, int* config_id, int* tile_m,
                           int* tile_n, int64_t* workgroups);

/*
 * fp8_linear_group_config writes the id of the GEMM kernel configuration of the single
 * launch that fp8_linear_run_group makes for these plans at m rows (6: persistent 256 x
 * 256 tiles over every problem; 5 or 7: the skinny weight stream over every problem's
 * column blocks), or -1 when each plan runs its own GEMM (fp8_linear_plan_config then
 * names each one; also for m == 0, which launches nothing). For tests and reports.
 * Returns FP8W8A8_ERR_INVALID_ARG for a NULL array, element or output pointer or an
 * nplans outside 1..FP8W8A8_MAX_GROUP, FP8W8A8_ERR_BAD_SHAPE for plans whose k differ
 * or an m outside 0 <= m < FP8W8A8_MAX_ROWS, FP8W8A8_ERR_BAD_DEVICE for plans on
 * different devices, as fp8_linear_run_group does.
 */
int fp8_linear_group_config(const fp8_linear_plan* const* plans, int nplans, int64_t m, int* config_id);

/* Number of GEMM kernel configurations compiled in (ids 0 .. count-1). */
int fp8_gemm_config_count(void);

/*
 * fp8_gemm_run_config - launch one named GEMM kernel configuration directly on
 * already-quantised operands, bypassing the selector: out = epilogue(qA x qW^T).
 * It exists so that tests can hold every compiled configuration to the same
 * parity bar; arguments follow fp8_linear_create / fp8_linear_run (E4M3 kind),
 * config_id must be in [0, fp8_gemm_config_count()).
 */
int fp8_gemm_run_config(int config_id, int64_t m, int64_t n, int64_t k, const void* qa,
                        const float* a_scale, const void* w_fp8, const float* w_scale,
                        const void* bias_bf16, void* out_bf16, void* stream);

/* ---- single-launch quantisation + GEMM -------------------------------------------
 *
 * The retrospective (section 3.2) counts run-time activation quantisation and its
 * extra memory traffic among the costs of the FP8 path. fp8_quant_gemm performs the
 * per-token quantisation (bit-identical to fp8_quant_rows) and the GEMM with its
 * epilogue (bit-identical to fp8_gemm_run_config's configuration 0, 256 x 256 tiles)
 * in ONE kernel launch: the first wave of workgroups quantises the tokens in shares
 * into the workspace and publishes a flag per share; every workgroup waits until the
 * shares that hold its own tile's tokens are published (quantising itself any such
 * share whose owner has not published within 100 us, so the wait ends even when not
 * all workgroups are resident), then runs its output tile on the codes. Same result
 * as fp8_quant_rows followed by the GEMM; on MI355X it is no faster than those two
 * launches (see the bench's quant_gemm record), so fp8_linear_run keeps the two
 * launches.
 *
 * A flag holds the launch's generation number, which the host picks per call and
 * passes to the kernel. A HIP graph would replay the recorded number, and from the
 * second replay on every flag would already match before its share is rewritten, so
 * a call on a stream that is being captured is refused with FP8W8A8_ERR_CAPTURE
 * (nothing is launched or recorded).
 *
 *   m, n, k    as fp8_linear_create / fp8_linear_run (0 <= m < FP8W8A8_MAX_ROWS)
 *   a_bf16     device, bf16 [m, k], 16-byte aligned
 *   w_fp8, w_scale, bias_bf16   as fp8_linear_create
 *   out_bf16   device, bf16 [m, n], 16-byte aligned, written
 *   workspace  device, 256-byte aligned, at least fp8_quant_gemm_workspace_bytes(m, k):
 *              the codes [m, k] (rounded up to 256 bytes), then the scales [m] (likewise),
 *              then the launch flags. After the call the codes and scales hold the
 *              quantised activation. Prior contents do not matter (no clearing needed);
 *              two calls that overlap in time must not share a workspace.
 *   stream     hipStream_t or NULL, not under graph capture; one launch, no synchronisation
 */
size_t fp8_quant_gemm_workspace_bytes(int64_t m, int64_t k);
int fp8_quant_gemm(int64_t m, int64_t n, int64_t k, const void* a_bf16, const void* w_fp8,
                   const float* w_scale, const void* bias_bf16, void* out_bf16, void* workspace,
                   size_t workspace_bytes, void* stream);

/* ---- per-tensor FP8 quantisation (state-dict conversion) -------------------------
 *
 * The QuantizeFP8Format page (runcomfy.com, "Quantize Model to FP8 Format")
 * converts each tensor to float8_e4m3fn or float8_e5m2 by scaling it (no formula
 * given); the Stable Diffusion 3.5 FP8 page (dn008.com.cn, section on FP8,
 * steps 1-4) gives the steps. One scale per tensor, fmax = 448 or 57344:
 *
 *   s   = fl32(amax / fmax)            (0 for an all-zero tensor)
 *   q   = rne_sat(fl32(x / s))         (signed-zero codes when s == 0)
 *   x'  = fl32(dec(q) * s)             (fp8_dequant_tensor)
 *
 * e5m2 is the OCP E5M2 encoding (bias 15, largest finite 57344, saturating; the
 * infinity and NaN codes are never produced for finite input).
 *
 *   x_bf16     device, bf16, numel elements (any shape, flattened), 16-byte aligned
 *   numel      0 <= numel < FP8W8A8_MAX_ROWS * FP8W8A8_MAX_DIM, numel % 16 == 0 (0 is a no-op)
 *   format     FP8W8A8_FMT_E4M3FN or FP8W8A8_FMT_E5M2 (else FP8W8A8_ERR_INVALID_ARG)
 *   q_out      device, u8 codes [numel], 16-byte aligned, written
 *   scale_out  device, one fp32, 4-byte aligned, written
 *   workspace  device, fp8_quant_tensor_workspace_bytes() bytes, 16-byte aligned, scratch
 *              (per-workgroup maxima); its contents need no initialisation; two
 *              calls that overlap in time must not share it
 * Two launches on `stream`. Inputs must be finite. A tensor that fits in the registers
 * of one workgroup per compute unit (numel <= 65536 x CUs: 16.8 M elements, 32 MiB of
 * bf16, on 256 CUs) is read once: a small launch marks the maxima unwritten,
 * then the workgroups hold their shares, publish their maxima, wait for the largest
 * and quantise what they hold. Other tensors are read twice (maxima, then codes).
 */
#define FP8W8A8_FMT_E4M3FN 0
#define FP8W8A8_FMT_E5M2 1

size_t fp8_quant_tensor_workspace_bytes(void);
int fp8_quant_tensor(const void* x_bf16, int64_t numel, int format, void* q_out, float* scale_out, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * fp8_quant_tensor_form - fp8_quant_tensor with its form chosen, a test and measurement
 * hook: FP8W8A8_TENSOR_FORM_AUTO (what fp8_quant_tensor does), _ONE_PASS (returns
 * FP8W8A8_ERR_BAD_SHAPE, launching nothing, for a tensor that does not fit), _TWO_PASS,
 * or _ONE_PASS_NO_WAIT: one pass in which no workgroup waits for the others; each reads
 * the whole input for the maximum itself (the path a workgroup takes if the others have
 * not arrived within 1 ms, e.g. while another stream's kernel holds CUs). Codes and
 * scale are identical in every form. Other arguments and statuses as fp8_quant_tensor;
 * an unknown form is FP8W8A8_ERR_INVALID_ARG.
 */
#define FP8W8A8_TENSOR_FORM_AUTO 0
#define FP8W8A8_TENSOR_FORM_ONE_PASS 1
#define FP8W8A8_TENSOR_FORM_TWO_PASS 2
#define FP8W8A8_TENSOR_FORM_ONE_PASS_NO_WAIT 3
int fp8_quant_tensor_form(int form, const void* x_bf16, int64_t numel, int format, void* q_out, float* scale_out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* out_f32[i] = fl32(dec(q[i]) * *scale). q 16-byte aligned, out_f32 16-byte aligned, scale device fp32. */
int fp8_dequant_tensor(const void* q, int64_t numel, int format, const float* scale, float* out_f32, void* stream);

/* ---- FP8 weight-only linear (W8A16) --------------------------------------------
 *
 * The FP8 weight-only pipeline of the LongCat avatar comparison page
 * (longcat-avatar-compare.pages.dev, speed overview table): the weight is stored as
 * FP8 codes with per-output-channel scales (fp8_quant_weights_per_channel; a
 * per-tensor scale from fp8_quant_tensor is the same scale repeated n times), the
 * activation stays bf16 and is not quantised. w_format selects the codes:
 * FP8W8A8_FMT_E4M3FN, or FP8W8A8_FMT_E5M2 (the state-dict converter's default):
 *
 *   out[m,n] = bf16_rne( fl32( sum_k a[m,k] * dec(qW[n,k]) ) * sW[n] + bias[n] )
 *
 * The product runs on the bf16 matrix cores (every e4m3fn value is exact in bf16)
 * with fp32 accumulation; the epilogue runs in fp32 and rounds once. Layouts,
 * ownership, streams and errors are as for fp8_linear_*: a [m, k] bf16 and out
 * [m, n] bf16 row-major, 16-byte aligned; the plan borrows qW [n, k], sW [n] and
 * bias [n] (or NULL), with the same shape and alignment rules as fp8_linear_create.
 * No workspace is needed.
 */
typedef struct fp8_w8a16_plan fp8_w8a16_plan;

int fp8_w8a16_create(int device, int64_t n, int64_t k, int w_format, const void* w_fp8, const float* w_scale,
                     const void* bias_bf16, fp8_w8a16_plan** out);

/* m == 0 is a no-op. a_bf16 and out_bf16 are device pointers, 16-byte aligned. As for
 * fp8_linear_run, the plan's device must be current (else FP8W8A8_ERR_BAD_DEVICE). */
int fp8_w8a16_run(const fp8_w8a16_plan* plan, int64_t m, const void* a_bf16, void* out_bf16, void* stream);

void fp8_w8a16_destroy(fp8_w8a16_plan* plan);

/* Introspection and the test hook, as fp8_linear_plan_config / fp8_gemm_*. */
int fp8_w8a16_plan_config(const fp8_w8a16_plan* plan, int64_t m, int* config_id, int* tile_m, int* tile_n,
                          int64_t* workgroups);
int fp8_w8a16_config_count(void);
int fp8_w8a16_run_config(int config_id, int w_format, int64_t m, int64_t n, int64_t k, const void* a_bf16,
                         const void* w_fp8, const float* w_scale, const void* bias_bf16, void* out_bf16, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8W8A8_H */
