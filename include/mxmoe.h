/*
 * mxmoe.h — C ABI of libmxmoe.so, a fused MXFP4 Mixture-of-Experts layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (article "MiniMax-M3.1 on AMD Instinct GPUs: Day-0 support and
 * optimization", section "MiniMax-M3.1 at a glance"; model card
 * "amd/MiniMax-M3.1-Flash-Quark-MXFP4", section "Model Overview"):
 *
 *   logits[t,e] = sum_h x[t,h] * Wr[e,h] (+ bias[e])     fp32 router ("high precision")
 *   ids[t,:]    = top-k experts by logit (k of E; 4 of 128 in the model)
 *   w[t,j]      = softmax over the k chosen logits
 *   xq          = MXFP4(x[t])                             dynamic activation quantization
 *   g, u        = xq . W13[e] gate rows, up rows           MXFP4 x MXFP4, fp32 accumulate
 *   a           = MXFP4(silu(g) * u)
 *   d[t,j]      = a . W2[e] rows
 *   s[t]        = the same FFN in MXFP8 (shared expert, every token passes through it)
 *   y[t]        = bf16( sum_j w[t,j] * d[t,j] + s[t] (+ residual[t]) )
 *
 * Element and scale formats are those of the OCP Microscaling Formats (MX) v1.0
 * specification: E2M1 (FP4) and E4M3 (FP8, max 448, no Inf) elements, blocks
 * of 32 consecutive elements along the reduction axis sharing one E8M0 scale
 * 2^(code-127).  Conversion: block exponent floor(log2(max|v|)) - emax_elem
 * (2 for E2M1, 8 for E4M3) clamped to [-127, 127] (-127 for an all-zero
 * block), elements rounded to nearest with ties to the even code, saturated
 * to the largest finite magnitude, sign kept (also when rounding to zero).
 *
 * Conventions for every call:
 *  - All data pointers are device memory owned by the caller.  The library
 *    never allocates, frees, synchronizes or reads device data on the host
 *    (except moe_decode_status, a diagnostic); every compute call only
 *    enqueues work on `stream` and is safe to capture into a HIP graph.
 *  - Arguments are validated before anything is enqueued.  A call that
 *    returns an error has enqueued nothing.  Kernel launch failures return
 *    MOE_ERR_HIP.
 *  - bf16 tensors are passed as uint16_t bit patterns, row-major.
 *  - Calls on one stream are ordered; calls that share a workspace must not
 *    run concurrently on different streams.
 */
#ifndef MXMOE_H
#define MXMOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = -1,   /* null pointer, bad size, misaligned pointer */
  MOE_ERR_UNSUPPORTED = -2,        /* valid request this entry point does not serve (e.g. decode T > 16) */
  MOE_ERR_WORKSPACE_TOO_SMALL = -3,
  MOE_ERR_HIP = -4,                /* a HIP runtime call or kernel launch failed */
  MOE_ERR_TIMEOUT = -5             /* reported by moe_decode_status: a device-side wait gave up */
} moe_status;

enum { MX_FMT_FP4 = 0, MX_FMT_FP8 = 1 };
enum { MX_LAYOUT_ROWMAJOR = 0, MX_LAYOUT_TILED = 1 };

/*
 * Tiled MX weight layout (MX_LAYOUT_TILED), the layout every weight pointer in
 * moe_layer_t uses.  A matrix W[N][K] (N % 16 == 0, K % 128 == 0, quantized
 * along K) is cut into tiles of 16 rows x 128 columns.  Tile (nt, kt) holds TB
 * bytes (1024 for FP4, 2048 for FP8) at byte offset (nt*(K/128) + kt)*TB.
 * Inside a tile, with l = 0..63, r = 16*nt + l%16, q = l/16, j = 0..15:
 *   FP4: byte 16*l + j            = W[r][128*kt + 32*q + 2*j] (low nibble),
 *                                   W[r][128*kt + 32*q + 2*j + 1] (high nibble)
 *   FP8: byte 1024*c + 16*l + j   = W[r][128*kt + 64*c + 16*q + j], c = 0, 1
 * Scales: KG = ceil(K/512) groups of four K-tiles per 16-row strip;
 *   byte ((nt*KG + g)*64 + l)*4 + i = E8M0 scale of W[r][32*(4*(4*g+i) + q) ...],
 *   127 where 4*g + i >= K/128.
 * Each tile is exactly one operand of the gfx950 scaled matrix instruction
 * (16x16x128), so a wavefront streams weights as whole 1 KiB rows of HBM.
 *
 * Row-major MX layout (MX_LAYOUT_ROWMAJOR): codes [N][K/2] for FP4 (element 2i
 * in the low nibble of byte i) or [N][K] for FP8; scales [N][K/32].
 */
size_t mx_codes_bytes(int rows, int cols, int fmt, int layout);
size_t mx_scales_bytes(int rows, int cols, int layout);

/*
 * Static MX quantization of fp32 weights (the model card's "Routed-expert
 * weight quantization: OCP MXFP4, Static"; the shared expert is MXFP8, article
 * section "MiniMax-M3.1 at a glance").  Run once at load time.
 *   w      [rows][cols] fp32, row-major, 16-byte aligned
 *   fmt    MX_FMT_FP4 or MX_FMT_FP8; layout MX_LAYOUT_ROWMAJOR or MX_LAYOUT_TILED
 *   codes  mx_codes_bytes(rows, cols, fmt, layout) bytes, 16-byte aligned
 *   scales mx_scales_bytes(rows, cols, layout) bytes, 4-byte aligned
 * Requires cols % 32 == 0 (row-major) or rows % 16 == 0 and cols % 128 == 0 (tiled).
 */
moe_status mx_quantize_weights(const float* w, int rows, int cols, int fmt, int layout,
                               uint8_t* codes, uint8_t* scales, hipStream_t stream);

/*
 * Re-quantization of an MXFP8 matrix to MXFP4 along the same 32-element
 * blocks: each element's exact value (E4M3 value times its E8M0 scale) goes
 * through the MX conversion again with the E2M1 element type.  This is how
 * the MXFP8 shared expert becomes the MXFP4 expert folded into the table (vLLM
 * PR #64273, section "Purpose": the shared-expert re-quantization is lossy).
 * Run once at load time.
 *   codes8, scales8  MXFP8 matrix [rows][cols] in `layout` (16- / 4-byte aligned)
 *   codes4, scales4  MXFP4 output in the same layout: mx_codes_bytes(rows, cols,
 *                    MX_FMT_FP4, layout) and mx_scales_bytes(rows, cols, layout)
 * Values must be finite in fp32 (scale code and element value together below
 * 2^128).  Shape requirements as for mx_quantize_weights.
 */
moe_status mx_requant_fp8_to_fp4(const uint8_t* codes8, const uint8_t* scales8, int rows, int cols, int layout,
                                 uint8_t* codes4, uint8_t* scales4, hipStream_t stream);

/*
 * NVFP4 -> MXFP4 re-quantization: the load-time conversion of the NVFP4
 * routed experts to the MXFP4 datapath (article "MiniMax-M3.1 on AMD Instinct
 * GPUs: Day-0 support and optimization", TL;DR and section "Day 0 support for
 * AMD Instinct GPUs"; vLLM PR #64273 squash commit, "Re-quantize the NVFP4
 * routed experts to MXFP8 (or MXFP4) at load").  The pages name NVFP4 without
 * defining it; the public definition is used: E2M1 elements in blocks of 16
 * consecutive elements along a row, each block with an E4M3 scale, and an fp32
 * second-level scale.  Values v = E2M1(c) * E4M3(s_block) * s_global, the
 * last product rounded once to fp32; these go through the MX conversion with
 * the E2M1 element type (32-element blocks, E8M0 scales).
 *   codes          [rows][cols/2] packed E2M1 (element 2i in the low nibble), 16-byte aligned
 *   block_scales   [rows][cols/16] E4M3
 *   global_scales  fp32, device memory: row r uses global_scales[r / rows_per_scale]
 *                  (rows_per_scale = rows for one per-tensor scale; I for a
 *                  gate/up matrix whose two halves carry their own)
 *   codes4, scales4 MXFP4 output in `layout` (sizes as mx_codes_bytes / mx_scales_bytes)
 * Requires cols % 32 == 0 (row-major) or rows % 16 == 0 and cols % 128 == 0 (tiled).
 */
moe_status mx_requant_nvfp4_to_fp4(const uint8_t* codes, const uint8_t* block_scales, const float* global_scales,
                                   int rows_per_scale, int rows, int cols, int layout, uint8_t* codes4,
                                   uint8_t* scales4, hipStream_t stream);

/*
 * Dynamic MXFP4 quantization of bf16 activations (model card "Model
 * Overview": "Routed-expert activation quantization: OCP MXFP4, Dynamic").
 *   x      [rows][cols] bf16, 16-byte aligned, cols % 32 == 0
 *   codes  [rows][cols/2] packed E2M1 (element 2i in the low nibble of byte i)
 *   scales [rows][cols/32] E8M0
 * Exact: each element is multiplied by 2^-e (a power of two, exact in fp32)
 * and converted by gfx950's scaled fp32 -> E2M1 instruction with a unit scale,
 * which rounds to nearest even and saturates; the block exponent comes from the
 * exponent bits of the block maximum.  Codes equal the specification's for
 * every finite bf16 input.
 */
moe_status mxfp4_quant_act(const uint16_t* x, int rows, int cols, uint8_t* codes,
                           uint8_t* scales, hipStream_t stream);

/*
 * One MoE layer's weights (device pointers, caller-owned, tiled layout).
 * Routed expert e's matrices start at e * mx_codes_bytes(rows, cols, FP4, TILED)
 * bytes from w13 / w2 (scales likewise with mx_scales_bytes).
 *
 * shared_folded = 1: the shared expert is folded into the expert table (the
 * AITER fused MoE "with the shared expert optionally folded into the expert
 * table", article "MiniMax-M3.1 on AMD Instinct GPUs: Day-0 support and
 * optimization", section "Serving with vLLM / What we Optimized"; MXFP4
 * shared experts, model card section "Experimental MXFP4 shared experts").
 * w13 / w2 then hold E + 1 experts; expert E (index num_experts) is the shared
 * expert in MXFP4 (mx_requant_fp8_to_fp4 makes it from the MXFP8 one) and is
 * selected for every token with weight 1, after the k routed choices:
 *   y[t] = bf16( sum_{j<k} w[t,j] d[t,j] + d_shared[t] (+ residual[t]) ).
 * The router still chooses among experts 0..E-1.  Requires shared_inter = 0
 * (the ws* pointers are ignored), top_k <= 7 and num_experts <= 255.
 * shared_folded = 0: an MXFP8 shared expert as given by shared_inter / ws*.
 *
 * norm_weight != NULL: the RMSNorm in front of the router is fused into the
 * layer call (mono decode fuses "the RMSNorm and router", article section
 * "Serving with vLLM / What we Optimized").  The call's input is then the
 * residual stream h, and with g = norm_weight
 *   r[t] = 1 / sqrtf(S[t] / H + norm_eps),  S[t] = sum_h h[t,h]^2 in fp32
 *          (lane l of a wavefront FMAs h = 256 i + 4 l + c, i ascending,
 *          c = 0..3, then a butterfly over lane distances 32 .. 1)
 *   x[t,h] = (h[t,h] * r[t]) * g[h]          two fp32 products, no bf16 step
 * x feeds the router and the MX quantizers, and h itself is added back:
 *   y[t] = bf16( h[t] + sum_j w[t,j] d[t,j] + s[t] ).
 * The residual argument of the layer calls must then be NULL.
 */
typedef struct {
  int32_t hidden;        /* H: multiple of 128 */
  int32_t inter;         /* I: routed expert intermediate size, multiple of 128 */
  int32_t num_experts;   /* E: 1..256 */
  int32_t top_k;         /* k: 1..min(E, 8) */
  int32_t shared_inter;  /* I_s: shared expert intermediate size, multiple of 128, or 0 for none */
  const float* router_w;      /* [E][H] fp32 row-major */
  const float* router_bias;   /* [E] fp32 added to the logits, or NULL */
  const uint8_t* w13;         /* E x tiled FP4 [2I][H]: rows 0..I-1 gate, I..2I-1 up */
  const uint8_t* w13_scale;
  const uint8_t* w2;          /* E x tiled FP4 [H][I] */
  const uint8_t* w2_scale;
  const uint8_t* ws13;        /* tiled FP8 [2I_s][H] (gate rows first), NULL if I_s == 0 */
  const uint8_t* ws13_scale;
  const uint8_t* ws2;         /* tiled FP8 [H][I_s], NULL if I_s == 0 */
  const uint8_t* ws2_scale;
  int32_t shared_folded;      /* 0 or 1, see above */
  const float* norm_weight;   /* [H] fp32 pre-router RMSNorm weight, or NULL (see below) */
  float norm_eps;             /* its epsilon */
} moe_layer_t;

/*
 * Router and top-k (article "MiniMax-M3.1 at a glance": 4 of 128 routed
 * experts per token; routers kept in high precision).
 *   x        [T][H] bf16
 *   logits   [T][E] fp32 output, or NULL.  Passing a buffer also selects the
 *            expert-parallel kernel (tiles of 16 rows x 32 experts over the
 *            whole GPU, then a top-k pass); without one, a workgroup takes 8
 *            rows and loops over all E experts, which is many times slower
 *            (about 290 us for up to 8 rows of the MiniMax-M3.1 router, against
 *            35 us for 64 rows with a buffer, on one MI355X).  Both give the
 *            same results bit for bit.
 *   topk_ids [T][k] int32: the k largest logits in descending order; equal
 *            logits go to the lower expert index
 *   topk_w   [T][k] fp32: softmax over the k chosen logits
 * Logit arithmetic (fixed, independent of T): lane l = 0..63 accumulates with
 * fp32 FMA, in order, the products x[t][h]*Wr[e][h] for h = 256*i + 4*l + c
 * (i ascending, c = 0..3); the 64 partial sums are added by a butterfly over
 * lane distances 32, 16, 8, 4, 2, 1; then bias[e] is added.  The fused decode
 * call uses the same arithmetic, so both produce identical logits.
 */
moe_status moe_router_topk(const moe_layer_t* layer, const uint16_t* x, int T, float* logits,
                           int32_t* topk_ids, float* topk_w, hipStream_t stream);

/*
 * Token sort by expert: a stable counting sort of the slots s = t*k + j by
 * topk_ids[t][j], each expert's segment padded to a multiple of block_m.
 * This is the step that turns routed tokens into per-expert row blocks for a
 * grouped fused-MoE GEMM (the AITER MXFP4 fused MoE the article "MiniMax-M3.1
 * on AMD Instinct GPUs: Day-0 support and optimization" runs outside mono
 * decode, section "Serving with vLLM / What we Optimized"; the pages do not
 * spell the sort out, so the padded counting sort is this library's reading).
 *   sorted_slots   moe_align_sort_capacity(T, k, E, block_m) int32: slots grouped
 *                  by expert (experts ascending, slots ascending inside), each
 *                  segment padded with T*k; entries past num_padded are T*k
 *   block_expert   capacity / block_m int32: expert owning each block of block_m
 *                  entries; -1 past the last block
 *   expert_offsets [E+1] int32: exclusive scan of the unpadded counts
 *   num_padded     [1] int32: total padded length
 *   ws             moe_align_sort_workspace_bytes(T, k, E) bytes of scratch
 */
size_t moe_align_sort_capacity(int T, int k, int E, int block_m);
size_t moe_align_sort_workspace_bytes(int T, int k, int E);
moe_status moe_align_sort(const int32_t* topk_ids, int T, int k, int E, int block_m,
                          int32_t* sorted_slots, int32_t* block_expert, int32_t* expert_offsets,
                          int32_t* num_padded, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Workspace for the fused calls.  path 0: fused_moe_mxfp4_decode (T <= 64; a
 * workspace sized for T <= 16 serves only steps of up to 16 rows, one sized for
 * 17 <= T <= 64 serves every step), path 1: fused_moe_mxfp4_grouped (any T).
 * Returns 0 for invalid arguments.
 * A decode workspace must be zero-filled once (moe_workspace_init) before its
 * first use.  Each decode call tags the words it hands between workgroups
 * with a 32-bit call counter kept in the workspace; the call that would make
 * the counter wrap clears every tagged word itself, so a workspace serves any
 * number of calls without re-initialization (and steps of any size in its
 * range).  After moe_decode_status reports
 * MOE_ERR_TIMEOUT the workspace must be zero-filled again: until then every
 * decode call on it writes NaN (bf16 0x7FC0) to y and computes nothing.
 */
size_t moe_workspace_bytes(const moe_layer_t* layer, int T, int path);
moe_status moe_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The whole layer for 1..64 rows in ONE kernel launch ("mono decode": one
 * fused kernel launch per MoE layer for a pure decode of at most 16 tokens,
 * article section "Serving with vLLM / What we Optimized"; the monokernel's
 * "rows (1..16)", vLLM PR #64273 section "Test Result"; and the wider steps
 * the article names as its next kernel item, section "What's next").  Steps
 * of 17..64 rows run an instance that takes every unit's rows in 16-row
 * groups on the same weight tiles, so a step still reads each selected
 * expert's weights once.
 *   x         [T][H] bf16, T in 1..64 (MOE_ERR_UNSUPPORTED otherwise, and for
 *             17..64 rows on shapes whose wide instance does not fit the LDS)
 *   residual  [T][H] bf16 added before the single bf16 rounding, or NULL
 *   y         [T][H] bf16 output; may alias residual, must not alias x
 *   ws        moe_workspace_bytes(layer, T, 0) bytes, zero-filled before first use
 *   topk_ids_out [T][k], topk_w_out [T][k]: routing result, or NULL
 * Arithmetic: every dot product is cut into NC K-chunks of 128-wide tiles (NC =
 * 4, else 2, else 1: the largest that divides K/128); a chunk is one chain of
 * scaled 16x16x128 matrix instructions from zero in tile order and the chunk
 * sums are added in chunk order in fp32; SwiGLU, re-quantization and the
 * combine order are those of the oracle.  fused_moe_mxfp4_grouped uses the same
 * arithmetic, so both give identical bits for the same rows.
 * Output row t depends only on x[t] (and residual[t]): results are bit-identical
 * for any T (1..64, either instance) and any row order.  Shapes whose gate/up K-chunk is longer than 6
 * tiles ((H/128)/NC > 6), or whose staged x and intermediates exceed the
 * 160 KiB of LDS, give MOE_ERR_UNSUPPORTED (the grouped call handles them).  The launch is a persistent grid sized to the
 * device's co-resident capacity; its device-side waits are bounded, and a wait
 * that gives up marks the workspace (see moe_decode_status) instead of hanging.
 */
moe_status fused_moe_mxfp4_decode(const moe_layer_t* layer, const uint16_t* x, int T,
                                  const uint16_t* residual, uint16_t* y, void* ws, size_t ws_bytes,
                                  int32_t* topk_ids_out, float* topk_w_out, hipStream_t stream);

/*
 * fused_moe_mxfp4_decode (steps of 1..16 rows) without a workspace argument,
 * for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is the library's own: a
 * static device array of 8 MiB per GPU, held until the process ends, whose
 * address is looked up once per device.  The first call on a device also
 * zero-fills it, with a kernel on `stream` ahead of the layer's launch.  This
 * call allocates nothing and calls no allocating routine.
 *   arguments, results and arithmetic as for fused_moe_mxfp4_decode.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (different streams, or concurrent host threads with their first
 * calls) race on it and must not be made.  The array keeps the last call's
 * contents; the call-tag protocol of the decode workspace makes that safe for
 * the next call.  A layer whose decode workspace (moe_workspace_bytes with
 * path 0) exceeds 8 MiB gives MOE_ERR_WORKSPACE_TOO_SMALL.  A timed-out wait
 * poisons the array for the rest of the process (outputs NaN, see
 * moe_workspace_bytes); moe_decode_status cannot inspect it.
 */
moe_status fused_moe_mxfp4_decode_noalloc(const moe_layer_t* layer, const uint16_t* x, int T,
                                          const uint16_t* residual, uint16_t* y, int32_t* topk_ids_out,
                                          float* topk_w_out, hipStream_t stream);

/*
 * The layer for any number of rows (prefill and steps wider than 16 rows,
 * which the pages keep on the standard path: article section "Performance,
 * mono decode on vs off").  Several launches: router + top-k, token sort,
 * activation quantization, grouped gate/up and down GEMMs on scaled FP4
 * matrix instructions, the MXFP8 shared expert, and the combine.
 *   x, residual, y as for the decode call; T >= 1
 *   ws  moe_workspace_bytes(layer, T, 1) bytes (no initialization needed)
 * The steps that do not depend on the routing (the quantization of x, the
 * shared gate/up GEMM) run on a second stream that the library creates on
 * each device at its first call there (default priority, kept until the
 * process ends), forked from `stream` before the router and joined back
 * into it before the steps that use their results: all of the call's work
 * is ordered after earlier work on `stream` and before later work on it, as
 * for a single stream.  Calls on one device from several host threads take turns on that
 * stream.  While `stream` is being captured into a graph every step runs on
 * `stream` itself.
 */
moe_status fused_moe_mxfp4_grouped(const moe_layer_t* layer, const uint16_t* x, int T,
                                   const uint16_t* residual, uint16_t* y, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/*
 * Diagnostic: fused_moe_mxfp4_grouped with every step on `stream`, in the
 * order below, an event recorded on `stream` before each of its launch steps
 * and one at the end, so that a caller can time them (hipEventElapsedTime).
 * events[0..7], caller-created, non-NULL:
 *   0 router and top-k, 1 token sort, 2 MX quantization of x, 3 routed
 *   gate/up GEMM, 4 routed down GEMM, 5 shared gate/up GEMM (the combine
 *   kernel when there is no shared expert), 6 shared down GEMM with the
 *   combine (nothing without a shared expert), 7 end.
 * Results and errors as for fused_moe_mxfp4_grouped.
 */
moe_status fused_moe_mxfp4_grouped_timed(const moe_layer_t* layer, const uint16_t* x, int T,
                                         const uint16_t* residual, uint16_t* y, void* ws, size_t ws_bytes,
                                         const hipEvent_t* events, hipStream_t stream);

/*
 * Diagnostic (synchronizes the device): MOE_OK if no fused decode call on this
 * workspace has given up a device-side wait, MOE_ERR_TIMEOUT otherwise.  A
 * call whose wait gives up writes NaN to the output columns it combines after
 * that point; later calls write NaN everywhere (see moe_workspace_bytes).
 */
moe_status moe_decode_status(const void* ws, size_t ws_bytes);

/*
 * Diagnostic (synchronizes the device): phase timestamps of the last fused
 * decode call on this workspace, in ticks of the device's 100 MHz constant
 * clock.  Workgroup g fills words [16g, 16g+16): 0 launch start; 1 its
 * router / shared gate/up units done; 2 all logits seen; 3 routing known; 4
 * its routed gate/up units done (0 if it had none); 5 its down units and
 * combines done; 6 end of its first router or shared unit (0 if it had none);
 * 7 its MXFP4 (and, in a shared unit, MXFP8) copy of x in LDS; 8 top-k done;
 * 9 expert list done; for its first routed gate/up unit 10 matrix products
 * done and 11 results stored; 12 a shared unit's matrix products done; 13 its
 * first routed gate/up unit released; 14 its first down unit's intermediate
 * staged (0 where it had no such unit); 15 the time its first load (the
 * call's epoch word) returned.
 * Copies at most n_words words to host memory and returns
 * the number of workgroups of that call (0 if none ran yet), or a negative
 * moe_status.
 */
int moe_decode_trace(const moe_layer_t* layer, const void* ws, size_t ws_bytes, uint64_t* host,
                     size_t n_words);

const char* moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MXMOE_H */
