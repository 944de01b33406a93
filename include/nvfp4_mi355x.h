/*
 * nvfp4_mi355x.h -- C ABI of the MI355X (gfx950) NVFP4 hot path.
 *
 * NVFP4 in this library: values in 16-element K-blocks; each block stores 16
 * E2M1 (FP4) codes packed two per byte (element 2i in bits 3..0, element 2i+1
 * in bits 7..4), one FP8-E4M3 block scale byte, and shares one FP32 global
 * scale per row (per token), per tensor or per expert.  The format and operand
 * shapes follow "Fused Nvfp4 GEMM All Reduce Plugin" (TensorRT-Edge-LLM C++
 * API), section "Baked-weight inputs": activation FP4 [B,K], activation_scale
 * FP32 [B,1,K/16] (the combined scale from DequantizeLinear), weight FP4 [N,K],
 * weight FP8 block scale [N,K/16], scalar FP32 global weight scale, FP16 [B,N]
 * output.  Per-token activation globals follow "perf: optimize per-token nvfp4
 * quantization kernel" (flashinfer pull request 3237), description.
 *
 * Quantization arithmetic (binary32, round-to-nearest-even, exact division):
 *   amax    = max |y| over the global group
 *   g_enc   = 2688 / amax   (2688 = 448 * 6), replaced by FLT_MAX if not finite
 *   g_dec   = 1 / g_enc     -- the FP32 global scale that is stored
 *   per block: sf = E4M3_RNE(min((amax_b / 6) * g_enc, 448))
 *              c  = e4m3(sf) * g_dec        -- combined scale, [rows,1,K/16]
 *              enc = (c == 0) ? 0 : 1 / c
 *   per element: code = E2M1_RNE_saturating(y * enc), sign kept (-0 -> 0x8)
 * Dequantization: activation x = e2m1(code) * c; weight w = e2m1(code) *
 * e4m3(sf) * g_dec.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless stated; the caller allocates every
 *    buffer and keeps it alive until the stream work completes.  The library
 *    never allocates or frees, and keeps a pointer past the call only for a
 *    registered external weight (until it is unregistered).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls are asynchronous and stream-ordered; they never synchronize.
 *  - Arguments are validated on the host before anything is launched: on any
 *    error status nothing has been written.  Kernel faults surface at the
 *    caller's next synchronization.
 *  - Rows and strides are dense and row-major; leading dimensions are
 *    flattened into rows by the caller.  Offsets are 64-bit.
 *  - Inputs that are not 16-byte aligned take a scalar path with identical
 *    results ("Building Custom TensorRT-LLM Plugins for Low-Latency FP8
 *    Inference at Scale", "Production Pitfalls & Hard Lessons", item 1).
 *  - Re-entrant; no mutable state besides a per-device property cache filled
 *    on first use and the external-weight registry (nvfp4_register_weight,
 *    guarded by a lock).  Temporary memory comes from the caller's workspace
 *    (same article, item 3).
 */
#ifndef NVFP4_MI355X_H
#define NVFP4_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define NVFP4_OK 0
#define NVFP4_EINVAL 1        /* null pointer, bad size, bad enum, K % 16 != 0 */
#define NVFP4_EUNSUPPORTED 2  /* current device is not gfx950, or size beyond limits */
#define NVFP4_EWORKSPACE 3    /* workspace missing or smaller than the query returns */
#define NVFP4_EHIP 4          /* a HIP runtime call or launch failed */
#define NVFP4_ESCRATCH 5      /* needs more than the fixed scratch of a no-allocation entry point */

/* Input element types. */
#define NVFP4_BF16 0
#define NVFP4_FP16 1

/* Activations fused in front of the quantizer. */
#define NVFP4_ACT_NONE 0
#define NVFP4_ACT_SWIGLU 1    /* y = silu(gate) * up; gate = first half of the row */
#define NVFP4_ACT_RELU2 2     /* y = max(x, 0)^2 */

/* Human-readable name of a status code (static string, never NULL). */
const char* nvfp4_status_string(int32_t status);

/*
 * nvfp4_quantize -- NVFP4-quantize x[rows, k] with one FP32 global per group
 * of `group_rows` consecutive rows: 1 = per token (activations), rows = per
 * tensor (the scalar weight_f32_scale of the plugin contract), rows/E = per
 * expert ("Nvfp4 A16 Blackwell Moe Runner", globalScales [E]).
 *   x          : [rows, k] bf16 or fp16 (dtype), device
 *   codes      : [rows, k/2] uint8 out
 *   sf         : [rows, k/16] uint8 out (E4M3 bytes)
 *   g_dec      : [rows / group_rows] float out (stored global scale)
 *   scale_out  : [rows, k/16] float out, combined scale c; may be NULL
 *   workspace  : device scratch of nvfp4_quantize_workspace_size() bytes
 *                (0 bytes when group_rows == 1; then may be NULL)
 * Requires rows >= 0, k > 0, k % 16 == 0, group_rows >= 1 dividing rows.
 * rows == 0 is a no-op.
 */
int32_t nvfp4_quantize(const void* x, int32_t dtype, int64_t rows, int64_t k, int64_t group_rows,
                       uint8_t* codes, uint8_t* sf, float* g_dec, float* scale_out,
                       void* workspace, size_t workspace_bytes, void* stream);
size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t k, int64_t group_rows);

/*
 * nvfp4_act_quant -- fused activation + per-token NVFP4 quantization: the
 * activation is evaluated in fp32 registers and never written back
 * ("Building Custom TensorRT-LLM Plugins for Low-Latency FP8 Inference at
 * Scale", "The Cost of Non-Fused Quantization" and "Fusing the Kernel in CUDA";
 * ReLU2 from "Nvfp4 A16 Blackwell Moe Runner").
 *   x       : [rows, 2*k_out] for SWIGLU (gate | up), else [rows, k_out]
 *   codes   : [rows, k_out/2], sf: [rows, k_out/16], g_dec: [rows],
 *   scale_out: [rows, k_out/16] or NULL.
 * SwiGLU's exp is a fixed binary32 evaluation: for x > 88.75 it is +inf, for
 * x < -87 it is 0, else with n = rint(x * fp32(log2 e)),
 * r = fma(-n, fp32(ln 2), x), r = fma(-n, fp32(ln 2 - fp32(ln 2)), r),
 * p = Horner-with-fma of sum_{k<=7} fp32(1/k!) r^k, result ldexp(p, n);
 * then silu(g) = g / (1 + exp(-g)) with exact division.
 * Requires k_out % 16 == 0, rows >= 0.
 */
int32_t nvfp4_act_quant(const void* x, int32_t dtype, int64_t rows, int64_t k_out, int32_t act,
                        uint8_t* codes, uint8_t* sf, float* g_dec, float* scale_out, void* stream);

/*
 * nvfp4_gemm -- y[B,N] (fp16) = sum_k deq(a)[B,k] * deq(w)[N,k], the GEMM of
 * "Fused Nvfp4 GEMM All Reduce Plugin" (baked-weight inputs 0..4, output 0)
 * on one rank's K-share; the all-reduce is not part of this library.
 *   a        : [B, K/2] uint8 activation codes
 *   a_scale  : [B, K/16] float combined activation scale ([B,1,K/16])
 *   w        : [N, K/2] uint8 weight codes
 *   w_sf     : [N, K/16] uint8 E4M3 weight block scales
 *   w_gscale : pointer to ONE float on the device, the global weight scale
 *   y        : [B, N] fp16 out (round-to-nearest-even from fp32 accumulation)
 *   workspace: nvfp4_gemm_workspace_size() bytes, 256-byte aligned (the size
 *              may be 0 -> NULL allowed); EWORKSPACE if smaller or misaligned
 * Requires B >= 0, N > 0, K > 0, K % 16 == 0 (whole 16-blocks, the [N, K/16]
 * block scale of the plugin contract); a_scale and w_gscale 4-byte aligned,
 * y 2-byte aligned (EINVAL otherwise).  w and w_sf may have any alignment:
 * weights whose rows are not 16-byte aligned (w not 16-byte aligned, w_sf
 * not 2-byte aligned, or K % 32 == 16) take a byte-load path with the same
 * arithmetic, so its results are bit-identical to those of the aligned path
 * on the same values ("Building Custom TensorRT-LLM Plugins for Low-Latency
 * FP8 Inference at Scale", "Production Pitfalls & Hard Lessons", item 1).
 * B == 0 is a no-op.
 */
int32_t nvfp4_gemm(const uint8_t* a, const float* a_scale, const uint8_t* w, const uint8_t* w_sf,
                   const float* w_gscale, void* y, int64_t B, int64_t N, int64_t K,
                   void* workspace, size_t workspace_bytes, void* stream);
size_t nvfp4_gemm_workspace_size(int64_t B, int64_t N, int64_t K);

/*
 * Pre-tiled weights: the offline reordering of the weight codes and E4M3
 * bytes into the order the GEMM's lanes read them -- the role of the baked
 * N128_K64 weight tiling of "Nvfp4 A16 Blackwell Moe Runner" (fc1/fc2 weight
 * layout) and of the weight shuffles of "feature: add fp4 mm using trtllm
 * backend", done for gfx950's lanes.  Layout: row group G = rows 16G..16G+15;
 * for each 128-k chunk c a 1 KiB tile of codes whose 16-byte lane l = r + 16q
 * (r < 16, q < 4) holds the 32 codes of row 16G + r at k = 128c + 32q .. +31
 * (same packing as [N, K/2]), and a 128-byte tile of E4M3 bytes whose 2-byte
 * lane l holds that row's two block scales for those 32 k.  Tiles are stored
 * row group by row group, chunk by chunk: codes [N/16][K/128][64][16 B] (N*K/2
 * bytes), E4M3 bytes [N/16][K/128][64][2 B] (N*K/16 bytes).
 *
 * nvfp4_pretile_weight -- writes that layout from [N, K/2] codes and
 * [N, K/16] E4M3 bytes (a permutation; the inputs are not modified).
 *   w_tiled : N*K/2 bytes, 16-byte aligned; sf_tiled: N*K/16 bytes, 4-byte aligned
 * Requires N % 16 == 0, K % 128 == 0, K <= 2^24; w 16-byte and w_sf 2-byte
 * aligned (EINVAL / EUNSUPPORTED otherwise).
 */
int32_t nvfp4_pretile_weight(const uint8_t* w, const uint8_t* w_sf, int64_t N, int64_t K,
                             uint8_t* w_tiled, uint8_t* sf_tiled, void* stream);
/*
 * nvfp4_gemm_pretiled -- nvfp4_gemm with the weight operands in the
 * pre-tiled layout.  Same arithmetic and results as nvfp4_gemm on the
 * untiled weights (bit-identical output), same workspace
 * (nvfp4_gemm_workspace_size, 256-byte aligned).  Requires N % 16 == 0,
 * K % 128 == 0, K <= 2^24, w_tiled 16-byte and sf_tiled 4-byte aligned.
 */
int32_t nvfp4_gemm_pretiled(const uint8_t* a, const float* a_scale, const uint8_t* w_tiled,
                            const uint8_t* sf_tiled, const float* w_gscale, void* y, int64_t B,
                            int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * External-weight mode of "Fused Nvfp4 GEMM All Reduce Plugin" (sections
 * "External-weight inputs", "Attributes" and the register / unregister
 * functions): the packed weight and its E4M3 block scale live outside the
 * call, registered once per (device, resource id); the GEMM then names the
 * resource instead of passing the two weight pointers.
 *
 * nvfp4_register_weight -- records (device, resource_id) -> (weight, scale,
 * out_features = N, in_features = K, scale_cols = K/16).  Host-only: no HIP
 * call, no copy; the pointers must stay valid for every GEMM that uses the
 * resource, and the caller unregisters before releasing the storage.
 *   weight : [N, K/2] uint8 device codes (any alignment, as for nvfp4_gemm)
 *   scale  : [N, K/16] uint8 device E4M3 bytes
 * Requires device >= 0, resource_id >= 0 (a negative id means baked-weight
 * mode in the plugin and is rejected here), N > 0, K > 0, K % 16 == 0,
 * scale_cols == K/16, and (device, resource_id) not registered yet; EINVAL
 * otherwise (the registry is unchanged on error).
 */
int32_t nvfp4_register_weight(int32_t device, int32_t resource_id, const uint8_t* weight,
                              const uint8_t* scale, int32_t out_features, int32_t in_features,
                              int32_t scale_cols);
/* Removes (device, resource_id); EINVAL if it is not registered. */
int32_t nvfp4_unregister_weight(int32_t device, int32_t resource_id);
/*
 * nvfp4_gemm_external -- nvfp4_gemm with the weight and block scale of the
 * resource registered for (current device, resource_id); the inputs are those
 * of the plugin's external-weight mode: activation codes [B, K/2], combined
 * activation scale [B, K/16], global weight scale (one device float).  N and
 * K must equal the registered out/in features (EINVAL otherwise, as for an
 * unknown resource).  Same kernels, results and workspace as nvfp4_gemm.
 */
int32_t nvfp4_gemm_external(const uint8_t* a, const float* a_scale, int32_t resource_id,
                            const float* w_gscale, void* y, int64_t B, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_moe_w4a16 -- routed MoE layer with NVFP4 weights and FP16
 * activations ("Nvfp4 A16 Blackwell Moe Runner", Nvfp4A16BlackwellMoeParams):
 * sigmoid group-top-k routing with a correction bias, then per chosen expert
 * out_t += w_tj * (relu(x_t . W1_e^T)^2) . W2_e^T.
 *   router_logits   : [tokens, experts] float
 *   correction_bias : [experts] float (used for selection only)
 *   x               : [tokens, hidden] fp16
 *   w1, w1_sf, w1_g : [experts, inter, hidden/2] u8, [experts, inter, hidden/16] u8,
 *                     [experts] float  (fc1, per-expert global)
 *   w2, w2_sf, w2_g : [experts, hidden, inter/2] u8, [experts, hidden, inter/16] u8,
 *                     [experts] float  (fc2)
 *   out             : [tokens, hidden] fp16
 *   topk_ids_out    : [tokens, top_k] int32 or NULL (chosen experts, best first)
 *   topk_w_out      : [tokens, top_k] float or NULL (their weights)
 * Routing: s = 1/(1+exp(-l)) (exp as for nvfp4_act_quant), b = s + bias;
 * group score = sum of the group's two best b; keep topk_group groups; pick
 * top_k experts by b inside them (ties to the lower index); weights s, divided
 * by their sum when norm_topk_prob, times routed_scaling.
 * Requires experts % n_group == 0, 1 <= topk_group <= n_group,
 * 1 <= top_k <= topk_group * experts / n_group, top_k <= 16, experts <= 256,
 * hidden % 64 == 0, inter % 64 == 0, inter <= 8192, hidden * inter <= 2^31,
 * tokens <= 2^24; x, w1, w2 16-byte aligned, out 8-byte aligned, block scales
 * 4-byte aligned (EINVAL otherwise).
 */
int32_t nvfp4_moe_w4a16(const float* router_logits, const float* correction_bias, const void* x,
                        const uint8_t* w1, const uint8_t* w1_sf, const float* w1_g,
                        const uint8_t* w2, const uint8_t* w2_sf, const float* w2_g, void* out,
                        int32_t* topk_ids_out, float* topk_w_out,
                        int32_t tokens, int32_t experts, int32_t top_k, int32_t hidden, int32_t inter,
                        int32_t n_group, int32_t topk_group, int32_t norm_topk_prob,
                        float routed_scaling, void* workspace, size_t workspace_bytes, void* stream);
size_t nvfp4_moe_w4a16_workspace_size(int32_t tokens, int32_t experts, int32_t top_k, int32_t hidden,
                                      int32_t inter);

/*
 * nvfp4_moe_w4a16_pretiled -- nvfp4_moe_w4a16 with the expert weights in the
 * pre-tiled layout (offline weight preparation, as for nvfp4_gemm_pretiled):
 *   w1, w1_sf : nvfp4_pretile_weight of the stacked fc1 weights viewed as one
 *               [experts * inter, hidden] matrix (codes [experts * inter,
 *               hidden/2], E4M3 bytes [experts * inter, hidden/16])
 *   w2, w2_sf : the same of the stacked fc2 weights [experts * hidden, inter]
 * A 16-row group never spans two experts, so expert e's tiles are the bytes
 * at the same offsets as its rows in the plain layout.  Same routing,
 * arithmetic and results as nvfp4_moe_w4a16 (bit-identical output), same
 * workspace.  Requires hidden % 128 == 0 and inter % 128 == 0 besides the
 * conditions of nvfp4_moe_w4a16 (EINVAL otherwise).
 */
int32_t nvfp4_moe_w4a16_pretiled(const float* router_logits, const float* correction_bias,
                                 const void* x, const uint8_t* w1, const uint8_t* w1_sf,
                                 const float* w1_g, const uint8_t* w2, const uint8_t* w2_sf,
                                 const float* w2_g, void* out, int32_t* topk_ids_out,
                                 float* topk_w_out, int32_t tokens, int32_t experts, int32_t top_k,
                                 int32_t hidden, int32_t inter, int32_t n_group,
                                 int32_t topk_group, int32_t norm_topk_prob, float routed_scaling,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_moe_w4a16_noalloc -- nvfp4_moe_w4a16 for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and the same results (bit-identical).  Its scratch is a fixed
 * device array of NVFP4_NOALLOC_SCRATCH_BYTES inside the library; each GPU the
 * library runs on holds its own copy from the first call until the process
 * ends.  The call allocates and frees nothing.
 *   Returns NVFP4_ESCRATCH (nothing launched) when
 *   nvfp4_moe_w4a16_workspace_size(tokens, experts, top_k, hidden, inter)
 *   exceeds NVFP4_NOALLOC_SCRATCH_BYTES (32 MiB: e.g. up to ~400 tokens at
 *   64 experts, top-8, hidden 2048, inter 1024); otherwise as nvfp4_moe_w4a16.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (concurrent streams, or host threads without ordering between
 * their streams) race and give undefined results.  No part of the scratch
 * needs to start at zero: every word a call reads was written earlier in the
 * same call, so contents left by the previous call do not matter.
 */
#define NVFP4_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
int32_t nvfp4_moe_w4a16_noalloc(const float* router_logits, const float* correction_bias,
                                const void* x, const uint8_t* w1, const uint8_t* w1_sf,
                                const float* w1_g, const uint8_t* w2, const uint8_t* w2_sf,
                                const float* w2_g, void* out, int32_t* topk_ids_out,
                                float* topk_w_out, int32_t tokens, int32_t experts, int32_t top_k,
                                int32_t hidden, int32_t inter, int32_t n_group, int32_t topk_group,
                                int32_t norm_topk_prob, float routed_scaling, void* stream);

/*
 * MXFP4 variant -- the UE8M0_SF switch of the block helper in "perf: optimize
 * per-token nvfp4 quantization kernel" (review): 32-element K-blocks whose
 * scale is one E8M0 byte b (value 2^(b-127)), the format gfx950's block-scaled
 * MFMA consumes directly.  Arithmetic as for NVFP4 (same global scale per
 * group of rows), except per block:
 *   sf = smallest power of two >= (amax_b / 6) * g_enc, saturating at 2^127
 *        (byte 254; also for NaN), at least 2^-127 (byte 0)
 *   c  = sf * g_dec,  enc = (c == 0) ? 0 : 1 / c,  code = E2M1_RNE_sat(y * enc)
 * so no element of a block saturates.  Dequantization: e2m1(code) * 2^(b-127)
 * * g_dec.
 *
 * MX tile layout (the operand order of the MFMA's lanes), for an operand of
 * R rows and K columns (K % 128 == 0): rows padded to R32 = 32*ceil(R/32);
 * row group G = rows 32G..32G+31.
 *   codes : per (G, 64-k chunk c) a 1 KiB tile; its 16-byte lane l = r + 32h
 *           (r < 32, h < 2) holds the 32 codes of row 32G + r at k = 64c + 32h
 *           .. +31, packed as in [R, K/2].  [R32/32][K/64][64][16 B] = R32*K/2 bytes.
 *   scales: per (G, 128-k chunk c) a 128-byte tile; its 2-byte lane l = r + 32h
 *           holds in byte j the E8M0 byte of block 4c + 2j + h of row 32G + r.
 *           [R32/32][K/128][64][2 B] = R32*K/32 bytes.
 * Padding rows hold zero codes and zero scale bytes.
 */
#define NVFP4_MX_ROWS 0    /* codes [rows, k/2], E8M0 bytes [rows, k/32] */
#define NVFP4_MX_TILED 1   /* the MX tile layout */

/*
 * nvfp4_mx_quantize -- MXFP4 quantization of x with the optional activation
 * of nvfp4_act_quant in front (act != NONE needs group_rows == 1).
 *   x         : [rows, k_in] bf16 or fp16, 16-byte aligned (k_in = 2*k for SWIGLU)
 *   layout    : NVFP4_MX_ROWS (k % 32 == 0) or NVFP4_MX_TILED (k % 128 == 0;
 *               codes R32*k/2 bytes, sf R32*k/32 bytes, padding rows written)
 *   codes, sf : outputs in that layout; codes 4-byte aligned
 *   g_dec     : [rows / group_rows] float out
 *   workspace : nvfp4_quantize_workspace_size(rows, k, group_rows) bytes
 * Requires k <= 32768 (the row is held in registers), rows % group_rows == 0.
 */
int32_t nvfp4_mx_quantize(const void* x, int32_t dtype, int64_t rows, int64_t k, int32_t act,
                          int64_t group_rows, int32_t layout, uint8_t* codes, uint8_t* sf,
                          float* g_dec, void* workspace, size_t workspace_bytes, void* stream);
/*
 * nvfp4_mx_tile -- writes the MX tile layout from [rows, k/2] codes and
 * [rows, k/32] E8M0 bytes (a permutation; padding rows zero).  Offline for
 * weights.  Requires k % 128 == 0, k <= 2^24; codes and codes_tiled 16-byte,
 * sf_tiled 2-byte aligned.
 */
int32_t nvfp4_mx_tile(const uint8_t* codes, const uint8_t* sf, int64_t rows, int64_t k,
                      uint8_t* codes_tiled, uint8_t* sf_tiled, void* stream);
/*
 * nvfp4_mx_gemm -- y[B,N] (fp16) = sum_k deq(a)[B,k] * deq(w)[N,k] for MXFP4
 * operands in the MX tile layout, on v_mfma_scale_f32_32x32x64_f8f6f4 (FP4 x
 * FP4 with the E8M0 bytes as the instruction's block scales; fp32
 * accumulation; y = fp16_RNE(acc * (a_g[row / a_group_rows] * w_gscale[0]))).
 *   a_tiled, a_sf_tiled : activation tiles (B rows), e.g. from nvfp4_mx_quantize
 *   a_g                 : [B / a_group_rows] float activation globals (1 = per token)
 *   w_tiled, w_sf_tiled : weight tiles (N rows), e.g. from nvfp4_mx_tile
 *   w_gscale            : one device float
 *   y                   : [B, N] fp16, 16-byte aligned
 * Requires N % 32 == 0, K % 128 == 0, K <= 2^24, B % a_group_rows == 0;
 * tiles 16-byte and scale tiles, a_g, w_gscale 4-byte aligned.  B == 0 is a no-op.
 */
int32_t nvfp4_mx_gemm(const uint8_t* a_tiled, const uint8_t* a_sf_tiled, const float* a_g,
                      int64_t a_group_rows, const uint8_t* w_tiled, const uint8_t* w_sf_tiled,
                      const float* w_gscale, void* y, int64_t B, int64_t N, int64_t K, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_MI355X_H */
