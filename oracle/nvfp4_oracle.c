/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for the NVFP4 hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * constant with the HIP kernels: every constant below is derived here from its
 * mathematical definition.
 *
 * Sources (web pages; no line numbers):
 *  [P1] "Fused Nvfp4 GEMM All Reduce Plugin" (TensorRT-Edge-LLM C++ API),
 *       section "Baked-weight inputs": activation FP4 [B,K], activation_scale
 *       FP32 [B,1,K/16] = combined scale from DequantizeLinear, weight FP4 [N,K],
 *       weight FP8 block scale [N,K/16], scalar FP32 global weight scale;
 *       output FP16 [B,N]; FP4 packed as UINT8.
 *  [P2] "Nvfp4 A16 Blackwell Moe Runner", struct Nvfp4A16BlackwellMoeParams:
 *       sigmoid group-top-k routing with correctionBias, nGroup, topkGroup,
 *       normTopkProb, routedScalingFactor; ReLU2; per-expert FP32 global scales;
 *       4 block scales per 64 K-elements (16-element blocks).
 *  [P3] "Building Custom TensorRT-LLM Plugins for Low-Latency FP8 Inference at
 *       Scale", sections "The Cost of Non-Fused Quantization" (SwiGLU input
 *       [N,2H] -> [N,H]) and "Fusing the Kernel in CUDA" (activation kept in
 *       fp32 registers, saturation at the E4M3 limit 448).
 *  [P4] "perf: optimize per-token nvfp4 quantization kernel" (flashinfer PR
 *       3237), description and review: per-token global scale, exact (not
 *       fast-math) reciprocal arithmetic, block helper taking the block max, the
 *       global scale and its reciprocal.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - global scale: g_enc = (448*6)/amax, replaced by FLT_MAX when not finite;
 *    the emitted FP32 global is the decode direction g_dec = 1/g_enc.
 *  - block scale: sf = E4M3_RNE_saturating((amax_b / 6) * g_enc).
 *  - combined scale c = decode(sf) * g_dec; encode factor enc = 1/c (0 if c==0).
 *  - element: v = y * enc; code = E2M1 round-to-nearest-even, saturating at 6,
 *    sign bit = sign of v (so -0 encodes as 0x8).
 *  - packing: element 2i in bits 3..0, element 2i+1 in bits 7..4.
 *  - SwiGLU: gate = first half of the row, up = second half;
 *    y = (g / (1 + exp(-g))) * u with the exp defined by oracle_exp below.
 *  - ReLU2: y = r*r with r = max(x, +0).
 *  - MXFP4 variant (the UE8M0_SF switch of the block helper in [P4], review;
 *    the pages show only the switch): 32-element blocks; the same global
 *    scale and block amax as above; the block scale is an E8M0 byte (value
 *    2^(b-127)), namely the smallest such power of two >= (amax_b / 6) * g_enc,
 *    so no element of a block saturates; at or above 2^127 (and for NaN) it
 *    is byte 254, at or below 2^-127 byte 0; c = e8m0(b) * g_dec, enc = 1/c,
 *    elements as above.
 * All float arithmetic is IEEE-754 binary32, round-to-nearest-even, one
 * rounding per operation, no contraction (build with -ffp-contract=off);
 * fmaf is used only where an fma is written explicitly.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Input element decoding (bf16 and fp16 are exact in binary32).        */
/* ------------------------------------------------------------------ */

static float bf16_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;  /* bf16 is the top half of a binary32 */
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static float fp16_to_float(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
  }
  return (float)(sign ? -v : v);
}

float oracle_input_to_float(uint16_t h, int dtype) {
  return dtype == 0 ? bf16_to_float(h) : fp16_to_float(h);
}

/* ------------------------------------------------------------------ */
/* FP8 E4M3 (OCP "FN" variant): bias 7, no infinities, 0x7F/0xFF = NaN,  */
/* largest finite 448 ([P3] "Fusing the Kernel in CUDA").               */
/* ------------------------------------------------------------------ */

double oracle_e4m3_decode(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 15;
  int m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);                  /* m/8 * 2^-6 */
  else
    v = ldexp((double)(8 + m), e - 10);        /* (1 + m/8) * 2^(e-7) */
  return sign ? -v : v;
}

/* Nearest finite non-negative E4M3 value, ties to the even code; anything at
 * or beyond 448 maps to 448 (saturation).  Brute force over all 127 finite
 * non-negative codes: codes are monotone in value, so an even code means an
 * even mantissa, which is what round-half-to-even asks for. */
uint8_t oracle_e4m3_encode(float x) {
  double xv = (double)x;
  if (!(xv > 0.0)) return 0;                   /* 0, -0 and (outside contract) NaN */
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double d = fabs(xv - oracle_e4m3_decode((uint8_t)c));
    if (d < bestd || (d == bestd && (c % 2) == 0)) {
      bestd = d;
      best = c;
    }
  }
  return (uint8_t)best;
}

/* ------------------------------------------------------------------ */
/* FP4 E2M1: magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign in bit 3.     */
/* ------------------------------------------------------------------ */

static const double kE2M1Mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_decode(uint8_t nib) {
  double v = kE2M1Mag[nib & 7];
  return (nib & 8) ? -v : v;
}

/* Nearest magnitude, ties to the even index; |v| >= 6 saturates to 6. */
uint8_t oracle_e2m1_encode(float v) {
  uint8_t sign = signbit(v) ? 8 : 0;
  double m = fabs((double)v);
  if (m >= 6.0) return sign | 7;
  int best = 0;
  double bestd = INFINITY;
  for (int i = 0; i < 8; ++i) {
    double d = fabs(m - kE2M1Mag[i]);
    if (d < bestd || (d == bestd && (i % 2) == 0)) {
      bestd = d;
      best = i;
    }
  }
  return sign | (uint8_t)best;
}

/* ------------------------------------------------------------------ */
/* exp: a fixed binary32 evaluation, defined here from the mathematics   */
/* (Cody & Waite argument reduction, 1980; Taylor series of e^r).        */
/*   x > 88.75          -> +inf   (e^x exceeds FLT_MAX well before)      */
/*   x < -87            -> 0      (keeps every result a normal number)    */
/*   n = rint(x * L2E)                        (ties to even)              */
/*   r = fma(-n, LN2_HI, x);  r = fma(-n, LN2_LO, r)                      */
/*   p = sum_{k=0..7} r^k/k!  by Horner with fma, coefficients rounded    */
/*   result = ldexp(p, n)  (exact while normal; overflows to +inf)        */
/* ------------------------------------------------------------------ */

static float f32_of(double d) { return (float)d; }

float oracle_exp(float x) {
  if (x != x) return x;                           /* NaN propagates (the reduction needs a number) */
  if (x > 88.75f) return INFINITY;
  if (x < -87.0f) return 0.0f;
  const double ln2 = 0.693147180559945309417232121458176568;
  const float L2E = f32_of(1.0 / ln2);            /* log2(e) rounded to fp32 */
  const float LN2_HI = f32_of(ln2);               /* ln 2 rounded to fp32 */
  const float LN2_LO = f32_of(ln2 - (double)LN2_HI);
  float c[8];
  double fact = 1.0;
  for (int k = 0; k < 8; ++k) {                   /* c[k] = fp32(1/k!) */
    if (k > 0) fact *= (double)k;
    c[k] = f32_of(1.0 / fact);
  }
  float t = x * L2E;
  float n = rintf(t);
  float r = fmaf(-n, LN2_HI, x);
  r = fmaf(-n, LN2_LO, r);
  float p = c[7];
  for (int k = 6; k >= 0; --k) p = fmaf(p, r, c[k]);
  return ldexpf(p, (int)n);
}

/* SwiGLU element: silu(g) * u with silu(g) = g / (1 + exp(-g)). */
float oracle_swiglu(float g, float u) {
  float e = oracle_exp(-g);
  float s = 1.0f + e;
  float q = g / s;
  return q * u;
}

/* ReLU^2 element. */
float oracle_relu2(float x) {
  float r = (x > 0.0f) ? x : 0.0f;
  return r * r;
}

/* ------------------------------------------------------------------ */
/* Quantizer.                                                          */
/* ------------------------------------------------------------------ */

enum { ACT_NONE = 0, ACT_SWIGLU = 1, ACT_RELU2 = 2 };

/* Global scale pair from a group amax. */
void oracle_global_scale(float amax, float* g_enc_out, float* g_dec_out) {
  float g_enc = 2688.0f / amax;                   /* 2688 = 448 * 6, exact */
  if (!isfinite(g_enc)) g_enc = FLT_MAX;
  *g_enc_out = g_enc;
  *g_dec_out = 1.0f / g_enc;
}

/* One 16-element block: given y[16], the group's g_enc and g_dec, returns the
 * E4M3 scale byte, the combined fp32 scale and writes 8 packed code bytes. */
void oracle_quantize_block(const float* y, float g_enc, float g_dec, uint8_t* sf_out,
                           float* c_out, uint8_t* codes8) {
  float amax_b = 0.0f;
  for (int i = 0; i < 16; ++i) amax_b = fmaxf(amax_b, fabsf(y[i]));
  float sf_f = (amax_b / 6.0f) * g_enc;
  uint8_t sf = oracle_e4m3_encode(sf_f);
  float sfd = (float)oracle_e4m3_decode(sf);     /* exact */
  float c = sfd * g_dec;
  float enc = (c == 0.0f) ? 0.0f : 1.0f / c;
  /* A zero element always encodes to a zero code with its own sign.  This only
     matters where 1/c overflows to +inf (c below 2^-128, rows whose amax is
     under about 1e-34), where the product 0 * inf would be NaN. */
  for (int i = 0; i < 8; ++i) {
    float v0 = (y[2 * i] == 0.0f) ? y[2 * i] : y[2 * i] * enc;
    float v1 = (y[2 * i + 1] == 0.0f) ? y[2 * i + 1] : y[2 * i + 1] * enc;
    codes8[i] = (uint8_t)(oracle_e2m1_encode(v0) | (oracle_e2m1_encode(v1) << 4));
  }
  *sf_out = sf;
  *c_out = c;
}

/* Activation output of row `r`, column `j` (j < k_out). */
static float act_value(const uint16_t* x, int dtype, int64_t k_in, int act, int64_t r,
                       int64_t j, int64_t k_out) {
  const uint16_t* row = x + r * k_in;
  if (act == ACT_SWIGLU) {
    float g = oracle_input_to_float(row[j], dtype);
    float u = oracle_input_to_float(row[k_out + j], dtype);
    return oracle_swiglu(g, u);
  }
  float v = oracle_input_to_float(row[j], dtype);
  if (act == ACT_RELU2) return oracle_relu2(v);
  return v;
}

/*
 * x      : [rows, k_in] bf16 (dtype 0) or fp16 (dtype 1), raw 16-bit patterns
 * act    : 0 none (k_out = k_in), 1 SwiGLU (k_out = k_in/2), 2 ReLU2
 * group_rows : rows sharing one global scale (1 = per token; rows = per
 *          tensor; rows/E = per expert).  Must divide rows.
 * codes  : [rows, k_out/2] packed E2M1
 * sf     : [rows, k_out/16] E4M3 bytes
 * g_dec  : [rows/group_rows] fp32 decode-direction global scale
 * c      : [rows, k_out/16] fp32 combined scale (may be NULL)
 * returns 0, or -1 on invalid arguments / allocation failure.
 */
int oracle_quantize(const uint16_t* x, int dtype, int64_t rows, int64_t k_in, int act,
                    int64_t group_rows, uint8_t* codes, uint8_t* sf, float* g_dec, float* c) {
  if (rows < 0 || k_in <= 0 || group_rows <= 0 || (rows % group_rows) != 0) return -1;
  int64_t k_out = (act == ACT_SWIGLU) ? k_in / 2 : k_in;
  if ((act == ACT_SWIGLU && (k_in % 2) != 0) || (k_out % 16) != 0) return -1;
  int64_t nb = k_out / 16;
  float* y = (float*)malloc(sizeof(float) * (size_t)k_out);
  if (!y) return -1;
  for (int64_t g0 = 0; g0 < rows; g0 += group_rows) {
    /* pass 1: the group's amax */
    float amax = 0.0f;
    for (int64_t r = g0; r < g0 + group_rows; ++r)
      for (int64_t j = 0; j < k_out; ++j)
        amax = fmaxf(amax, fabsf(act_value(x, dtype, k_in, act, r, j, k_out)));
    float g_enc, gd;
    oracle_global_scale(amax, &g_enc, &gd);
    g_dec[g0 / group_rows] = gd;
    /* pass 2: blocks */
    for (int64_t r = g0; r < g0 + group_rows; ++r) {
      for (int64_t j = 0; j < k_out; ++j) y[j] = act_value(x, dtype, k_in, act, r, j, k_out);
      for (int64_t b = 0; b < nb; ++b) {
        float cb;
        oracle_quantize_block(y + 16 * b, g_enc, gd, sf + r * nb + b, &cb,
                              codes + r * (k_out / 2) + 8 * b);
        if (c) c[r * nb + b] = cb;
      }
    }
  }
  free(y);
  return 0;
}

/* Only the activation stage (for tests): y[rows, k_out] fp32. */
int oracle_activation(const uint16_t* x, int dtype, int64_t rows, int64_t k_in, int act,
                      float* y) {
  int64_t k_out = (act == ACT_SWIGLU) ? k_in / 2 : k_in;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < k_out; ++j) y[r * k_out + j] = act_value(x, dtype, k_in, act, r, j, k_out);
  return 0;
}

/* ------------------------------------------------------------------ */
/* MoE routing ([P2] Nvfp4A16BlackwellMoeParams): sigmoid scores, bias   */
/* used for selection only, group score = sum of the group's two best   */
/* biased scores, keep topk_group groups, pick top_k experts among      */
/* them; ties go to the lower index; weights are the unbiased sigmoid   */
/* scores, optionally divided by their sum (added in rank order), then  */
/* multiplied by routed_scaling.                                        */
/* ------------------------------------------------------------------ */

float oracle_sigmoid(float l) {
  float e = oracle_exp(-l);
  float d = 1.0f + e;
  return 1.0f / d;
}

/* Is (va, ia) ranked before (vb, ib)? Higher value first, lower index on ties. */
static int ranks_before(float va, int ia, float vb, int ib) {
  return (va > vb) || (va == vb && ia < ib);
}

int oracle_route(const float* logits, const float* bias, int tokens, int experts, int top_k,
                 int n_group, int topk_group, int norm_topk_prob, float routed_scaling,
                 int32_t* ids, float* weights) {
  if (tokens < 0 || experts <= 0 || n_group <= 0 || experts % n_group != 0) return -1;
  int gsize = experts / n_group;
  if (topk_group <= 0 || topk_group > n_group || top_k <= 0 || top_k > topk_group * gsize) return -1;
  float* s = (float*)malloc(sizeof(float) * experts);
  float* b = (float*)malloc(sizeof(float) * experts);
  float* gs = (float*)malloc(sizeof(float) * n_group);
  int* keep = (int*)malloc(sizeof(int) * n_group);
  int* used = (int*)malloc(sizeof(int) * experts);
  if (!s || !b || !gs || !keep || !used) { free(s); free(b); free(gs); free(keep); free(used); return -1; }
  for (int t = 0; t < tokens; ++t) {
    for (int e = 0; e < experts; ++e) {
      s[e] = oracle_sigmoid(logits[(int64_t)t * experts + e]);
      b[e] = s[e] + bias[e];
      /* the pages give no order for NaN: a NaN score ranks below every number */
      if (b[e] != b[e]) b[e] = -INFINITY;
    }
    /* group scores: sum of the two best biased scores (one if gsize == 1) */
    for (int g = 0; g < n_group; ++g) {
      int i1 = -1, i2 = -1;
      for (int e = g * gsize; e < (g + 1) * gsize; ++e) {
        if (i1 < 0 || ranks_before(b[e], e, b[i1], i1)) { i2 = i1; i1 = e; }
        else if (i2 < 0 || ranks_before(b[e], e, b[i2], i2)) { i2 = e; }
      }
      gs[g] = (i2 >= 0) ? b[i1] + b[i2] : b[i1];
      /* a NaN group score (+inf and -inf biased scores summed) ranks below
       * every number, as a NaN expert score does */
      if (gs[g] != gs[g]) gs[g] = -INFINITY;
      keep[g] = 0;
    }
    /* keep topk_group groups, by repeated selection of the best remaining */
    for (int k = 0; k < topk_group; ++k) {
      int best = -1;
      for (int g = 0; g < n_group; ++g)
        if (!keep[g] && (best < 0 || ranks_before(gs[g], g, gs[best], best))) best = g;
      keep[best] = 1;
    }
    for (int e = 0; e < experts; ++e) used[e] = 0;
    for (int k = 0; k < top_k; ++k) {
      int best = -1;
      for (int e = 0; e < experts; ++e) {
        if (!keep[e / gsize] || used[e]) continue;
        if (best < 0 || ranks_before(b[e], e, b[best], best)) best = e;
      }
      used[best] = 1;
      ids[(int64_t)t * top_k + k] = best;
      weights[(int64_t)t * top_k + k] = s[best];
    }
    if (norm_topk_prob) {
      float sum = 0.0f;
      for (int k = 0; k < top_k; ++k) sum = sum + weights[(int64_t)t * top_k + k];
      for (int k = 0; k < top_k; ++k)
        weights[(int64_t)t * top_k + k] = weights[(int64_t)t * top_k + k] / sum;
    }
    for (int k = 0; k < top_k; ++k)
      weights[(int64_t)t * top_k + k] = weights[(int64_t)t * top_k + k] * routed_scaling;
  }
  free(s); free(b); free(gs); free(keep); free(used);
  return 0;
}

/* ------------------------------------------------------------------ */
/* MXFP4 variant: E8M0 block scales over 32 elements ([P4] review, the  */
/* UE8M0_SF switch of the block helper; readings in the header).        */
/* ------------------------------------------------------------------ */

/* E8M0: byte b is 2^(b - 127); 255 is NaN and never produced here. */
double oracle_e8m0_decode(uint8_t b) {
  if (b == 255) return NAN;
  return ldexp(1.0, (int)b - 127);
}

/* Smallest E8M0 value >= x, by search over the 255 finite codes (the values
 * increase with the code).  x above 2^127 or NaN gives 254. */
uint8_t oracle_e8m0_encode_up(float x) {
  double xv = (double)x;
  if (!(xv <= ldexp(1.0, 127))) return 254;
  for (int b = 0; b <= 254; ++b)
    if (oracle_e8m0_decode((uint8_t)b) >= xv) return (uint8_t)b;
  return 254;
}

/* One 32-element block: E8M0 byte, combined scale c, 16 packed code bytes. */
void oracle_mx_quantize_block(const float* y, float g_enc, float g_dec, uint8_t* sf_out,
                              float* c_out, uint8_t* codes16) {
  float amax_b = 0.0f;
  for (int i = 0; i < 32; ++i) amax_b = fmaxf(amax_b, fabsf(y[i]));
  float sf_f = (amax_b / 6.0f) * g_enc;
  uint8_t sf = oracle_e8m0_encode_up(sf_f);
  float c = (float)oracle_e8m0_decode(sf) * g_dec;   /* one binary32 rounding */
  float enc = (c == 0.0f) ? 0.0f : 1.0f / c;
  for (int i = 0; i < 16; ++i) {
    float v0 = (y[2 * i] == 0.0f) ? y[2 * i] : y[2 * i] * enc;
    float v1 = (y[2 * i + 1] == 0.0f) ? y[2 * i + 1] : y[2 * i + 1] * enc;
    codes16[i] = (uint8_t)(oracle_e2m1_encode(v0) | (oracle_e2m1_encode(v1) << 4));
  }
  *sf_out = sf;
  *c_out = c;
}

/*
 * Same arguments as oracle_quantize, with 32-element blocks:
 * codes [rows, k_out/2], sf [rows, k_out/32] E8M0 bytes, g_dec [rows/group_rows].
 */
int oracle_mx_quantize(const uint16_t* x, int dtype, int64_t rows, int64_t k_in, int act,
                       int64_t group_rows, uint8_t* codes, uint8_t* sf, float* g_dec) {
  if (rows < 0 || k_in <= 0 || group_rows <= 0 || (rows % group_rows) != 0) return -1;
  int64_t k_out = (act == ACT_SWIGLU) ? k_in / 2 : k_in;
  if ((act == ACT_SWIGLU && (k_in % 2) != 0) || (k_out % 32) != 0) return -1;
  int64_t nb = k_out / 32;
  float* y = (float*)malloc(sizeof(float) * (size_t)k_out);
  if (!y) return -1;
  for (int64_t g0 = 0; g0 < rows; g0 += group_rows) {
    float amax = 0.0f;
    for (int64_t r = g0; r < g0 + group_rows; ++r)
      for (int64_t j = 0; j < k_out; ++j)
        amax = fmaxf(amax, fabsf(act_value(x, dtype, k_in, act, r, j, k_out)));
    float g_enc, gd;
    oracle_global_scale(amax, &g_enc, &gd);
    g_dec[g0 / group_rows] = gd;
    for (int64_t r = g0; r < g0 + group_rows; ++r) {
      for (int64_t j = 0; j < k_out; ++j) y[j] = act_value(x, dtype, k_in, act, r, j, k_out);
      for (int64_t b = 0; b < nb; ++b) {
        float cb;
        oracle_mx_quantize_block(y + 32 * b, g_enc, gd, sf + r * nb + b, &cb,
                                 codes + r * (k_out / 2) + 16 * b);
      }
    }
  }
  free(y);
  return 0;
}
