/*
 * oracle_sanitize_driver.c -- drives every exported function of the C oracle
 * (oracle/nvfp4_oracle.c) over ordinary and edge inputs and prints one
 * FNV-1a checksum of all results.  Built twice by the test suite: plainly,
 * and with AddressSanitizer + UndefinedBehaviorSanitizer (including
 * float-to-int cast overflow); both builds must exit 0 and print the same
 * checksum.  Test infrastructure only.
 *
 * Edge inputs: zero, negative-zero and subnormal rows; rows whose amax is tiny
 * enough that the encode factor overflows; huge bf16 values (ReLU2 and SwiGLU
 * overflow to inf); inf and NaN inputs (outside the quantizer's contract, but
 * they must not reach undefined behaviour); NaN router logits; every E4M3,
 * E2M1 and E8M0 byte.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e4m3_decode(uint8_t b);
uint8_t oracle_e4m3_encode(float x);
double oracle_e2m1_decode(uint8_t nib);
uint8_t oracle_e2m1_encode(float v);
float oracle_exp(float x);
float oracle_swiglu(float g, float u);
float oracle_relu2(float x);
float oracle_sigmoid(float l);
float oracle_input_to_float(uint16_t h, int dtype);
void oracle_global_scale(float amax, float* g_enc_out, float* g_dec_out);
void oracle_quantize_block(const float* y, float g_enc, float g_dec, uint8_t* sf_out, float* c_out,
                           uint8_t* codes8);
int oracle_quantize(const uint16_t* x, int dtype, int64_t rows, int64_t k_in, int act,
                    int64_t group_rows, uint8_t* codes, uint8_t* sf, float* g_dec, float* c);
int oracle_activation(const uint16_t* x, int dtype, int64_t rows, int64_t k_in, int act, float* y);
int oracle_route(const float* logits, const float* bias, int tokens, int experts, int top_k,
                 int n_group, int topk_group, int norm_topk_prob, float routed_scaling,
                 int32_t* ids, float* weights);
double oracle_e8m0_decode(uint8_t b);
uint8_t oracle_e8m0_encode_up(float x);
void oracle_mx_quantize_block(const float* y, float g_enc, float g_dec, uint8_t* sf_out,
                              float* c_out, uint8_t* codes16);
int oracle_mx_quantize(const uint16_t* x, int dtype, int64_t rows, int64_t k_in, int act,
                       int64_t group_rows, uint8_t* codes, uint8_t* sf, float* g_dec);

static uint64_t h = 1469598103934665603ull;
static void mix(const void* p, size_t n) {
  const unsigned char* b = (const unsigned char*)p;
  for (size_t i = 0; i < n; ++i) { h ^= b[i]; h *= 1099511628211ull; }
}
/* NaN payloads and signs are not specified by IEEE arithmetic (they may differ
   between builds), so every NaN is hashed as one pattern. */
static void mixf(float f) { if (f != f) f = NAN; mix(&f, 4); }
static void mixfa(const float* a, size_t n) { for (size_t i = 0; i < n; ++i) mixf(a[i]); }
static void mixd(double d) { if (d != d) d = 12345.0; mix(&d, 8); }

static uint32_t rs = 2463534242u;   /* xorshift32: fixed sequence, no libc rand */
static uint32_t nxt(void) { rs ^= rs << 13; rs ^= rs >> 17; rs ^= rs << 5; return rs; }

static float bits_f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* A row of 16-bit patterns of kind `kind` (see main). */
static void fill(uint16_t* x, int64_t n, int kind) {
  for (int64_t i = 0; i < n; ++i) {
    uint16_t v;
    switch (kind) {
      case 0: v = (uint16_t)nxt(); if ((v & 0x7F80u) == 0x7F80u) v &= 0xBFFFu; break;  /* any finite bf16 */
      case 1: v = 0; break;                                                           /* zeros */
      case 2: v = (uint16_t)(0x8000u | (nxt() & 1u)); break;                          /* -0 and -min subnormal */
      case 3: v = (uint16_t)(nxt() & 0x807Fu); break;                                 /* bf16 subnormals */
      case 4: v = (uint16_t)((nxt() & 0x8000u) | 0x7F00u | (nxt() & 0x7Fu)); break;   /* huge bf16 */
      case 5: v = (i % 7 == 3) ? 0x7F80u : (i % 11 == 5) ? 0x7FC1u : (uint16_t)(nxt() & 0x3FFFu); break;  /* inf / NaN */
      default: v = (uint16_t)(nxt() & 0x7BFFu); break;                                 /* finite fp16 */
    }
    x[i] = v;
  }
}

int main(void) {
  /* formats, every byte */
  for (int b = 0; b < 256; ++b) {
    mixd(oracle_e4m3_decode((uint8_t)b));
    mixd(oracle_e8m0_decode((uint8_t)b));
    if (b < 16) mixd(oracle_e2m1_decode((uint8_t)b));
  }
  const float special[] = {0.0f, -0.0f, 1e-45f, 1e-40f, 0x1p-9f, 0.25f, 0.75f, 5.0f, 6.0f, 448.0f,
                           464.0f, 3.4e38f, INFINITY, -INFINITY, NAN, -5.5f, 0x1p127f, 0x1p-127f};
  for (size_t i = 0; i < sizeof(special) / sizeof(special[0]); ++i) {
    float v = special[i];
    mix(&(uint8_t){oracle_e4m3_encode(v)}, 1);
    mix(&(uint8_t){oracle_e2m1_encode(v)}, 1);
    mix(&(uint8_t){oracle_e8m0_encode_up(v)}, 1);
    mixf(oracle_exp(v)); mixf(oracle_sigmoid(v)); mixf(oracle_relu2(v)); mixf(oracle_swiglu(v, 1.5f));
    float ge, gd;
    oracle_global_scale(v, &ge, &gd);
    mixf(ge); mixf(gd);
  }
  for (int i = 0; i < 20000; ++i) {
    const float v = bits_f(nxt());
    mix(&(uint8_t){oracle_e4m3_encode(v)}, 1);
    mix(&(uint8_t){oracle_e2m1_encode(v)}, 1);
    mix(&(uint8_t){oracle_e8m0_encode_up(v)}, 1);
    mixf(oracle_exp(v));
    mixf(oracle_input_to_float((uint16_t)nxt(), i & 1));
  }
  /* single blocks with extreme scales */
  {
    float y[32];
    uint8_t sf, codes[16];
    float c;
    for (int t = 0; t < 64; ++t) {
      for (int i = 0; i < 32; ++i) y[i] = (t % 4 == 0) ? 0.0f : bits_f(nxt() & 0xBFFFFFFFu);
      const float ge = (t % 3 == 0) ? 3.4028235e38f : bits_f(nxt() & 0x7F7FFFFFu);
      const float gd = 1.0f / ge;
      oracle_quantize_block(y, ge, gd, &sf, &c, codes);
      mix(&sf, 1); mixf(c); mix(codes, 8);
      oracle_mx_quantize_block(y, ge, gd, &sf, &c, codes);
      mix(&sf, 1); mixf(c); mix(codes, 16);
    }
  }
  /* whole quantizations: dtypes x activations x groupings x input kinds */
  const int64_t rows = 8, k = 64;
  uint16_t* x = (uint16_t*)malloc(sizeof(uint16_t) * rows * 2 * k);
  uint8_t* codes = (uint8_t*)malloc(rows * k / 2);
  uint8_t* sf = (uint8_t*)malloc(rows * k / 16);
  float* g = (float*)malloc(sizeof(float) * rows);
  float* cs = (float*)malloc(sizeof(float) * rows * k / 16);
  float* y = (float*)malloc(sizeof(float) * rows * 2 * k);
  if (!x || !codes || !sf || !g || !cs || !y) return 3;
  for (int kind = 0; kind <= 6; ++kind) {
    for (int dt = 0; dt < 2; ++dt) {
      for (int act = 0; act < 3; ++act) {
        const int64_t k_in = act == 1 ? 2 * k : k;
        /* inf/NaN inputs (kind 5; kind 4 read as fp16 is NaN) are outside the
           quantizer's contract: they run under the sanitizers, but the sign
           a NaN takes through the arithmetic depends on operand order, which
           the compiler may change, so their results are not hashed */
        const int hashed = !(kind == 5 || (kind == 4 && dt == 1));
        for (int gr = 1; gr <= 8; gr *= 8) {
          fill(x, rows * k_in, kind == 0 && dt == 1 ? 6 : kind);
          if (oracle_quantize(x, dt, rows, k_in, act, gr, codes, sf, g, cs) != 0) return 4;
          if (hashed) { mix(codes, rows * k / 2); mix(sf, rows * k / 16); mixfa(g, rows / gr); mixfa(cs, rows * k / 16); }
          if (oracle_mx_quantize(x, dt, rows, k_in, act, gr, codes, sf, g) != 0) return 5;
          if (hashed) { mix(codes, rows * k / 2); mix(sf, rows * k / 32); mixfa(g, rows / gr); }
        }
        if (oracle_activation(x, dt, rows, k_in, act, y) != 0) return 6;
        if (hashed) mixfa(y, rows * k);
      }
    }
  }
  /* argument rejection (no writes) */
  if (oracle_quantize(x, 0, 3, 64, 0, 2, codes, sf, g, cs) != -1) return 7;
  if (oracle_quantize(x, 0, 2, 40, 0, 1, codes, sf, g, cs) != -1) return 8;
  if (oracle_mx_quantize(x, 0, 2, 48, 0, 1, codes, sf, g) != -1) return 9;
  /* routing: several configurations, some NaN logits */
  {
    const int cfg[][5] = {{8, 2, 1, 3, 0}, {64, 8, 4, 8, 0}, {256, 16, 4, 16, 1}, {16, 1, 1, 4, 0},
                          {12, 4, 2, 4, 1}};
    for (size_t ci = 0; ci < sizeof(cfg) / sizeof(cfg[0]); ++ci) {
      const int E = cfg[ci][0], ng = cfg[ci][1], tg = cfg[ci][2], tk = cfg[ci][3], nan = cfg[ci][4];
      const int T = 33;
      float* lg = (float*)malloc(sizeof(float) * T * E);
      float* bs = (float*)malloc(sizeof(float) * E);
      int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * T * tk);
      float* w = (float*)malloc(sizeof(float) * T * tk);
      if (!lg || !bs || !ids || !w) return 10;
      for (int i = 0; i < T * E; ++i)
        lg[i] = (nan && i % 5 == 0) ? NAN : (float)((int)(nxt() % 2001) - 1000) / 250.0f;
      for (int e = 0; e < E; ++e) bs[e] = (float)((int)(nxt() % 201) - 100) / 1000.0f;
      for (int norm = 0; norm < 2; ++norm) {
        if (oracle_route(lg, bs, T, E, tk, ng, tg, norm, 2.5f, ids, w) != 0) return 11;
        mix(ids, sizeof(int32_t) * T * tk); mixfa(w, (size_t)T * tk);
      }
      if (oracle_route(lg, bs, T, E, tk + E, ng, tg, 1, 1.0f, ids, w) != -1) return 12;
      free(lg); free(bs); free(ids); free(w);
    }
  }
  free(x); free(codes); free(sf); free(g); free(cs); free(y);
  printf("%016llx\n", (unsigned long long)h);
  return 0;
}
