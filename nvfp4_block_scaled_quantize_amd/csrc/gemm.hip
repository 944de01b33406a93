// gemm.hip -- block-scaled NVFP4 GEMM y[B,N] = deq(a)[B,K] . deq(w)[N,K]^T with
// FP16 output, the operation of "Fused Nvfp4 GEMM All Reduce Plugin"
// (baked-weight inputs 0..4, output 0), for gfx950.
//
// Why FP16 MFMA for the prefill kernels: gfx950's scaled f8f6f4 MFMA applies
// power-of-two (E8M0) scales per 32 K-elements, while NVFP4 carries an E4M3
// scale per 16 elements and the activation side an arbitrary FP32 scale per
// 16 elements.  The dequantized weight e2m1 * e4m3 has at most 6 significant
// bits and lies in [2^-10, 2688], so it is EXACT in FP16; the global weight
// scale moves to the epilogue.  The activation q * c is rounded once to FP16
// after a power-of-two normalization (per row for the prefill kernels, per
// row and half round of 256 k in the FP16 decode kernel) so that no value can
// overflow FP16; the power of two returns in FP32 after the MFMAs.  Products
// accumulate in FP32.
//
// Three kernel families, chosen by the batch size:
//  * gemm_skinny4 (B <= 4, decode): the raw FP4 codes of both operands on the
//    FP4 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4, E8M0 scales 1).
//    The activation operand is block-diagonal -- each operand row is one
//    (token, 16-k block) pair -- so each output is one block's unscaled dot
//    product (exact in FP32), scaled in FP32 by the weight's E4M3 byte and the
//    token's combined scale.  One workgroup per 32 weight rows, each wave one
//    interleaved eighth of K, 16-byte weight loads straight into the MFMA
//    operand; nothing is dequantized.
//  * gemm_skinny16 (4 < B <= 16, decode): the same work split; every lane
//    converts its 32 FP4 weight codes with v_cvt_scalef32_pk_f16_fp4 and one
//    packed FP16 multiply by the E4M3 scale and feeds v_mfma_f32_16x16x32_f16
//    with the (up to 16) activation rows as the other operand, so the
//    arithmetic per weight does not grow with B.
//    Both decode kernels load and stage the activations of each wave's own K
//    slice through a private LDS region, in order with its weights, so no
//    workgroup barrier precedes the MFMAs; the eight K slices are summed in
//    LDS in a fixed order (deterministic).
//  * gemm_wide (larger B, prefill, 16-byte weight rows, K % 64 == 0, or the
//    pre-tiled layout): a prologue kernel writes the normalized FP16
//    activations once; the main kernel computes 128 x 512 output tiles with 8
//    waves (128 x 64 each, v_mfma_f32_32x32x16_f16), streaming FP16
//    activations, packed FP4 weight codes and E4M3 bytes from global memory
//    straight into four LDS stages; weights are dequantized in registers
//    right before each MFMA.  gemm_tiled (256 x 256 tiles, register staging)
//    serves the other shapes: K % 64 != 0, and weights at any alignment with
//    K % 16 == 0 (byte loads).
//
// K permutation: inside each MFMA group the hardware sums over all k of the
// instruction, so the assignment of actual k values to MFMA k-slots is free as
// long as both operands use the same one.  Each lane group takes 32
// consecutive k (one 16-byte load of codes, two E4M3 bytes) and spreads them
// over four MFMAs.
#include "device_common.h"
#include "internal.h"
#include "lds_dma.h"

#include <mutex>
#include <type_traits>

namespace nvfp4 {

namespace {

// ------------------------------------------------------------ shared helpers

// Exponent e with max_c * 2^-e in [1, 2) (0 for a zero row).
__device__ __forceinline__ int row_exponent(float cmax) {
  if (!(cmax > 0.0f)) return 0;
  return (int)((__float_as_uint(cmax) >> 23) & 0xFFu) - 127;
}

// Eight FP4 codes (one dword) -> eight FP16 values q * scale16 (exact when
// scale16 is an E4M3 value).
__device__ __forceinline__ v8h dequant8_f16(uint32_t codes, _Float16 scale16) {
  const v2h s2 = {scale16, scale16};
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
  v8h r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Eight FP4 activation codes times an fp32 scale, each product rounded to FP16.
__device__ __forceinline__ v8h dequant8_act(uint32_t codes, float c) {
  const v2f q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  const v2f q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  const v2f q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  const v2f q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  v8h r;
  r[0] = (_Float16)(q0.x * c); r[1] = (_Float16)(q0.y * c);
  r[2] = (_Float16)(q1.x * c); r[3] = (_Float16)(q1.y * c);
  r[4] = (_Float16)(q2.x * c); r[5] = (_Float16)(q2.y * c);
  r[6] = (_Float16)(q3.x * c); r[7] = (_Float16)(q3.y * c);
  return r;
}

// E4M3 bytes 0 and 1 of a word -> two FP16 values (every E4M3 value is exact
// in FP32 and in FP16).
__device__ __forceinline__ v2h e4m3_pair_f16(uint32_t word) {
  const v2f f = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
  return v2h{(_Float16)f.x, (_Float16)f.y};
}

// Eight FP4 codes times an FP16 scale pair {s, s}.
__device__ __forceinline__ v8h dequant8_f16x2(uint32_t codes, v2h s2) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
  v8h r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// E4M3 byte 0 / byte 1 of a word -> FP16 (every E4M3 value is exact in FP16).
__device__ __forceinline__ _Float16 e4m3_b0_f16(uint32_t word) {
  return (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)word, 0);
}
__device__ __forceinline__ _Float16 e4m3_b1_f16(uint32_t word) {
  return (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)word, 1);
}

__device__ __forceinline__ uint32_t load_u32_bytes(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

// The 32 codes (16 bytes) of a row at byte p by byte loads, any alignment;
// when only the first 16 of the 32 k are inside the row (K % 32 == 16 at
// the row end), the upper 8 bytes are zero and are not read.
__device__ __forceinline__ uint4 load_codes32_bytes(const uint8_t* p, bool full) {
  uint4 r;
  r.x = load_u32_bytes(p);
  r.y = load_u32_bytes(p + 4);
  r.z = full ? load_u32_bytes(p + 8) : 0u;
  r.w = full ? load_u32_bytes(p + 12) : 0u;
  return r;
}

// 8 bytes at a 4-byte aligned address (one dwordx2 load), or by byte loads.
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
__device__ __forceinline__ u32x2 load_u32x2_a4(const uint8_t* p) {
  return *reinterpret_cast<const u32x2_a4*>(p);
}
__device__ __forceinline__ u32x2 load_u32x2_bytes(const uint8_t* p) {
  return u32x2{load_u32_bytes(p), load_u32_bytes(p + 4)};
}

// Weight operand layouts of the GEMM kernels.
constexpr int kWPlain = 0;   // [N, K/2] codes, 16-byte aligned rows (K % 32 == 0)
constexpr int kWTiled = 1;   // the pre-tiled layout
constexpr int kWBytes = 2;   // [N, K/2] codes at any alignment, K % 16 == 0 (byte loads)

// ------------------------------------------------------------ skinny (decode)

constexpr int kSkThreads = 512;   // 8 waves
constexpr int kSkWaves = kSkThreads / 64;
constexpr int kSkRows = 32;       // weight rows per workgroup: two 16-row MFMA groups
constexpr int kSkPF = 4;          // 128-k chunks per round (all loads of a round in flight)
constexpr int kSkHalves = 2;      // activation load groups per round (one 2^e per row each in
                                  // the FP16 kernel)
constexpr int kSkHC = kSkPF / kSkHalves;        // chunks per half round
constexpr int kScaleOne = 0x7F7F7F7F;          // E8M0 1.0 in every byte: the MFMA's own scales unused

// Per-wave LDS of the skinny kernel for NP token pairs: a half round's
// activation operand rows (kSkHC chunks x NP pairs x 16 rows x 16 B: the
// row's block in its half of the 32 k, zeros in the other half), as many zero
// bytes (read by the lanes whose 32 k do not hold their row's block), the
// half round's activation scales (kSkHC x NP x 4 lane groups x 16 B) and a
// 16-byte slot that takes the writes of items past the last token.  The
// K-slice reduction reuses the space after a barrier.
constexpr int sk_aop_bytes(int np) { return kSkHC * np * 16 * 16; }
constexpr int sk_wave_bytes(int np) { return 2 * sk_aop_bytes(np) + kSkHC * np * 64 + 16; }
constexpr size_t skinny4_lds_bytes(int np) { return (size_t)kSkWaves * sk_wave_bytes(np); }
constexpr size_t skinny4_red_bytes(int np) { return (size_t)kSkWaves * kSkRows * 2 * np * 4; }
static_assert(skinny4_lds_bytes(1) >= skinny4_red_bytes(1) && skinny4_lds_bytes(2) >= skinny4_red_bytes(2),
              "the reduction fits the stages");

// Sum of a value over the four 16-lane rows of a wave, the same in every lane
// and added in the same order: v_permlane16_swap pairs rows (0, 1) and (2, 3),
// v_permlane32_swap the two halves.
__device__ __forceinline__ float fold_lane_groups(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// The FP4 operand of a scaled MFMA: 32 codes in the low four registers.
typedef int v8i __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v8i fp4_op(u32x4 v) {
  return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

// Decode: one workgroup = 32 weight rows x all of K on the FP4 matrix cores
// (v_mfma_scale_f32_16x16x128_f8f6f4, both operands E2M1, the instruction's
// E8M0 scales fixed at 1).  The hardware sums over all 128 k of an
// instruction, while every 16 k carry their own scales on both sides, so the
// activation operand is block-diagonal: operand row m = 4 G + u stands for
// token 2 p + u / 2 and 16-k block 2 G + u % 2 of the chunk and holds that
// block's codes, zeros elsewhere.  Output (m, n) of one instruction is then
// the unscaled dot product of block (2 G + u % 2) of that token and weight row
// n: a sum of 16 E2M1 x E2M1 products, a multiple of 1/4 below 2^10, exact in
// FP32 whatever the summation order.  The lane holding rows 4 G .. 4 G + 3 of
// column n multiplies each by its weight's E4M3 scale times the token's FP32
// combined scale (one rounding each) and adds it to an FP32 total per (row,
// token).  No dequantization, no FP16 rounding, no normalization.
// The weight operand is 16 raw code bytes per lane (lane r + 16 g: row r,
// k = 32 g .. 32 g + 31 of the chunk), exactly as stored; the activation
// operand uses the same (lane group, byte) positions for the same k.
//
// Wave w owns the interleaved 128-k chunks w, w + 8, ... in rounds of kSkPF
// chunks.  A round issues its loads half round by half round -- the half's
// activation items (16 B of codes = 32 k of one token; 16 B of combined
// scales = 4 blocks of one token), then the half's weight codes and E4M3
// bytes -- so with the in-order load counter each half's activations arrive
// before its weights and the first half is processed while the second
// streams in.  The activation items are written into the wave's own LDS
// region at their operand positions (the zero positions are written once at
// the start) and read back one 16-byte operand per lane and pair: LDS
// operations of one wave run in order, so no barrier.  At the end the four
// lane groups' totals are folded in registers (cross-row lane swaps) and the
// eight K slices summed in LDS, both in a fixed order (deterministic).
// Rounds that lie inside K and the wave's range run without validity selects;
// the last partial round clamps its addresses and zeroes codes and scales
// outside (scales too, so that no NaN from an unused byte can enter).
// AV: activation codes and scales 16-byte aligned with K % 64 == 0 (16-byte
// loads), else byte and dword loads.  NP: token pairs (B <= 2 NP).
// WL: weight layout (kWPlain, kWTiled = pre-tiled, each wave-load of 16 rows
// x 128 k one contiguous KiB of codes / 128 B of E4M3 bytes, kWBytes = any
// alignment and K % 16 == 0 by byte loads, the upper 16 k of a half-filled
// last 32-k group zero).  All run the same arithmetic on the same values:
// bit-identical results.
// One workgroup per CU (256 workgroups fill the chip for N = 8192), so two
// waves per SIMD: the registers go to loads in flight.
template <bool AV, int NP, int WL>
__global__ void __launch_bounds__(kSkThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_skinny4(const uint8_t* __restrict__ a, const float* __restrict__ a_scale,
            const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_sf,
            const float* __restrict__ w_g, _Float16* __restrict__ y, int B, int N, int K) {
  constexpr int TP = 2 * NP;                       // token slots
  constexpr int CL = (kSkHC * TP * 4 + 63) / 64;   // code items per lane and half round
  static_assert(kSkHC * TP * 2 <= 64, "one scale item per lane and half round");
  constexpr int kWB = sk_wave_bytes(NP);
  constexpr int kAop = sk_aop_bytes(NP);   // operand rows at 0, zeros at kAop
  constexpr int kSc = 2 * kAop;            // activation scales
  constexpr int kDummy = kWB - 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  unsigned char* st = smem + (size_t)wave * kWB;
  float* red = reinterpret_cast<float*>(smem);   // after the last round

  const int r16 = lane & 15, g = lane >> 4;
  const int nch = (K + 127) >> 7;
  const int cnt = wave < nch ? (nch - 1 - wave) / kSkWaves + 1 : 0;   // chunk(m) for m < cnt
  auto chunk = [&](int m) { return wave + kSkWaves * m; };
  const int64_t kb2 = K / 2, kb16 = K / 16;

  int nrow[2];                                   // rows past N re-read row N-1 (not stored)
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const int n = blockIdx.x * kSkRows + rg * 16 + r16;
    nrow[rg] = n < N ? n : N - 1;
  }
  // code item j of the lane: (chunk ii of the half, token t, 32-k part s);
  // its block 2 s + v is operand row 4 s + 2 (t & 1) + v of pair t / 2, read
  // by the lanes of group s (bytes 8 v .. 8 v + 7 of their 16).  Items past
  // the last token go to the dummy.
  int ct[CL], cii[CL], cs[CL], cdst[CL][2];
#pragma unroll
  for (int j = 0; j < CL; ++j) {
    const int item = lane + 64 * j;
    const int s = item & 3, t = (item >> 2) % TP, ii = (item >> 2) / TP;
    const bool ok = ii < kSkHC && t < B;
    ct[j] = t < B ? t : B - 1;
    cii[j] = ii < kSkHC ? ii : 0;
    cs[j] = s;
#pragma unroll
    for (int v = 0; v < 2; ++v)
      cdst[j][v] = ok ? ((ii * NP + (t >> 1)) * 16 + 4 * s + 2 * (t & 1) + v) * 16 : kDummy;
  }
  // scale item of the lane: (ii, token t, half s of the chunk's blocks):
  // blocks 4 s + 2 u, 4 s + 2 u + 1 go to the scale slot of (ii, pair t / 2,
  // lane group 2 s + u) at floats 2 (t & 1), 2 (t & 1) + 1
  int sdst[2];
  const int ss = lane & 1, stk = (lane >> 1) % TP, sii = (lane >> 1) / TP;
  const int sto = stk < B ? stk : B - 1;
  {
    const bool ok = sii < kSkHC && stk < B;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      sdst[u] = ok ? kSc + ((sii * NP + (stk >> 1)) * 4 + 2 * ss + u) * 16 + 8 * (stk & 1) : kDummy;
  }
  const int sii_c = sii < kSkHC ? sii : 0;
  // the zero rows, written once; operand row r16 of a pair is read from the
  // stage by lane group r16 / 4 (whose 32 k hold the row's block), from the
  // zeros by the other three.  Scale slots of tokens past B are never written:
  // they meet only operand rows of those tokens, whose totals are not stored.
  for (int o = 16 * lane; o < kAop; o += 1024) *reinterpret_cast<u32x4*>(st + kAop + o) = u32x4{0u, 0u, 0u, 0u};
  const int abase = ((r16 >> 2) == g ? 0 : kAop) + 16 * r16;

  v2f tot[2][NP];   // per row group and pair: FP32 totals of tokens 2 p, 2 p + 1
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
#pragma unroll
    for (int p = 0; p < NP; ++p) tot[rg][p] = v2f{0.0f, 0.0f};

  // FULL: all kSkPF chunks of the round inside the wave's list and inside K
  auto round = [&](int mb, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    u32x4 acode[kSkHalves][CL];
    v4f ascl[kSkHalves];
    uint4 wc[kSkPF][2];
    uint32_t wsv[kSkPF][2];
    // 1. loads, half by half: the half's activation items, then its weights.
    //    In a partial round, addresses outside the range or past K are
    //    clamped to k = 0 and the values are zeroed.
#pragma unroll
    for (int h = 0; h < kSkHalves; ++h) {
#pragma unroll
      for (int j = 0; j < CL; ++j) {
        const int mi = mb + kSkHC * h + cii[j];
        const int k0 = chunk(FULL ? mi : (mi < cnt ? mi : cnt - 1)) * 128 + 32 * cs[j];
        const uint8_t* pa = a + (int64_t)ct[j] * kb2;
        if (FULL) {
          if constexpr (AV) {
            acode[h][j] = *reinterpret_cast<const u32x4*>(pa + k0 / 2);
          } else {
            const uint4 q = load_codes32_bytes(pa + k0 / 2, true);
            acode[h][j] = u32x4{q.x, q.y, q.z, q.w};
          }
        } else {
          const bool v0 = mi < cnt && k0 < K, v1 = mi < cnt && k0 + 16 < K;
          const uint8_t* p = pa + (v0 ? k0 / 2 : 0);
          u32x4 q;
          if constexpr (AV) {
            q = *reinterpret_cast<const u32x4*>(p);   // K % 64 == 0: v1 == v0
          } else {
            const uint4 r = load_codes32_bytes(p, v1);
            q = u32x4{r.x, r.y, r.z, r.w};
          }
          acode[h][j] = u32x4{v0 ? q.x : 0u, v0 ? q.y : 0u, v1 ? q.z : 0u, v1 ? q.w : 0u};
        }
      }
      {
        const int mi = mb + kSkHC * h + sii_c;
        const int kb = chunk(FULL ? mi : (mi < cnt ? mi : cnt - 1)) * 8 + 4 * ss;   // first block
        const float* ps = a_scale + (int64_t)sto * kb16;
        if (FULL) {
          if constexpr (AV) ascl[h] = *reinterpret_cast<const v4f*>(ps + kb);
          else ascl[h] = v4f{ps[kb], ps[kb + 1], ps[kb + 2], ps[kb + 3]};
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const bool ok = mi < cnt && kb + u < kb16;
            const float f = ps[ok ? kb + u : 0];
            ascl[h][u] = ok ? f : 0.0f;
          }
        }
      }
#pragma unroll
      for (int ii = 0; ii < kSkHC; ++ii) {
        const int i = kSkHC * h + ii;
        const int c = chunk(FULL ? mb + i : (mb + i < cnt ? mb + i : cnt - 1));
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
          if constexpr (WL == kWTiled) {
            // tile (row group, chunk), lane order r16 + 16 g (K % 128 == 0)
            const int64_t t = ((int64_t)(nrow[rg] >> 4) * nch + c) * 64 + lane;
            wc[i][rg] = *reinterpret_cast<const uint4*>(w + t * 16);
            wsv[i][rg] = (uint32_t)*reinterpret_cast<const uint16_t*>(w_sf + t * 2);
          } else {
            const int k0 = c * 128 + 32 * g;
            const int k = FULL ? k0 : (k0 < K ? k0 : 0);
            const uint8_t* wr = w + (int64_t)nrow[rg] * kb2 + k / 2;
            const uint8_t* sr = w_sf + (int64_t)nrow[rg] * kb16 + k / 16;
            if constexpr (WL == kWBytes) {
              const bool full = FULL || k + 16 < K;
              wc[i][rg] = load_codes32_bytes(wr, full);
              wsv[i][rg] = (uint32_t)sr[0] | (full ? (uint32_t)sr[1] << 8 : 0u);
            } else {
              wc[i][rg] = *reinterpret_cast<const uint4*>(wr);
              wsv[i][rg] = (uint32_t)*reinterpret_cast<const uint16_t*>(sr);
            }
          }
        }
      }
      // issue order = arrival order: keep the halves' load groups apart, and
      // every load of the round ahead of the first use
      __builtin_amdgcn_sched_barrier(0);
    }

#pragma unroll
    for (int h = 0; h < kSkHalves; ++h) {
      // 2. the half's activation items into their operand positions
      //    (unconditional stores: a branch would move the loads into it)
#pragma unroll
      for (int j = 0; j < CL; ++j) {
        *reinterpret_cast<u32x4*>(st + cdst[j][0]) = u32x4{acode[h][j].x, acode[h][j].y, 0u, 0u};
        *reinterpret_cast<u32x4*>(st + cdst[j][1]) = u32x4{0u, 0u, acode[h][j].z, acode[h][j].w};
      }
      *reinterpret_cast<v2f*>(st + sdst[0]) = v2f{ascl[h][0], ascl[h][1]};
      *reinterpret_cast<v2f*>(st + sdst[1]) = v2f{ascl[h][2], ascl[h][3]};
      __builtin_amdgcn_sched_barrier(0);   // staging first: it waits only for the half's activations
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // 3. per chunk and pair one MFMA per row group, scaled into the totals
#pragma unroll
      for (int ii = 0; ii < kSkHC; ++ii) {
        const int i = kSkHC * h + ii;
        v2f swf[2];   // E4M3 scales of blocks 2 g, 2 g + 1 of each row group's row
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
          uint32_t sb = wsv[i][rg];
          if (!FULL) {
            const int k0 = chunk(mb + i) * 128 + 32 * g;
            const bool cv = mb + i < cnt;
            sb = (cv && k0 < K ? (sb & 0xFFu) : 0u) | (cv && k0 + 16 < K ? (sb & 0xFF00u) : 0u);
          }
          swf[rg] = __builtin_amdgcn_cvt_pk_f32_fp8((int)sb, false);
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const u32x4 aop = *reinterpret_cast<const u32x4*>(st + abase + (ii * NP + p) * 256);
          const v4f sa = *reinterpret_cast<const v4f*>(st + kSc + ((ii * NP + p) * 4 + g) * 16);
#pragma unroll
          for (int rg = 0; rg < 2; ++rg) {
            const uint4 wq = wc[i][rg];
            const v4f c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                fp4_op(aop), fp4_op(u32x4{wq.x, wq.y, wq.z, wq.w}), v4f{0.0f, 0.0f, 0.0f, 0.0f}, 4, 4, 0,
                kScaleOne, 0, kScaleOne);
            float t0 = tot[rg][p][0], t1 = tot[rg][p][1];
            t0 = __builtin_fmaf(c[0], swf[rg][0] * sa[0], t0);
            t0 = __builtin_fmaf(c[1], swf[rg][1] * sa[1], t0);
            t1 = __builtin_fmaf(c[2], swf[rg][0] * sa[2], t1);
            t1 = __builtin_fmaf(c[3], swf[rg][1] * sa[3], t1);
            tot[rg][p] = v2f{t0, t1};
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // the next half's staging after this half's reads
    }
  };

  int mb = 0;
  for (; mb + kSkPF <= cnt && (chunk(mb + kSkPF - 1) + 1) * 128 <= K; mb += kSkPF) round(mb, std::true_type{});
  if (mb < cnt) round(mb, std::false_type{});   // wave-uniform

  // fold the four lane groups' partial totals in registers (every lane ends
  // with the same sum, added in the same order), then sum the eight K slices
  // in LDS in a fixed order, scale, round to FP16
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int v = 0; v < 2; ++v) tot[rg][p][v] = fold_lane_groups(tot[rg][p][v]);
  __syncthreads();   // every wave is done with its stage
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int v = 0; v < 2; ++v)
        if ((((rg * NP + p) * 2 + v) & 3) == g) red[(wave * TP + 2 * p + v) * kSkRows + rg * 16 + r16] = tot[rg][p][v];
  __syncthreads();
  const float gw = *w_g;
  for (int t = tid; t < TP * kSkRows; t += kSkThreads) {
    const int b = t / kSkRows, nl = t % kSkRows;
    const int n = blockIdx.x * kSkRows + nl;
    if (b < B && n < N) {
      float s = red[b * kSkRows + nl];
#pragma unroll
      for (int q = 1; q < kSkWaves; ++q) s += red[(q * TP + b) * kSkRows + nl];
      y[(int64_t)b * N + n] = (_Float16)(s * gw);
    }
  }
}


constexpr int kSkPitch = kSkPF * 128 + 8;        // halves per staged activation row
constexpr int kSkRedRow = kSkRows + 1;          // K-slice reduction: [wave][token][row], rows padded
constexpr int kSkRedPitch = 16 * kSkRedRow;      // floats per wave

// Dynamic LDS of the skinny kernel for IPL activation items per lane: per wave
// a stage of 4 IPL + 1 rows x kSkPitch halves and as many FP32 powers of two
// (the K-slice reduction reuses the stages after a barrier).
constexpr size_t skinny16_lds_bytes(int ipl) {
  return (size_t)kSkWaves * (size_t)(4 * ipl + 1) * (kSkPitch * 2 + 4 * kSkHalves);
}
static_assert(skinny16_lds_bytes(2) >= (size_t)kSkWaves * kSkRedPitch * 4, "reduction fits the stages");

// Decode with more tokens (4 < B <= 16): the weights dequantized once per
// chunk serve every token through v_mfma_f32_16x16x32_f16, so the
// arithmetic per weight does not grow with B (the FP4 kernel's scaling
// epilogue does, by two operations per token, block and row).
// One workgroup = 32 weight rows x all of K; wave w owns the interleaved
// 128-k chunks w, w + 8, ... for both 16-row groups, in rounds of kSkPF
// chunks.  A round:
//  1. issues its loads half round by half round: the half's activation items
//     (IPL per lane, each 16 codes of one row and their FP32 combined scale;
//     the 16 lanes of a row cover the half's 2 x 128 k), then the half's
//     weight tiles.  With the in-order load counter, each half's activations
//     arrive before its weights and the first half is processed while the
//     second streams in -- no workgroup barrier and no prologue precede the
//     MFMAs;
//  2. per half, the row maximum of the combined scales (DPP over the 16-lane
//     row holding the row's items) gives a power of two 2^e per row; the
//     items are dequantized as q * (c 2^-e), rounded
//     once to FP16 (|value| < 12), into a stage in the wave's own LDS region,
//     read back in MFMA layout (LDS operations of one wave run in order, so
//     no barrier);
//  3. per chunk the weights are dequantized in registers (e2m1 * e4m3 is exact
//     in FP16) and feed one v_mfma_f32_16x16x32_f16 chain per row group over
//     the half; the chain result times 2^e is added to the FP32 total.
// At the end the eight K slices are summed in LDS in a fixed order.
// Rounds that lie inside K and the wave's range run without any per-item
// validity selects and with constant address offsets; the last partial round
// re-loads valid addresses and zeroes what lies outside.
// A4: activation codes 4-byte aligned (dword loads), else byte loads.
// IPL: activation items per lane per chunk; B <= 4 * IPL.
// WL: weight layout (kWPlain, kWTiled = pre-tiled, each wave-load of 16 rows
// x 128 k one contiguous KiB of codes / 128 B of E4M3 bytes, kWBytes = any
// alignment and K % 16 == 0 by byte loads, the upper 16 k of a half-filled
// last 32-k group zero).  All three run the same arithmetic on the same
// values: bit-identical results.
// One workgroup per CU (256 workgroups fill the chip for N = 8192), so two
// waves per SIMD: the registers go to loads in flight and operand buffers.
template <bool A4, int IPL, int WL>
__global__ void __launch_bounds__(kSkThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_skinny16(const uint8_t* __restrict__ a, const float* __restrict__ a_scale,
            const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_sf,
            const float* __restrict__ w_g, _Float16* __restrict__ y, int B, int N, int K) {
  constexpr int R = 4 * IPL;                  // staged activation rows; row R takes the
                                              // writes of items past row B-1
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  _Float16* st = reinterpret_cast<_Float16*>(smem) + (size_t)wave * (R + 1) * kSkPitch;
  float* sexp = reinterpret_cast<float*>(smem + (size_t)kSkWaves * (R + 1) * kSkPitch * 2) +
                wave * (R + 1) * kSkHalves;
  float* red = reinterpret_cast<float*>(smem);   // after the last round

  const int r16 = lane & 15, g = lane >> 4;
  const int nch = (K + 127) >> 7;
  // this wave's chunks: chunk(m) for m < cnt
  // interleaved chunks: waves side by side on the same 128-byte segments of
  // plain weight rows read faster than contiguous K slices per wave (and every
  // layout keeps the same summation order)
  constexpr bool kInterleave = true;
  const int cnt = kInterleave ? (wave < nch ? (nch - 1 - wave) / kSkWaves + 1 : 0)
                              : (wave + 1) * nch / kSkWaves - wave * nch / kSkWaves;
  const int cbase = kInterleave ? wave : wave * nch / kSkWaves;
  auto chunk = [&](int m) { return kInterleave ? cbase + kSkWaves * m : cbase + m; };
  const int64_t kb2 = K / 2, kb16 = K / 16;
  const int rb = r16 < B ? r16 : B - 1;       // activation row of this lane's MFMA column

  int nrow[2];                                // rows past N re-read row N-1 (not stored)
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const int n = blockIdx.x * kSkRows + rg * 16 + r16;
    nrow[rg] = n < N ? n : N - 1;
  }
  // activation items: per half round (two chunks), item j of lane l is row
  // l / 16 + 4 j, the 16 codes at k = 16 (l % 8) .. +15 of the half's chunk
  // (l % 16) / 8 (8 B of codes, one FP32 combined scale)
  int arow[IPL], srow[IPL];
#pragma unroll
  for (int j = 0; j < IPL; ++j) {
    const int b = (lane >> 4) + 4 * j;
    arow[j] = b < B ? b : B - 1;
    srow[j] = b < B ? b : R;
  }
  const int ich = (lane & 15) >> 3, ik = 16 * (lane & 7);

  v4f tot[2];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) tot[rg] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // FULL: all kSkPF chunks of the round inside the wave's list and inside K
  auto round = [&](int mb, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    u32x2 acode[kSkHalves][IPL];
    float ascl[kSkHalves][IPL];
    uint4 wc[kSkPF][2];
    uint32_t wsv[kSkPF][2];
    int ka[kSkHalves];
    // 1. loads, half by half: the half's activation items, then its weight
    //    tiles.  In a partial round, codes and scales outside the range or
    //    past K are not read (addresses clamped to k = 0) and are zeroed below.
#pragma unroll
    for (int h = 0; h < kSkHalves; ++h) {
      const int mi = mb + kSkHC * h + ich;
      ka[h] = chunk(FULL ? mi : (mi < cnt ? mi : cnt - 1)) * 128 + ik;   // first k of the item
#pragma unroll
      for (int j = 0; j < IPL; ++j) {
        const uint8_t* pa = a + (int64_t)arow[j] * kb2;
        const float* ps = a_scale + (int64_t)arow[j] * kb16;
        if (FULL) {
          acode[h][j] = A4 ? load_u32x2_a4(pa + ka[h] / 2) : load_u32x2_bytes(pa + ka[h] / 2);
          ascl[h][j] = ps[ka[h] / 16];
        } else {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int k = ka[h] + 8 * q < K ? ka[h] + 8 * q : 0;
            acode[h][j][q] = A4 ? *reinterpret_cast<const uint32_t*>(pa + k / 2) : load_u32_bytes(pa + k / 2);
          }
          ascl[h][j] = ps[ka[h] < K ? ka[h] / 16 : 0];
        }
      }
#pragma unroll
      for (int ii = 0; ii < kSkHC; ++ii) {
        const int i = kSkHC * h + ii;
        const int c = chunk(FULL ? mb + i : (mb + i < cnt ? mb + i : cnt - 1));
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
          if constexpr (WL == kWTiled) {
            // tile (row group, chunk), lane order r16 + 16 g (K % 128 == 0)
            const int64_t t = ((int64_t)(nrow[rg] >> 4) * nch + c) * 64 + lane;
            wc[i][rg] = *reinterpret_cast<const uint4*>(w + t * 16);
            wsv[i][rg] = (uint32_t)*reinterpret_cast<const uint16_t*>(w_sf + t * 2);
          } else {
            const int k0 = c * 128 + 32 * g;
            const int k = FULL ? k0 : (k0 < K ? k0 : 0);
            const uint8_t* wr = w + (int64_t)nrow[rg] * kb2 + k / 2;
            const uint8_t* sr = w_sf + (int64_t)nrow[rg] * kb16 + k / 16;
            if constexpr (WL == kWBytes) {
              const bool full = FULL || k + 16 < K;
              wc[i][rg] = load_codes32_bytes(wr, full);
              wsv[i][rg] = (uint32_t)sr[0] | (full ? (uint32_t)sr[1] << 8 : 0u);
            } else {
              wc[i][rg] = *reinterpret_cast<const uint4*>(wr);
              wsv[i][rg] = (uint32_t)*reinterpret_cast<const uint16_t*>(sr);
            }
          }
        }
      }
      // issue order = arrival order: keep the halves' load groups apart, and
      // every load of the round ahead of the first use (the scheduler would
      // otherwise reorder them or sink later loads below earlier work)
      __builtin_amdgcn_sched_barrier(0);
    }

#pragma unroll
    for (int h = 0; h < kSkHalves; ++h) {
      // 2. stage the half's activations, normalized per row by 2^-e; items
      //    outside the range or past K stage zeros.  Stores are unconditional
      //    (a branch would move the loads into it, behind a wait for all loads).
      const bool iv = FULL || mb + kSkHC * h + ich < cnt;   // the item's chunk is in the wave's list
#pragma unroll
      for (int j = 0; j < IPL; ++j) {
        const float sc = (FULL || (iv && ka[h] < K)) ? ascl[h][j] : 0.0f;
        uint32_t code[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) code[q] = (FULL || (iv && ka[h] + 8 * q < K)) ? acode[h][j][q] : 0u;
        const int e = row_exponent(row16_max(__builtin_fabsf(sc)));
        const float c = sc * __builtin_ldexpf(1.0f, -e);
        _Float16* dst = st + srow[j] * kSkPitch + 128 * (kSkHC * h + ich) + ik;
        *reinterpret_cast<v8h*>(dst) = dequant8_act(code[0], c);
        *reinterpret_cast<v8h*>(dst + 8) = dequant8_act(code[1], c);
        sexp[h * (R + 1) + srow[j]] = __builtin_ldexpf(1.0f, e);   // the same value from the row's 16 lanes
      }
      __builtin_amdgcn_sched_barrier(0);   // staging first: it waits only for the half's activations
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // 3. the half's weights chunk by chunk, one MFMA chain per row group
      v4f acc[2];
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) acc[rg] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ii = 0; ii < kSkHC; ++ii) {
        const int i = kSkHC * h + ii;
        v8h bf[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
          bf[m] = *reinterpret_cast<const v8h*>(st + rb * kSkPitch + 128 * i + 32 * g + 8 * m);
        // weight codes past K (a partial last chunk) or of chunks past the
        // range are zeroed; their activations are zero as well
        const bool kv = FULL || (mb + i < cnt && chunk(mb + i) * 128 + 32 * g < K);
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
          const v2h sp = e4m3_pair_f16(wsv[i][rg]);
          const v2h s0 = {sp[0], sp[0]}, s1 = {sp[1], sp[1]};
          const uint32_t cw[4] = {kv ? wc[i][rg].x : 0u, kv ? wc[i][rg].y : 0u, kv ? wc[i][rg].z : 0u,
                                  kv ? wc[i][rg].w : 0u};
#pragma unroll
          for (int m = 0; m < 4; ++m)
            acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant8_f16x2(cw[m], m < 2 ? s0 : s1), bf[m], acc[rg], 0, 0, 0);
        }
      }
      const float es = sexp[h * (R + 1) + rb];
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[rg][r] += acc[rg][r] * es;
      __builtin_amdgcn_sched_barrier(0);   // the next half's staging after this half's work
    }
  };

  int mb = 0;
  for (; mb + kSkPF <= cnt && (chunk(mb + kSkPF - 1) + 1) * 128 <= K; mb += kSkPF) round(mb, std::true_type{});
  if (mb < cnt) round(mb, std::false_type{});   // wave-uniform

  // sum the eight K slices in a fixed order, scale, round to FP16
  __syncthreads();   // every wave is done with its stage
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave * kSkRedPitch + r16 * kSkRedRow + rg * 16 + 4 * g + r] = tot[rg][r];
  __syncthreads();
  const float gw = *w_g;
  for (int t = tid; t < B * kSkRows; t += kSkThreads) {
    const int b = t / kSkRows, nl = t % kSkRows;
    const int n = blockIdx.x * kSkRows + nl;
    if (n < N) {
      float s = red[b * kSkRedRow + nl];
#pragma unroll
      for (int q = 1; q < kSkWaves; ++q) s += red[q * kSkRedPitch + b * kSkRedRow + nl];
      y[(int64_t)b * N + n] = (_Float16)(s * gw);
    }
  }
}

typedef void (*SkinnyFn)(const uint8_t*, const float*, const uint8_t*, const uint8_t*, const float*,
                         _Float16*, int, int, int);

// B <= 4: the FP4 kernel with NP token pairs; 4 < B <= 16: the FP16 kernel
// with IPL activation items per lane (B <= 4 IPL).
constexpr int kSkFp4MaxB = 4;
int skinny_np(int B) { return B <= 2 ? 1 : 2; }
int skinny_ipl(int B) { return B <= 8 ? 2 : 4; }
size_t skinny_lds(int B) { return B <= kSkFp4MaxB ? skinny4_lds_bytes(skinny_np(B)) : skinny16_lds_bytes(skinny_ipl(B)); }

template <bool X, int WL>
SkinnyFn skinny_kernel_x(int B) {
  if (B <= kSkFp4MaxB) return skinny_np(B) == 1 ? gemm_skinny4<X, 1, WL> : gemm_skinny4<X, 2, WL>;
  return skinny_ipl(B) == 2 ? gemm_skinny16<X, 2, WL> : gemm_skinny16<X, 4, WL>;
}
// x: the activation flag of the kernel family (FP4: 16-byte code and scale
// loads; FP16: 4-byte aligned codes).  The byte-load weight path of the FP16
// kernel uses byte loads for the activation codes too.
SkinnyFn skinny_kernel(int B, bool x, int wl) {
  if (wl == kWBytes) {
    if (B > kSkFp4MaxB) return skinny_kernel_x<false, kWBytes>(B);
    return x ? skinny_kernel_x<true, kWBytes>(B) : skinny_kernel_x<false, kWBytes>(B);
  }
  if (wl == kWTiled) return x ? skinny_kernel_x<true, kWTiled>(B) : skinny_kernel_x<false, kWTiled>(B);
  return x ? skinny_kernel_x<true, kWPlain>(B) : skinny_kernel_x<false, kWPlain>(B);
}

// ------------------------------------------------------------ tiled (prefill)

// Prologue: one workgroup per activation row -> normalized FP16 row and its
// power of two.  A lane's unit is half a block (8 codes, 16 bytes of output),
// so the lanes of a store instruction write one contiguous run (with whole
// blocks per lane the run had 16-byte holes that the next store filled:
// 17.3 -> 14.8 us for [4096, 8192]).  Rows of up to 256 * kA16Items blocks
// keep every unit's combined scale and codes in registers, loaded before the
// row maximum is formed (one pass over the row, all loads in flight
// together); longer rows take a second pass.  A8: activation code rows
// 8-byte aligned (dword loads of 8 codes), else byte loads.  The same
// arithmetic either way.
constexpr int kA16Items = 4;
template <bool A8>
__global__ void __launch_bounds__(256)
a_to_f16_rows(const uint8_t* __restrict__ a, const float* __restrict__ a_scale,
              _Float16* __restrict__ a16, float* __restrict__ rowscale, int K) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int kb16 = K / 16;
  const float* sc = a_scale + row * kb16;
  const uint8_t* ar = a + row * (K / 2);
  _Float16* out = a16 + row * K;
  // half-block units: unit u = 8 codes of block u / 2, so consecutive lanes
  // store consecutive 16 bytes (one contiguous run per store instruction)
  const int nu = 2 * kb16;
  const bool held = nu <= 256 * 2 * kA16Items;   // block-uniform
  float cs[2 * kA16Items];
  uint32_t cc[2 * kA16Items];
  float m = 0.0f;
  auto code4 = [&](int u) -> uint32_t {
    if constexpr (A8) return *reinterpret_cast<const uint32_t*>(ar + 4 * u);
    else return load_u32_bytes(ar + 4 * u);
  };
  if (held) {
#pragma unroll
    for (int i = 0; i < 2 * kA16Items; ++i) {
      const int u = threadIdx.x + 256 * i;
      const int uu = u < nu ? u : 0;
      cs[i] = sc[uu >> 1];
      cc[i] = code4(uu);
    }
#pragma unroll
    for (int i = 0; i < 2 * kA16Items; ++i)
      if (threadIdx.x + 256 * i < nu) m = __builtin_fmaxf(m, cs[i]);
  } else {
    for (int j = threadIdx.x; j < kb16; j += 256) m = __builtin_fmaxf(m, sc[j]);
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  const int e = row_exponent(m);
  const float inv = __builtin_ldexpf(1.0f, -e);
  if (threadIdx.x == 0) rowscale[row] = __builtin_ldexpf(1.0f, e);
  if (held) {
#pragma unroll
    for (int i = 0; i < 2 * kA16Items; ++i) {
      const int u = threadIdx.x + 256 * i;
      if (u < nu) {
        const float c = cs[i] * inv;
        *reinterpret_cast<v8h*>(out + 8 * u) = dequant8_act(cc[i], c);
      }
    }
  } else {
    for (int u = threadIdx.x; u < nu; u += 256) {
      const float c = sc[u >> 1] * inv;
      *reinterpret_cast<v8h*>(out + 8 * u) = dequant8_act(code4(u), c);
    }
  }
}

constexpr int kTM = 256, kTN = 256, kTK = 64;
constexpr int kTThreads = 256;
constexpr int kAStride = kTM + 1;                 // 16-byte rows per A column chunk (+1 pad)
constexpr int kWStride = kTN + 1;
constexpr size_t kAStage = (size_t)8 * kAStride * 16;
constexpr size_t kWStage = (size_t)2 * kWStride * 16;
constexpr size_t kSStage = (size_t)kTN * 4;
constexpr size_t kStage = kAStage + kWStage + kSStage;
constexpr size_t kTiledLds = 2 * kStage;

// WB: the weight codes at any alignment and K % 16 == 0 (byte loads; the
// upper 16 k of a half-filled last 32-k group read as zero codes).  Same
// products in the same order as gemm_wide, so bit-identical results.
template <bool WB>
__global__ void __launch_bounds__(kTThreads)
gemm_tiled(const _Float16* __restrict__ a16, const float* __restrict__ rowscale,
           const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_sf,
           const float* __restrict__ w_g, _Float16* __restrict__ y, int B, int N, int K,
           int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int tile = blockIdx.x;
  const int tm = tile / tiles_n, tn = tile % tiles_n;
  const int m0 = tm * kTM, n0 = tn * kTN;
  const int64_t kb2 = K / 2, kb16 = K / 16;
  const int nsteps = (K + kTK - 1) / kTK;

  uint4 ra[8], rw[2];
  uint32_t rsf;
  auto gload = [&](int s) {
    const int k0 = s * kTK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = tid + kTThreads * i;
      const int row = p >> 3, c = p & 7;
      const int gr = m0 + row, k = k0 + 8 * c;
      ra[i] = (gr < B && k < K) ? *reinterpret_cast<const uint4*>(a16 + (int64_t)gr * K + k)
                                : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + kTThreads * i;
      const int row = p >> 1, hh = p & 1;
      const int gn = n0 + row, k = k0 + 32 * hh;
      if constexpr (WB)
        rw[i] = (gn < N && k < K) ? load_codes32_bytes(w + (int64_t)gn * kb2 + k / 2, k + 16 < K)
                                  : make_uint4(0, 0, 0, 0);
      else
        rw[i] = (gn < N && k < K) ? *reinterpret_cast<const uint4*>(w + (int64_t)gn * kb2 + k / 2)
                                  : make_uint4(0, 0, 0, 0);
    }
    {
      const int gn = n0 + tid;
      uint32_t v = 0;
      if (gn < N) {
        const uint8_t* p = w_sf + (int64_t)gn * kb16 + k0 / 16;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (k0 + 16 * j < K) v |= (uint32_t)p[j] << (8 * j);
      }
      rsf = v;
    }
  };
  auto lstore = [&](int buf) {
    unsigned char* st = smem + buf * kStage;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = tid + kTThreads * i;
      const int row = p >> 3, c = p & 7;
      *reinterpret_cast<uint4*>(st + ((size_t)c * kAStride + row) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + kTThreads * i;
      const int row = p >> 1, hh = p & 1;
      *reinterpret_cast<uint4*>(st + kAStage + ((size_t)hh * kWStride + row) * 16) = rw[i];
    }
    *reinterpret_cast<uint32_t*>(st + kAStage + kWStage + (size_t)tid * 4) = rsf;
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) gload(s + 1);
    const unsigned char* st = smem + buf * kStage;
    uint4 wcode[4];
    _Float16 wsc0[4], wsc1[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int nl = wn * 128 + nt * 32 + l32;
      wcode[nt] = *reinterpret_cast<const uint4*>(st + kAStage + ((size_t)h * kWStride + nl) * 16);
      // this lane group's two blocks are bytes 2h and 2h+1 of the row's scale word
      const uint32_t sw = *reinterpret_cast<const uint32_t*>(st + kAStage + kWStage + (size_t)nl * 4) >> (16 * h);
      wsc0[nt] = e4m3_b0_f16(sw);
      wsc1[nt] = e4m3_b1_f16(sw);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v8h af[4], bf[4];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const int rl = wm * 128 + bt * 32 + l32;
        af[bt] = *reinterpret_cast<const v8h*>(st + ((size_t)(4 * h + m) * kAStride + rl) * 16);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const uint32_t cw = (m == 0) ? wcode[nt].x : (m == 1) ? wcode[nt].y : (m == 2) ? wcode[nt].z : wcode[nt].w;
        bf[nt] = dequant8_f16(cw, m < 2 ? wsc0[nt] : wsc1[nt]);
      }
#pragma unroll
      for (int bt = 0; bt < 4; ++bt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[bt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[bt], bf[nt], acc[bt][nt], 0, 0, 0);
    }
    if (s + 1 < nsteps) lstore(buf ^ 1);
    __syncthreads();
  }

  const float gw = *w_g;
#pragma unroll
  for (int bt = 0; bt < 4; ++bt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * 128 + bt * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
      if (row >= B) continue;
      const float rsc = rowscale[row] * gw;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int col = n0 + wn * 128 + nt * 32 + l32;
        if (col < N) y[(int64_t)row * N + col] = (_Float16)(acc[bt][nt][r] * rsc);
      }
    }
  }
}


// ------------------------------------------------------------ tiled, LDS-DMA pipeline
//
// The operands go straight from global memory into LDS with
// global_load_lds_dwordx4 / _dword (no staging registers), several LDS stages
// deep, one barrier per 64-k stage.  Requires K % 64 == 0.

constexpr int kP2Threads = 512;

// 128 x 512 output tiles, eight waves side by side in N (128 x 64 each: four
// 32-row x two 32-column v_mfma_f32_32x32x16_f16 blocks), four LDS stages
// (three in flight).  Per 64-k stage the tile needs 16 KB of FP16 activations
// and 16 KB of FP4 weights + 2 KB of E4M3 bytes -- about a sixth fewer bytes
// per MAC than 256 x 256, because the weights are the cheap operand -- and the
// smaller stage leaves room for the fourth buffer.  LDS layouts, chosen so
// that every copy instruction reads whole row segments and the MFMA operand
// reads are free of bank conflicts for both 8-lane (128 B) and 16-lane
// (256 B) groups:
//   A: blocks of 8 rows x 128 B; 16-byte chunk c of row r sits at position
//      c ^ (r & 7) ^ ((r >> 3) & 1) of its row;
//   W: 32 B per row; chunk h of row n at position h ^ (((n >> 2) ^ (n >> 3)) & 1).
// Workgroup order: each XCD takes 64 consecutive tiles, walked 4 M-tiles at a
// time, so its 32 resident workgroups share 4 activation row stripes and 8
// weight column stripes in its L2.
constexpr int kXM = 128, kXN = 512;
constexpr int kXAOff = 0;                          // A: 128 rows x 128 B
constexpr int kXWOff = kXAOff + kXM * 128;         // W: 512 rows x 32 B
constexpr int kXSOff = kXWOff + kXN * 32;          // S: 512 rows x 4 B
constexpr int kXStage = kXSOff + kXN * 4;

// TILED: weights in the pre-tiled layout, where the 16 rows of a row group
// are interleaved so that one 64-k stage of a row group is one contiguous
// 512 B (codes) / 64 B (E4M3 bytes); the copies then read 512 B segments and
// the LDS holds each row group in that order (row r16 + 16 h, h = 32-k half).
template <bool TILED>
__global__ void __launch_bounds__(kP2Threads)
gemm_wide(const _Float16* __restrict__ a16, const float* __restrict__ rowscale,
          const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_sf,
          const float* __restrict__ w_g, _Float16* __restrict__ y, int B, int N, int K,
          int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) unsigned char lds0[kXStage];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[kXStage];
  __shared__ __attribute__((aligned(16))) unsigned char lds2[kXStage];
  __shared__ __attribute__((aligned(16))) unsigned char lds3[kXStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // N slice of 64 columns
  const int l32 = lane & 31, h = lane >> 5;
  const int ntiles = tiles_m * tiles_n;
  int tm, tn;
  {
    const int t = blockIdx.x;
    if (ntiles % 512 == 0 && tiles_m % 4 == 0 && tiles_n % 16 == 0) {
      // groups of 64 tiles (4 M-tiles x 16 N-tiles, N-tiles outer), one group
      // per XCD at a time (consecutive ids go to different XCDs)
      const int xcd = t % 8, l = t / 8 % 64, grp = t / 512;
      const int g = grp * 8 + xcd;
      const int lm = l % 4, ln = l / 4;
      const int groups_n = tiles_n / 16;
      tm = (g / groups_n) * 4 + lm;
      tn = (g % groups_n) * 16 + ln;
    } else {
      tm = t / tiles_n;
      tn = t % tiles_n;
    }
  }
  const int m0 = tm * kXM, n0 = tn * kXN;
  const int nsteps = K / kTK;

  // DMA work of this wave per stage: A blocks 2w, 2w+1 (8 rows each), W rows
  // 64w .. 64w+63 (two copies of 32 rows), E4M3 bytes of rows 64w .. 64w+63.
  // The tile's first row goes into the 64-bit scalar base; the 32-bit lane
  // offsets are relative to it (< 512 rows x K bytes), so no size wraps.
  uint32_t aofs[2], wofs[2], sofs;
  int alds[2], wlds[2], slds;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int blk = wave * 2 + j, r8 = lane >> 3, c = (lane & 7) ^ r8 ^ (blk & 1);
    {
      int r = m0 + 8 * blk + r8;
      r = r < B ? r : B - 1;
      aofs[j] = (uint32_t)(r - m0) * (uint32_t)K * 2u + 16u * c;
      alds[j] = kXAOff + (wave * 2 + j) * 1024;
    }
  }
  if constexpr (TILED) {
    // row group G of the tile (16 rows): K*8 bytes of codes, K bytes of
    // E4M3 bytes; stage st at st*512 / st*64 inside it
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int grp = n0 / 16 + (wave * 2 + j) * 2 + (lane >> 5);
      grp = grp < N / 16 ? grp : N / 16 - 1;
      wofs[j] = (uint32_t)(grp - n0 / 16) * (uint32_t)K * 8u + 16u * (lane & 31);
      wlds[j] = kXWOff + (wave * 2 + j) * 1024;
    }
    {
      int grp = n0 / 16 + wave * 4 + (lane >> 4);
      grp = grp < N / 16 ? grp : N / 16 - 1;
      sofs = (uint32_t)(grp - n0 / 16) * (uint32_t)K + 4u * (lane & 15);
      slds = kXSOff + wave * 256;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rl = 64 * wave + 32 * j + (lane >> 1);
      int r = n0 + rl;
      r = r < N ? r : N - 1;
      wofs[j] = (uint32_t)(r - n0) * (uint32_t)(K / 2) + 16u * ((lane & 1) ^ (((rl >> 2) ^ (rl >> 3)) & 1));
      wlds[j] = kXWOff + (wave * 2 + j) * 1024;
    }
    {
      int r = n0 + 64 * wave + lane;
      r = r < N ? r : N - 1;
      sofs = (uint32_t)(r - n0) * (uint32_t)(K / 16);
      slds = kXSOff + wave * 256;
    }
  }
  const unsigned char* abase = reinterpret_cast<const unsigned char*>(a16) + (size_t)m0 * K * 2;
  const uint8_t* wbase = w + (size_t)n0 * (K / 2);
  const uint8_t* sbase = w_sf + (size_t)n0 * (K / 16);

  auto issue = [&](unsigned char* buf, int st) {
    const int k0 = st * kTK;
    const unsigned char* ab = abase + (size_t)k0 * 2;
    const uint32_t l0 = lds_addr(buf);
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(ab, aofs[j], l0 + alds[j]);
    const uint8_t* wst = TILED ? wbase + (size_t)st * 512 : wbase + k0 / 2;
    const uint8_t* sst = TILED ? sbase + (size_t)st * 64 : sbase + k0 / 16;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(wst, wofs[j], l0 + wlds[j]);
    dma4(sst, sofs, l0 + slds);
  };
  constexpr int kLoads = 5;   // per wave per stage

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto a_off = [](int rl, int c) {
    return kXAOff + (rl >> 3) * 1024 + 16 * (8 * (rl & 7) + (c ^ (rl & 7) ^ ((rl >> 3) & 1)));
  };

  auto compute = [&](const unsigned char* st) {
    uint4 wcode[2];
    v2h wsc[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int nl = wave * 64 + nt * 32 + l32;
      uint32_t sw;
      if constexpr (TILED) {
        const int pos = (nl >> 4) * 32 + (nl & 15) + 16 * h;   // lane order of the row group
        wcode[nt] = *reinterpret_cast<const uint4*>(st + kXWOff + pos * 16);
        sw = *reinterpret_cast<const uint16_t*>(st + kXSOff + pos * 2);
      } else {
        wcode[nt] = *reinterpret_cast<const uint4*>(st + kXWOff + nl * 32 + 16 * (h ^ (((nl >> 2) ^ (nl >> 3)) & 1)));
        sw = *reinterpret_cast<const uint32_t*>(st + kXSOff + nl * 4) >> (16 * h);
      }
      wsc[nt][0] = e4m3_b0_f16(sw);
      wsc[nt][1] = e4m3_b1_f16(sw);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v8h af[4], bf[2];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) af[bt] = *reinterpret_cast<const v8h*>(st + a_off(bt * 32 + l32, 4 * h + m));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const uint32_t cw = (m == 0) ? wcode[nt].x : (m == 1) ? wcode[nt].y : (m == 2) ? wcode[nt].z : wcode[nt].w;
        bf[nt] = dequant8_f16(cw, wsc[nt][m >> 1]);
      }
#pragma unroll
      for (int bt = 0; bt < 4; ++bt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[bt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[bt], bf[nt], acc[bt][nt], 0, 0, 0);
    }
  };
  // one 64-k stage: wait for its DMA (stages s+1, s+2 may stay in flight),
  // barrier, start stage s+3's DMA into the buffer freed by stage s-1, compute
  auto step = [&](const unsigned char* cur, unsigned char* next3, int s) {
    if (s + 2 < nsteps) wait_vmcnt_le<2 * kLoads>();
    else if (s + 1 < nsteps) wait_vmcnt_le<kLoads>();
    else wait_vmcnt_le<0>();
    __builtin_amdgcn_s_barrier();
    if (s + 3 < nsteps) issue(next3, s + 3);
    compute(cur);
  };

  issue(lds0, 0);
  if (nsteps > 1) issue(lds1, 1);
  if (nsteps > 2) issue(lds2, 2);
  for (int s = 0; s < nsteps; s += 4) {
    step(lds0, lds3, s);
    if (s + 1 < nsteps) step(lds1, lds0, s + 1);
    if (s + 2 < nsteps) step(lds2, lds1, s + 2);
    if (s + 3 < nsteps) step(lds3, lds2, s + 3);
  }

  const float gw = *w_g;
#pragma unroll
  for (int bt = 0; bt < 4; ++bt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + bt * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
      if (row >= B) continue;
      const float rsc = rowscale[row] * gw;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int col = n0 + wave * 64 + nt * 32 + l32;
        if (col < N) y[(int64_t)row * N + col] = (_Float16)(acc[bt][nt][r] * rsc);
      }
    }
  }
}

bool use_skinny(int64_t B) { return B <= 16; }

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

// Workspace of the tiled paths: [FP16 activations] [row powers of two].
size_t gemm_workspace_bytes(int64_t B, int64_t N, int64_t K) {
  (void)N;
  if (use_skinny(B)) return 0;
  return align256((size_t)B * (size_t)K * 2) + align256((size_t)B * 4);
}

// Pre-tiled weight layout (offline, once per weight): row group G = rows
// 16G .. 16G+15; for each 128-k chunk c a 1 KiB tile of codes whose 16-byte
// lane l = r + 16 q holds the 32 codes of row 16G + r at k = 128c + 32q ..
// +31, and a 128-byte tile of E4M3 bytes whose 2-byte lane l holds that
// row's bytes for the same 32 k.  Tiles are stored (G, c) row-major, so a row
// group's codes are contiguous (K*8 bytes), as are its E4M3 bytes (K bytes).
// One thread per lane: a plain permutation of 16-byte and 2-byte pieces.
__global__ void __launch_bounds__(256)
pretile_weight(const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_sf, int64_t ntiles,
               int nch, int K, uint8_t* __restrict__ wt, uint8_t* __restrict__ st) {
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= ntiles) return;
  const int l = threadIdx.x & 63;
  const int64_t grp = tile / nch;
  const int c = (int)(tile - grp * nch);
  const int64_t r = 16 * grp + (l & 15);
  const int k = 128 * c + 32 * (l >> 4);
  *reinterpret_cast<uint4*>(wt + (tile * 64 + l) * 16) =
      *reinterpret_cast<const uint4*>(w + r * (K / 2) + k / 2);
  *reinterpret_cast<uint16_t*>(st + (tile * 64 + l) * 2) =
      *reinterpret_cast<const uint16_t*>(w_sf + r * (K / 16) + k / 16);
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, []() {
    for (int wl = kWPlain; wl <= kWBytes && attr_err == hipSuccess; ++wl)
      for (int a4 = 0; a4 < 2 && attr_err == hipSuccess; ++a4)
        for (int B : {1, 3, 5, 9})   // one B per kernel instance
          if (attr_err == hipSuccess)
            attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(skinny_kernel(B, a4 != 0, wl)),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)skinny_lds(B));
    if (attr_err == hipSuccess)
      attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_tiled<false>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kTiledLds);
    if (attr_err == hipSuccess)
      attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_tiled<true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kTiledLds);

  });
  if (attr_err != hipSuccess) return attr_err;
  const int B = (int)g.B, N = (int)g.N, K = (int)g.K;
  _Float16* y = reinterpret_cast<_Float16*>(g.y);
  // 16-byte weight rows and 2-byte scale rows, else the byte-load path
  const bool w_rows16 = ((uintptr_t)g.w % 16) == 0 && (K % 32) == 0 && ((uintptr_t)g.w_sf % 2) == 0;
  const int wl = g.tiled ? kWTiled : (w_rows16 ? kWPlain : kWBytes);
  if (use_skinny(g.B)) {
    const unsigned grid = (unsigned)((N + kSkRows - 1) / kSkRows);
    // FP4 kernel: 16-byte activation code and scale loads (16-byte aligned
    // rows and bases); FP16 kernel: 4-byte aligned activation codes
    const bool x = B <= kSkFp4MaxB
                       ? ((uintptr_t)g.a % 16) == 0 && ((uintptr_t)g.a_scale % 16) == 0 && K % 64 == 0
                       : ((uintptr_t)g.a % 4) == 0;
    const SkinnyFn fn = skinny_kernel(B, x, wl);
    hipLaunchKernelGGL(fn, dim3(grid), dim3(kSkThreads), skinny_lds(B), s, g.a, g.a_scale, g.w,
                       g.w_sf, g.w_g, y, B, N, K);
    return hipGetLastError();
  }
  unsigned char* ws = reinterpret_cast<unsigned char*>(g.workspace);
  _Float16* a16 = reinterpret_cast<_Float16*>(ws);
  float* rowscale = reinterpret_cast<float*>(ws + align256((size_t)B * (size_t)K * 2));
  // gemm_wide's copies take 32-bit lane offsets of up to 512 rows x K bytes
  const bool wide = g.tiled || (w_rows16 && K % kTK == 0 && ((uintptr_t)g.w_sf % 4) == 0 && g.K <= (1 << 24));
  if ((uintptr_t)g.a % 8 == 0)
    hipLaunchKernelGGL(a_to_f16_rows<true>, dim3((unsigned)B), dim3(256), 0, s, g.a, g.a_scale, a16, rowscale, K);
  else
    hipLaunchKernelGGL(a_to_f16_rows<false>, dim3((unsigned)B), dim3(256), 0, s, g.a, g.a_scale, a16, rowscale, K);
  if (wide) {
    const int wtm = (B + kXM - 1) / kXM, wtn = (N + kXN - 1) / kXN;
    if (g.tiled)
      hipLaunchKernelGGL(gemm_wide<true>, dim3((unsigned)(wtm * wtn)), dim3(kP2Threads), 0, s, a16,
                         rowscale, g.w, g.w_sf, g.w_g, y, B, N, K, wtm, wtn);
    else
      hipLaunchKernelGGL(gemm_wide<false>, dim3((unsigned)(wtm * wtn)), dim3(kP2Threads), 0, s, a16,
                         rowscale, g.w, g.w_sf, g.w_g, y, B, N, K, wtm, wtn);
  } else {
    const int tiles_m = (B + kTM - 1) / kTM, tiles_n = (N + kTN - 1) / kTN;
    hipLaunchKernelGGL(w_rows16 ? gemm_tiled<false> : gemm_tiled<true>, dim3((unsigned)(tiles_m * tiles_n)),
                       dim3(kTThreads), kTiledLds, s, a16, rowscale, g.w, g.w_sf, g.w_g, y, B, N, K, tiles_n);
  }
  return hipGetLastError();
}

hipError_t launch_pretile(const uint8_t* w, const uint8_t* w_sf, int64_t N, int64_t K,
                          uint8_t* w_tiled, uint8_t* sf_tiled, hipStream_t s) {
  const int nch = (int)(K / 128);
  const int64_t ntiles = N / 16 * nch;
  hipLaunchKernelGGL(pretile_weight, dim3((unsigned)((ntiles + 3) / 4)), dim3(256), 0, s, w, w_sf, ntiles,
                     nch, (int)K, w_tiled, sf_tiled);
  return hipGetLastError();
}

}  // namespace nvfp4
