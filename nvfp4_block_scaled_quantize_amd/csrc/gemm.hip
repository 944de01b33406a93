// gemm.hip -- block-scaled NVFP4 GEMM y[B,N] = deq(a)[B,K] . deq(w)[N,K]^T with
// FP16 output, the operation of "Fused Nvfp4 GEMM All Reduce Plugin"
// (baked-weight inputs 0..4, output 0), for gfx950.
//
// Why FP16 MFMA: gfx950's scaled f8f6f4 MFMA applies power-of-two (E8M0)
// scales per 32 K-elements, while NVFP4 carries an E4M3 scale per 16 elements
// and the activation side an arbitrary FP32 scale per 16 elements.  The
// dequantized weight e2m1 * e4m3 has at most 6 significant bits and lies in
// [2^-10, 2688], so it is EXACT in FP16; the global weight scale moves to the
// epilogue.  The activation q * c is rounded once to FP16 after a per-row
// power-of-two normalization (so no row can overflow FP16), and the row's
// power of two returns in the epilogue.  Products accumulate in FP32.
//
// Two kernels, chosen by the batch size:
//  * gemm_skinny (B <= 16, decode): a streaming GEMV-like pass over the weight
//    matrix.  Each wave owns 16 weight rows and one quarter of K; every lane
//    issues 16-byte loads of 32 consecutive FP4 codes of its row (eight loads in
//    flight per lane), converts them with v_cvt_scalef32_pk_f16_fp4 and one
//    packed FP16 multiply by the E4M3 scale, and feeds v_mfma_f32_16x16x32_f16
//    with the (up to 16) activation rows as the other operand.  The activations
//    are dequantized once per workgroup into LDS while the first weight chunks
//    are in flight.  The four K quarters are summed in LDS in a fixed order
//    (deterministic).
//  * gemm_wide (larger B, prefill, K % 64 == 0): a prologue kernel writes the
//    normalized FP16 activations once; the main kernel computes 128 x 512
//    output tiles with 8 waves (128 x 64 each, v_mfma_f32_32x32x16_f16),
//    streaming FP16 activations, packed FP4 weight codes and E4M3 bytes from
//    global memory straight into four LDS stages; weights are dequantized in
//    registers right before each MFMA.  gemm_tiled (256 x 256 tiles, register
//    staging) serves K % 64 != 0.
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

// Weight operand layouts of the GEMM kernels.
constexpr int kWPlain = 0;   // [N, K/2] codes, 16-byte aligned rows (K % 32 == 0)
constexpr int kWTiled = 1;   // the pre-tiled layout
constexpr int kWBytes = 2;   // [N, K/2] codes at any alignment, K % 16 == 0 (byte loads)

// ------------------------------------------------------------ skinny (decode)

constexpr int kSkThreads = 512;   // 8 waves
constexpr int kSkNsub = 2;        // 16-row subtiles per workgroup
constexpr int kSkKs = 4;          // K quarters per workgroup
constexpr int kSkRows = 16 * kSkNsub;
constexpr int kSkPF = 8;          // 128-k chunks loaded per round per wave
constexpr int kSkItems = 16;      // activation items (8 codes) per thread
constexpr int kSkEarly = 5;       // weight chunks loaded before the activation prologue
constexpr size_t kSkRedBytes = (size_t)kSkKs * kSkRows * 16 * sizeof(float);

// One workgroup = 8 waves = 2 sixteen-row weight subtiles x 4 K quarters.
// Order of work, chosen against the memory latency chain of one workgroup:
//  1. every thread issues the loads of its activation items (a few codes +
//     combined scales; shared by all workgroups, so they hit L2), the global
//     weight scale, and the weight loads of the first kSkEarly chunks;
//  2. row maxima of the combined scales (wave reduction + LDS integer max),
//     the per-row power of two, and the FP16 activations in LDS -- three
//     barriers, which wait only for the issue of the few loads above (a wave
//     whose weight loads are throttled by HBM would hold every barrier);
//  3. the remaining weight loads of the round, then MFMAs chunk by chunk as the
//     data arrives (in-order load counter).  The first round is straight-line
//     code: inside a loop the compiler drained every outstanding load at the
//     loop head, so the later chunks' loads waited a full memory latency;
//  4. the four K quarters are summed in LDS in a fixed order.
// A4: activation codes 4-byte aligned (dword loads), else byte loads.
// NI: activation items (units of eight codes) per thread, >= B * ceil(K/8 / 512).
// WL = kWTiled: the weights are in the pre-tiled layout (nvfp4_pretile_weight):
// each wave-load of 16 rows x 128 k is one contiguous KiB (codes) / 128 B (E4M3
// bytes) instead of 16 row segments.  WL = kWBytes: the scalar path for
// weights at any alignment and K % 16 == 0: the same arithmetic on the same
// values (bit-identical results), with byte loads, and both operands zeroed
// for the k past the row end of a half-filled last 32-k group.
template <bool A4, int NI, int WL>
__global__ void __launch_bounds__(kSkThreads)
gemm_skinny(const uint8_t* __restrict__ a, const float* __restrict__ a_scale,
            const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_sf,
            const float* __restrict__ w_g, _Float16* __restrict__ y, int B, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ float rs[16];
  __shared__ float rinv[16];
  __shared__ uint32_t rmax[16];
  const int pitch = K + 8;   // halves; keeps consecutive activation rows 16 B apart in bank space
  _Float16* As = reinterpret_cast<_Float16*>(smem);
  float* red = reinterpret_cast<float*>(smem + (((size_t)B * pitch * 2 + 15) / 16) * 16);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int nsub = wave % kSkNsub, ks = wave / kSkNsub;
  const int r16 = lane & 15, g = lane >> 4;
  const int nrow = blockIdx.x * kSkRows + nsub * 16 + r16;
  const int64_t kb2 = K / 2, kb16 = K / 16;
  const int nchunks = (K + 127) >> 7;
  if (tid < 16) rmax[tid] = 0u;

  // 1a. this thread's activation items: item j is unit q8 = tid + 512 i (eight
  //     codes) of row b, (b, i) running over (0, 0), (0, 1), ..., (0, ipr-1),
  //     (1, 0), ... (wave-uniform counters).  Loads are unconditional: items
  //     past the last row or the row end re-load a valid unit (masked later).
  const int per_row = K / 8;
  const int ipr = (per_row + kSkThreads - 1) / kSkThreads;
  uint32_t acode[NI];
  float ascl[NI];
  {
    int b = 0, i = 0;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int q8 = tid + kSkThreads * i;
      const int bb = b < B ? b : B - 1;
      const int qq = q8 < per_row ? q8 : 0;
      const uint8_t* pa = a + (int64_t)bb * kb2 + 4 * (int64_t)qq;
      acode[j] = A4 ? *reinterpret_cast<const uint32_t*>(pa) : load_u32_bytes(pa);
      ascl[j] = a_scale[(int64_t)bb * kb16 + qq / 2];
      if (++i == ipr) { i = 0; ++b; }
    }
  }
  const float gw = *w_g;

  // 1b. weight loads.  Rows past N re-load row N-1 (their outputs are not
  //     stored); chunks past the end of K re-load chunk 0 and are skipped.
  const uint8_t* wr = w + (int64_t)(nrow < N ? nrow : N - 1) * kb2;
  const uint8_t* sr = w_sf + (int64_t)(nrow < N ? nrow : N - 1) * kb16;
  uint4 wc[kSkPF];
  uint32_t wsv[kSkPF];
  auto load_chunks = [&](int c0, int i0, int i1) {
#pragma unroll
    for (int i = 0; i < kSkPF; ++i) {
      if (i < i0 || i >= i1) continue;
      const int c = c0 + i * kSkKs;
      if constexpr (WL == kWTiled) {
        // tile (row group, chunk), lane order r16 + 16 g (K % 128 == 0)
        const int64_t t = ((int64_t)(nrow < N ? nrow : N - 1) / 16 * nchunks + (c < nchunks ? c : 0)) * 64 + lane;
        wc[i] = *reinterpret_cast<const uint4*>(w + t * 16);
        wsv[i] = (uint32_t)*reinterpret_cast<const uint16_t*>(w_sf + t * 2);
      } else if constexpr (WL == kWBytes) {
        const int k0 = c * 128 + 32 * g;
        const int k = (c < nchunks && k0 < K) ? k0 : 0;
        const bool full = k + 16 < K;
        wc[i] = load_codes32_bytes(wr + k / 2, full);
        wsv[i] = (uint32_t)sr[k / 16] | (full ? (uint32_t)sr[k / 16 + 1] << 8 : 0u);
      } else {
        const int k0 = c * 128 + 32 * g;
        const int k = (c < nchunks && k0 < K) ? k0 : 0;
        wc[i] = *reinterpret_cast<const uint4*>(wr + k / 2);
        wsv[i] = (uint32_t)*reinterpret_cast<const uint16_t*>(sr + k / 16);
      }
    }
  };
  load_chunks(ks, 0, kSkEarly);
  __syncthreads();   // rmax cleared

  // 2. per-row power-of-two normalization: row max of the (non-negative)
  //    combined scales as an integer max of their bits, per wave then in LDS
  {
    float cur = 0.0f;
    int b = 0, i = 0;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const bool v = tid + kSkThreads * i < per_row;
      cur = __builtin_fmaxf(cur, v ? ascl[j] : 0.0f);
      if (i + 1 == ipr || j == NI - 1) {
        if (b < B) {
          const float m = wave_max_dpp(cur);
          if (lane == 0) atomicMax(&rmax[b], __float_as_uint(m) & 0x7FFFFFFFu);
        }
        cur = 0.0f;
      }
      if (++i == ipr) { i = 0; ++b; }
    }
  }
  __syncthreads();
  if (tid < B) {
    const int e = row_exponent(__uint_as_float(rmax[tid]));
    rs[tid] = __builtin_ldexpf(1.0f, e);
    rinv[tid] = __builtin_ldexpf(1.0f, -e);
  }
  __syncthreads();
  {
    int b = 0, i = 0;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int q8 = tid + kSkThreads * i;
      if (b < B && q8 < per_row)
        *reinterpret_cast<v8h*>(As + (int64_t)b * pitch + 8 * q8) = dequant8_act(acode[j], ascl[j] * rinv[b]);
      if (++i == ipr) { i = 0; ++b; }
    }
  }
  __syncthreads();

  // 3. stream the weights.  Batch columns past B read row B-1 of the LDS
  //    activations; their outputs are never stored.
  load_chunks(ks, kSkEarly, kSkPF);
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const _Float16* arow = As + (r16 < B ? r16 : B - 1) * pitch;
  auto compute_round = [&](int c0) {
#pragma unroll
    for (int i = 0; i < kSkPF; ++i) {
      const int c = c0 + i * kSkKs;
      if (c < nchunks) {   // wave-uniform
        const int k = c * 128 + 32 * g;
        const bool kv = k < K;   // false only in a partial last chunk
        v8h bf[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) bf[m] = *reinterpret_cast<const v8h*>(arow + (kv ? k : 0) + 8 * m);
        if constexpr (WL == kWBytes) {
          // k + 16 .. k + 31 past the row end: the LDS there is not this row
          if (k + 16 >= K) { bf[2] = v8h{}; bf[3] = v8h{}; }
        }
        const _Float16 s0 = e4m3_b0_f16(wsv[i]), s1 = e4m3_b1_f16(wsv[i]);
        const uint32_t cw[4] = {kv ? wc[i].x : 0u, kv ? wc[i].y : 0u, kv ? wc[i].z : 0u, kv ? wc[i].w : 0u};
#pragma unroll
        for (int m = 0; m < 4; ++m)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(dequant8_f16(cw[m], m < 2 ? s0 : s1), bf[m], acc, 0, 0, 0);
      }
    }
  };
  // the first round straight-line (its loads were issued above), later rounds
  // (K > 4096) in a loop
  compute_round(ks);
  for (int c0 = ks + kSkPF * kSkKs; c0 < nchunks; c0 += kSkPF * kSkKs) {
    load_chunks(c0, 0, kSkPF);
    compute_round(c0);
  }

  // 4. sum the K quarters in a fixed order, scale, round to FP16
#pragma unroll
  for (int r = 0; r < 4; ++r) red[(ks * kSkRows + nsub * 16 + 4 * g + r) * 16 + r16] = acc[r];
  __syncthreads();
  for (int t = tid; t < 16 * kSkRows; t += kSkThreads) {
    const int b = t / kSkRows, nl = t % kSkRows;
    const int n = blockIdx.x * kSkRows + nl;
    if (b < B && n < N) {
      float s = red[(0 * kSkRows + nl) * 16 + b];
#pragma unroll
      for (int q = 1; q < kSkKs; ++q) s += red[(q * kSkRows + nl) * 16 + b];
      y[(int64_t)b * N + n] = (_Float16)((s * rs[b]) * gw);
    }
  }
}

typedef void (*SkinnyFn)(const uint8_t*, const float*, const uint8_t*, const uint8_t*, const float*,
                         _Float16*, int, int, int);

// The instantiation with the fewest activation items per thread covering ni.
template <bool A4, int WL>
SkinnyFn skinny_kernel_a(int ni) {
  if (ni <= 1) return gemm_skinny<A4, 1, WL>;
  if (ni <= 2) return gemm_skinny<A4, 2, WL>;
  if (ni <= 4) return gemm_skinny<A4, 4, WL>;
  if (ni <= 8) return gemm_skinny<A4, 8, WL>;
  return gemm_skinny<A4, kSkItems, WL>;
}
// The byte-load weight path uses byte loads for the activation codes too.
SkinnyFn skinny_kernel(bool a4, int ni, int wl) {
  if (wl == kWBytes) return skinny_kernel_a<false, kWBytes>(ni);
  if (wl == kWTiled) return a4 ? skinny_kernel_a<true, kWTiled>(ni) : skinny_kernel_a<false, kWTiled>(ni);
  return a4 ? skinny_kernel_a<true, kWPlain>(ni) : skinny_kernel_a<false, kWPlain>(ni);
}

size_t skinny_lds_bytes(int64_t B, int64_t K) {
  return (((size_t)B * (size_t)(K + 8) * 2 + 15) / 16) * 16 + kSkRedBytes;
}

// Dynamic LDS budget of the skinny kernel (its static LDS is 192 bytes).
constexpr size_t kSkinnyDynMax = 160 * 1024 - 1024;

// ------------------------------------------------------------ tiled (prefill)

// Prologue: one workgroup per activation row -> normalized FP16 row and its
// power of two.
__global__ void __launch_bounds__(256)
a_to_f16_rows(const uint8_t* __restrict__ a, const float* __restrict__ a_scale,
              _Float16* __restrict__ a16, float* __restrict__ rowscale, int K) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int64_t kb16 = K / 16;
  const float* sc = a_scale + row * kb16;
  float m = 0.0f;
  for (int64_t j = threadIdx.x; j < kb16; j += 256) m = __builtin_fmaxf(m, sc[j]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  const int e = row_exponent(m);
  const float inv = __builtin_ldexpf(1.0f, -e);
  if (threadIdx.x == 0) rowscale[row] = __builtin_ldexpf(1.0f, e);
  const uint8_t* ar = a + row * (K / 2);
  for (int64_t j = threadIdx.x; j < kb16; j += 256) {
    const float c = sc[j] * inv;
    const uint32_t c0 = load_u32_bytes(ar + 8 * j), c1 = load_u32_bytes(ar + 8 * j + 4);
    _Float16* out = a16 + row * K + 16 * j;
    *reinterpret_cast<v8h*>(out) = dequant8_act(c0, c);
    *reinterpret_cast<v8h*>(out + 8) = dequant8_act(c1, c);
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

bool use_skinny(int64_t B, int64_t K) {
  const int64_t ipr = (K / 8 + kSkThreads - 1) / kSkThreads;
  return B <= 16 && skinny_lds_bytes(B, K) <= kSkinnyDynMax && B * ipr <= kSkItems;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

// Workspace of the tiled paths: [FP16 activations] [row powers of two].
size_t gemm_workspace_bytes(int64_t B, int64_t N, int64_t K) {
  (void)N;
  if (use_skinny(B, K)) return 0;
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
        for (int ni = 1; ni <= kSkItems && attr_err == hipSuccess; ni *= 2)
          attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(skinny_kernel(a4 != 0, ni, wl)),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSkinnyDynMax);
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
  if (use_skinny(g.B, g.K)) {
    const unsigned grid = (unsigned)((N + kSkRows - 1) / kSkRows);
    const int ni = B * ((K / 8 + kSkThreads - 1) / kSkThreads);
    const SkinnyFn fn = skinny_kernel(((uintptr_t)g.a % 4) == 0, ni, wl);
    hipLaunchKernelGGL(fn, dim3(grid), dim3(kSkThreads), skinny_lds_bytes(B, K), s, g.a, g.a_scale,
                       g.w, g.w_sf, g.w_g, y, B, N, K);
    return hipGetLastError();
  }
  unsigned char* ws = reinterpret_cast<unsigned char*>(g.workspace);
  _Float16* a16 = reinterpret_cast<_Float16*>(ws);
  float* rowscale = reinterpret_cast<float*>(ws + align256((size_t)B * (size_t)K * 2));
  // gemm_wide's copies take 32-bit lane offsets of up to 512 rows x K bytes
  const bool wide = g.tiled || (w_rows16 && K % kTK == 0 && ((uintptr_t)g.w_sf % 4) == 0 && g.K <= (1 << 24));
  hipLaunchKernelGGL(a_to_f16_rows, dim3((unsigned)B), dim3(256), 0, s, g.a, g.a_scale, a16,
                     rowscale, K);
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
