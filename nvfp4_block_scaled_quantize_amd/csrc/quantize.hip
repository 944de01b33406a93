// quantize.hip -- NVFP4 quantization kernels for gfx950.
//
// Per-token path (one workgroup per row): the row is read from HBM once and
// kept in VGPRs between the amax pass and the encode pass -- the role the
// shared-memory caching of input vectors plays in "perf: optimize per-token
// nvfp4 quantization kernel" (flashinfer pull request 3237, review).  A lane
// loads units of 8 consecutive values with one 16-byte load, consecutive lanes
// read consecutive units (each wave load is one contiguous 1 KiB span), so a
// 16-element block spans an adjacent lane pair and its amax is an in-lane max
// plus one pair exchange; only the row amax needs a wave + LDS reduction.
// Each lane writes the 4 code bytes of its unit with one 4-byte store
// ("Building Custom TensorRT-LLM Plugins for Low-Latency FP8 Inference at
// Scale", "Fusing the Kernel in CUDA": vector loads, fused encode).
//
// The optional activation (SwiGLU: gate = first half of the row, up = second
// half; ReLU^2) runs in fp32 registers in front of the quantizer, so the
// activation output never reaches HBM (same article, "The Cost of Non-Fused
// Quantization").
//
// SwiGLU on bf16 inputs with many rows: silu depends only on the 16-bit gate
// pattern, so each workgroup first tabulates silu in LDS for every bf16 gate
// with |g| in [2^-24, 256) (8192 entries: both signs, 32 exponents, 128
// mantissas) using the same binary32 evaluation as the direct path, then
// streams rows persistently, replacing exp + division by one LDS read.  Gates
// outside the table (tiny, huge, non-finite) are recomputed directly, so the
// output is bit-identical to the direct evaluation.
//
// Per-group path (per tensor / per expert): a partial-amax kernel writes at
// most 1024 partial maxima per group into the workspace, a second kernel
// reduces them to one maximum per group, and the row kernel uses that instead
// of its own row's.
//
// MXFP4 variant (the UE8M0_SF switch of the block helper in the same pull
// request): the same row kernel with 32-element blocks -- four adjacent lanes'
// units -- and an E8M0 scale byte per block, the smallest power of two at or
// above (amax_b / 6) * g_enc.  It can write the MX tile layout the
// block-scaled MFMA GEMM reads (32-row groups, one 16-byte lane piece per 32
// codes); then the padding rows of the last group are written as zeros.
//
// A scalar fallback handles inputs that are not 16-byte aligned (or codes not
// 4-byte aligned) and rows longer than the register cache, with identical
// results (same article, "Production Pitfalls & Hard Lessons", item 1).
#include "device_common.h"
#include "internal.h"

namespace nvfp4 {

namespace {

constexpr int kMaxThreads = 256;     // per-row kernel and fallback
constexpr int kMaxUnits = 16;        // 8-value units per thread held in registers
constexpr int kTabUnits = 2;         // persistent SwiGLU kernel: units per thread,
constexpr int kTabThreads = 1024;    // at most this many threads per workgroup
constexpr uint32_t kTabE0 = 103;     // smallest tabulated biased exponent: |g| >= 2^-24
constexpr int kTabHalf = 32 * 128;   // entries per sign: exponents 103..134 (|g| < 256)
constexpr int kTabMinRows = 1024;    // below this the per-workgroup table does not pay off

// Raw 16-byte loads of this thread's L units of a row (gate and, for SwiGLU,
// up).  Units past the row end load the row's last unit instead, so every
// load is issued unconditionally and all of them are in flight together; the
// caller masks those units out.
template <int ACT, int L>
__device__ __forceinline__ void load_units(const uint16_t* __restrict__ xr, int64_t k_out, int units,
                                           int tid, int T, u32x4 (&g)[L], u32x4 (&u)[L]) {
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int q0 = tid + i * T;
    const int q = q0 < units ? q0 : units - 1;
    g[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + 8 * (int64_t)q));
    if constexpr (ACT == kActSwiglu)
      u[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + k_out + 8 * (int64_t)q));
  }
}

// The eight activation outputs of one unit from its raw words.
template <int DT, int ACT>
__device__ __forceinline__ void unit_values(const u32x4& g, const u32x4& u, float* y) {
  const uint32_t w[4] = {g.x, g.y, g.z, g.w};
  if constexpr (ACT == kActSwiglu) {
    const uint32_t v[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float ga, gb, ua, ub;
      unpack2<DT>(w[i], ga, gb);
      unpack2<DT>(v[i], ua, ub);
      y[2 * i] = swiglu_f32(ga, ua);
      y[2 * i + 1] = swiglu_f32(gb, ub);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a0, a1;
      unpack2<DT>(w[i], a0, a1);
      if constexpr (ACT == kActRelu2) { a0 = relu2_f32(a0); a1 = relu2_f32(a1); }
      y[2 * i] = a0;
      y[2 * i + 1] = a1;
    }
  }
}

template <int DT, int ACT>
__device__ __forceinline__ void load_block_scalar(const uint16_t* __restrict__ xr, int64_t k_out,
                                                  int64_t j, float* y) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    int64_t k = 16 * j + e;
    if constexpr (ACT == kActSwiglu) {
      y[e] = swiglu_f32(unpack1<DT>(xr[k]), unpack1<DT>(xr[k_out + k]));
    } else {
      float v = unpack1<DT>(xr[k]);
      y[e] = (ACT == kActRelu2) ? relu2_f32(v) : v;
    }
  }
}

// Block-wide max; every thread gets the result.  `red` holds one float per
// wave; the caller separates reuses of `red` by a barrier.
__device__ __forceinline__ float block_max(float v, float* red) {
  const float w = wave_max_dpp(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = w;
  __syncthreads();
  float m = red[0];
  const int nw = (blockDim.x + 63) >> 6;
  for (int i = 1; i < nw; ++i) m = __builtin_fmaxf(m, red[i]);
  return m;
}

// Global scales of this row: its own amax (per token) or its group's partials.
__device__ __forceinline__ float partials_max(const float* __restrict__ parts, int64_t row,
                                              int64_t group_rows, int nparts) {
  const float* pp = parts + (row / group_rows) * (int64_t)nparts;
  float m = 0.0f;
  for (int p = threadIdx.x; p < nparts; p += blockDim.x) m = __builtin_fmaxf(m, pp[p]);
  return m;
}

// Block amax of a unit from its own 8 values and its pair lane's.
__device__ __forceinline__ float unit_pair_max(const float* y) {
  float m = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(y[e]));
  return __builtin_fmaxf(m, dpp_f32<0xB1>(m));
}

// Encodes this thread's L units of a row.  Unit i of the two lanes of a pair
// is one 16-block; the pair splits the block scales between them (the lane
// of parity p evaluates the blocks of units i = p, p+2, ...) and exchanges
// the encode factors, so each block's scale is computed once and each lane
// stores the scale bytes of the blocks it evaluated.
template <int L>
__device__ __forceinline__ void encode_units(const float (&y)[L][8], const float (&am)[L], float g_enc,
                                             float gd, int tid, int T, int units,
                                             uint8_t* __restrict__ cr, uint8_t* __restrict__ sr,
                                             float* __restrict__ scr) {
  constexpr int J = (L + 1) / 2;
  const int p = tid & 1;
  const uint32_t pmask = 0u - (uint32_t)p;   // all ones on odd lanes
  float enc_own[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i_odd = (2 * j + 1 < L) ? 2 * j + 1 : 2 * j;
    // bit select rather than a lane-dependent array index, which the compiler
    // would turn into a memory access
    const float amb = __uint_as_float((__float_as_uint(am[i_odd]) & pmask) |
                                      (__float_as_uint(am[2 * j]) & ~pmask));
    float c, enc;
    const uint32_t sbyte = block_scale(amb, g_enc, gd, c, enc);
    enc_own[j] = enc;
    const int i = 2 * j + p;
    const int q = tid + i * T;
    if (i < L && q < units) {
      sr[q >> 1] = (uint8_t)sbyte;
      if (scr) scr[q >> 1] = c;
    }
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const float other = dpp_f32<0xB1>(enc_own[j]);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int i = 2 * j + b;
      if (i >= L) continue;
      const float enc = (b == p) ? enc_own[j] : other;
      const int q = tid + i * T;
      if (q < units)
        __builtin_nontemporal_store(pack8_e2m1(y[i], enc), reinterpret_cast<uint32_t*>(cr + 4 * (int64_t)q));
    }
  }
}

// Row kernel with the row cached in registers: L units per thread, one row
// per workgroup, blockDim.x a multiple of 64 (so unit pairs share a wave).
template <int DT, int ACT, int L>
__global__ void __launch_bounds__(kMaxThreads)
quant_rows_vec(const uint16_t* __restrict__ x, int64_t k_out, int units,
               uint8_t* __restrict__ codes, uint8_t* __restrict__ sf, float* __restrict__ g_dec,
               float* __restrict__ scale_out, const float* __restrict__ parts, int64_t group_rows,
               int nparts) {
  __shared__ float red[kMaxThreads / 64];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, T = blockDim.x;
  const int64_t k_in = (ACT == kActSwiglu) ? 2 * k_out : k_out;
  const uint16_t* xr = x + row * k_in;
  u32x4 rg[L], ru[L];
  load_units<ACT, L>(xr, k_out, units, tid, T, rg, ru);
  float y[L][8];
  float am[L];
  float tmax = 0.0f;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    unit_values<DT, ACT>(rg[i], ru[i], y[i]);
    const float m = unit_pair_max(y[i]);
    am[i] = (tid + i * T < units) ? m : 0.0f;
    tmax = __builtin_fmaxf(tmax, am[i]);
  }
  if (parts != nullptr) tmax = partials_max(parts, row, group_rows, nparts);
  const float amax = block_max(tmax, red);
  float g_enc, gd;
  global_scales(amax, g_enc, gd);
  if (tid == 0) {
    if (group_rows == 1) g_dec[row] = gd;
    else if (row % group_rows == 0) g_dec[row / group_rows] = gd;
  }
  uint8_t* cr = codes + row * (k_out / 2);
  uint8_t* sr = sf + row * (k_out / 16);
  float* scr = scale_out ? scale_out + row * (k_out / 16) : nullptr;
  encode_units<L>(y, am, g_enc, gd, tid, T, units, cr, sr, scr);
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// silu of the two bf16 gates of one dword from the LDS table.  With
// t = h - (kTabE0 << 7) per 16-bit half, a gate is in the table iff bits
// 12..14 of t are clear (t in [0, 0x1000) for +, [0x8000, 0x9000) for -); the
// entry is (t & 0xFFF) + 0x1000 * sign.  `acc` collects t for the miss test.
__device__ __forceinline__ void silu_tab2(uint32_t w, const float* tab, uint32_t& acc, float& lo,
                                          float& hi) {
  const u16x2 k0 = {(uint16_t)(kTabE0 << 7), (uint16_t)(kTabE0 << 7)};
  const uint32_t t = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, w) - k0);
  acc |= t;
  const uint32_t idx = (t & 0x0FFF0FFFu) | ((t >> 3) & 0x10001000u);
  lo = tab[idx & 0xFFFFu];
  hi = tab[idx >> 16];
}

// One row of the tabulated SwiGLU kernel from its raw gate/up words.
template <int L>
__device__ __forceinline__ void swiglu_tab_row(const u32x4 (&rg)[L], const u32x4 (&ru)[L],
                                               const float* tab, float* red, int64_t row,
                                               int64_t k_out, int units, uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ sf, float* __restrict__ g_dec,
                                               float* __restrict__ scale_out) {
  const int tid = threadIdx.x, T = blockDim.x;
  float y[L][8];
  uint32_t miss = 0;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const uint32_t gw[4] = {rg[i].x, rg[i].y, rg[i].z, rg[i].w};
    const uint32_t uw[4] = {ru[i].x, ru[i].y, ru[i].z, ru[i].w};
    uint32_t acc = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float slo, shi;
      silu_tab2(gw[e], tab, acc, slo, shi);
      y[i][2 * e] = slo * bf16_lo(uw[e]);
      y[i][2 * e + 1] = shi * bf16_hi(uw[e]);
    }
    if (tid + i * T < units) miss |= acc;   // padding units are never recomputed
  }
  if (miss & 0x70007000u) {   // a gate outside the table in this lane: evaluate directly
#pragma unroll
    for (int i = 0; i < L; ++i) unit_values<kBf16, kActSwiglu>(rg[i], ru[i], y[i]);
  }
  float am[L];
  float tmax = 0.0f;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const float m = unit_pair_max(y[i]);
    am[i] = (tid + i * T < units) ? m : 0.0f;
    tmax = __builtin_fmaxf(tmax, am[i]);
  }
  const float amax = block_max(tmax, red);
  float g_enc, gd;
  global_scales(amax, g_enc, gd);
  if (tid == 0) g_dec[row] = gd;
  uint8_t* cr = codes + row * (k_out / 2);
  uint8_t* sr = sf + row * (k_out / 16);
  float* scr = scale_out ? scale_out + row * (k_out / 16) : nullptr;
  encode_units<L>(y, am, g_enc, gd, tid, T, units, cr, sr, scr);
}

// Persistent fused SwiGLU + per-token quantize for bf16 rows.  Rows rotate
// through three register buffers: the loads of the next two rows are in
// flight while a row is reduced and encoded.  Rows past the end re-load the
// last row (never used), so loads stay unconditional.  red[0..2] belong to
// the three buffers, so two barriers separate consecutive uses of one.
template <int L>
__global__ void __launch_bounds__(kTabThreads)
swiglu_quant_tab(const uint16_t* __restrict__ x, int64_t rows, int64_t k_out, int units,
                 uint8_t* __restrict__ codes, uint8_t* __restrict__ sf, float* __restrict__ g_dec,
                 float* __restrict__ scale_out) {
  __shared__ float tab[2 * kTabHalf];
  __shared__ float red[3][kTabThreads / 64];
  const int tid = threadIdx.x, T = blockDim.x;
  for (int i = tid; i < 2 * kTabHalf; i += T) {
    const uint32_t h = ((uint32_t)(i >= kTabHalf) << 15) | ((kTabE0 << 7) + (uint32_t)(i & (kTabHalf - 1)));
    tab[i] = silu_f32(__uint_as_float(h << 16));
  }
  __syncthreads();

  const int64_t G = gridDim.x;
  auto rowptr = [&](int64_t r) { return x + (r < rows ? r : rows - 1) * 2 * k_out; };
  u32x4 ag[L], au[L], bg[L], bu[L], cg[L], cu[L];
  int64_t row = blockIdx.x;
  load_units<kActSwiglu, L>(rowptr(row), k_out, units, tid, T, ag, au);
  load_units<kActSwiglu, L>(rowptr(row + G), k_out, units, tid, T, bg, bu);
  for (; row < rows; row += 3 * G) {
    load_units<kActSwiglu, L>(rowptr(row + 2 * G), k_out, units, tid, T, cg, cu);
    swiglu_tab_row<L>(ag, au, tab, red[0], row, k_out, units, codes, sf, g_dec, scale_out);
    if (row + G >= rows) break;
    load_units<kActSwiglu, L>(rowptr(row + 3 * G), k_out, units, tid, T, ag, au);
    swiglu_tab_row<L>(bg, bu, tab, red[1], row + G, k_out, units, codes, sf, g_dec, scale_out);
    if (row + 2 * G >= rows) break;
    load_units<kActSwiglu, L>(rowptr(row + 4 * G), k_out, units, tid, T, bg, bu);
    swiglu_tab_row<L>(cg, cu, tab, red[2], row + 2 * G, k_out, units, codes, sf, g_dec, scale_out);
  }
}

// Fallback: any alignment, any row length; two streaming passes per row.
template <int DT, int ACT>
__global__ void __launch_bounds__(kMaxThreads)
quant_rows_generic(const uint16_t* __restrict__ x, int64_t k_out, uint8_t* __restrict__ codes,
                   uint8_t* __restrict__ sf, float* __restrict__ g_dec, float* __restrict__ scale_out,
                   const float* __restrict__ parts, int64_t group_rows, int nparts) {
  __shared__ float red[kMaxThreads / 64];
  const int64_t row = blockIdx.x;
  const int64_t k_in = (ACT == kActSwiglu) ? 2 * k_out : k_out;
  const int64_t nb = k_out / 16;
  const uint16_t* xr = x + row * k_in;
  float tmax = 0.0f;
  if (parts != nullptr) {
    tmax = partials_max(parts, row, group_rows, nparts);
  } else {
    for (int64_t j = threadIdx.x; j < nb; j += blockDim.x) {
      float y[16];
      load_block_scalar<DT, ACT>(xr, k_out, j, y);
      for (int e = 0; e < 16; ++e) tmax = __builtin_fmaxf(tmax, __builtin_fabsf(y[e]));
    }
  }
  const float amax = block_max(tmax, red);
  float g_enc, gd;
  global_scales(amax, g_enc, gd);
  if (threadIdx.x == 0 && (row % group_rows) == 0) g_dec[row / group_rows] = gd;
  for (int64_t j = threadIdx.x; j < nb; j += blockDim.x) {
    float y[16];
    load_block_scalar<DT, ACT>(xr, k_out, j, y);
    float amb = 0.0f;
    for (int e = 0; e < 16; ++e) amb = __builtin_fmaxf(amb, __builtin_fabsf(y[e]));
    float c, enc;
    const uint32_t s = block_scale(amb, g_enc, gd, c, enc);
    const uint32_t w0 = pack8_e2m1(&y[0], enc), w1 = pack8_e2m1(&y[8], enc);
    uint8_t* cr = codes + row * (k_out / 2) + 8 * j;
    for (int b = 0; b < 4; ++b) {
      cr[b] = (uint8_t)(w0 >> (8 * b));
      cr[4 + b] = (uint8_t)(w1 >> (8 * b));
    }
    sf[row * nb + j] = (uint8_t)s;
    if (scale_out) scale_out[row * nb + j] = c;
  }
}

// Partial maxima of |x| over `nparts` slices of each group of elements.  A
// slice is read with 16-byte loads (four in flight per lane) when the group
// and the slice start are 16-byte aligned, element by element otherwise.
template <int DT>
__global__ void __launch_bounds__(kMaxThreads)
group_amax_parts(const uint16_t* __restrict__ x, int64_t group_elems, int64_t chunk, int nparts,
                 float* __restrict__ parts) {
  __shared__ float red[kMaxThreads / 64];
  const int64_t g = blockIdx.y;
  const int p = blockIdx.x;
  const uint16_t* base = x + g * group_elems;
  const int64_t lo = (int64_t)p * chunk;
  const int64_t hi = (lo + chunk < group_elems) ? lo + chunk : group_elems;
  float m = 0.0f;
  int64_t e = lo;
  if (hi > lo && (((uintptr_t)(base + lo)) & 15) == 0) {
    const u32x4* v = reinterpret_cast<const u32x4*>(base + lo);
    const int64_t nv = (hi - lo) / 8;
    for (int64_t i = threadIdx.x; i < nv; i += 4 * kMaxThreads) {
      u32x4 q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t j = i + u * kMaxThreads;
        q[u] = __builtin_nontemporal_load(v + (j < nv ? j : i));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t w4[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float a, b;
          unpack2<DT>(w4[t], a, b);
          m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fabsf(a), __builtin_fabsf(b)));
        }
      }
    }
    e = lo + nv * 8;
  }
  for (int64_t i = e + threadIdx.x; i < hi; i += blockDim.x)
    m = __builtin_fmaxf(m, __builtin_fabsf(unpack1<DT>(base[i])));
  m = block_max(m, red);
  if (threadIdx.x == 0) parts[g * nparts + p] = m;
}

// Maximum over each group's partial maxima: gmax[g].
__global__ void __launch_bounds__(kMaxThreads)
group_amax_final(const float* __restrict__ parts, int nparts, float* __restrict__ gmax) {
  __shared__ float red[kMaxThreads / 64];
  const float* pp = parts + (int64_t)blockIdx.x * nparts;
  float m = 0.0f;
  for (int i = threadIdx.x; i < nparts; i += blockDim.x) m = __builtin_fmaxf(m, pp[i]);
  m = block_max(m, red);
  if (threadIdx.x == 0) gmax[blockIdx.x] = m;
}

template <int DT, int ACT, int L>
void launch_vec(const QuantArgs& a, int units, int threads, hipStream_t s) {
  hipLaunchKernelGGL((quant_rows_vec<DT, ACT, L>), dim3((unsigned)a.rows), dim3(threads), 0, s,
                     (const uint16_t*)a.x, a.k_out, units, a.codes, a.sf, a.g_dec, a.scale_out,
                     a.parts, a.group_rows, a.nparts);
}

template <int DT, int ACT>
void dispatch_vec(const QuantArgs& a, int units, int L, int threads, hipStream_t s) {
  switch (L) {
    case 1: launch_vec<DT, ACT, 1>(a, units, threads, s); break;
    case 2: launch_vec<DT, ACT, 2>(a, units, threads, s); break;
    case 3: launch_vec<DT, ACT, 3>(a, units, threads, s); break;
    case 4: launch_vec<DT, ACT, 4>(a, units, threads, s); break;
    case 5: launch_vec<DT, ACT, 5>(a, units, threads, s); break;
    case 6: launch_vec<DT, ACT, 6>(a, units, threads, s); break;
    case 7: launch_vec<DT, ACT, 7>(a, units, threads, s); break;
    case 8: launch_vec<DT, ACT, 8>(a, units, threads, s); break;
    case 9: case 10: launch_vec<DT, ACT, 10>(a, units, threads, s); break;
    case 11: case 12: launch_vec<DT, ACT, 12>(a, units, threads, s); break;
    default: launch_vec<DT, ACT, kMaxUnits>(a, units, threads, s); break;
  }
}

void launch_tab(const QuantArgs& a, int units, int threads, hipStream_t s) {
  const int64_t grid = a.rows < a.num_cus ? a.rows : a.num_cus;
  hipLaunchKernelGGL((swiglu_quant_tab<kTabUnits>), dim3((unsigned)grid), dim3(threads), 0, s,
                     (const uint16_t*)a.x, a.rows, a.k_out, units, a.codes, a.sf, a.g_dec, a.scale_out);
}

int round64(int64_t n) { return (int)(((n + 63) / 64) * 64); }

template <int DT, int ACT>
void launch_rows(const QuantArgs& a, hipStream_t s) {
  const int64_t units = a.k_out / 8;
  const bool aligned = ((uintptr_t)a.x % 16 == 0) && ((uintptr_t)a.codes % 4 == 0);
  if (DT == kBf16 && ACT == kActSwiglu && aligned && a.parts == nullptr && a.rows >= kTabMinRows &&
      units <= (int64_t)kTabThreads * kTabUnits && a.num_cus > 0) {
    launch_tab(a, (int)units, round64((units + kTabUnits - 1) / kTabUnits), s);
    return;
  }
  if (aligned && units <= (int64_t)kMaxThreads * kMaxUnits) {
    const int L = (int)((units + kMaxThreads - 1) / kMaxThreads);
    const int threads = round64((units + L - 1) / L);
    dispatch_vec<DT, ACT>(a, (int)units, L, threads, s);
  } else {
    hipLaunchKernelGGL((quant_rows_generic<DT, ACT>), dim3((unsigned)a.rows), dim3(kMaxThreads), 0,
                       s, (const uint16_t*)a.x, a.k_out, a.codes, a.sf, a.g_dec, a.scale_out,
                       a.parts, a.group_rows, a.nparts);
  }
}

// ---------------------------------------------------------------- MXFP4 variant

// E8M0 byte of a 32-block and its encode factor: the smallest power of two x
// >= (amax_b / 6) * g_enc, at most 2^127 (byte 254, also for NaN), at least
// 2^-127 (byte 0); c = x * g_dec, enc = 1 / c (0 if c == 0).
__device__ __forceinline__ uint32_t mx_block_scale(float amax_b, float g_enc, float g_dec,
                                                   float& enc) {
  const float sf_f = __builtin_fminf(div6_f32(amax_b) * g_enc, 0x1p127f);
  const uint32_t b = __float_as_uint(sf_f);   // sf_f >= +0: amax_b >= 0, g_enc >= 0
  uint32_t e;
  if (b <= 0x00400000u) e = 0;                // at most 2^-127 (and +0)
  else if (b < 0x00800000u) e = 1;            // subnormal above 2^-127: 2^-126
  else e = (b >> 23) + ((b & 0x7FFFFFu) != 0u ? 1u : 0u);
  const float x = (e == 0) ? 0x1p-127f : __uint_as_float(e << 23);
  const float c = x * g_dec;
  enc = (c == 0.0f) ? 0.0f : 1.0f / c;
  return e;
}

// Byte offsets of unit q (8 codes, k = 8q) and of block b of row r in the MX
// tile layout (nch64 = K/64 code tiles and nch128 = K/128 scale tiles per
// 32-row group).
__device__ __forceinline__ int64_t mx_code_pos(int64_t r, int q, int nch64) {
  const int64_t tile = (r >> 5) * nch64 + (q >> 3);
  return (tile * 64 + (r & 31) + 32 * ((q >> 2) & 1)) * 16 + 4 * (q & 3);
}
__device__ __forceinline__ int64_t mx_scale_pos(int64_t r, int b, int nch128) {
  const int64_t tile = (r >> 5) * nch128 + (b >> 2);
  return (tile * 64 + (r & 31) + 32 * (b & 1)) * 2 + ((b >> 1) & 1);
}

// MXFP4 row kernel: as quant_rows_vec, with the block amax over a lane quad.
template <int DT, int ACT, int L, bool TILED>
__global__ void __launch_bounds__(kMaxThreads)
mx_quant_rows(const uint16_t* __restrict__ x, int64_t rows, int64_t k_out, int units,
              uint8_t* __restrict__ codes, uint8_t* __restrict__ sf, float* __restrict__ g_dec,
              const float* __restrict__ parts, int64_t group_rows, int nparts) {
  __shared__ float red[kMaxThreads / 64];
  int64_t row = blockIdx.x;
  if constexpr (TILED) {
    // the 32 rows of a row group run on one XCD (consecutive workgroup ids go
    // to different XCDs), so each tile's 16-byte pieces meet in one L2 and
    // leave it as whole lines; ids past the last group exit
    const int64_t xcd = row & 7, slot = row >> 3;
    row = ((slot >> 5) * 8 + xcd) * 32 + (slot & 31);
    if (row >= (rows + 31) / 32 * 32) return;
  }
  const int tid = threadIdx.x, T = blockDim.x;
  const int nch64 = (int)(k_out / 64), nch128 = (int)(k_out / 128);
  if (TILED && row >= rows) {   // padding row of the last 32-row group
    for (int q = tid; q < units; q += T)
      *reinterpret_cast<uint32_t*>(codes + mx_code_pos(row, q, nch64)) = 0u;
    for (int b = tid; b < units / 4; b += T) sf[mx_scale_pos(row, b, nch128)] = 0;
    return;
  }
  const int64_t k_in = (ACT == kActSwiglu) ? 2 * k_out : k_out;
  const uint16_t* xr = x + row * k_in;
  u32x4 rg[L], ru[L];
  load_units<ACT, L>(xr, k_out, units, tid, T, rg, ru);
  float y[L][8];
  float am[L];
  float tmax = 0.0f;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    unit_values<DT, ACT>(rg[i], ru[i], y[i]);
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(y[i][e]));
    m = __builtin_fmaxf(m, dpp_f32<0xB1>(m));   // lane ^ 1
    m = __builtin_fmaxf(m, dpp_f32<0x4E>(m));   // lane ^ 2: the quad holds one 32-block
    am[i] = (tid + i * T < units) ? m : 0.0f;
    tmax = __builtin_fmaxf(tmax, am[i]);
  }
  if (parts != nullptr) tmax = partials_max(parts, row, group_rows, nparts);
  const float amax = block_max(tmax, red);
  float g_enc, gd;
  global_scales(amax, g_enc, gd);
  if (tid == 0) {
    if (group_rows == 1) g_dec[row] = gd;
    else if (row % group_rows == 0) g_dec[row / group_rows] = gd;
  }
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int q = tid + i * T;
    if (q >= units) continue;
    float enc;
    const uint32_t sbyte = mx_block_scale(am[i], g_enc, gd, enc);
    const uint32_t w = pack8_e2m1(y[i], enc);
    if constexpr (TILED) {
      // a plain store: the 16-byte pieces of a tile's lines come from 32
      // workgroups and must merge in L2 (a streaming store would send each
      // piece to memory as a partial line)
      *reinterpret_cast<uint32_t*>(codes + mx_code_pos(row, q, nch64)) = w;
      if ((tid & 3) == 0) sf[mx_scale_pos(row, q >> 2, nch128)] = (uint8_t)sbyte;
    } else {
      __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(codes + row * (k_out / 2) + 4 * (int64_t)q));
      if ((tid & 3) == 0) sf[row * (k_out / 32) + (q >> 2)] = (uint8_t)sbyte;
    }
  }
}

template <int DT, int ACT, bool TILED>
void launch_mx_rows(const QuantArgs& a, hipStream_t s) {
  const int units = (int)(a.k_out / 8);
  int L = (units + kMaxThreads - 1) / kMaxThreads;
  L = L <= 1 ? 1 : L <= 2 ? 2 : L <= 4 ? 4 : L <= 8 ? 8 : kMaxUnits;
  const int threads = round64((units + L - 1) / L);
  const int64_t grid = TILED ? (a.rows + 255) / 256 * 256 : a.rows;   // whole sets of 8 row groups
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, s, (const uint16_t*)a.x, a.rows,
                       a.k_out, units, a.codes, a.sf, a.g_dec, a.parts, a.group_rows, a.nparts);
  };
  switch (L) {
    case 1: go(mx_quant_rows<DT, ACT, 1, TILED>); break;
    case 2: go(mx_quant_rows<DT, ACT, 2, TILED>); break;
    case 4: go(mx_quant_rows<DT, ACT, 4, TILED>); break;
    case 8: go(mx_quant_rows<DT, ACT, 8, TILED>); break;
    default: go(mx_quant_rows<DT, ACT, kMaxUnits, TILED>); break;
  }
}

template <int DT, int ACT>
void launch_mx(const QuantArgs& a, hipStream_t s) {
  if (a.tiled) launch_mx_rows<DT, ACT, true>(a, s);
  else launch_mx_rows<DT, ACT, false>(a, s);
}

}  // namespace

int quant_num_parts(int64_t group_elems) {
  int64_t p = (group_elems + 16383) / 16384;
  return (int)(p < 1 ? 1 : (p > 1024 ? 1024 : p));
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  QuantArgs b = a;
  if (a.group_rows > 1) {
    // slices of whole 8-element units, so every slice start stays 16-byte
    // aligned when the group start is
    const int64_t ge = a.group_rows * a.k_out;
    const int64_t chunk = ((ge + a.nparts - 1) / a.nparts + 7) / 8 * 8;
    const int64_t groups = a.rows / a.group_rows;
    const dim3 grid((unsigned)a.nparts, (unsigned)groups);
    if (a.dtype == kBf16)
      hipLaunchKernelGGL(group_amax_parts<0>, grid, dim3(kMaxThreads), 0, s, (const uint16_t*)a.x,
                         ge, chunk, a.nparts, a.parts);
    else
      hipLaunchKernelGGL(group_amax_parts<1>, grid, dim3(kMaxThreads), 0, s, (const uint16_t*)a.x,
                         ge, chunk, a.nparts, a.parts);
    float* gmax = a.parts + groups * a.nparts;
    hipLaunchKernelGGL(group_amax_final, dim3((unsigned)groups), dim3(kMaxThreads), 0, s, a.parts,
                       a.nparts, gmax);
    b.parts = gmax;
    b.nparts = 1;
  } else {
    b.parts = nullptr;
  }
  if (a.mx) {
    if (a.dtype == kBf16) {
      switch (a.act) {
        case kActSwiglu: launch_mx<0, kActSwiglu>(b, s); break;
        case kActRelu2: launch_mx<0, kActRelu2>(b, s); break;
        default: launch_mx<0, kActNone>(b, s); break;
      }
    } else {
      switch (a.act) {
        case kActSwiglu: launch_mx<1, kActSwiglu>(b, s); break;
        case kActRelu2: launch_mx<1, kActRelu2>(b, s); break;
        default: launch_mx<1, kActNone>(b, s); break;
      }
    }
    return hipGetLastError();
  }
  if (a.dtype == kBf16) {
    switch (a.act) {
      case kActSwiglu: launch_rows<0, kActSwiglu>(b, s); break;
      case kActRelu2: launch_rows<0, kActRelu2>(b, s); break;
      default: launch_rows<0, kActNone>(b, s); break;
    }
  } else {
    switch (a.act) {
      case kActSwiglu: launch_rows<1, kActSwiglu>(b, s); break;
      case kActRelu2: launch_rows<1, kActRelu2>(b, s); break;
      default: launch_rows<1, kActNone>(b, s); break;
    }
  }
  return hipGetLastError();
}

}  // namespace nvfp4
