// quantize.hip -- NVFP4 quantization kernels for gfx950.
//
// Per-token path (one workgroup per row): the row is read from HBM once and
// kept in VGPRs between the amax pass and the encode pass -- the role the
// shared-memory caching of input vectors plays in "perf: optimize per-token
// nvfp4 quantization kernel" (flashinfer pull request 3237, review).  Each lane
// owns whole 16-element blocks, so the block amax is an in-lane max and only
// the row amax needs a wave (DPP/permute) + LDS reduction.  Loads are 16-byte
// vectors ("Building Custom TensorRT-LLM Plugins for Low-Latency FP8 Inference
// at Scale", "Fusing the Kernel in CUDA"), consecutive lanes read consecutive
// 32-byte blocks, and each lane writes its 8 code bytes with one 8-byte store.
//
// The optional activation (SwiGLU: gate = first half of the row, up = second
// half; ReLU^2) runs in fp32 registers in front of the quantizer, so the
// activation output never reaches HBM (same article, "The Cost of Non-Fused
// Quantization").
//
// Per-group path (per tensor / per expert): a partial-amax kernel writes at
// most 256 partial maxima per group into the workspace; the row kernel then
// reduces its group's partials instead of its own row.
//
// A scalar fallback handles inputs that are not 16-byte aligned (or codes not
// 8-byte aligned) and rows longer than the register cache, with identical
// results (same article, "Production Pitfalls & Hard Lessons", item 1).
#include "device_common.h"
#include "internal.h"

namespace nvfp4 {

namespace {

constexpr int kMaxThreads = 256;

// Loads the 16 activation outputs of block j of a row into y[16].
template <int DT, int ACT>
__device__ __forceinline__ void load_block_vec(const uint16_t* __restrict__ xr, int64_t k_out, int j,
                                               float* y) {
  if constexpr (ACT == kActSwiglu) {
    const u32x4* pg = reinterpret_cast<const u32x4*>(xr + 16 * (int64_t)j);
    const u32x4* pu = reinterpret_cast<const u32x4*>(xr + k_out + 16 * (int64_t)j);
    const u32x4 g0 = __builtin_nontemporal_load(pg);
    const u32x4 g1 = __builtin_nontemporal_load(pg + 1);
    const u32x4 u0 = __builtin_nontemporal_load(pu);
    const u32x4 u1 = __builtin_nontemporal_load(pu + 1);
    const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const uint32_t uw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float ga, gb, ua, ub;
      unpack2<DT>(gw[i], ga, gb);
      unpack2<DT>(uw[i], ua, ub);
      y[2 * i] = swiglu_f32(ga, ua);
      y[2 * i + 1] = swiglu_f32(gb, ub);
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(xr + 16 * (int64_t)j);
    const u32x4 a0 = __builtin_nontemporal_load(p);
    const u32x4 a1 = __builtin_nontemporal_load(p + 1);
    const uint32_t w[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float a, b;
      unpack2<DT>(w[i], a, b);
      if constexpr (ACT == kActRelu2) { a = relu2_f32(a); b = relu2_f32(b); }
      y[2 * i] = a;
      y[2 * i + 1] = b;
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

// Block-wide max; every thread gets the result.  blockDim.x <= 256.
__device__ __forceinline__ float block_max(float v, float* red) {
  float w = wave_max(v);
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

// Row kernel with the row cached in registers: NB blocks per thread, T
// threads per row (blockDim.x = T rounded up to a wave).
template <int DT, int ACT, int NB>
__global__ void __launch_bounds__(kMaxThreads)
quant_rows_fast(const uint16_t* __restrict__ x, int64_t k_out, int nb, int T,
                uint8_t* __restrict__ codes, uint8_t* __restrict__ sf, float* __restrict__ g_dec,
                float* __restrict__ scale_out, const float* __restrict__ parts, int64_t group_rows,
                int nparts) {
  __shared__ float red[kMaxThreads / 64];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t k_in = (ACT == kActSwiglu) ? 2 * k_out : k_out;
  const uint16_t* xr = x + row * k_in;
  float y[NB][16];
  float am[NB];
  float tmax = 0.0f;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int j = tid + i * T;
    am[i] = 0.0f;
    if (tid < T && j < nb) {
      load_block_vec<DT, ACT>(xr, k_out, j, y[i]);
#pragma unroll
      for (int e = 0; e < 16; ++e) am[i] = __builtin_fmaxf(am[i], __builtin_fabsf(y[i][e]));
      tmax = __builtin_fmaxf(tmax, am[i]);
    }
  }
  if (parts != nullptr) tmax = partials_max(parts, row, group_rows, nparts);
  const float amax = block_max(tmax, red);
  float g_enc, gd;
  global_scales(amax, g_enc, gd);
  if (tid == 0 && (row % group_rows) == 0) g_dec[row / group_rows] = gd;
  uint8_t* cr = codes + row * (k_out / 2);
  uint8_t* sr = sf + row * (int64_t)nb;
  float* scr = scale_out ? scale_out + row * (int64_t)nb : nullptr;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int j = tid + i * T;
    if (tid < T && j < nb) {
      float c, enc;
      const uint32_t s = block_scale(am[i], g_enc, gd, c, enc);
      u32x2 o;
      o.x = pack8_e2m1(&y[i][0], enc);
      o.y = pack8_e2m1(&y[i][8], enc);
      __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(cr + 8 * (int64_t)j));
      sr[j] = (uint8_t)s;
      if (scr) scr[j] = c;
    }
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

// Partial maxima of |x| over `nparts` slices of each group of elements.
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
  for (int64_t e = lo + threadIdx.x; e < hi; e += blockDim.x)
    m = __builtin_fmaxf(m, __builtin_fabsf(unpack1<DT>(base[e])));
  m = block_max(m, red);
  if (threadIdx.x == 0) parts[g * nparts + p] = m;
}

template <int DT, int ACT, int NB>
void launch_fast(const QuantArgs& a, int T, hipStream_t s) {
  const int threads = ((T + 63) / 64) * 64;
  hipLaunchKernelGGL((quant_rows_fast<DT, ACT, NB>), dim3((unsigned)a.rows), dim3(threads), 0, s,
                     (const uint16_t*)a.x, a.k_out, (int)(a.k_out / 16), T, a.codes, a.sf, a.g_dec,
                     a.scale_out, a.parts, a.group_rows, a.nparts);
}

template <int DT, int ACT>
void dispatch_nb(const QuantArgs& a, int nb_per_thread, int T, hipStream_t s) {
  switch (nb_per_thread) {
    case 1: launch_fast<DT, ACT, 1>(a, T, s); break;
    case 2: launch_fast<DT, ACT, 2>(a, T, s); break;
    case 3: launch_fast<DT, ACT, 3>(a, T, s); break;
    case 4: launch_fast<DT, ACT, 4>(a, T, s); break;
    case 5: launch_fast<DT, ACT, 5>(a, T, s); break;
    case 6: launch_fast<DT, ACT, 6>(a, T, s); break;
    case 7: launch_fast<DT, ACT, 7>(a, T, s); break;
    default: launch_fast<DT, ACT, 8>(a, T, s); break;
  }
}

template <int DT, int ACT>
void launch_rows(const QuantArgs& a, hipStream_t s) {
  const int64_t nb = a.k_out / 16;
  const bool aligned = ((uintptr_t)a.x % 16 == 0) && ((uintptr_t)a.codes % 8 == 0);
  const int64_t per = (nb + kMaxThreads - 1) / kMaxThreads;
  if (aligned && per <= 8) {
    const int nbt = (int)(per < 1 ? 1 : per);
    const int T = (int)((nb + nbt - 1) / nbt);
    dispatch_nb<DT, ACT>(a, nbt, T, s);
  } else {
    hipLaunchKernelGGL((quant_rows_generic<DT, ACT>), dim3((unsigned)a.rows), dim3(kMaxThreads), 0,
                       s, (const uint16_t*)a.x, a.k_out, a.codes, a.sf, a.g_dec, a.scale_out,
                       a.parts, a.group_rows, a.nparts);
  }
}

}  // namespace

int quant_num_parts(int64_t group_elems) {
  int64_t p = (group_elems + 4095) / 4096;
  return (int)(p < 1 ? 1 : (p > 256 ? 256 : p));
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  QuantArgs b = a;
  if (a.group_rows > 1) {
    const int64_t ge = a.group_rows * a.k_out;
    const int64_t chunk = (ge + a.nparts - 1) / a.nparts;
    const dim3 grid((unsigned)a.nparts, (unsigned)(a.rows / a.group_rows));
    if (a.dtype == kBf16)
      hipLaunchKernelGGL(group_amax_parts<0>, grid, dim3(kMaxThreads), 0, s, (const uint16_t*)a.x,
                         ge, chunk, a.nparts, a.parts);
    else
      hipLaunchKernelGGL(group_amax_parts<1>, grid, dim3(kMaxThreads), 0, s, (const uint16_t*)a.x,
                         ge, chunk, a.nparts, a.parts);
  } else {
    b.parts = nullptr;
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
