// internal.h -- launcher interfaces between the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kBf16 = 0;
constexpr int kFp16 = 1;
constexpr int kActNone = 0;
constexpr int kActSwiglu = 1;
constexpr int kActRelu2 = 2;

struct QuantArgs {
  const void* x;
  int dtype;
  int act;
  int64_t rows;
  int64_t k_out;       // quantized row length (input row is 2*k_out for SwiGLU)
  int64_t group_rows;  // rows sharing one global scale
  uint8_t* codes;
  uint8_t* sf;
  float* g_dec;
  float* scale_out;    // may be null
  float* parts;        // workspace: [groups, nparts] partial maxima (group_rows > 1)
  int nparts;
  int num_cus;         // compute units of the current device (persistent grids)
  int mx;              // MXFP4 variant: 32-element blocks with E8M0 scale bytes
  int tiled;           // MXFP4 only: codes / scale bytes in the MX tile layout
};

// Number of partial maxima per group the per-group path uses.
int quant_num_parts(int64_t group_elems);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);

struct GemmArgs {
  const uint8_t* a;
  const float* a_scale;
  const uint8_t* w;
  const uint8_t* w_sf;
  const float* w_g;
  void* y;
  int64_t B, N, K;
  void* workspace;
  size_t workspace_bytes;
  int tiled;           // w / w_sf in the pre-tiled layout (N % 16 == 0, K % 128 == 0)
};

size_t gemm_workspace_bytes(int64_t B, int64_t N, int64_t K);
hipError_t launch_pretile(const uint8_t* w, const uint8_t* w_sf, int64_t N, int64_t K,
                          uint8_t* w_tiled, uint8_t* sf_tiled, hipStream_t s);
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s);

struct MoeArgs {
  const float* logits;
  const float* bias;
  const void* x;
  const uint8_t* w1;
  const uint8_t* w1_sf;
  const float* w1_g;
  const uint8_t* w2;
  const uint8_t* w2_sf;
  const float* w2_g;
  void* out;
  int32_t* ids_out;
  float* w_out;
  int tokens, experts, top_k, hidden, inter, n_group, topk_group, norm;
  float scaling;
  void* workspace;
  size_t workspace_bytes;
  int num_cus;         // compute units of the current device (work split)
  int tiled_weights;   // w1/w2 codes and E4M3 bytes in the pre-tiled layout
};

// MXFP4 variant: the MX tile permutation and the block-scaled MFMA GEMM.
struct MxGemmArgs {
  const uint8_t* a;    // activation code tiles
  const uint8_t* as;   // activation scale tiles
  const float* ag;     // activation globals, one per a_group_rows rows
  int64_t a_group_rows;
  const uint8_t* w;    // weight code tiles
  const uint8_t* ws;   // weight scale tiles
  const float* wg;     // one weight global
  void* y;             // [B, N] fp16
  int64_t B, N, K;
};

hipError_t launch_mx_tile(const uint8_t* codes, const uint8_t* sf, int64_t rows, int64_t K,
                          uint8_t* codes_tiled, uint8_t* sf_tiled, hipStream_t s);
hipError_t launch_mx_gemm(const MxGemmArgs& g, hipStream_t s);

size_t moe_workspace_bytes(int tokens, int experts, int top_k, int hidden, int inter);
hipError_t launch_moe(const MoeArgs& m, hipStream_t s);
// The fixed no-allocation scratch of the current device (address and size).
hipError_t moe_noalloc_scratch(void** ptr, size_t* bytes);

}  // namespace nvfp4
