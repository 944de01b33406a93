// api.hip -- the C ABI of include/nvfp4_mi355x.h: host-side validation, the
// per-device gfx950 check, workspace checks, stream-ordered launches and the
// external-weight registry.  Nothing here allocates device memory or
// synchronizes; only the registry keeps (caller-owned) pointers.
#include <mutex>
#include <string.h>
#include <unordered_map>

#include "../../include/nvfp4_mi355x.h"
#include "internal.h"

namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
  int ok;        // 1 if gfx950, 0 if not
  int num_cus;   // compute units
};

// Properties of the current device, queried once per device; nullptr if HIP
// reports an error.
const DeviceInfo* current_device() {
  static std::once_flag once[kMaxDevices];
  static DeviceInfo info[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(once[dev], [dev]() {
    hipDeviceProp_t p;
    const bool got = hipGetDeviceProperties(&p, dev) == hipSuccess;
    info[dev].ok = (got && strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 0;
    info[dev].num_cus = got ? p.multiProcessorCount : 0;
  });
  return &info[dev];
}

int32_t device_status() {
  const DeviceInfo* d = current_device();
  if (!d) return NVFP4_EHIP;
  return d->ok ? NVFP4_OK : NVFP4_EUNSUPPORTED;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP; }

bool aligned4(const void* p) { return ((uintptr_t)p % 4) == 0; }
bool aligned256(const void* p) { return ((uintptr_t)p % 256) == 0; }

// External weights of "Fused Nvfp4 GEMM All Reduce Plugin" (external-weight
// mode): (device, resource id) -> the caller's weight and scale pointers.
struct ExternalWeight {
  const uint8_t* weight;
  const uint8_t* scale;
  int32_t out_features, in_features;
};

struct Registry {
  std::mutex mu;
  std::unordered_map<uint64_t, ExternalWeight> map;
};

Registry& registry() {
  static Registry r;
  return r;
}

uint64_t registry_key(int32_t device, int32_t resource_id) {
  return ((uint64_t)(uint32_t)device << 32) | (uint32_t)resource_id;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(int32_t status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_EINVAL: return "invalid argument";
    case NVFP4_EUNSUPPORTED: return "unsupported device or size";
    case NVFP4_EWORKSPACE: return "workspace missing or too small";
    case NVFP4_EHIP: return "HIP runtime error";
    case NVFP4_ESCRATCH: return "problem larger than the fixed scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t k, int64_t group_rows) {
  if (rows <= 0 || k <= 0 || group_rows <= 1 || rows % group_rows != 0) return 0;
  const int np = nvfp4::quant_num_parts(group_rows * k);
  return (size_t)(rows / group_rows) * (size_t)(np + 1) * sizeof(float);
}

static int32_t quantize_common(const void* x, int32_t dtype, int64_t rows, int64_t k_out,
                               int32_t act, int64_t group_rows, uint8_t* codes, uint8_t* sf,
                               float* g_dec, float* scale_out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (dtype != NVFP4_BF16 && dtype != NVFP4_FP16) return NVFP4_EINVAL;
  if (act != NVFP4_ACT_NONE && act != NVFP4_ACT_SWIGLU && act != NVFP4_ACT_RELU2) return NVFP4_EINVAL;
  if (rows < 0 || k_out <= 0 || (k_out % 16) != 0 || group_rows < 1) return NVFP4_EINVAL;
  if (rows > 0 && (rows % group_rows) != 0) return NVFP4_EINVAL;
  if (rows == 0) return NVFP4_OK;
  if (!x || !codes || !sf || !g_dec) return NVFP4_EINVAL;
  if (!aligned4(g_dec) || (scale_out && !aligned4(scale_out))) return NVFP4_EINVAL;
  if (((uintptr_t)x % 2) != 0) return NVFP4_EINVAL;
  if (rows > 0x7FFFFFFFLL) return NVFP4_EUNSUPPORTED;                // grid.x limit
  const int64_t k_in = (act == NVFP4_ACT_SWIGLU) ? 2 * k_out : k_out;
  if (k_in > (int64_t)1 << 40) return NVFP4_EUNSUPPORTED;
  nvfp4::QuantArgs a{};
  a.x = x; a.dtype = dtype; a.act = act; a.rows = rows; a.k_out = k_out; a.group_rows = group_rows;
  a.codes = codes; a.sf = sf; a.g_dec = g_dec; a.scale_out = scale_out; a.parts = nullptr;
  a.nparts = 0;
  if (group_rows > 1) {
    if ((rows / group_rows) > 65535) return NVFP4_EUNSUPPORTED;   // grid.y limit of the partial pass
    const size_t need = nvfp4_quantize_workspace_size(rows, k_out, group_rows);
    if (!workspace || workspace_bytes < need || !aligned4(workspace)) return NVFP4_EWORKSPACE;
    a.parts = (float*)workspace;
    a.nparts = nvfp4::quant_num_parts(group_rows * k_out);
  }
  const int32_t ds = device_status();
  if (ds != NVFP4_OK) return ds;
  a.num_cus = current_device()->num_cus;
  return hip_status(nvfp4::launch_quantize(a, (hipStream_t)stream));
}

int32_t nvfp4_quantize(const void* x, int32_t dtype, int64_t rows, int64_t k, int64_t group_rows,
                       uint8_t* codes, uint8_t* sf, float* g_dec, float* scale_out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return quantize_common(x, dtype, rows, k, NVFP4_ACT_NONE, group_rows, codes, sf, g_dec,
                         scale_out, workspace, workspace_bytes, stream);
}

int32_t nvfp4_mx_quantize(const void* x, int32_t dtype, int64_t rows, int64_t k_out, int32_t act,
                          int64_t group_rows, int32_t layout, uint8_t* codes, uint8_t* sf,
                          float* g_dec, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != NVFP4_BF16 && dtype != NVFP4_FP16) return NVFP4_EINVAL;
  if (act != NVFP4_ACT_NONE && act != NVFP4_ACT_SWIGLU && act != NVFP4_ACT_RELU2) return NVFP4_EINVAL;
  if (layout != NVFP4_MX_ROWS && layout != NVFP4_MX_TILED) return NVFP4_EINVAL;
  if (rows < 0 || k_out <= 0 || group_rows < 1) return NVFP4_EINVAL;
  if ((k_out % (layout == NVFP4_MX_TILED ? 128 : 32)) != 0) return NVFP4_EINVAL;
  if (act != NVFP4_ACT_NONE && group_rows != 1) return NVFP4_EINVAL;
  if (rows > 0 && (rows % group_rows) != 0) return NVFP4_EINVAL;
  if (rows == 0) return NVFP4_OK;
  if (!x || !codes || !sf || !g_dec) return NVFP4_EINVAL;
  if (((uintptr_t)x % 16) != 0 || !aligned4(codes) || !aligned4(g_dec)) return NVFP4_EINVAL;
  if (k_out > 32768 || rows > 0x7FFFFF00LL) return NVFP4_EUNSUPPORTED;   // grid of whole 256-row sets
  nvfp4::QuantArgs a{};
  a.x = x; a.dtype = dtype; a.act = act; a.rows = rows; a.k_out = k_out; a.group_rows = group_rows;
  a.codes = codes; a.sf = sf; a.g_dec = g_dec; a.scale_out = nullptr; a.parts = nullptr;
  a.nparts = 0; a.mx = 1; a.tiled = (layout == NVFP4_MX_TILED) ? 1 : 0;
  if (group_rows > 1) {
    if ((rows / group_rows) > 65535) return NVFP4_EUNSUPPORTED;   // grid.y limit of the partial pass
    const size_t need = nvfp4_quantize_workspace_size(rows, k_out, group_rows);
    if (!workspace || workspace_bytes < need || !aligned4(workspace)) return NVFP4_EWORKSPACE;
    a.parts = (float*)workspace;
    a.nparts = nvfp4::quant_num_parts(group_rows * k_out);
  }
  const int32_t ds = device_status();
  if (ds != NVFP4_OK) return ds;
  a.num_cus = current_device()->num_cus;
  return hip_status(nvfp4::launch_quantize(a, (hipStream_t)stream));
}

int32_t nvfp4_mx_tile(const uint8_t* codes, const uint8_t* sf, int64_t rows, int64_t k,
                      uint8_t* codes_tiled, uint8_t* sf_tiled, void* stream) {
  if (rows < 0 || k <= 0 || (k % 128) != 0) return NVFP4_EINVAL;
  if (rows == 0) return NVFP4_OK;
  if (!codes || !sf || !codes_tiled || !sf_tiled) return NVFP4_EINVAL;
  if (((uintptr_t)codes % 16) != 0 || ((uintptr_t)codes_tiled % 16) != 0 ||
      ((uintptr_t)sf_tiled % 2) != 0)
    return NVFP4_EINVAL;
  // four 1 KiB tiles per workgroup of the permutation: grid.x < 2^31
  if (k > (1LL << 24) || (rows + 31) / 32 * (k / 64) > (1LL << 32)) return NVFP4_EUNSUPPORTED;
  const int32_t ds = device_status();
  if (ds != NVFP4_OK) return ds;
  return hip_status(nvfp4::launch_mx_tile(codes, sf, rows, k, codes_tiled, sf_tiled,
                                          (hipStream_t)stream));
}

int32_t nvfp4_mx_gemm(const uint8_t* a_tiled, const uint8_t* a_sf_tiled, const float* a_g,
                      int64_t a_group_rows, const uint8_t* w_tiled, const uint8_t* w_sf_tiled,
                      const float* w_gscale, void* y, int64_t B, int64_t N, int64_t K, void* stream) {
  if (B < 0 || N <= 0 || K <= 0 || (N % 32) != 0 || (K % 128) != 0 || a_group_rows < 1)
    return NVFP4_EINVAL;
  if (B > 0 && (B % a_group_rows) != 0) return NVFP4_EINVAL;
  if (B == 0) return NVFP4_OK;
  if (!a_tiled || !a_sf_tiled || !a_g || !w_tiled || !w_sf_tiled || !w_gscale || !y) return NVFP4_EINVAL;
  if (((uintptr_t)a_tiled % 16) != 0 || ((uintptr_t)w_tiled % 16) != 0 || !aligned4(a_sf_tiled) ||
      !aligned4(w_sf_tiled) || !aligned4(a_g) || !aligned4(w_gscale) || ((uintptr_t)y % 16) != 0)
    return NVFP4_EINVAL;
  if (B > 0x7FFFFFE0LL || N > 0x7FFFFFE0LL || K > (1LL << 24)) return NVFP4_EUNSUPPORTED;
  if (((B + 255) / 256) * ((N + 255) / 256) > 0x7FFFFFFFLL) return NVFP4_EUNSUPPORTED;
  const int32_t ds = device_status();
  if (ds != NVFP4_OK) return ds;
  nvfp4::MxGemmArgs g{a_tiled, a_sf_tiled, a_g, a_group_rows, w_tiled, w_sf_tiled, w_gscale, y, B, N, K};
  return hip_status(nvfp4::launch_mx_gemm(g, (hipStream_t)stream));
}

int32_t nvfp4_act_quant(const void* x, int32_t dtype, int64_t rows, int64_t k_out, int32_t act,
                        uint8_t* codes, uint8_t* sf, float* g_dec, float* scale_out, void* stream) {
  return quantize_common(x, dtype, rows, k_out, act, 1, codes, sf, g_dec, scale_out, nullptr, 0,
                         stream);
}

size_t nvfp4_gemm_workspace_size(int64_t B, int64_t N, int64_t K) {
  if (B <= 0 || N <= 0 || K <= 0) return 0;
  return nvfp4::gemm_workspace_bytes(B, N, K);
}

int32_t nvfp4_gemm(const uint8_t* a, const float* a_scale, const uint8_t* w, const uint8_t* w_sf,
                   const float* w_gscale, void* y, int64_t B, int64_t N, int64_t K,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || N <= 0 || K <= 0 || (K % 16) != 0) return NVFP4_EINVAL;
  if (B == 0) return NVFP4_OK;
  if (!a || !a_scale || !w || !w_sf || !w_gscale || !y) return NVFP4_EINVAL;
  if (!aligned4(a_scale) || !aligned4(w_gscale) || ((uintptr_t)y % 2) != 0) return NVFP4_EINVAL;
  if (B > 0x7FFFFFFFLL || N > 0x7FFFFFFFLL || K > 0x7FFFFFFFLL) return NVFP4_EUNSUPPORTED;
  const size_t need = nvfp4::gemm_workspace_bytes(B, N, K);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned256(workspace)))
    return NVFP4_EWORKSPACE;
  const int32_t ds = device_status();
  if (ds != NVFP4_OK) return ds;
  nvfp4::GemmArgs g{a, a_scale, w, w_sf, w_gscale, y, B, N, K, workspace, workspace_bytes, 0};
  return hip_status(nvfp4::launch_gemm(g, (hipStream_t)stream));
}

int32_t nvfp4_pretile_weight(const uint8_t* w, const uint8_t* w_sf, int64_t N, int64_t K,
                             uint8_t* w_tiled, uint8_t* sf_tiled, void* stream) {
  if (N <= 0 || K <= 0 || (N % 16) != 0 || (K % 128) != 0) return NVFP4_EINVAL;
  if (!w || !w_sf || !w_tiled || !sf_tiled) return NVFP4_EINVAL;
  if (((uintptr_t)w % 16) != 0 || ((uintptr_t)w_tiled % 16) != 0 || ((uintptr_t)w_sf % 2) != 0 ||
      ((uintptr_t)sf_tiled % 4) != 0)
    return NVFP4_EINVAL;
  if (N > 0x7FFFFFFFLL || K > (1LL << 24)) return NVFP4_EUNSUPPORTED;
  const int32_t ds = device_status();
  if (ds != NVFP4_OK) return ds;
  return hip_status(nvfp4::launch_pretile(w, w_sf, N, K, w_tiled, sf_tiled, (hipStream_t)stream));
}

int32_t nvfp4_gemm_pretiled(const uint8_t* a, const float* a_scale, const uint8_t* w_tiled,
                            const uint8_t* sf_tiled, const float* w_gscale, void* y, int64_t B,
                            int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (B < 0 || N <= 0 || K <= 0 || (N % 16) != 0 || (K % 128) != 0) return NVFP4_EINVAL;
  if (B == 0) return NVFP4_OK;
  if (!a || !a_scale || !w_tiled || !sf_tiled || !w_gscale || !y) return NVFP4_EINVAL;
  if (!aligned4(a_scale) || !aligned4(w_gscale) || ((uintptr_t)y % 2) != 0) return NVFP4_EINVAL;
  if (((uintptr_t)w_tiled % 16) != 0 || ((uintptr_t)sf_tiled % 4) != 0) return NVFP4_EINVAL;
  if (B > 0x7FFFFFFFLL || N > 0x7FFFFFFFLL || K > (1LL << 24)) return NVFP4_EUNSUPPORTED;
  const size_t need = nvfp4::gemm_workspace_bytes(B, N, K);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned256(workspace)))
    return NVFP4_EWORKSPACE;
  const int32_t ds = device_status();
  if (ds != NVFP4_OK) return ds;
  nvfp4::GemmArgs g{a, a_scale, w_tiled, sf_tiled, w_gscale, y, B, N, K, workspace, workspace_bytes, 1};
  return hip_status(nvfp4::launch_gemm(g, (hipStream_t)stream));
}

int32_t nvfp4_register_weight(int32_t device, int32_t resource_id, const uint8_t* weight,
                              const uint8_t* scale, int32_t out_features, int32_t in_features,
                              int32_t scale_cols) {
  if (device < 0 || resource_id < 0 || !weight || !scale) return NVFP4_EINVAL;
  if (out_features <= 0 || in_features <= 0 || (in_features % 16) != 0 ||
      scale_cols != in_features / 16)
    return NVFP4_EINVAL;
  Registry& r = registry();
  std::lock_guard<std::mutex> lock(r.mu);
  const bool inserted =
      r.map.emplace(registry_key(device, resource_id),
                    ExternalWeight{weight, scale, out_features, in_features}).second;
  return inserted ? NVFP4_OK : NVFP4_EINVAL;
}

int32_t nvfp4_unregister_weight(int32_t device, int32_t resource_id) {
  if (device < 0 || resource_id < 0) return NVFP4_EINVAL;
  Registry& r = registry();
  std::lock_guard<std::mutex> lock(r.mu);
  return r.map.erase(registry_key(device, resource_id)) == 1 ? NVFP4_OK : NVFP4_EINVAL;
}

int32_t nvfp4_gemm_external(const uint8_t* a, const float* a_scale, int32_t resource_id,
                            const float* w_gscale, void* y, int64_t B, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (resource_id < 0) return NVFP4_EINVAL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return NVFP4_EHIP;
  ExternalWeight ew;
  {
    Registry& r = registry();
    std::lock_guard<std::mutex> lock(r.mu);
    const auto it = r.map.find(registry_key(dev, resource_id));
    if (it == r.map.end()) return NVFP4_EINVAL;
    ew = it->second;
  }
  if (N != ew.out_features || K != ew.in_features) return NVFP4_EINVAL;
  return nvfp4_gemm(a, a_scale, ew.weight, ew.scale, w_gscale, y, B, N, K, workspace,
                    workspace_bytes, stream);
}

size_t nvfp4_moe_w4a16_workspace_size(int32_t tokens, int32_t experts, int32_t top_k,
                                      int32_t hidden, int32_t inter) {
  if (tokens <= 0 || experts <= 0 || top_k <= 0 || hidden <= 0 || inter <= 0) return 0;
  return nvfp4::moe_workspace_bytes(tokens, experts, top_k, hidden, inter);
}

// Argument checks shared by both MoE entry points (everything but the
// workspace); NVFP4_OK for tokens == 0 too (the caller returns early).
static int32_t moe_check(const float* router_logits, const float* correction_bias, const void* x,
                         const uint8_t* w1, const uint8_t* w1_sf, const float* w1_g,
                         const uint8_t* w2, const uint8_t* w2_sf, const float* w2_g, void* out,
                         int32_t tokens, int32_t experts, int32_t top_k, int32_t hidden,
                         int32_t inter, int32_t n_group, int32_t topk_group) {
  if (tokens < 0 || tokens > (1 << 24) || experts <= 0 || experts > 256 || n_group <= 0 ||
      experts % n_group != 0)
    return NVFP4_EINVAL;
  const int gsize = experts / n_group;
  if (topk_group < 1 || topk_group > n_group || top_k < 1 || top_k > 16 ||
      top_k > topk_group * gsize)
    return NVFP4_EINVAL;
  if (hidden <= 0 || inter <= 0 || hidden % 64 != 0 || inter % 64 != 0 || inter > 8192 ||
      (int64_t)hidden * inter > (int64_t(1) << 31))
    return NVFP4_EINVAL;
  if (tokens == 0) return NVFP4_OK;
  if (!router_logits || !correction_bias || !x || !w1 || !w1_sf || !w1_g || !w2 || !w2_sf ||
      !w2_g || !out)
    return NVFP4_EINVAL;
  if (((uintptr_t)x % 16) != 0 || ((uintptr_t)out % 8) != 0 || ((uintptr_t)w1 % 16) != 0 ||
      ((uintptr_t)w2 % 16) != 0 || !aligned4(w1_sf) || !aligned4(w2_sf) ||
      !aligned4(router_logits) || !aligned4(correction_bias) || !aligned4(w1_g) || !aligned4(w2_g))
    return NVFP4_EINVAL;
  return NVFP4_OK;
}

int32_t nvfp4_moe_w4a16(const float* router_logits, const float* correction_bias, const void* x,
                        const uint8_t* w1, const uint8_t* w1_sf, const float* w1_g,
                        const uint8_t* w2, const uint8_t* w2_sf, const float* w2_g, void* out,
                        int32_t* topk_ids_out, float* topk_w_out, int32_t tokens, int32_t experts,
                        int32_t top_k, int32_t hidden, int32_t inter, int32_t n_group,
                        int32_t topk_group, int32_t norm_topk_prob, float routed_scaling,
                        void* workspace, size_t workspace_bytes, void* stream) {
  const int32_t st = moe_check(router_logits, correction_bias, x, w1, w1_sf, w1_g, w2, w2_sf, w2_g,
                               out, tokens, experts, top_k, hidden, inter, n_group, topk_group);
  if (st != NVFP4_OK || tokens == 0) return st;
  const size_t need = nvfp4::moe_workspace_bytes(tokens, experts, top_k, hidden, inter);
  if (!workspace || workspace_bytes < need || !aligned256(workspace)) return NVFP4_EWORKSPACE;
  const int32_t ds = device_status();
  if (ds != NVFP4_OK) return ds;
  nvfp4::MoeArgs m{router_logits, correction_bias, x, w1, w1_sf, w1_g, w2, w2_sf, w2_g, out,
                   topk_ids_out, topk_w_out, tokens, experts, top_k, hidden, inter, n_group,
                   topk_group, norm_topk_prob ? 1 : 0, routed_scaling, workspace, workspace_bytes,
                   current_device()->num_cus, 0};
  return hip_status(nvfp4::launch_moe(m, (hipStream_t)stream));
}

int32_t nvfp4_moe_w4a16_pretiled(const float* router_logits, const float* correction_bias,
                                 const void* x, const uint8_t* w1, const uint8_t* w1_sf,
                                 const float* w1_g, const uint8_t* w2, const uint8_t* w2_sf,
                                 const float* w2_g, void* out, int32_t* topk_ids_out,
                                 float* topk_w_out, int32_t tokens, int32_t experts, int32_t top_k,
                                 int32_t hidden, int32_t inter, int32_t n_group,
                                 int32_t topk_group, int32_t norm_topk_prob, float routed_scaling,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  const int32_t st = moe_check(router_logits, correction_bias, x, w1, w1_sf, w1_g, w2, w2_sf, w2_g,
                               out, tokens, experts, top_k, hidden, inter, n_group, topk_group);
  if (st != NVFP4_OK) return st;
  if (hidden % 128 != 0 || inter % 128 != 0) return NVFP4_EINVAL;   // whole 128-k chunks
  if (tokens == 0) return NVFP4_OK;
  const size_t need = nvfp4::moe_workspace_bytes(tokens, experts, top_k, hidden, inter);
  if (!workspace || workspace_bytes < need || !aligned256(workspace)) return NVFP4_EWORKSPACE;
  const int32_t ds = device_status();
  if (ds != NVFP4_OK) return ds;
  nvfp4::MoeArgs m{router_logits, correction_bias, x, w1, w1_sf, w1_g, w2, w2_sf, w2_g, out,
                   topk_ids_out, topk_w_out, tokens, experts, top_k, hidden, inter, n_group,
                   topk_group, norm_topk_prob ? 1 : 0, routed_scaling, workspace, workspace_bytes,
                   current_device()->num_cus, 1};
  return hip_status(nvfp4::launch_moe(m, (hipStream_t)stream));
}

int32_t nvfp4_moe_w4a16_noalloc(const float* router_logits, const float* correction_bias,
                                const void* x, const uint8_t* w1, const uint8_t* w1_sf,
                                const float* w1_g, const uint8_t* w2, const uint8_t* w2_sf,
                                const float* w2_g, void* out, int32_t* topk_ids_out,
                                float* topk_w_out, int32_t tokens, int32_t experts, int32_t top_k,
                                int32_t hidden, int32_t inter, int32_t n_group, int32_t topk_group,
                                int32_t norm_topk_prob, float routed_scaling, void* stream) {
  const int32_t st = moe_check(router_logits, correction_bias, x, w1, w1_sf, w1_g, w2, w2_sf, w2_g,
                               out, tokens, experts, top_k, hidden, inter, n_group, topk_group);
  if (st != NVFP4_OK || tokens == 0) return st;
  const size_t need = nvfp4::moe_workspace_bytes(tokens, experts, top_k, hidden, inter);
  if (need > (size_t)NVFP4_NOALLOC_SCRATCH_BYTES) return NVFP4_ESCRATCH;
  const int32_t ds = device_status();
  if (ds != NVFP4_OK) return ds;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  if (nvfp4::moe_noalloc_scratch(&scratch, &scratch_bytes) != hipSuccess || scratch_bytes < need)
    return NVFP4_EHIP;
  nvfp4::MoeArgs m{router_logits, correction_bias, x, w1, w1_sf, w1_g, w2, w2_sf, w2_g, out,
                   topk_ids_out, topk_w_out, tokens, experts, top_k, hidden, inter, n_group,
                   topk_group, norm_topk_prob ? 1 : 0, routed_scaling, scratch, scratch_bytes,
                   current_device()->num_cus, 0};
  return hip_status(nvfp4::launch_moe(m, (hipStream_t)stream));
}

}  // extern "C"
