// moe.hip -- routed MoE layer with NVFP4 weights and FP16 activations
// ("Nvfp4 A16 Blackwell Moe Runner", Nvfp4A16BlackwellMoeParams: sigmoid
// group-top-k routing with a correction bias, ReLU^2, NVFP4 fc1/fc2 with
// per-expert FP32 global scales), for gfx950.
//
// Four launches, all deterministic (no floating-point atomics):
//  1. route      : one wave per token.  Lanes hold experts; sigmoid scores
//                  (the same binary32 exp as the quantizer), biased scores,
//                  group scores = sum of the group's two best, repeated wave
//                  argmax for the kept groups and the top-k experts (ties to
//                  the lower index), weights normalized in rank order.
//  2. fc1        : grid (inter/128, experts).  Each workgroup finds the pairs
//                  (token, rank) routed to its expert by a ballot scan of the
//                  routing table in pair order, then computes
//                  h = relu(x . W1^T * g1)^2 for 128 weight rows with
//                  v_mfma_f32_32x32x16_f16 (weights dequantized in registers,
//                  exact in FP16; token rows gathered from x as the other
//                  operand).  h is stored in fp32 per pair, and the largest h
//                  of each pair is folded into a per-pair maximum (integer
//                  max on the fp32 bits: order independent).
//  3. fc2        : grid (hidden/128, experts).  Same structure on h, which is
//                  converted to FP16 after scaling by 2^-e (e = exponent of
//                  the pair's maximum, so no pair can overflow FP16);
//                  o = h . W2^T * g2 * 2^e, stored in fp32 per pair.
//  4. combine    : out[t] = sum_j w[t,j] * o[t*top_k + j] in rank order, FP16.
#include "device_common.h"
#include "internal.h"

#include <mutex>

namespace nvfp4 {

namespace {

constexpr int kFcThreads = 256;        // 4 waves x 32 weight rows
constexpr int kFcRows = 128;
constexpr int kTokTiles = 4;           // token tiles of 32 held in registers per pass

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct MoeWs {
  int32_t* ids;
  float* wts;
  uint32_t* pmax;
  float* h;
  float* o;
};

MoeWs carve(void* base, int P, int hidden, int inter) {
  unsigned char* p = reinterpret_cast<unsigned char*>(base);
  MoeWs w;
  w.ids = reinterpret_cast<int32_t*>(p); p += align256((size_t)P * 4);
  w.wts = reinterpret_cast<float*>(p); p += align256((size_t)P * 4);
  w.pmax = reinterpret_cast<uint32_t*>(p); p += align256((size_t)P * 4);
  w.h = reinterpret_cast<float*>(p); p += align256((size_t)P * inter * 4);
  w.o = reinterpret_cast<float*>(p);
  return w;
}

// (value, index) pair ordering: higher value first, lower index on ties.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return (va > vb) || (va == vb && ia < ib);
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off, 64);
    const int oi = __shfl_xor(i, off, 64);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
  }
}

constexpr int kMaxExpertsPerLane = 4;   // experts <= 256

__global__ void __launch_bounds__(256)
moe_route(const float* __restrict__ logits, const float* __restrict__ bias, int T, int E,
          int top_k, int n_group, int topk_group, int norm, float scaling,
          int32_t* __restrict__ ids, float* __restrict__ wts, uint32_t* __restrict__ pmax,
          int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  __shared__ float sb[4][256];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t_raw = blockIdx.x * 4 + wv;
  const bool tv = t_raw < T;             // waves past the last token idle but reach the barriers
  const int t = tv ? t_raw : 0;
  const float ninf = -__builtin_inff();
  const int gsize = E / n_group;
  float s[kMaxExpertsPerLane], b[kMaxExpertsPerLane];
#pragma unroll
  for (int i = 0; i < kMaxExpertsPerLane; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      s[i] = sigmoid_f32(logits[(int64_t)t * E + e]);
      b[i] = s[i] + bias[e];
      sb[wv][e] = b[i];
    } else {
      s[i] = 0.0f;
      b[i] = ninf;
    }
  }
  __syncthreads();
  // group scores: lane g sums its group's two best biased scores
  float gs[kMaxExpertsPerLane];
#pragma unroll
  for (int i = 0; i < kMaxExpertsPerLane; ++i) {
    const int g = lane + 64 * i;
    gs[i] = ninf;
    if (g < n_group) {
      float v1 = ninf, v2 = ninf;
      int i1 = -1, i2 = -1;
      for (int e = g * gsize; e < (g + 1) * gsize; ++e) {
        const float v = sb[wv][e];
        if (i1 < 0 || better(v, e, v1, i1)) { v2 = v1; i2 = i1; v1 = v; i1 = e; }
        else if (i2 < 0 || better(v, e, v2, i2)) { v2 = v; i2 = e; }
      }
      gs[i] = (i2 >= 0) ? v1 + v2 : v1;
    }
  }
  // keep topk_group groups
  bool keep[kMaxExpertsPerLane] = {false, false, false, false};
  for (int k = 0; k < topk_group; ++k) {
    float bv = ninf;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxExpertsPerLane; ++i) {
      const int g = lane + 64 * i;
      if (g < n_group && !keep[i] && better(gs[i], g, bv, bi)) { bv = gs[i]; bi = g; }
    }
    wave_argmax(bv, bi);
#pragma unroll
    for (int i = 0; i < kMaxExpertsPerLane; ++i)
      if (lane + 64 * i == bi) keep[i] = true;
  }
  // the kept-group flag of each of this lane's experts
  __shared__ int kg[4][256];
#pragma unroll
  for (int i = 0; i < kMaxExpertsPerLane; ++i) {
    const int g = lane + 64 * i;
    if (g < n_group) kg[wv][g] = keep[i] ? 1 : 0;
  }
  __syncthreads();
  bool cand[kMaxExpertsPerLane];
#pragma unroll
  for (int i = 0; i < kMaxExpertsPerLane; ++i) {
    const int e = lane + 64 * i;
    cand[i] = (e < E) && kg[wv][e / gsize];
  }
  // top_k experts among the kept groups
  float wsel = 0.0f;      // lane j < top_k ends up holding rank j's weight
  int isel = 0;
  for (int k = 0; k < top_k; ++k) {
    float bv = ninf;
    int bi = 0x7FFFFFFF;
    float sv = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxExpertsPerLane; ++i) {
      const int e = lane + 64 * i;
      if (cand[i] && better(b[i], e, bv, bi)) { bv = b[i]; bi = e; }
    }
    wave_argmax(bv, bi);
#pragma unroll
    for (int i = 0; i < kMaxExpertsPerLane; ++i)
      if (lane + 64 * i == bi) { cand[i] = false; sv = s[i]; }
    // broadcast the chosen expert's unbiased score from its owner lane
    sv = __shfl(sv, bi & 63, 64);
    if (lane == k) { wsel = sv; isel = bi; }
  }
  // normalize in rank order (sequential sum on lane 0), then scale
  float sum = 0.0f;
  for (int k = 0; k < top_k; ++k) sum = sum + __shfl(wsel, k, 64);
  if (tv && lane < top_k) {
    float wgt = norm ? wsel / sum : wsel;
    wgt = wgt * scaling;
    const int64_t p = (int64_t)t * top_k + lane;
    ids[p] = isel;
    wts[p] = wgt;
    pmax[p] = 0u;
    if (ids_out) ids_out[p] = isel;
    if (w_out) w_out[p] = wgt;
  }
}

// Pairs routed to expert e, in pair order, into LDS; returns their count.
__device__ int gather_pairs(const int32_t* __restrict__ ids, int P, int e, int* plist) {
  __shared__ int cnt_sh;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int cnt = 0;
    for (int base = 0; base < P; base += 64) {
      const int p = base + lane;
      const bool hit = (p < P) && ids[p] == e;
      const uint64_t m = __ballot(hit);
      if (hit) plist[cnt + __popcll(m & ((1ull << lane) - 1ull))] = p;
      cnt += __popcll(m);
    }
    if (lane == 0) cnt_sh = cnt;
  }
  __syncthreads();
  return cnt_sh;
}

// Pairs routed to expert e, in pair order: plist[i] = pair index, tlist[i] =
// its token (pair / top_k).  Every wave scans a contiguous share of the
// routing table (its ids are loaded in one round), a prefix over the waves
// orders the shares, a second ballot pass writes the lists.
constexpr int kGatherRegs = 8;   // routing-table chunks of 64 held per wave per round

__device__ int gather_pairs_all(const int32_t* __restrict__ ids, int P, int top_k, int e,
                                int* plist, int* tlist) {
  __shared__ int wcnt[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int nchunks = (P + 63) / 64;
  const int per = (nchunks + nw - 1) / nw;
  const int c0 = wave * per, c1 = (c0 + per < nchunks) ? c0 + per : nchunks;
  uint64_t masks[kGatherRegs];
  int cnt = 0;
  const bool inreg = (c1 - c0) <= kGatherRegs;
  if (inreg) {
    int v[kGatherRegs];
#pragma unroll
    for (int i = 0; i < kGatherRegs; ++i) {
      const int p = (c0 + i) * 64 + lane;
      v[i] = (c0 + i < c1 && p < P) ? ids[p] : -1;
    }
#pragma unroll
    for (int i = 0; i < kGatherRegs; ++i) {
      masks[i] = __ballot(v[i] == e);
      cnt += __popcll(masks[i]);
    }
  } else {
    for (int c = c0; c < c1; ++c) {
      const int p = c * 64 + lane;
      cnt += __popcll(__ballot((p < P) && ids[p] == e));
    }
  }
  if (lane == 0) wcnt[wave] = cnt;
  __syncthreads();
  int base = 0, total = 0;
  for (int i = 0; i < nw; ++i) {
    if (i < wave) base += wcnt[i];
    total += wcnt[i];
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  if (inreg) {
#pragma unroll
    for (int i = 0; i < kGatherRegs; ++i) {
      const int p = (c0 + i) * 64 + lane;
      if ((masks[i] >> lane) & 1ull) {
        const int slot = base + __popcll(masks[i] & lt);
        plist[slot] = p;
        tlist[slot] = p / top_k;
      }
      base += __popcll(masks[i]);
    }
  } else {
    for (int c = c0; c < c1; ++c) {
      const int p = c * 64 + lane;
      const bool hit = (p < P) && ids[p] == e;
      const uint64_t m = __ballot(hit);
      if (hit) {
        const int slot = base + __popcll(m & lt);
        plist[slot] = p;
        tlist[slot] = p / top_k;
      }
      base += __popcll(m);
    }
  }
  __syncthreads();
  return total;
}

__device__ __forceinline__ v8h dequant8_w(uint32_t codes, _Float16 s16) {
  const v2h s2 = {s16, s16};
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
  v8h r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// FC = 1: act = x fp16 [T, K] (row = pair / top_k); out = h fp32 [P, N] + pmax.
// FC = 2: act = h fp32 [P, K] scaled by 2^-e(pmax[p]); out = o fp32 [P, N].
template <int FC>
__global__ void __launch_bounds__(kFcThreads)
moe_fc(const void* __restrict__ act, const int32_t* __restrict__ ids, int P, int top_k,
       uint32_t* __restrict__ pmax, const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_sf,
       const float* __restrict__ w_g, int N, int K, float* __restrict__ out) {
  extern __shared__ int plist[];
  const int e = blockIdx.y;
  const int cnt = gather_pairs(ids, P, e, plist);
  if (cnt == 0) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int n0 = blockIdx.x * kFcRows + wv * 32;
  const int nrow = n0 + l32;
  const bool nvalid = nrow < N;
  const int64_t kb2 = K / 2, kb16 = K / 16;
  const uint8_t* wr = w + ((int64_t)e * N + (nvalid ? nrow : 0)) * kb2;
  const uint8_t* sr = w_sf + ((int64_t)e * N + (nvalid ? nrow : 0)) * kb16;
  const float ge = w_g[e];
  const v8h zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

  for (int t0 = 0; t0 < cnt; t0 += 32 * kTokTiles) {
    // this lane's token slot in each tile, its activation row and scale
    const void* arow[kTokTiles];
    float ainv[kTokTiles];
    bool avalid[kTokTiles];
#pragma unroll
    for (int tt = 0; tt < kTokTiles; ++tt) {
      const int slot = t0 + tt * 32 + l32;
      avalid[tt] = slot < cnt;
      const int p = avalid[tt] ? plist[slot] : 0;
      if constexpr (FC == 1) {
        arow[tt] = reinterpret_cast<const _Float16*>(act) + (int64_t)(p / top_k) * K;
        ainv[tt] = 1.0f;
      } else {
        arow[tt] = reinterpret_cast<const float*>(act) + (int64_t)p * K;
        const uint32_t mb = pmax[p];
        const int ex = (mb == 0u) ? 0 : (int)((mb >> 23) & 0xFFu) - 127;
        ainv[tt] = __builtin_ldexpf(1.0f, -ex);
      }
    }
    const int ntiles = (cnt - t0 + 31) / 32;
    v16f acc[kTokTiles];
#pragma unroll
    for (int tt = 0; tt < kTokTiles; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tt][r] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += 64) {
      const int k = k0 + 32 * h;
      const bool kv = k < K;
      const uint4 wc = (nvalid && kv) ? *reinterpret_cast<const uint4*>(wr + k / 2) : make_uint4(0, 0, 0, 0);
      const uint32_t sw = (nvalid && kv) ? (uint32_t)*reinterpret_cast<const uint16_t*>(sr + k / 16) : 0u;
      const _Float16 s0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)sw, 0);
      const _Float16 s1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)sw, 1);
      v8h wf[4];
      wf[0] = dequant8_w(wc.x, s0);
      wf[1] = dequant8_w(wc.y, s0);
      wf[2] = dequant8_w(wc.z, s1);
      wf[3] = dequant8_w(wc.w, s1);
#pragma unroll
      for (int tt = 0; tt < kTokTiles; ++tt) {
        if (tt >= ntiles) break;
        const bool v = avalid[tt] && kv;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          v8h af;
          if constexpr (FC == 1) {
            af = v ? *reinterpret_cast<const v8h*>(reinterpret_cast<const _Float16*>(arow[tt]) + k + 8 * m)
                   : zero8;
          } else {
            if (v) {
              const float* src = reinterpret_cast<const float*>(arow[tt]) + k + 8 * m;
              const float4 lo = *reinterpret_cast<const float4*>(src);
              const float4 hi = *reinterpret_cast<const float4*>(src + 4);
              const float sc = ainv[tt];
              af[0] = (_Float16)(lo.x * sc); af[1] = (_Float16)(lo.y * sc);
              af[2] = (_Float16)(lo.z * sc); af[3] = (_Float16)(lo.w * sc);
              af[4] = (_Float16)(hi.x * sc); af[5] = (_Float16)(hi.y * sc);
              af[6] = (_Float16)(hi.z * sc); af[7] = (_Float16)(hi.w * sc);
            } else {
              af = zero8;
            }
          }
          // weights are the A operand (rows = weight rows), tokens the B operand
          acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[m], af, acc[tt], 0, 0, 0);
        }
      }
    }

    // epilogue: D[i][j] -> weight row n0 + i, token slot t0 + tt*32 + j
#pragma unroll
    for (int tt = 0; tt < kTokTiles; ++tt) {
      if (tt >= ntiles) break;
      const int slot = t0 + tt * 32 + l32;
      const bool sv = slot < cnt;
      const int p = sv ? plist[slot] : 0;
      float vmax = 0.0f;
      float scale = ge;
      if constexpr (FC == 2) scale = ge / ainv[tt];   // ge * 2^e, exact power-of-two scaling
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = (r >> 2) * 8 + h * 4 + (r & 3);
        const int n = n0 + i;
        float v = acc[tt][r] * scale;
        if constexpr (FC == 1) {
          v = relu2_f32(v);
          vmax = __builtin_fmaxf(vmax, v);
        }
        if (sv && n < N) out[(int64_t)p * N + n] = v;
      }
      if constexpr (FC == 1) {
        vmax = __builtin_fmaxf(vmax, __shfl_xor(vmax, 32, 64));
        if (sv && h == 0) atomicMax(pmax + p, __float_as_uint(vmax));
      }
    }
  }
}

// Streaming version of fc1/fc2 (the one launched).  One workgroup = 4 waves
// = 64 weight rows of one expert, each wave 16 rows over the whole K (two
// workgroups fit a CU, so one computes while the other waits on memory).
// Each lane issues all of its weight-code loads (32 codes + 2 E4M3 bytes per
// 128-k chunk, up to 2048 k) before any arithmetic.  The expert's token rows
// are staged in LDS as FP16 in 256-k chunks (fc2 applies the per-pair power
// of two while staging), double-buffered, and feed v_mfma_f32_16x16x32_f16 as
// the second operand, 64 tokens per pass.
constexpr int kMsThreads = 256;
constexpr int kMsRows = 64;
constexpr int kMsKC = 256;               // staged k per LDS chunk
constexpr int kMsTok = 64;               // tokens per pass (4 tiles of 16)
constexpr int kMsSB = 2048;              // k per register superblock (16 chunks of 128)
constexpr int kMsPitch = kMsKC + 8;      // halves per staged token row (+16 B skew)

size_t moe_stream_lds(int tokens) {
  return 2 * align256((size_t)tokens * 4) + 2 * (size_t)kMsTok * kMsPitch * 2;
}

template <int FC>
__global__ void __launch_bounds__(kMsThreads)
moe_fc_stream(const void* __restrict__ act, const int32_t* __restrict__ ids, int P, int top_k,
              uint32_t* __restrict__ pmax, const uint8_t* __restrict__ w,
              const uint8_t* __restrict__ w_sf, const float* __restrict__ w_g, int N, int K,
              float* __restrict__ out, int tok_off) {
  extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
  int* plist = reinterpret_cast<int*>(sm);
  int* tlist = reinterpret_cast<int*>(sm + tok_off / 2);
  _Float16* xsb[2] = {reinterpret_cast<_Float16*>(sm + tok_off),
                      reinterpret_cast<_Float16*>(sm + tok_off + kMsTok * kMsPitch * 2)};
  const int e = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int nbase = blockIdx.x * kMsRows + wave * 16;
  const int nrow = nbase + r16;
  const bool nvalid = nrow < N;
  const int64_t kb2 = K / 2, kb16 = K / 16;
  const uint8_t* wr = w + ((int64_t)e * N + (nvalid ? nrow : 0)) * kb2;
  const uint8_t* sr = w_sf + ((int64_t)e * N + (nvalid ? nrow : 0)) * kb16;
  const v8h zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  constexpr int kStageVec = (kMsTok * kMsKC / 8) / kMsThreads;   // 8-element vectors per thread

  const int cnt = gather_pairs_all(ids, P, top_k, e, plist, tlist);
  if (cnt == 0) return;
  const float ge = w_g[e];

  uint4 wc[16];
  uint32_t ws[16];
  auto load_w = [&](int kb) {
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int k = kb + 128 * c + 32 * g;
      const bool v = nvalid && k < K;
      wc[c] = v ? *reinterpret_cast<const uint4*>(wr + k / 2) : make_uint4(0, 0, 0, 0);
      ws[c] = v ? (uint32_t)*reinterpret_cast<const uint16_t*>(sr + k / 16) : 0u;
    }
  };

  // staging of token rows: global -> registers -> LDS (FP16)
  v8h stg[kStageVec];
  auto stage_load = [&](int t0, int kc) {
#pragma unroll
    for (int i = 0; i < kStageVec; ++i) {
      const int v = tid + kMsThreads * i;
      const int slot = v / (kMsKC / 8), kq = v % (kMsKC / 8);
      const int k = kc + 8 * kq;
      v8h val = zero8;
      if (t0 + slot < cnt && k < K) {
        if constexpr (FC == 1) {
          val = *reinterpret_cast<const v8h*>(reinterpret_cast<const _Float16*>(act) +
                                              (int64_t)tlist[t0 + slot] * K + k);
        } else {
          const int p = plist[t0 + slot];
          const uint32_t mb = pmax[p];
          const int ex = (mb == 0u) ? 0 : (int)((mb >> 23) & 0xFFu) - 127;
          const float sc = __builtin_ldexpf(1.0f, -ex);
          const float* src = reinterpret_cast<const float*>(act) + (int64_t)p * K + k;
          const float4 lo = *reinterpret_cast<const float4*>(src);
          const float4 hi = *reinterpret_cast<const float4*>(src + 4);
          val[0] = (_Float16)(lo.x * sc); val[1] = (_Float16)(lo.y * sc);
          val[2] = (_Float16)(lo.z * sc); val[3] = (_Float16)(lo.w * sc);
          val[4] = (_Float16)(hi.x * sc); val[5] = (_Float16)(hi.y * sc);
          val[6] = (_Float16)(hi.z * sc); val[7] = (_Float16)(hi.w * sc);
        }
      }
      stg[i] = val;
    }
  };
  auto stage_store = [&](_Float16* xs) {
#pragma unroll
    for (int i = 0; i < kStageVec; ++i) {
      const int v = tid + kMsThreads * i;
      const int slot = v / (kMsKC / 8), kq = v % (kMsKC / 8);
      *reinterpret_cast<v8h*>(xs + slot * kMsPitch + 8 * kq) = stg[i];
    }
  };

  // one superblock of up to 2048 k for tokens [t0, t0+64)
  auto superblock = [&](int t0, int kb, v4f* acc) {
    stage_store(xsb[0]);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kMsSB / kMsKC; ++q) {
      const int kc = kb + q * kMsKC;
      if (kc >= K) break;
      const bool more = (q + 1 < kMsSB / kMsKC) && (kc + kMsKC < K);
      if (more) stage_load(t0, kc + kMsKC);        // next chunk's loads in flight
      const _Float16* xs = xsb[q & 1];
#pragma unroll
      for (int c2 = 0; c2 < kMsKC / 128; ++c2) {
        const int c = q * (kMsKC / 128) + c2;     // chunk within the superblock
        const int k = kc + 128 * c2 + 32 * g;
        if (kc + 128 * c2 >= K) break;
        const _Float16 s0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)ws[c], 0);
        const _Float16 s1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)ws[c], 1);
        v8h af[4];
        af[0] = dequant8_w(wc[c].x, s0);
        af[1] = dequant8_w(wc[c].y, s0);
        af[2] = dequant8_w(wc[c].z, s1);
        af[3] = dequant8_w(wc[c].w, s1);
        const bool kv = k < K;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          if (t0 + 16 * tt >= cnt) break;
          const _Float16* xrow = xs + (16 * tt + r16) * kMsPitch + 128 * c2 + 32 * g;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const v8h bf = kv ? *reinterpret_cast<const v8h*>(xrow + 8 * m) : zero8;
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[m], bf, acc[tt], 0, 0, 0);
          }
        }
      }
      if (more) stage_store(xsb[(q + 1) & 1]);
      __syncthreads();
    }
  };

  auto epilogue = [&](int t0, const v4f* acc) {
    // D[i][j] -> weight row nbase + 4g + r, token slot t0 + 16tt + (lane & 15)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      if (t0 + 16 * tt >= cnt) break;
      const int slot = t0 + 16 * tt + r16;
      const bool sv = slot < cnt;
      const int p = sv ? plist[slot] : 0;
      float scale = ge;
      if constexpr (FC == 2) {
        const uint32_t mb = pmax[p];
        const int ex = (mb == 0u) ? 0 : (int)((mb >> 23) & 0xFFu) - 127;
        scale = __builtin_ldexpf(ge, ex);
      }
      float vmax = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = nbase + 4 * g + r;
        float v = acc[tt][r] * scale;
        if constexpr (FC == 1) {
          v = relu2_f32(v);
          vmax = __builtin_fmaxf(vmax, v);
        }
        if (sv && n < N) out[(int64_t)p * N + n] = v;
      }
      if constexpr (FC == 1) {
        vmax = __builtin_fmaxf(vmax, __shfl_xor(vmax, 16, 64));
        vmax = __builtin_fmaxf(vmax, __shfl_xor(vmax, 32, 64));
        if (sv && g == 0) atomicMax(pmax + p, __float_as_uint(vmax));
      }
    }
  };

  if (cnt <= kMsTok && K <= kMsSB) {
    // common case: one pass, one superblock, straight-line
    load_w(0);
    stage_load(0, 0);
    v4f acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    superblock(0, 0, acc);
    epilogue(0, acc);
    return;
  }
  for (int t0 = 0; t0 < cnt; t0 += kMsTok) {
    v4f acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int kb = 0; kb < K; kb += kMsSB) {
      load_w(kb);
      stage_load(t0, kb);
      superblock(t0, kb, acc);
    }
    epilogue(t0, acc);
  }
}

// out[t] = sum_j w[t,j] * o[t*top_k + j], four outputs per thread.
__global__ void __launch_bounds__(256)
moe_combine4(const float* __restrict__ o, const float* __restrict__ wts, int top_k, int H,
             _Float16* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int n = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (n >= H) return;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < top_k; ++j) {
    const float wj = wts[t * top_k + j];
    const float4 v = *reinterpret_cast<const float4*>(o + (t * top_k + j) * H + n);
    s.x += wj * v.x; s.y += wj * v.y; s.z += wj * v.z; s.w += wj * v.w;
  }
  v4h r = {(_Float16)s.x, (_Float16)s.y, (_Float16)s.z, (_Float16)s.w};
  *reinterpret_cast<v4h*>(out + t * H + n) = r;
}

__global__ void __launch_bounds__(256)
moe_combine(const float* __restrict__ o, const float* __restrict__ wts, int top_k, int H,
            _Float16* __restrict__ out) {
  const int64_t t = blockIdx.x;
  for (int n = threadIdx.x; n < H; n += blockDim.x) {
    float s = 0.0f;
    for (int j = 0; j < top_k; ++j) s += wts[t * top_k + j] * o[(t * top_k + j) * H + n];
    out[t * H + n] = (_Float16)s;
  }
}

}  // namespace

size_t moe_workspace_bytes(int tokens, int experts, int top_k, int hidden, int inter) {
  (void)experts;
  const size_t P = (size_t)tokens * top_k;
  return 3 * align256(P * 4) + align256(P * inter * 4) + align256(P * hidden * 4);
}

hipError_t launch_moe(const MoeArgs& m, hipStream_t s) {
  const int P = m.tokens * m.top_k;
  if (m.tokens > 16384) return hipErrorNotSupported;   // the per-expert pair list lives in LDS
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, []() {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_fc_stream<1>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 1024);
    if (attr_err == hipSuccess)
      attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_fc_stream<2>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 1024);
  });
  if (attr_err != hipSuccess) return attr_err;
  MoeWs ws = carve(m.workspace, P, m.hidden, m.inter);
  hipLaunchKernelGGL(moe_route, dim3((m.tokens + 3) / 4), dim3(256), 0, s, m.logits, m.bias,
                     m.tokens, m.experts, m.top_k, m.n_group, m.topk_group, m.norm, m.scaling,
                     ws.ids, ws.wts, ws.pmax, m.ids_out, m.w_out);
  const size_t lds = moe_stream_lds(m.tokens);
  const int tok_off = 2 * (int)align256((size_t)m.tokens * 4);
  hipLaunchKernelGGL(moe_fc_stream<1>, dim3((m.inter + kMsRows - 1) / kMsRows, m.experts),
                     dim3(kMsThreads), lds, s, m.x, ws.ids, P, m.top_k, ws.pmax, m.w1, m.w1_sf,
                     m.w1_g, m.inter, m.hidden, ws.h, tok_off);
  hipLaunchKernelGGL(moe_fc_stream<2>, dim3((m.hidden + kMsRows - 1) / kMsRows, m.experts),
                     dim3(kMsThreads), lds, s, ws.h, ws.ids, P, m.top_k, ws.pmax, m.w2, m.w2_sf,
                     m.w2_g, m.hidden, m.inter, ws.o, tok_off);
  hipLaunchKernelGGL(moe_combine4, dim3(m.tokens, (m.hidden + 1023) / 1024), dim3(256), 0, s, ws.o,
                     ws.wts, m.top_k, m.hidden, reinterpret_cast<_Float16*>(m.out));
  return hipGetLastError();
}

}  // namespace nvfp4
