// moe.hip -- routed MoE layer with NVFP4 weights and FP16 activations
// ("Nvfp4 A16 Blackwell Moe Runner", Nvfp4A16BlackwellMoeParams: sigmoid
// group-top-k routing with a correction bias, ReLU^2, NVFP4 fc1/fc2 with
// per-expert FP32 global scales), for gfx950.
//
// Five launches, all deterministic (no floating-point atomics):
//  1. route      : one wave per token.  Lanes hold experts; sigmoid scores
//                  (the same binary32 exp as the quantizer), biased scores,
//                  group scores = sum of the group's two best; kept groups and
//                  top-k experts by rank counts in the order "higher score
//                  first, lower index on ties"; weights normalized in rank
//                  order.
//  2. lists      : one workgroup per expert writes the pairs (token, rank)
//                  routed to it, in pair order, and their count.
//  3. fc1        : grid (inter/256 row tiles, experts, token passes), 8 waves
//                  x 32 weight rows, v_mfma_f32_32x32x16_f16.  Weights are
//                  dequantized in registers (exact in FP16) and loaded three
//                  128-k chunks ahead; the expert's tokens are gathered from x
//                  three chunks ahead and staged in LDS, in balanced passes of
//                  at most 64 tokens (an expert with more tokens spreads over
//                  several workgroups).  h = relu(x . W1^T * g1)^2 is stored
//                  as FP16 scaled by 2^-et per (pair, 256-row tile), et the
//                  exponent of the tile's largest h; the pair's overall
//                  largest h is an integer max of fp32 bits (order
//                  independent).
//  4. fc2        : grid (hidden/256 row tiles, experts, token passes).  Same
//                  structure on h, each tile rescaled by 2^(et - e) while
//                  staged (e = exponent of the pair's largest h, so no pair
//                  can overflow FP16); o = h . W2^T * g2 * 2^e in fp32 per
//                  pair.
//  5. combine    : out[t] = sum_j w[t,j] * o[t*top_k + j] in rank order, FP16.
#include "device_common.h"
#include "internal.h"
#include "../../include/nvfp4_mi355x.h"

#include <mutex>

// Fixed device scratch of nvfp4_moe_w4a16_noalloc, for callers that cannot
// allocate.  Each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` is only a host-side stand-in: the
// device address comes from moe_noalloc_scratch() below and is what the
// kernels receive.
static __device__ __align__(256) unsigned char scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

namespace nvfp4 {

namespace {

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Expert FFN kernels (moe_fc_wide below): work split and staging.
constexpr int kFwThreads = 512;
constexpr int kFwRows = 256;              // weight rows per tile (32 per wave)
constexpr int kFwKC = 128;                // k per chunk
constexpr int kFwTT = 2;                  // 32-token MFMA tiles per pass
constexpr int kFwTok = 32 * kFwTT;        // tokens per pass at most
constexpr int kFwPitch = kFwKC + 8;       // halves per staged token row (+16 B skew)
constexpr int kFwVec = kFwTok * kFwKC / 8 / kFwThreads;   // staged 8-element vectors per thread
constexpr int kFwRowThreads = kFwKC / 8;  // threads staging one token row of a chunk
constexpr int kFwSlotsPerVec = kFwThreads / kFwRowThreads;   // token slots per staged vector index
constexpr int kFwWBuf = 4;                // weight register buffers (loads three chunks ahead)
constexpr int kFwMaxZ = 1024;             // grid z (more passes handled in a loop)
constexpr int kFwMaxT1 = 8192 / kFwRows;  // fc1 row tiles (inter <= 8192)
constexpr int kFwPerCU = 512 / kFwThreads;   // workgroups resident per compute unit
static_assert(kFwVec * kFwSlotsPerVec == kFwTok, "staging covers the pass's token slots");
static_assert(kFwRows == 32 * (kFwThreads / 64), "one 32-row MFMA tile per wave");

struct MoeWs {
  int32_t* ids;      // [P] expert of each pair
  float* wts;        // [P] its weight
  uint32_t* pmax;    // [P] largest h of the pair (fp32 bits)
  int32_t* counts;   // [E] pairs per expert
  int32_t* plists;   // [E, T] pairs of each expert
  int32_t* tlists;   // [E, T] their tokens
  int32_t* etile;    // [P, nt1] exponent of each fc1 row tile's largest h
  _Float16* h;       // [P, inter] scaled per fc1 row tile
  float* o;          // [P, hidden]
};

int fc1_tiles(int inter) { return (inter + kFwRows - 1) / kFwRows; }

MoeWs carve(void* base, int T, int E, int P, int hidden, int inter) {
  unsigned char* p = reinterpret_cast<unsigned char*>(base);
  MoeWs w;
  w.ids = reinterpret_cast<int32_t*>(p); p += align256((size_t)P * 4);
  w.wts = reinterpret_cast<float*>(p); p += align256((size_t)P * 4);
  w.pmax = reinterpret_cast<uint32_t*>(p); p += align256((size_t)P * 4);
  w.counts = reinterpret_cast<int32_t*>(p); p += align256((size_t)E * 4);
  w.plists = reinterpret_cast<int32_t*>(p); p += align256((size_t)E * T * 4);
  w.tlists = reinterpret_cast<int32_t*>(p); p += align256((size_t)E * T * 4);
  w.etile = reinterpret_cast<int32_t*>(p); p += align256((size_t)P * fc1_tiles(inter) * 4);
  w.h = reinterpret_cast<_Float16*>(p); p += align256((size_t)P * inter * 2);
  w.o = reinterpret_cast<float*>(p);
  (void)hidden;
  return w;
}

// (value, index) pair ordering: higher value first, lower index on ties.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return (va > vb) || (va == vb && ia < ib);
}

constexpr int kMaxExpertsPerLane = 4;   // experts <= 256

// One wave per token.  Each selection is made by counting, for every
// contender, how many others come before it in the (value desc, index asc)
// order -- the same order as taking repeated maxima with ties to the lower
// index -- so no serial chain of cross-lane reductions is needed.
__global__ void __launch_bounds__(256)
moe_route(const float* __restrict__ logits, const float* __restrict__ bias, int T, int E,
          int top_k, int n_group, int topk_group, int norm, float scaling,
          int32_t* __restrict__ ids, float* __restrict__ wts, uint32_t* __restrict__ pmax,
          int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  __shared__ float sb[4][256];      // biased scores
  __shared__ float sg[4][256];      // group scores
  __shared__ int kg[4][256];        // kept-group flags
  __shared__ float cb[4][256];      // candidates (experts of kept groups): biased score
  __shared__ int ce[4][256];        // ... and expert index, in expert order
  __shared__ int sel_e[4][16];      // chosen experts by rank
  __shared__ float sel_s[4][16];    // their unbiased scores
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
      if (b[i] != b[i]) b[i] = ninf;   // a NaN score ranks below every number
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
#pragma unroll 8
      for (int e = g * gsize; e < (g + 1) * gsize; ++e) {
        const float v = sb[wv][e];
        if (i1 < 0 || better(v, e, v1, i1)) { v2 = v1; i2 = i1; v1 = v; i1 = e; }
        else if (i2 < 0 || better(v, e, v2, i2)) { v2 = v; i2 = e; }
      }
      gs[i] = (i2 >= 0) ? v1 + v2 : v1;
      sg[wv][g] = gs[i];
    }
  }
  __syncthreads();
  // a group is kept when fewer than topk_group groups come before it
#pragma unroll
  for (int i = 0; i < kMaxExpertsPerLane; ++i) {
    const int g = lane + 64 * i;
    if (g < n_group) {
      int r = 0;
#pragma unroll 8
      for (int g2 = 0; g2 < n_group; ++g2) r += better(sg[wv][g2], g2, gs[i], g) ? 1 : 0;
      kg[wv][g] = r < topk_group ? 1 : 0;
    }
  }
  __syncthreads();
  // compact the candidates in expert order
  const uint64_t below = (1ull << lane) - 1ull;
  int nc = 0;
  bool cand[kMaxExpertsPerLane];
  int cpos[kMaxExpertsPerLane];
#pragma unroll
  for (int i = 0; i < kMaxExpertsPerLane; ++i) {
    const int e = lane + 64 * i;
    cand[i] = (e < E) && kg[wv][e / gsize] != 0;
    const uint64_t m = __ballot(cand[i]);
    cpos[i] = nc + __popcll(m & below);
    if (cand[i]) { cb[wv][cpos[i]] = b[i]; ce[wv][cpos[i]] = e; }
    nc += __popcll(m);
  }
  __syncthreads();
  // a candidate is chosen at rank r = number of candidates before it
#pragma unroll
  for (int i = 0; i < kMaxExpertsPerLane; ++i) {
    if (cand[i]) {
      const int e = lane + 64 * i;
      int r = 0;
#pragma unroll 8
      for (int c = 0; c < nc; ++c) r += better(cb[wv][c], ce[wv][c], b[i], e) ? 1 : 0;
      if (r < top_k) { sel_e[wv][r] = e; sel_s[wv][r] = s[i]; }
    }
  }
  __syncthreads();
  // normalize in rank order (every lane forms the same sequential sum), then scale
  float sum = 0.0f;
#pragma unroll 8
  for (int k = 0; k < top_k; ++k) sum = sum + sel_s[wv][k];
  if (tv && lane < top_k) {
    const float wsel = sel_s[wv][lane];
    const int isel = sel_e[wv][lane];
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

// Pairs routed to expert e, in pair order, written to lists + e*T (pair
// index) and tlists + e*T (its token); counts[e] = their number.  One
// workgroup per expert: every wave scans a contiguous share of the routing
// table (ids loaded in one round), a prefix over the waves orders the
// shares, a second ballot pass writes the lists.  An expert appears at most
// once per token, so T entries always suffice.
constexpr int kListThreads = 256;
constexpr int kListRegs = 16;   // routing-table chunks of 64 held per wave

__global__ void __launch_bounds__(kListThreads)
moe_lists(const int32_t* __restrict__ ids, int P, int T, int top_k, int32_t* __restrict__ plists,
          int32_t* __restrict__ tlists, int32_t* __restrict__ counts) {
  __shared__ int wcnt[kListThreads / 64];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = kListThreads / 64;
  const int nchunks = (P + 63) / 64;
  const int per = (nchunks + nw - 1) / nw;
  const int c0 = wave * per, c1 = (c0 + per < nchunks) ? c0 + per : nchunks;
  int32_t* pl = plists + (int64_t)e * T;
  int32_t* tl = tlists + (int64_t)e * T;
  const uint64_t lt = (1ull << lane) - 1ull;
  int cnt = 0;
  // the branch depends on `per` only (block-uniform), so every wave reaches
  // the same barrier; each wave's share c1 - c0 is at most `per`
  if (per <= kListRegs) {
    uint64_t masks[kListRegs];
    int v[kListRegs];
#pragma unroll
    for (int i = 0; i < kListRegs; ++i) {
      const int p = (c0 + i) * 64 + lane;
      v[i] = (c0 + i < c1 && p < P) ? ids[p] : -1;
    }
#pragma unroll
    for (int i = 0; i < kListRegs; ++i) {
      masks[i] = __ballot(v[i] == e);
      cnt += __popcll(masks[i]);
    }
    if (lane == 0) wcnt[wave] = cnt;
    __syncthreads();
    int base = 0, total = 0;
    for (int i = 0; i < nw; ++i) {
      if (i < wave) base += wcnt[i];
      total += wcnt[i];
    }
#pragma unroll
    for (int i = 0; i < kListRegs; ++i) {
      const int p = (c0 + i) * 64 + lane;
      if ((masks[i] >> lane) & 1ull) {
        const int slot = base + __popcll(masks[i] & lt);
        pl[slot] = p;
        tl[slot] = p / top_k;
      }
      base += __popcll(masks[i]);
    }
    if (threadIdx.x == 0) counts[e] = total;
  } else {
    for (int c = c0; c < c1; ++c) {
      const int p = c * 64 + lane;
      cnt += __popcll(__ballot((p < P) && ids[p] == e));
    }
    if (lane == 0) wcnt[wave] = cnt;
    __syncthreads();
    int base = 0, total = 0;
    for (int i = 0; i < nw; ++i) {
      if (i < wave) base += wcnt[i];
      total += wcnt[i];
    }
    for (int c = c0; c < c1; ++c) {
      const int p = c * 64 + lane;
      const bool hit = (p < P) && ids[p] == e;
      const uint64_t m = __ballot(hit);
      if (hit) {
        const int slot = base + __popcll(m & lt);
        pl[slot] = p;
        tl[slot] = p / top_k;
      }
      base += __popcll(m);
    }
    if (threadIdx.x == 0) counts[e] = total;
  }
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

// Expert FFN layer.  A unit of work is (expert e, tile of 256 weight rows,
// pass of up to kFwTok of the expert's tokens); an expert with more tokens is
// cut into balanced passes.  Workgroup (x, e, z) takes passes z, z +
// gridDim.z, ... and, within each pass, R consecutive row tiles streamed back
// to back (R > 1 when the units number four or more per workgroup slot).
// 8 waves x one 32-row v_mfma_f32_32x32x16_f16 tile, kFwTT 32-token tiles.
// K goes in 128-k chunks; lane (row r, half h) owns the 64 k at 64 h of a
// chunk: two 16-byte code loads and one 4-byte load of its four E4M3 bytes,
// issued three chunks ahead (across row tiles) into registers and used as
// loaded (no widening or packing that would make the compiler wait for them
// early).  MFMA m of a chunk takes k = 64 h + 8 m .. + 7 from both operands.  The FP16 activations
// of a chunk are loaded three chunks ahead into registers and written to LDS
// one chunk ahead.  Loads are issued in the order they are needed and the
// chunk barrier waits for LDS traffic only, so each wait covers just what the
// next step uses.  Requires K % 64 == 0.
// FC = 1: act = x [T, K] (row = token).  out = h [P, N] FP16 with, per pair
//         and row tile, h scaled by 2^-et (et = exponent of the tile's
//         largest h, stored in etile [P, nt1]); pmax[p] = largest h (fp32
//         bits, integer max: order independent).
// FC = 2: act = h [P, K]; staging rescales each 256-k tile by 2^(et - e),
//         e = exponent of pmax[p], so the pair's values share one scale and
//         none can overflow FP16.  out = o [P, N] fp32 = h . W^T * g * 2^e.


template <int V> struct IntC { static constexpr int value = V; };

struct WChunk {
  uint4 q0, q1;     // 64 codes
  uint32_t sc;      // their four E4M3 block scales
};


__device__ __forceinline__ int exponent_of(uint32_t bits) {
  return bits == 0u ? 0 : (int)((bits >> 23) & 0xFFu) - 127;
}

template <int FC>
__global__ void __launch_bounds__(kFwThreads)
moe_fc_wide(const _Float16* __restrict__ act, const int32_t* __restrict__ plists,
            const int32_t* __restrict__ tlists, const int32_t* __restrict__ counts, int T,
            uint32_t* __restrict__ pmax, int32_t* __restrict__ etile, int nt1,
            const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_sf,
            const float* __restrict__ w_g, int N, int K, int R, void* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) _Float16 xs[2][kFwTok * kFwPitch];
  __shared__ int spair[kFwTok];   // pair of each token slot of the pass
  __shared__ int srow[kFwTok];    // its activation row
  __shared__ int sexp[kFwTok];    // fc2: exponent e of the pair's largest h
  __shared__ float redmax[FC == 1 ? kFwThreads / 64 : 1][kFwTok];   // fc1: per-wave largest h
  // fc2: factor 2^(et - e) of each fc1 row tile t of each slot's pair
  __shared__ _Float16 sfac[FC == 2 ? kFwMaxT1 : 1][kFwTok];
  // workgroups of one expert on one XCD (consecutive workgroup ids go to
  // consecutive XCDs), so the expert's activations are fetched into one L2
  int bx = blockIdx.x, e = blockIdx.y;
  if ((gridDim.y & 7) == 0) {
    const int L = blockIdx.x + gridDim.x * blockIdx.y;
    const int slot = L >> 3;
    bx = slot % gridDim.x;
    e = (slot / gridDim.x) * 8 + (L & 7);
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int32_t* pl = plists + (int64_t)e * T;
  const int32_t* tl = tlists + (int64_t)e * T;
  // the first pass starts at the list head: load it together with the count
  int lp = 0, lt = 0;
  if (blockIdx.z == 0 && tid < kFwTok) {
    const int idx = tid < T ? tid : T - 1;
    lp = pl[idx];
    if (FC == 1) lt = tl[idx];
  }
  const int cnt = counts[e];
  const int np = (cnt + kFwTok - 1) / kFwTok;   // passes
  if ((int)blockIdx.z >= np) return;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, h = lane >> 5;
  const int nch = (K + kFwKC - 1) / kFwKC;
  const int nchp = (nch + kFwWBuf - 1) / kFwWBuf * kFwWBuf;   // whole rounds of four (extra chunks are zero)
  const int tiles = (N + kFwRows - 1) / kFwRows;
  const int xt0 = bx * R;
  const int ntile = (tiles - xt0 < R) ? tiles - xt0 : R;
  const float ge = w_g[e];
  const uint8_t* we = w + (int64_t)e * N * (K / 2);
  const uint8_t* se = w_sf + (int64_t)e * N * (K / 16);

  // this lane's weight row in row tile ti (rows past N re-read row N-1;
  // they are not stored)
  auto wrow = [&](int ti, const uint8_t*& wr, const uint8_t*& sr) __attribute__((always_inline)) {
    int n = (xt0 + ti) * kFwRows + wave * 32 + r32;
    n = n < N ? n : N - 1;
    wr = we + (int64_t)n * (K / 2);
    sr = se + (int64_t)n * (K / 16);
  };
  WChunk wb[kFwWBuf];
  // chunk c of a row (chunks past K re-read k = 0; compute() zeroes them)
  auto load_w = [&](const uint8_t* wr, const uint8_t* sr, int c, WChunk& d) __attribute__((always_inline)) {
    int k = c * kFwKC + 64 * h;
    k = k < K ? k : 0;
    d.q0 = *reinterpret_cast<const uint4*>(wr + k / 2);
    d.q1 = *reinterpret_cast<const uint4*>(wr + k / 2 + 16);
    d.sc = *reinterpret_cast<const uint32_t*>(sr + k / 16);
  };

  // staging: vector i of a thread = token slot kFwSlotsPerVec * i + tid /
  // kFwRowThreads, 8 k at 8 (tid % kFwRowThreads); only the pass's token
  // tiles are staged
  v8h stg[kFwWBuf][kFwVec];
  const int kq = tid % (kFwKC / 8);
  int64_t abase[kFwVec];     // element offset of the slot's activation row
  bool sval[kFwVec];
  // All kFwVec loads are issued whatever the pass's token count (slots past
  // it read a valid row and are never stored), so every step issues the same
  // number of loads and the compiler's load-counter waits stay exact; with a
  // count-dependent number of loads it waits conservatively, for loads issued
  // only one step earlier.
  auto stage_load = [&](int c, v8h (&dst)[kFwVec]) __attribute__((always_inline)) {
    const int k0 = c * kFwKC + 8 * kq;
    const int k = k0 < K ? k0 : 8 * kq;
#pragma unroll
    for (int i = 0; i < kFwVec; ++i) dst[i] = *reinterpret_cast<const v8h*>(act + abase[i] + k);
  };
  auto stage_store = [&](int c, const v8h (&src)[kFwVec], _Float16* xb, int ntt) __attribute__((always_inline)) {
    const bool kv = c * kFwKC + 8 * kq < K;
    const int ct = c * kFwKC / kFwRows;   // fc2: fc1 row tile of the chunk
    const int t = ct < nt1 ? ct : nt1 - 1;
#pragma unroll
    for (int i = 0; i < kFwVec; ++i) {
      if (kFwSlotsPerVec * i / 32 < ntt) {
        v8h val = src[i];
        if constexpr (FC == 2) {
          const _Float16 f = sfac[t][kFwSlotsPerVec * i + tid / kFwRowThreads];
          const v2h f2 = {f, f};
          v2h* pv = reinterpret_cast<v2h*>(&val);
          pv[0] = pv[0] * f2; pv[1] = pv[1] * f2; pv[2] = pv[2] * f2; pv[3] = pv[3] * f2;
        }
        if (!(kv && sval[i])) val = v8h{0, 0, 0, 0, 0, 0, 0, 0};
        *reinterpret_cast<v8h*>(xb + (kFwSlotsPerVec * i + tid / kFwRowThreads) * kFwPitch + 8 * kq) = val;
      }
    }
  };

  v16f acc[kFwTT];
  auto compute = [&](int c, const _Float16* xb, const WChunk& d, int ntt) __attribute__((always_inline)) {
    const bool kv = c * kFwKC + 64 * h < K;
    const uint32_t words[8] = {d.q0.x, d.q0.y, d.q0.z, d.q0.w, d.q1.x, d.q1.y, d.q1.z, d.q1.w};
    _Float16 s16[4];
    s16[0] = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)d.sc, 0);
    s16[1] = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)d.sc, 1);
    s16[2] = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)d.sc, 2);
    s16[3] = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)d.sc, 3);
    // the chunk's eight weight fragments once, then per token tile its eight
    // activation fragments read together before its eight MFMAs (one LDS
    // round trip per tile rather than per MFMA; each accumulator still sums
    // its fragments in the order m = 0..7)
    v8h af[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) af[m] = dequant8_w(kv ? words[m] : 0u, s16[m >> 1]);
#pragma unroll
    for (int tt = 0; tt < kFwTT; ++tt) {
      if (tt >= ntt) break;   // wave-uniform
      v8h bf[8];
#pragma unroll
      for (int m = 0; m < 8; ++m)
        bf[m] = *reinterpret_cast<const v8h*>(xb + (32 * tt + r32) * kFwPitch + 64 * h + 8 * m);
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[m], bf[m], acc[tt], 0, 0, 0);
    }
  };

  // results of row tile ti: acc[tt][r] = weight row n0 + 8 (r / 4) + 4 h +
  // r % 4, token slot 32 tt + r32
  auto epilogue = [&](int ti, int ntok, int ntt) __attribute__((always_inline)) {
    const int xt = xt0 + ti;
    const int n0 = xt * kFwRows + wave * 32;
    if constexpr (FC == 1) {
#pragma unroll
      for (int tt = 0; tt < kFwTT; ++tt) {
        if (tt >= ntt) break;
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) m = __builtin_fmaxf(m, relu2_f32(acc[tt][r] * ge));
        if (n0 >= N) m = 0.0f;
        m = __builtin_fmaxf(m, __shfl_xor(m, 32, 64));
        if (h == 0) redmax[wave][32 * tt + r32] = m;
      }
      lds_barrier();
#pragma unroll
      for (int tt = 0; tt < kFwTT; ++tt) {
        if (tt >= ntt) break;
        const int slot = 32 * tt + r32;
        float tmax = redmax[0][slot];
#pragma unroll
        for (int wv = 1; wv < kFwThreads / 64; ++wv) tmax = __builtin_fmaxf(tmax, redmax[wv][slot]);
        const int ex = exponent_of(__float_as_uint(tmax));
        const float sc = __builtin_ldexpf(1.0f, -ex);
        const bool sv = slot < ntok;
        const int p = spair[slot];
        if (sv && n0 < N) {
          _Float16* hp = reinterpret_cast<_Float16*>(out) + (int64_t)p * N + n0 + 4 * h;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v4h o4;
            o4[0] = (_Float16)(relu2_f32(acc[tt][4 * q + 0] * ge) * sc);
            o4[1] = (_Float16)(relu2_f32(acc[tt][4 * q + 1] * ge) * sc);
            o4[2] = (_Float16)(relu2_f32(acc[tt][4 * q + 2] * ge) * sc);
            o4[3] = (_Float16)(relu2_f32(acc[tt][4 * q + 3] * ge) * sc);
            *reinterpret_cast<v4h*>(hp + 8 * q) = o4;
          }
        }
        if (sv && wave == 0 && h == 0) {
          etile[(int64_t)p * nt1 + xt] = ex;
          atomicMax(pmax + p, __float_as_uint(tmax));
        }
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < kFwTT; ++tt) {
        if (tt >= ntt) break;
        const int slot = 32 * tt + r32;
        const float scale = __builtin_ldexpf(ge, sexp[slot]);
        if (slot < ntok && n0 < N) {
          float* op = reinterpret_cast<float*>(out) + (int64_t)spair[slot] * N + n0 + 4 * h;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float4 v;
            v.x = acc[tt][4 * q + 0] * scale;
            v.y = acc[tt][4 * q + 1] * scale;
            v.z = acc[tt][4 * q + 2] * scale;
            v.w = acc[tt][4 * q + 3] * scale;
            *reinterpret_cast<float4*>(op + 8 * q) = v;
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < kFwTT; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tt][r] = 0.0f;
  };

#pragma unroll
  for (int tt = 0; tt < kFwTT; ++tt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[tt][r] = 0.0f;
  for (int z = blockIdx.z; z < np; z += gridDim.z) {
    // balanced passes: the first cnt % np passes take one token more
    const int base = cnt / np, rem = cnt % np;
    const int ntok = base + (z < rem ? 1 : 0);
    const int t0 = z * base + (z < rem ? z : rem);
    const int ntt = (ntok + 31) / 32;
    if (z != (int)blockIdx.z) __syncthreads();   // a previous pass is done with the LDS buffers
    if (t0 != 0 && tid < kFwTok) {
      lp = pl[t0 + (tid < ntok ? tid : 0)];
      if (FC == 1) lt = tl[t0 + (tid < ntok ? tid : 0)];
    }
    // slots past the pass use token 0 / pair 0 (computed, never stored)
    if (tid < kFwTok) {
      const int p = tid < ntok ? lp : 0;
      spair[tid] = p;
      srow[tid] = FC == 1 ? (tid < ntok ? lt : 0) : p;
    }
    // weights of chunks 0..2, then (fc2) the pairs' maxima and the
    // activations of chunks 0 and 1, all in flight together
    const uint8_t *wr, *sr;
    wrow(0, wr, sr);
    load_w(wr, sr, 0, wb[0]);
    load_w(wr, sr, 1, wb[1]);
    load_w(wr, sr, 2, wb[2]);
    lds_barrier();
#pragma unroll
    for (int i = 0; i < kFwVec; ++i) {
      const int slot = kFwSlotsPerVec * i + tid / kFwRowThreads;
      sval[i] = slot < ntok;
      abase[i] = (int64_t)srow[slot] * K;
    }
    stage_load(0, stg[0]);
    stage_load(1, stg[1]);
    stage_load(2, stg[2]);
    if constexpr (FC == 2) {
      // each slot's exponent e and the factors of its fc1 row tiles
      // (d = et - e <= 0; d > 0 only for an all-zero tile; factors below
      // FP16's range are 0)
      for (int idx = tid; idx < kFwTok * nt1; idx += kFwThreads) {
        const int t = idx / kFwTok, slot = idx - t * kFwTok;
        const int p = spair[slot];
        const int ex = exponent_of(pmax[p]);
        int d = etile[(int64_t)p * nt1 + t] - ex;
        d = d > 0 ? 0 : d;
        sfac[t][slot] = d < -24 ? (_Float16)0.0f : (_Float16)__builtin_ldexpf(1.0f, d);
        if (t == 0) sexp[slot] = ex;
      }
      lds_barrier();
    }
    stage_store(0, stg[0], xs[0], ntt);
    lds_barrier();
    // chunk c of a tile uses weight and staging register buffers c % 4 and
    // LDS buffer c % 2 (nchp is a multiple of four, so this holds across
    // tiles).  Step c loads the activations and the weights of chunk c + 3,
    // past the tile's end those of the next tile (of this one past the last:
    // re-read, unused), so both have two steps of other work before use.
    for (int ti = 0; ti < ntile; ++ti) {
      const uint8_t *wn, *sn;
      wrow(ti + 1 < ntile ? ti + 1 : ti, wn, sn);
      auto step = [&](int c, auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        stage_load(c + 3 < nchp ? c + 3 : c + 3 - nchp, stg[(j + 3) % kFwWBuf]);
        const bool nx = c + 3 >= nchp;
        load_w(nx ? wn : wr, nx ? sn : sr, nx ? c + 3 - nchp : c + 3, wb[(j + 3) % kFwWBuf]);
        compute(c, xs[j & 1], wb[j], ntt);
        stage_store(c + 1 < nchp ? c + 1 : 0, stg[(j + 1) % kFwWBuf], xs[(j + 1) & 1], ntt);
        lds_barrier();
      };
      for (int c = 0; c < nchp; c += kFwWBuf) {
        step(c, IntC<0>{});
        step(c + 1, IntC<1>{});
        step(c + 2, IntC<2>{});
        step(c + 3, IntC<3>{});
      }
      epilogue(ti, ntok, ntt);
      wr = wn;
      sr = sn;
    }
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

}  // namespace

size_t moe_workspace_bytes(int tokens, int experts, int top_k, int hidden, int inter) {
  const size_t P = (size_t)tokens * top_k;
  const size_t ET = (size_t)experts * tokens;
  return 3 * align256(P * 4) + align256((size_t)experts * 4) + 2 * align256(ET * 4) +
         align256(P * fc1_tiles(inter) * 4) + align256(P * inter * 2) + align256(P * hidden * 4);
}

// Row tiles per workgroup.  One while the (expert, row tile) units number
// less than four per workgroup slot: smaller units finish the layer in fewer
// unit-lengths (for the 64-expert, 2048-row fc2 layer, 512 units of one tile
// beat 256 of two by ~3 us); beyond that, R tiles streamed back to back share
// one prologue.
static int tiles_per_wg(int experts, int n, int num_cus) {
  const int units = experts * ((n + kFwRows - 1) / kFwRows);
  const int slots = num_cus * kFwPerCU;
  int r = slots > 0 ? units / (2 * slots) : 1;
  return r < 1 ? 1 : (r > 8 ? 8 : r);
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
hipError_t moe_noalloc_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDev = 64;
  static std::once_flag once[kMaxDev];
  static void* addr[kMaxDev];
  static hipError_t err[kMaxDev];
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev]() {
    void* p = nullptr;
    err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    addr[dev] = (err[dev] == hipSuccess) ? p : nullptr;
  });
  if (err[dev] != hipSuccess) return err[dev];
  *ptr = addr[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}

hipError_t launch_moe(const MoeArgs& m, hipStream_t s) {
  const int P = m.tokens * m.top_k;
  MoeWs ws = carve(m.workspace, m.tokens, m.experts, P, m.hidden, m.inter);
  const int nt1 = fc1_tiles(m.inter);
  hipLaunchKernelGGL(moe_route, dim3((m.tokens + 3) / 4), dim3(256), 0, s, m.logits, m.bias,
                     m.tokens, m.experts, m.top_k, m.n_group, m.topk_group, m.norm, m.scaling,
                     ws.ids, ws.wts, ws.pmax, m.ids_out, m.w_out);
  hipLaunchKernelGGL(moe_lists, dim3(m.experts), dim3(kListThreads), 0, s, ws.ids, P, m.tokens,
                     m.top_k, ws.plists, ws.tlists, ws.counts);
  const int zs = (m.tokens + kFwTok - 1) / kFwTok < kFwMaxZ ? (m.tokens + kFwTok - 1) / kFwTok : kFwMaxZ;
  const int r1 = tiles_per_wg(m.experts, m.inter, m.num_cus);
  const int r2 = tiles_per_wg(m.experts, m.hidden, m.num_cus);
  hipLaunchKernelGGL(moe_fc_wide<1>, dim3((nt1 + r1 - 1) / r1, m.experts, zs), dim3(kFwThreads), 0, s,
                     reinterpret_cast<const _Float16*>(m.x), ws.plists, ws.tlists, ws.counts,
                     m.tokens, ws.pmax, ws.etile, nt1, m.w1, m.w1_sf, m.w1_g, m.inter, m.hidden, r1,
                     reinterpret_cast<void*>(ws.h));
  const int t2 = (m.hidden + kFwRows - 1) / kFwRows;
  hipLaunchKernelGGL(moe_fc_wide<2>, dim3((t2 + r2 - 1) / r2, m.experts, zs), dim3(kFwThreads), 0, s,
                     ws.h, ws.plists, ws.tlists, ws.counts, m.tokens, ws.pmax, ws.etile, nt1, m.w2,
                     m.w2_sf, m.w2_g, m.hidden, m.inter, r2, reinterpret_cast<void*>(ws.o));
  hipLaunchKernelGGL(moe_combine4, dim3(m.tokens, (m.hidden + 1023) / 1024), dim3(256), 0, s, ws.o,
                     ws.wts, m.top_k, m.hidden, reinterpret_cast<_Float16*>(m.out));
  return hipGetLastError();
}

}  // namespace nvfp4
