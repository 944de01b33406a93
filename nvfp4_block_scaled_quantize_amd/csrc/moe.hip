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
//  3. fc1        : units of (expert, 128 weight rows, pass of up to 64 of
//                  the expert's tokens), four waves each,
//                  v_mfma_f32_32x32x16_f16 with weights dequantized in
//                  registers (exact in FP16); operands copied global -> LDS
//                  by global_load_lds, several 64-k stages ahead.
//                  h = relu(x . W1^T * g1)^2 is stored as FP16 scaled by
//                  2^-et per (pair, 128-row tile), et the exponent of the
//                  tile's largest h; the pair's overall largest h is an
//                  integer max of fp32 bits (order independent).
//                  Weights in the plain [E, N, K/2] layout or pre-tiled
//                  (nvfp4_pretile_weight of the stacked [E N, K] matrix), in
//                  which each 64-k stage of a unit is whole cache lines.
//  4. fc2        : the same units on h.  The activations of each 128-k
//                  range (one fc1 tile) are multiplied by 2^(et - e) in FP16,
//                  e = exponent of the pair's largest h; o = acc * g2 * 2^e
//                  in fp32 per pair.
//  5. combine    : out[t] = sum_j w[t,j] * o[t*top_k + j] in rank order, FP16.
#include "device_common.h"
#include "internal.h"
#include "lds_dma.h"
#include "../../include/nvfp4_mi355x.h"

#include <mutex>
#include <type_traits>

// Fixed device scratch of nvfp4_moe_w4a16_noalloc, for callers that cannot
// allocate.  Each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` is only a host-side stand-in: the
// device address comes from moe_noalloc_scratch() below and is what the
// kernels receive.
static __device__ __align__(256) unsigned char scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

namespace nvfp4 {

namespace {

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// fc1 row tiles: the granularity of the per-tile exponents of h (etile)
constexpr int kFc1Rows = 128;

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

int fc1_tiles(int inter) { return (inter + kFc1Rows - 1) / kFc1Rows; }

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
// Evaluated with bitwise operations, so it compiles to compares and mask
// operations without branches.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return (va > vb) | ((va == vb) & (ia < ib));
}

constexpr int kMaxExpertsPerLane = 4;   // experts <= 256

// One token per workgroup of one wave; lane l holds experts l + 64 i.  Each
// selection counts, for every contender, how many others come before it in
// the (value desc, index asc) order -- the same order as taking repeated
// maxima with ties to the lower index -- so no serial chain of cross-lane
// reductions is needed.  The comparisons are branch-free and the LDS reads of
// a phase do not depend on one another, so each phase's reads are issued
// together; the kept groups travel as ballot masks.
__global__ void __launch_bounds__(64)
moe_route(const float* __restrict__ logits, const float* __restrict__ bias, int T, int E,
          int top_k, int n_group, int topk_group, int norm, float scaling,
          int32_t* __restrict__ ids, float* __restrict__ wts, uint32_t* __restrict__ pmax,
          int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  __shared__ float sb[64 * kMaxExpertsPerLane];   // biased scores
  __shared__ float sg[64 * kMaxExpertsPerLane];   // group scores
  __shared__ float cb[64 * kMaxExpertsPerLane];   // candidates (experts of kept groups): biased score
  __shared__ int ce[64 * kMaxExpertsPerLane];     // ... and expert index, in expert order
  __shared__ int sel_e[16];                       // chosen experts by rank
  __shared__ float sel_s[16];                     // their unbiased scores
  const int lane = threadIdx.x;
  const int t = blockIdx.x;
  if (t >= T) return;   // whole workgroup
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
      sb[e] = b[i];
    } else {
      s[i] = 0.0f;
      b[i] = ninf;
    }
  }
  __syncthreads();
  // group scores: lane g sums its group's two best biased scores (one if the
  // group has one expert)
  float gs[kMaxExpertsPerLane];
#pragma unroll
  for (int i = 0; i < kMaxExpertsPerLane; ++i) {
    const int g = lane + 64 * i;
    gs[i] = ninf;
    if (g < n_group) {
      float v1 = ninf, v2 = ninf;
      int i1 = -1, i2 = -1;
      const int e0 = g * gsize;
#pragma unroll 8
      for (int j = 0; j < gsize; ++j) {
        const int e = e0 + j;
        const float v = sb[e];
        const bool n1 = (i1 < 0) | better(v, e, v1, i1);
        const bool n2 = !n1 & ((i2 < 0) | better(v, e, v2, i2));
        v2 = n1 ? v1 : (n2 ? v : v2);
        i2 = n1 ? i1 : (n2 ? e : i2);
        v1 = n1 ? v : v1;
        i1 = n1 ? e : i1;
      }
      gs[i] = (i2 >= 0) ? v1 + v2 : v1;
      if (gs[i] != gs[i]) gs[i] = ninf;   // +inf + -inf: a NaN group score ranks below every number
      sg[g] = gs[i];
    }
  }
  __syncthreads();
  // a group is kept when fewer than topk_group groups come before it
  uint64_t kmask[kMaxExpertsPerLane];
#pragma unroll
  for (int i = 0; i < kMaxExpertsPerLane; ++i) {
    const int g = lane + 64 * i;
    bool kept = false;
    if (g < n_group) {
      int r = 0;
#pragma unroll 8
      for (int g2 = 0; g2 < n_group; ++g2) r += better(sg[g2], g2, gs[i], g) ? 1 : 0;
      kept = r < topk_group;
    }
    kmask[i] = __ballot(kept);
  }
  // compact the candidates in expert order
  const uint64_t below = (1ull << lane) - 1ull;
  int nc = 0;
  bool cand[kMaxExpertsPerLane];
#pragma unroll
  for (int i = 0; i < kMaxExpertsPerLane; ++i) {
    const int e = lane + 64 * i;
    const int g = e / gsize;
    const uint64_t km = g < 64 ? kmask[0] : g < 128 ? kmask[1] : g < 192 ? kmask[2] : kmask[3];
    cand[i] = (e < E) && ((km >> (g & 63)) & 1ull);
    const uint64_t m = __ballot(cand[i]);
    const int pos = nc + __popcll(m & below);
    if (cand[i]) { cb[pos] = b[i]; ce[pos] = e; }
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
      for (int c = 0; c < nc; ++c) r += better(cb[c], ce[c], b[i], e) ? 1 : 0;
      if (r < top_k) { sel_e[r] = e; sel_s[r] = s[i]; }
    }
  }
  __syncthreads();
  // normalize in rank order (every lane forms the same sequential sum), then scale
  float sum = 0.0f;
#pragma unroll 8
  for (int k = 0; k < top_k; ++k) sum = sum + sel_s[k];
  if (lane < top_k) {
    const float wsel = sel_s[lane];
    const int isel = sel_e[lane];
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

// Expert FFN layers (fc1, fc2).  A unit of work is (expert e, tile of 128
// weight rows, pass of up to 64 of the expert's tokens); an expert with more
// tokens is cut into balanced passes.  Workgroups are small (four waves,
// about 52 KiB of LDS), so three run on each compute unit and the hardware
// dispatcher spreads the many short units evenly; the units of one expert
// are dispatched next to each other on one XCD (its activations, and for
// several passes its weight rows, are then read from that XCD's L2).
// Wave w computes the weight rows 32 w .. 32 w + 31 of the tile
// (v_mfma_f32_32x32x16_f16, weights as the A operand, dequantized in
// registers -- exact in FP16) for every 32-token tile of the pass.
//
// K goes in 64-k stages copied global -> LDS by global_load_lds into two
// rings: waves 0-1 copy the weights (FP4 codes 32 B and E4M3 bytes 4 B per
// row and stage) through a 5-stage ring whose first four stages are issued
// before the token count is read; waves 2-3 gather the FP16 token rows
// (128 B per token and stage; 64-bit addresses) through a 6-stage ring for
// one token tile, 3 for two.  Each wave's copies are the same for every
// stage, so its vector-memory counter waits are exact; one barrier per stage
// publishes both.  LDS layouts (16 consecutive lanes of an operand read hit
// 16 distinct bank groups, and 8 lanes 8):
//   codes: 32 B per row, piece j of row r at j ^ (((r >> 2) ^ (r >> 3)) & 1);
//   E4M3 bytes: 4 B per row;
//   TW (weights in the pre-tiled layout of nvfp4_pretile_weight, applied to
//   the stacked [E N, K] matrix: per 16-row group and 128-k chunk 1 KiB of
//   codes, lane l = r + 16 g holding row r, k = 32 g .. 32 g + 31, and 128 B
//   of E4M3 pairs in the same lane order): a stage is the half of each of
//   its eight groups' tiles, 512 B of codes and 64 B of E4M3 bytes each,
//   copied as they are (a stage is then 36 whole cache lines instead of
//   touching 128 rows' lines twice): codes piece h of row r at
//   32 (r / 16) + 16 h + r % 16, the pair of bytes at 64 (r / 16) + 32 h +
//   2 (r % 16);
//   activations: 128 B per token slot, piece j of slot s at (j + rot(s)) mod
//   8, rot(s) = s + (s / 8) mod 4 (the same for slots s and s + 32) -- a
//   lane's four pieces of a stage are its slot base plus a constant, minus
//   128 B past the wrap.
// Lane (row r32, half h) owns the 32 k at 32 h of a stage: MFMA m of a stage
// takes k = 32 h + 8 m .. + 7 from both operands.  Requires K % 64 == 0,
// N % 64 == 0 and N K / 2 < 2^32.
// FC = 1: act = x [T, K] (row = token).  out = h [P, N] FP16 with, per pair
//         and 128-row tile, h scaled by 2^-et (et = exponent of the tile's
//         largest h, stored in etile [P, nt1]); pmax[p] = largest h (fp32
//         bits, integer max: order independent).
// FC = 2: act = h [P, K].  The activation fragments of each 128-k range (one
//         fc1 row tile) are multiplied by 2^(et - e) in FP16 before the
//         MFMA, e = exponent of pmax[p], so the pair's values share one scale
//         and none can overflow FP16 (values below 2^-24 of the pair's
//         largest h flush to zero).  out = o [P, N] fp32 = acc * g * 2^e.
constexpr int kMfThreads = 256;            // four waves
constexpr int kMfRows = 128;               // weight rows per tile (32 per wave)
constexpr int kMfKC = 64;                  // k per stage
constexpr int kMfMaxT = 2;                 // 32-token tiles per pass
constexpr int kMfTok = 32 * kMfMaxT;       // tokens per pass at most
constexpr int kMfCodeB = kMfRows * kMfKC / 2;        // 4096
constexpr int kMfWB = kMfCodeB + kMfRows * kMfKC / 16;   // codes + E4M3 bytes per stage
constexpr int kMfTileB = 32 * kMfKC * 2;   // activations of one token tile per stage
constexpr int kMfWBufs = 5;                // weight ring
constexpr int kMfABufs1 = 6, kMfABufs2 = 3;   // activation ring for one / two token tiles
constexpr int kMfMaxT1 = 8192 / kMfRows;   // fc1 row tiles (inter <= 8192)
constexpr int kMfMaxZ = 1024;              // passes in the grid (more handled in a loop)
constexpr int kMfWOps = 3;                 // weight copies per copying thread and stage
static_assert(kMfABufs1 * kMfTileB == kMfABufs2 * 2 * kMfTileB, "one activation ring size");
static_assert(kMfCodeB == 2 * 16 * 128 && kMfRows * 4 == 4 * 128, "weight copies: waves 0-1");

__device__ __forceinline__ int exponent_of(uint32_t bits) {
  return bits == 0u ? 0 : (int)((bits >> 23) & 0xFFu) - 127;
}

// s_waitcnt vmcnt(n) for a run-time n in [0, 23] (larger n: 23, which waits
// at least as long).
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
  switch (n) {
#define NVFP4_WCASE(i) case i: wait_vmcnt_le<i>(); break;
    NVFP4_WCASE(0) NVFP4_WCASE(1) NVFP4_WCASE(2) NVFP4_WCASE(3) NVFP4_WCASE(4) NVFP4_WCASE(5)
    NVFP4_WCASE(6) NVFP4_WCASE(7) NVFP4_WCASE(8) NVFP4_WCASE(9) NVFP4_WCASE(10) NVFP4_WCASE(11)
    NVFP4_WCASE(12) NVFP4_WCASE(13) NVFP4_WCASE(14) NVFP4_WCASE(15) NVFP4_WCASE(16)
    NVFP4_WCASE(17) NVFP4_WCASE(18) NVFP4_WCASE(19) NVFP4_WCASE(20) NVFP4_WCASE(21)
    NVFP4_WCASE(22)
#undef NVFP4_WCASE
    default: wait_vmcnt_le<23>(); break;
  }
}

template <int FC, bool TW>
__global__ void __launch_bounds__(kMfThreads, 3)
moe_fc(const _Float16* __restrict__ act, const int32_t* __restrict__ plists,
       const int32_t* __restrict__ tlists, const int32_t* __restrict__ counts, int T,
       uint32_t* __restrict__ pmax, int32_t* __restrict__ etile, int nt1, int tiles,
       const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_sf,
       const float* __restrict__ w_g, int N, int K, void* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kMfWBufs * kMfWB + kMfABufs1 * kMfTileB];
  __shared__ int srow[kMfTok];     // activation row of each token slot of the pass
  __shared__ int spair[kMfTok];    // its pair
  __shared__ int scnt;             // the expert's token count
  __shared__ int sexp[FC == 2 ? kMfTok : 1];                    // fc2: exponent e of the pair's largest h
  __shared__ signed char sdif[FC == 2 ? kMfMaxT1 : 1][kMfTok];  // fc2: et - e per fc1 row tile
  __shared__ float redmax[FC == 1 ? 4 : 1][kMfTok];             // fc1: largest h per wave

  // grid x = (pass, row tile), y = expert; the workgroups of one expert run
  // on one XCD (consecutive workgroup ids go to consecutive XCDs), its passes
  // of one row tile one XCD round apart
  int bxz = blockIdx.x, e = blockIdx.y;
  if ((gridDim.y & 7) == 0) {
    const int L = blockIdx.x + gridDim.x * blockIdx.y;
    const int slot = L >> 3;
    bxz = slot % gridDim.x;
    e = (slot / gridDim.x) * 8 + (L & 7);
  }
  const int bx = bxz % tiles, z0 = bxz / tiles, zs = gridDim.x / tiles;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool wcopy = wave < 2;                   // waves 0-1 copy weights, 2-3 activations
  const int ct = tid & 127;                      // index among the copying threads
  const int r32 = lane & 31, h = lane >> 5;
  const int nst = K / kMfKC;
  const int n0 = bx * kMfRows;
  const uint8_t* we = w + (int64_t)e * N * (K / 2);
  const uint8_t* se = w_sf + (int64_t)e * N * (K / 16);
  const uint32_t l0 = lds_addr(lds);
  const uint32_t la = l0 + kMfWBufs * kMfWB;     // activation ring
  const float ge = w_g[e];

  // weight copies (waves 0-1): code copy i fills LDS piece i * 128 + ct of
  // the stage (row (i * 128 + ct) / 2), the E4M3 copy the dword of row ct;
  // rows past N re-read row N - 1 (their results are not stored)
  uint32_t cofs[2], sofs;
  constexpr uint32_t kCStep = TW ? 512u : 32u, kSStep = TW ? 64u : 4u;   // bytes per stage
  if constexpr (TW) {
    // piece i * 128 + ct of the stage: group G = piece / 32, tile lane
    // 32 (c % 2) + piece % 32; the stage's offset in a tile is 512 c mod
    // 1 KiB plus 1 KiB per chunk, i.e. 512 c (64 c for the E4M3 pairs).
    // Groups past N re-read the last group (their results are not stored).
    const uint32_t nch2 = (uint32_t)(K / 128), gl = (uint32_t)(N / 16 - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pos = i * 128 + ct;
      const uint32_t gg = (uint32_t)(n0 / 16 + (pos >> 5));
      cofs[i] = (gg < gl ? gg : gl) * nch2 * 1024u + 16u * (uint32_t)(pos & 31);
    }
    const uint32_t gs = (uint32_t)(n0 / 16 + (ct >> 4));
    sofs = (gs < gl ? gs : gl) * nch2 * 128u + 4u * (uint32_t)(ct & 15);
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pos = i * 128 + ct, r = pos >> 1;
      const int j = (pos & 1) ^ (((r >> 2) ^ (r >> 3)) & 1);
      const uint32_t n = (uint32_t)(n0 + r < N ? n0 + r : N - 1);
      cofs[i] = n * (uint32_t)(K / 2) + 16u * j;
    }
    sofs = (uint32_t)(n0 + ct < N ? n0 + ct : N - 1) * (uint32_t)(K / 16);
  }
  auto issue_w = [&](int c) __attribute__((always_inline)) {
    const uint32_t lb = l0 + (c % kMfWBufs) * kMfWB;
    dma16(we, cofs[0] + kCStep * c, lb + 16 * (0 * 128 + 64 * wave));
    dma16(we, cofs[1] + kCStep * c, lb + 16 * (1 * 128 + 64 * wave));
    dma4(se, sofs + kSStep * c, lb + kMfCodeB + 4 * 64 * wave);
  };

  const bool first_z = z0 == 0;
  // the weights of the first stages depend on nothing else: in flight before
  // the token count is known (a z > 0 workgroup is usually idle: it waits)
  if (first_z && wcopy) {
    for (int c = 0; c < kMfWBufs - 1 && c < nst; ++c) issue_w(c);
  }
  // the count, the lists and (fc2) the exponents are read by waves 2-3 only:
  // a load of waves 0-1 would make the compiler wait for their copies
  const int32_t* pl = plists + (int64_t)e * T;
  const int32_t* tl = tlists + (int64_t)e * T;
  // the first pass starts at the list head: wave 2 reads it together with
  // the count (entries past the count are never used)
  int hp = 0, ht = 0;
  if (z0 == 0 && wave == 2) {
    const int i = lane < T ? lane : T - 1;
    hp = pl[i];
    if (FC == 1) ht = tl[i];
  }
  if (tid == 128) scnt = counts[e];
  lds_barrier();
  const int cnt = scnt;
  const int np = (cnt + kMfTok - 1) / kMfTok;   // passes
  if (z0 >= np) {
    wait_vmcnt_le<0>();   // no copy into LDS outlives the workgroup
    return;
  }
  // operand read offsets (bytes within a stage buffer)
  const int r = 32 * wave + r32;
  // code piece h of row r; the E4M3 dword of row r (plain) or its pair for
  // this lane's 32 k (TW)
  const uint32_t ca = TW ? 16u * (32 * (r >> 4) + 16 * h + (r & 15))
                         : 16u * (2 * r + (h ^ (((r >> 2) ^ (r >> 3)) & 1)));
  const uint32_t sa = TW ? kMfCodeB + 64u * (r >> 4) + 32u * h + 2u * (r & 15) : kMfCodeB + 4u * r;
  const int rot = (r32 + ((r32 >> 3) & 3)) & 7;  // rotation of slots r32 and 32 + r32
  const int b4 = (4 * h + rot) & 7;              // position of the lane's first piece
  const uint32_t ab0 = 128u * r32 + 16u * b4;    // slot r32 of tile 0, piece 4h
  typedef const __attribute__((address_space(3))) unsigned char* lptr;

  for (int z = z0; z < np; z += zs) {
    const bool wpre = first_z && z == z0;   // the first weight stages are issued
    // balanced passes: the first cnt % np passes take one token more
    const int base = cnt / np, rem = cnt % np;
    const int ntok = base + (z < rem ? 1 : 0);
    const int t0 = z * base + (z < rem ? z : rem);
    const int ntt = (ntok + 31) / 32;                    // token tiles of the pass
    if (z != z0) lds_barrier();   // the previous pass is done with the LDS
    // slots past the pass take the pass's first token (computed, never stored)
    if (wave == 2) {
      int p, t;
      if (z == 0) {
        const int p0 = __shfl(hp, 0, 64), t0h = __shfl(ht, 0, 64);
        p = lane < ntok ? hp : p0;
        t = lane < ntok ? ht : t0h;
      } else {
        const int idx = t0 + (lane < ntok ? lane : 0);
        p = pl[idx];
        t = FC == 1 ? tl[idx] : 0;
      }
      spair[lane] = p;
      srow[lane] = FC == 1 ? t : p;
    }
    lds_barrier();
    if constexpr (FC == 2) {
      // each slot's exponent e and, per fc1 row tile, et - e (> 0 only for an
      // all-zero tile, whose products are zero: clamped to 0)
      if (!wcopy) {
        for (int idx = ct; idx < kMfTok * nt1; idx += 128) {
          const int t = idx / kMfTok, slot = idx - t * kMfTok;
          const int p = spair[slot];
          const int ex = exponent_of(pmax[p]);
          int d = etile[(int64_t)p * nt1 + t] - ex;
          d = d > 0 ? 0 : (d < -126 ? -126 : d);
          sdif[t][slot] = (signed char)d;
          if (t == 0) sexp[slot] = ex;
        }
      }
    }
    // everything below is instantiated for one and for two token tiles, so
    // the accumulators stay in the same registers through the stage loop
    auto run = [&](auto nc) __attribute__((always_inline)) {
    constexpr int NTT = nc;
    constexpr int abufs = NTT == 1 ? kMfABufs1 : kMfABufs2;
    constexpr uint32_t abuf = NTT * kMfTileB;
    // activation copies (waves 2-3): copy i fills LDS piece i * 128 + ct of
    // the stage (slot (i * 128 + ct) / 8; the slot's piece (ct - rot) mod 8)
    const _Float16* aptr[2 * kMfMaxT];
#pragma unroll
    for (int i = 0; i < 2 * kMfMaxT; ++i) {
      const int pos = i * 128 + ct, s = pos >> 3;
      const int j = ((pos & 7) - (s + ((s >> 3) & 3))) & 7;
      aptr[i] = act + (int64_t)srow[s < kMfTok ? s : 0] * K + 8 * j;
    }
    auto issue_a = [&](int c) __attribute__((always_inline)) {
      const uint32_t lb = la + (c % abufs) * abuf;
#pragma unroll
      for (int i = 0; i < 2 * kMfMaxT; ++i)
        if (i < 2 * NTT) dma16_at(aptr[i] + kMfKC * c, lb + 16 * (i * 128 + 64 * (wave - 2)));
    };
    if (wcopy) {
      if (!wpre)
        for (int c = 0; c < kMfWBufs - 1 && c < nst; ++c) issue_w(c);
    } else {
      for (int c = 0; c < abufs - 1 && c < nst; ++c) issue_a(c);
    }
    if constexpr (FC == 2) lds_barrier();   // sexp / sdif written

    v16f acc[kMfMaxT];
#pragma unroll
    for (int i = 0; i < kMfMaxT; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][q] = 0.0f;
    _Float16 fac[kMfMaxT];   // fc2: factors of the current 128-k range

    auto compute = [&](uint32_t st, uint32_t sta, auto nwc) __attribute__((always_inline)) {
      constexpr int NW = nwc;
      // per-stage bases kept opaque, so every operand read below is a base
      // plus an immediate; all of the stage's reads are issued before the
      // first dequantization (the scheduling barrier keeps them there)
      uint32_t bw = st, b0 = sta + ab0, b1 = b0 - 128u;
      asm volatile("" : "+v"(bw), "+v"(b0), "+v"(b1));
      const lptr pw = (lptr)(uintptr_t)bw;
      const u32x4 cw = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(pw + ca);
      uint32_t sw;
      if constexpr (TW) sw = *reinterpret_cast<const __attribute__((address_space(3))) uint16_t*>(pw + sa);
      else sw = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(pw + sa);
      v8h bf[4][NW];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const lptr pa = (lptr)(uintptr_t)(m < 8 - b4 ? b0 : b1);
#pragma unroll
        for (int i = 0; i < NW; ++i)
          bf[m][i] = *reinterpret_cast<const __attribute__((address_space(3))) v8h*>(pa + 16 * m + 32 * 128 * i);
      }
      __builtin_amdgcn_sched_barrier(0);
      // this lane's two 16-blocks: bytes 2h and 2h + 1 of the row's dword
      // (TW: the pair itself)
      const uint32_t sh = TW ? sw : sw >> (16 * h);
      const _Float16 s0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)sh, 0);
      const _Float16 s1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)sh, 1);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const v8h a = dequant8_w(cw[m], m < 2 ? s0 : s1);
#pragma unroll
        for (int i = 0; i < NW; ++i) {
          v8h b = bf[m][i];
          if constexpr (FC == 2) {
            const v2h f2 = {fac[i], fac[i]};
            v2h* pb = reinterpret_cast<v2h*>(&b);
            pb[0] = pb[0] * f2; pb[1] = pb[1] * f2; pb[2] = pb[2] * f2; pb[3] = pb[3] * f2;
          }
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[i], 0, 0, 0);
        }
      }
    };

    for (int c = 0; c < nst; ++c) {
      // this wave's copies of stage c landed: at most those of the stages
      // issued after it remain
      if (wcopy) {
        const int k = (nst - 1 - c) < kMfWBufs - 2 ? nst - 1 - c : kMfWBufs - 2;
        wait_vmcnt_rt(k * kMfWOps);
      } else {
        const int k = (nst - 1 - c) < abufs - 2 ? nst - 1 - c : abufs - 2;
        wait_vmcnt_rt(k * 2 * NTT);
      }
      lds_barrier();   // every copy of stage c landed; stage c - 1 is no longer read
      if (wcopy) {
        if (c + kMfWBufs - 1 < nst) issue_w(c + kMfWBufs - 1);
      } else {
        if (c + abufs - 1 < nst) issue_a(c + abufs - 1);
      }
      if constexpr (FC == 2) {
        if ((c & 1) == 0) {   // a new 128-k range: fc1 row tile c / 2
#pragma unroll
          for (int i = 0; i < kMfMaxT; ++i) {
            const int d = sdif[c >> 1][32 * i + r32];
            fac[i] = d < -24 ? (_Float16)0.0f : (_Float16)__builtin_ldexpf(1.0f, d);
          }
        }
      }
      const uint32_t st = l0 + (c % kMfWBufs) * kMfWB, sta = la + (c % abufs) * abuf;
      compute(st, sta, nc);
    }

    // results: acc[i][q] = weight row n0 + 32 wave + 8 (q / 4) + 4 h + q % 4,
    // token slot 32 i + r32
    const bool rv = n0 + 32 * wave < N;   // N % 64 == 0: a wave's 32 rows are all in or all out
    if constexpr (FC == 1) {
#pragma unroll
      for (int i = 0; i < kMfMaxT; ++i) {
        if (i < ntt) {
          float mx = 0.0f;
#pragma unroll
          for (int q = 0; q < 16; ++q) mx = __builtin_fmaxf(mx, relu2_f32(acc[i][q] * ge));
          if (!rv) mx = 0.0f;
          mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, 64));
          if (h == 0) redmax[wave][32 * i + r32] = mx;
        }
      }
      lds_barrier();
#pragma unroll
      for (int i = 0; i < kMfMaxT; ++i) {
        const int slot = 32 * i + r32;
        if (i < ntt && slot < ntok) {
          const float tmax = __builtin_fmaxf(__builtin_fmaxf(redmax[0][slot], redmax[1][slot]),
                                             __builtin_fmaxf(redmax[2][slot], redmax[3][slot]));
          const int ex = exponent_of(__float_as_uint(tmax));
          const float sc = __builtin_ldexpf(1.0f, -ex);
          const int p = spair[slot];
          if (rv) {
            _Float16* hp = reinterpret_cast<_Float16*>(out) + (int64_t)p * N + n0 + 32 * wave + 4 * h;
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
              v4h o4;
              o4[0] = (_Float16)(relu2_f32(acc[i][4 * qd + 0] * ge) * sc);
              o4[1] = (_Float16)(relu2_f32(acc[i][4 * qd + 1] * ge) * sc);
              o4[2] = (_Float16)(relu2_f32(acc[i][4 * qd + 2] * ge) * sc);
              o4[3] = (_Float16)(relu2_f32(acc[i][4 * qd + 3] * ge) * sc);
              *reinterpret_cast<v4h*>(hp + 8 * qd) = o4;
            }
          }
          if (wave == 0 && h == 0) {
            etile[(int64_t)p * nt1 + bx] = ex;
            atomicMax(pmax + p, __float_as_uint(tmax));
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kMfMaxT; ++i) {
        const int slot = 32 * i + r32;
        if (i < ntt && slot < ntok && rv) {
          const float scale = __builtin_ldexpf(ge, sexp[slot]);
          float* op = reinterpret_cast<float*>(out) + (int64_t)spair[slot] * N + n0 + 32 * wave + 4 * h;
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            float4 v;
            v.x = acc[i][4 * qd + 0] * scale;
            v.y = acc[i][4 * qd + 1] * scale;
            v.z = acc[i][4 * qd + 2] * scale;
            v.w = acc[i][4 * qd + 3] * scale;
            *reinterpret_cast<float4*>(op + 8 * qd) = v;
          }
        }
      }
    }
    };
    if (ntt == 2) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 1>{});
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
  // one wave (one token) per workgroup
  hipLaunchKernelGGL(moe_route, dim3(m.tokens), dim3(64), 0, s, m.logits, m.bias,
                     m.tokens, m.experts, m.top_k, m.n_group, m.topk_group, m.norm, m.scaling,
                     ws.ids, ws.wts, ws.pmax, m.ids_out, m.w_out);
  hipLaunchKernelGGL(moe_lists, dim3(m.experts), dim3(kListThreads), 0, s, ws.ids, P, m.tokens,
                     m.top_k, ws.plists, ws.tlists, ws.counts);
  // fc1 and fc2: 128-row tiles x passes of up to 64 tokens; grid x = (pass,
  // row tile), y = expert
  const int zt = (m.tokens + kMfTok - 1) / kMfTok;
  const int zs = zt < kMfMaxZ ? zt : kMfMaxZ;
  const int t1 = (m.inter + kMfRows - 1) / kMfRows, t2 = (m.hidden + kMfRows - 1) / kMfRows;
  auto fc1 = m.tiled_weights ? moe_fc<1, true> : moe_fc<1, false>;
  auto fc2 = m.tiled_weights ? moe_fc<2, true> : moe_fc<2, false>;
  hipLaunchKernelGGL(fc1, dim3(t1 * zs, m.experts), dim3(kMfThreads), 0, s,
                     reinterpret_cast<const _Float16*>(m.x), ws.plists, ws.tlists, ws.counts, m.tokens,
                     ws.pmax, ws.etile, nt1, t1, m.w1, m.w1_sf, m.w1_g, m.inter, m.hidden,
                     reinterpret_cast<void*>(ws.h));
  hipLaunchKernelGGL(fc2, dim3(t2 * zs, m.experts), dim3(kMfThreads), 0, s, ws.h, ws.plists,
                     ws.tlists, ws.counts, m.tokens, ws.pmax, ws.etile, nt1, t2, m.w2, m.w2_sf, m.w2_g,
                     m.hidden, m.inter, reinterpret_cast<void*>(ws.o));
  hipLaunchKernelGGL(moe_combine4, dim3(m.tokens, (m.hidden + 1023) / 1024), dim3(256), 0, s, ws.o,
                     ws.wts, m.top_k, m.hidden, reinterpret_cast<_Float16*>(m.out));
  return hipGetLastError();
}

}  // namespace nvfp4
