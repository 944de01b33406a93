// mx_gemm.hip -- MXFP4 variant of the block-scaled GEMM on gfx950's scaled
// MFMA: y[B,N] (fp16) = g_a[row] * g_w * sum_k q_a 2^(e_a-127) q_w 2^(e_w-127),
// with FP4 (E2M1) codes and E8M0 scale bytes over 32-element K-blocks (the
// UE8M0_SF switch of the block helper in "perf: optimize per-token nvfp4
// quantization kernel", review).  v_mfma_scale_f32_32x32x64_f8f6f4 with FP4
// operands on both sides applies one E8M0 byte per lane, i.e. per row and
// 32-k half of its 64-k step, so the E2M1 x E2M1 products and the block
// scales are exact in the instruction and only the fp32 accumulation and the
// final fp16 rounding round.  Measured on gfx950: an 8-pass instruction (one
// every 32 clocks per SIMD); op_sel k picks byte k of a lane's scale register.
//
// Both operands come in the MX tile layout: rows padded to a multiple of 32;
// per (32-row group G, 64-k chunk c) a 1 KiB code tile whose 16-byte lane
// l = r + 32h is exactly the FP4 operand of MFMA lane l (row 32G + r, k =
// 64c + 32h .. +31); per (G, 128-k chunk) a 128 B scale tile whose 2-byte lane
// l holds that lane's E8M0 bytes for the chunk's two 64-k steps (op_sel 0, 1).
// Tiles are stored (G, chunk) row-major, so a group's codes (K*16 bytes) and
// scale bytes (K bytes) are contiguous.  The weight is the MFMA's first
// operand, so each lane's output holds four consecutive columns of a row.
//
//  * mx_gemm_wide (B > 32): 256 x 256 output tiles, four waves of 128 x 128
//    (4 x 4 MFMA blocks, the accumulators in AGPRs), 128-k stages copied
//    global -> LDS by global_load_lds_dwordx4/_dword, four LDS buffers (three
//    stages in flight), one barrier per stage.  Every copy reads whole 1 KiB
//    code tiles / 256 B of scale tiles, and every MFMA operand read is one
//    contiguous 1 KiB ds_read_b128 (no bank conflicts).  The fp16 output goes
//    through LDS so that each store instruction writes whole row segments.
//  * mx_gemm_skinny (B <= 32, decode): one workgroup per 32-row weight group,
//    eight waves splitting K; each wave streams its code and scale tiles
//    straight into registers, all of them issued before the first MFMA, and
//    the eight partial 32 x 32 blocks are summed through LDS.
#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "lds_dma.h"

namespace nvfp4 {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i fp4_operand(u32x4 v) {
  v8i r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  return r;
}

template <int KK>
__device__ __forceinline__ v16f mfma_mx(const v8i& w, const v8i& a, const v16f& acc, uint32_t sw,
                                        uint32_t sa) {
  // format code 4 = FP4 E2M1 for both operands; op_sel KK picks the scale
  // byte of 64-k step KK of the 128-k chunk
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, a, acc, 4, 4, KK, (int)sw, KK, (int)sa);
}

// Four fp16 outputs (consecutive columns) of one row.
__device__ __forceinline__ void store4(_Float16* p, float a, float b, float c, float d, float s) {
  v4h o = {(_Float16)(a * s), (_Float16)(b * s), (_Float16)(c * s), (_Float16)(d * s)};
  *reinterpret_cast<v4h*>(p) = o;
}

// ------------------------------------------------------------ wide (prefill)

constexpr int kMwThreads = 256;
constexpr int kMwTile = 256;                 // rows of each operand per tile
constexpr int kMwWOff = 0;                   // weight codes: [group 8][k-step 2][1 KiB]
constexpr int kMwAOff = 16384;               // activation codes: same
constexpr int kMwWSOff = 32768;              // weight scale tiles: [group 8][128 B]
constexpr int kMwASOff = 32768 + 1024;       // activation scale tiles
constexpr int kMwStage = 32768 + 2048;
constexpr int kMwLoads = 10;                 // copy instructions per wave per stage

__global__ void __launch_bounds__(kMwThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mx_gemm_wide(const uint8_t* __restrict__ a, const uint8_t* __restrict__ as,
             const float* __restrict__ ag, int64_t a_group_rows, const uint8_t* __restrict__ w,
             const uint8_t* __restrict__ ws, const float* __restrict__ wg,
             _Float16* __restrict__ y, int B, int N, int K, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) unsigned char lds0[kMwStage];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[kMwStage];
  __shared__ __attribute__((aligned(16))) unsigned char lds2[kMwStage];
  __shared__ __attribute__((aligned(16))) unsigned char lds3[kMwStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;   // this wave's 128-row halves of the tile
  int tm, tn;
  {
    const int t = blockIdx.x;
    if (tiles_m % 4 == 0 && tiles_n % 8 == 0 && (tiles_m * tiles_n) % 256 == 0) {
      // consecutive ids go to different XCDs; each XCD walks chunks of
      // 4 M-tiles x 8 N-tiles, so its 32 resident workgroups share 4
      // activation and 8 weight row stripes in its L2
      const int xcd = t & 7, l = t >> 3;
      const int chunk = (l >> 5) * 8 + xcd, within = l & 31;
      const int chunks_n = tiles_n / 8;
      tm = (chunk / chunks_n) * 4 + (within & 3);
      tn = (chunk % chunks_n) * 8 + (within >> 2);
    } else {
      tm = t / tiles_n;
      tn = t % tiles_n;
    }
  }
  const int gm0 = tm * (kMwTile / 32), gn0 = tn * (kMwTile / 32);   // first row groups
  const int gm_last = (B + 31) / 32 - 1, gn_last = N / 32 - 1;
  const int nstages = K / 128;

  // Copy work of this wave per stage: code tiles (group 2w + j/2, k-step j%2)
  // of both operands, and the scale tiles of groups 2w, 2w+1 of both.  Groups
  // past the operand's end re-read its last group (their outputs are never
  // stored).  Lane offsets are relative to the tile's first group (< 8 x 16K
  // bytes), the stage offset goes into the 64-bit scalar base.
  uint32_t wofs[4], aofs[4], wsofs, asofs;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int g = 2 * wave + (j >> 1), kk = j & 1;
    const int gw = min(gn0 + g, gn_last), ga = min(gm0 + g, gm_last);
    wofs[j] = (uint32_t)(gw - gn0) * (uint32_t)K * 16u + 1024u * kk + 16u * lane;
    aofs[j] = (uint32_t)(ga - gm0) * (uint32_t)K * 16u + 1024u * kk + 16u * lane;
  }
  {
    const int g = 2 * wave + (lane >> 5);
    const int gw = min(gn0 + g, gn_last), ga = min(gm0 + g, gm_last);
    wsofs = (uint32_t)(gw - gn0) * (uint32_t)K + 4u * (lane & 31);
    asofs = (uint32_t)(ga - gm0) * (uint32_t)K + 4u * (lane & 31);
  }
  const uint8_t* wbase = w + (size_t)gn0 * K * 16;
  const uint8_t* abase = a + (size_t)gm0 * K * 16;
  const uint8_t* wsbase = ws + (size_t)gn0 * K;
  const uint8_t* asbase = as + (size_t)gm0 * K;

  // copy instructions [lo, hi) of stage st (0-3 weight codes, 4-7 activation
  // codes, 8 weight scales, 9 activation scales) into buffer buf
  auto issue_part = [&](unsigned char* buf, int st, int lo, int hi) __attribute__((always_inline)) {
    const uint32_t l0 = lds_addr(buf);
#pragma unroll
    for (int idx = 0; idx < kMwLoads; ++idx) {
      if (idx < lo || idx >= hi) continue;
      if (idx < 4)
        dma16(wbase + (size_t)st * 2048, wofs[idx], l0 + kMwWOff + (4 * wave + idx) * 1024);
      else if (idx < 8)
        dma16(abase + (size_t)st * 2048, aofs[idx - 4], l0 + kMwAOff + (4 * wave + idx - 4) * 1024);
      else if (idx == 8)
        dma4(wsbase + (size_t)st * 128, wsofs, l0 + kMwWSOff + wave * 256);
      else
        dma4(asbase + (size_t)st * 128, asofs, l0 + kMwASOff + wave * 256);
    }
  };
  auto issue = [&](unsigned char* buf, int st) __attribute__((always_inline)) {
    issue_part(buf, st, 0, kMwLoads);
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Operand fragments of one 64-k step (four weight and four activation
  // 32-row blocks) and the scale registers of a stage.
  struct Frags {
    v8i w[4], a[4];
  };
  struct Scales {
    uint32_t w[4], a[4];
  };
  auto read_frags = [&](const unsigned char* st, int kk, Frags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.w[i] = fp4_operand(*reinterpret_cast<const u32x4*>(st + kMwWOff + ((4 * wn + i) * 2 + kk) * 1024 + 16 * lane));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      f.a[j] = fp4_operand(*reinterpret_cast<const u32x4*>(st + kMwAOff + ((4 * wm + j) * 2 + kk) * 1024 + 16 * lane));
  };
  auto read_scales = [&](const unsigned char* st, Scales& c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c.w[i] = *reinterpret_cast<const uint16_t*>(st + kMwWSOff + (4 * wn + i) * 128 + 2 * lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) c.a[j] = *reinterpret_cast<const uint16_t*>(st + kMwASOff + (4 * wm + j) * 128 + 2 * lane);
  };
  // Empty volatile asm taking accumulators as inputs: the MFMAs producing
  // them stay above it (volatile asm keeps its order against the copies and
  // the barrier, which plain MFMA builtins do not).
  auto pin_row = [&](int i) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" ::"a"(acc[i][j]));
  };
  auto mfmas = [&](const Frags& f, const Scales& c, auto kkc) __attribute__((always_inline)) {
    constexpr int KK = decltype(kkc)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_mx<KK>(f.w[i], f.a[j], acc[i][j], c.w[i], c.a[j]);
#pragma unroll
    for (int i = 0; i < 4; ++i) pin_row(i);
  };
  // The same MFMAs in four groups of four with stage st's copies issued
  // between the groups, so the copy instructions' issue time overlaps the
  // matrix pipe instead of idling it.
  auto mfmas_copy = [&](const Frags& f, const Scales& c, auto kkc, unsigned char* buf, int st)
                        __attribute__((always_inline)) {
    constexpr int KK = decltype(kkc)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the group's weight scale passes through an empty volatile asm placed
      // after the previous copies, so the compiler cannot hoist the group's
      // MFMAs above them
      uint32_t sw = c.w[i];
      if (i > 0) asm volatile("" : "+v"(sw));
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_mx<KK>(f.w[i], f.a[j], acc[i][j], sw, c.a[j]);
      pin_row(i);
      __builtin_amdgcn_sched_barrier(0);
      if (st < nstages) issue_part(buf, st, (i * kMwLoads) / 4, ((i + 1) * kMwLoads) / 4);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Stage s (buffer cur): the fragments of its first 64-k step are already
  // in registers (f0, c0).  Read the second step's fragments, run the first
  // step's 16 MFMAs; then wait for stage s+1's copies, barrier (every wave
  // is past its reads of stage s-1), start stage s+3's copies into stage
  // s-1's buffer, read stage s+1's first-step fragments into (f0n, c0n), and
  // run the second step's MFMAs while those reads land.
  auto stage = [&](const unsigned char* cur, const unsigned char* next1, unsigned char* next3, int s,
                   Frags& f0, Scales& c0, Frags& f0n, Scales& c0n) __attribute__((always_inline)) {
    // (the scheduling barriers keep the compiler from hoisting the barrier
    // and the next stage's reads above the first step's MFMAs)
    // the second step's reads go out after the first four MFMAs, so the wait
    // for the first step's operands (read during the previous stage) does not
    // also wait for them
    Frags f1;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[0][j] = mfma_mx<0>(f0.w[0], f0.a[j], acc[0][j], c0.w[0], c0.a[j]);
    pin_row(0);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(cur, 1, f1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      uint32_t sw = c0.w[i];
      asm volatile("" : "+v"(sw));
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_mx<0>(f0.w[i], f0.a[j], acc[i][j], sw, c0.a[j]);
      pin_row(i);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < nstages) {
      if (s + 2 < nstages) wait_vmcnt_le<kMwLoads>();
      else wait_vmcnt_le<0>();
      __builtin_amdgcn_s_barrier();
      read_scales(next1, c0n);
      read_frags(next1, 0, f0n);
    }
    __builtin_amdgcn_sched_barrier(0);
    mfmas_copy(f1, c0, std::integral_constant<int, 1>(), next3, s + 3);
    __builtin_amdgcn_sched_barrier(0);
  };

  issue(lds0, 0);
  if (nstages > 1) issue(lds1, 1);
  if (nstages > 2) issue(lds2, 2);
  if (nstages > 2) wait_vmcnt_le<2 * kMwLoads>();
  else if (nstages > 1) wait_vmcnt_le<kMwLoads>();
  else wait_vmcnt_le<0>();
  __builtin_amdgcn_s_barrier();
  Frags fa, fb;
  Scales ca, cb;
  read_frags(lds0, 0, fa);
  read_scales(lds0, ca);
  for (int s = 0; s < nstages; s += 4) {
    stage(lds0, lds1, lds3, s, fa, ca, fb, cb);
    if (s + 1 < nstages) stage(lds1, lds2, lds0, s + 1, fb, cb, fa, ca);
    if (s + 2 < nstages) stage(lds2, lds3, lds1, s + 2, fa, ca, fb, cb);
    if (s + 3 < nstages) stage(lds3, lds0, lds2, s + 3, fb, cb, fa, ca);
  }

  // Epilogue through LDS: each wave writes its 128 x 128 block, scaled and
  // rounded to fp16, row-major into its own stage buffer (row pitch 272 B:
  // 128 rows x 272 B is exactly one buffer; the 16-byte skew per row spreads
  // the 32 rows a store instruction touches over the banks), then stores it
  // with 16-byte lanes, 4 rows x 256 contiguous bytes per instruction,
  // instead of 16-byte pieces of 32 rows.  The barrier keeps the buffers'
  // last stage intact until every wave has read it.
  // Accumulator layout: lane holds row m = lane & 31 of block j and columns
  // n = 8q + 4h + 0..3 of block i in registers 4q .. 4q+3.
  __syncthreads();
  unsigned char* eb = wave == 0 ? lds0 : wave == 1 ? lds1 : wave == 2 ? lds2 : lds3;
  constexpr int kPitch = 272;
  const float gwv = *wg;
  const int h = lane >> 5;
  const int mw = tm * kMwTile + 128 * wm;     // first activation row of this wave's block
  const int nw = tn * kMwTile + 128 * wn;     // first weight row (output column)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ml = 32 * j + (lane & 31);
    const int m = min(mw + ml, B - 1);        // rows past B are written to LDS, never stored
    const float s = ag[m / a_group_rows] * gwv;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v4h o = {(_Float16)(acc[i][j][4 * q] * s), (_Float16)(acc[i][j][4 * q + 1] * s),
                 (_Float16)(acc[i][j][4 * q + 2] * s), (_Float16)(acc[i][j][4 * q + 3] * s)};
        *reinterpret_cast<v4h*>(eb + ml * kPitch + 2 * (32 * i + 8 * q + 4 * h)) = o;
      }
  }
  // only this wave reads what it wrote: a wave-local LDS wait suffices
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const int cr = lane >> 4, cc = lane & 15;   // 4 rows x 16 chunks of 16 bytes per instruction
#pragma unroll 4
  for (int r0 = 0; r0 < 128; r0 += 4) {
    const int m = mw + r0 + cr, n = nw + 8 * cc;
    const u32x4 v = *reinterpret_cast<const u32x4*>(eb + (r0 + cr) * kPitch + 16 * cc);
    if (m < B && n < N) *reinterpret_cast<u32x4*>(y + (int64_t)m * N + n) = v;
  }
}

// ------------------------------------------------------------ skinny (decode)

constexpr int kMsWaves = 8;
constexpr int kMsBatch = 4;                  // 128-k chunks per wave in flight

__global__ void __launch_bounds__(kMsWaves * 64)
mx_gemm_skinny(const uint8_t* __restrict__ a, const uint8_t* __restrict__ as,
               const float* __restrict__ ag, int64_t a_group_rows, const uint8_t* __restrict__ w,
               const uint8_t* __restrict__ ws, const float* __restrict__ wg,
               _Float16* __restrict__ y, int B, int N, int K) {
  __shared__ float red[kMsWaves][16][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x;                  // weight row group
  const int nch = K / 128;
  const int c0 = wave * nch / kMsWaves, c1 = (wave + 1) * nch / kMsWaves;
  const uint8_t* wg_codes = w + (size_t)g * K * 16 + 16 * lane;
  const uint8_t* wg_scales = ws + (size_t)g * K + 2 * lane;
  // activation columns past B (padding rows of the tile) read column 0 of
  // their half instead: the same addresses as that lane, one cache line per
  // load; their outputs are not stored
  const int alane = (lane & 31) < B ? lane : (lane & 32);
  const uint8_t* a_codes = a + 16 * alane;
  const uint8_t* a_scales = as + 2 * alane;
  v16f acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  for (int c = c0; c < c1; c += kMsBatch) {
    u32x4 wq[kMsBatch][2], aq[kMsBatch][2];
    uint32_t sw[kMsBatch], sa[kMsBatch];
#pragma unroll
    for (int b = 0; b < kMsBatch; ++b) {
      const int cc = min(c + b, c1 - 1);     // chunks past the range re-read the last one
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        wq[b][kk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wg_codes + (size_t)(2 * cc + kk) * 1024));
        aq[b][kk] = *reinterpret_cast<const u32x4*>(a_codes + (size_t)(2 * cc + kk) * 1024);
      }
      sw[b] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(wg_scales + (size_t)cc * 128));
      sa[b] = *reinterpret_cast<const uint16_t*>(a_scales + (size_t)cc * 128);
    }
#pragma unroll
    for (int b = 0; b < kMsBatch; ++b) {
      if (c + b < c1) {
        acc = mfma_mx<0>(fp4_operand(wq[b][0]), fp4_operand(aq[b][0]), acc, sw[b], sa[b]);
        acc = mfma_mx<1>(fp4_operand(wq[b][1]), fp4_operand(aq[b][1]), acc, sw[b], sa[b]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  if (tid < 256) {
    const int l = tid & 63, q = tid >> 6;    // lane of the MFMA block, register quad
    const int m = l & 31, h = l >> 5;
    if (m < B) {
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float sum = 0.0f;
#pragma unroll
        for (int wv = 0; wv < kMsWaves; ++wv) sum += red[wv][4 * q + t][l];
        v[t] = sum;
      }
      const float s = ag[m / a_group_rows] * *wg;
      store4(y + (int64_t)m * N + 32 * g + 8 * q + 4 * h, v[0], v[1], v[2], v[3], s);
    }
  }
}

// ------------------------------------------------------------ tile permutation

// One thread per 16-byte code piece; the threads of even chunks also move the
// two scale bytes of their lane in the matching 128-k scale tile.  Rows past
// the end are written as zero codes and zero scale bytes.
__global__ void __launch_bounds__(256)
mx_tile_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ sf, int64_t rows,
               int K, int64_t ntiles, uint8_t* __restrict__ ct, uint8_t* __restrict__ st) {
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= ntiles) return;
  const int l = threadIdx.x & 63, nch = K / 64;
  const int64_t grp = tile / nch;
  const int c = (int)(tile - grp * nch);
  const int64_t r = 32 * grp + (l & 31);
  const int h = l >> 5;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (r < rows) v = *reinterpret_cast<const u32x4*>(codes + r * (K / 2) + 32 * c + 16 * h);
  *reinterpret_cast<u32x4*>(ct + (tile * 64 + l) * 16) = v;
  if ((c & 1) == 0) {
    uint32_t s2 = 0;
    if (r < rows) {
      const uint8_t* sr = sf + r * (K / 32) + 2 * c + h;   // block 4(c/2) + 2j + h
      s2 = (uint32_t)sr[0] | ((uint32_t)sr[2] << 8);
    }
    const int64_t stile = grp * (K / 128) + c / 2;
    *reinterpret_cast<uint16_t*>(st + (stile * 64 + l) * 2) = (uint16_t)s2;
  }
}

}  // namespace

hipError_t launch_mx_tile(const uint8_t* codes, const uint8_t* sf, int64_t rows, int64_t K,
                          uint8_t* codes_tiled, uint8_t* sf_tiled, hipStream_t s) {
  const int64_t ntiles = (rows + 31) / 32 * (K / 64);
  if (ntiles == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_tile_kernel, dim3((unsigned)((ntiles + 3) / 4)), dim3(256), 0, s, codes, sf,
                     rows, (int)K, ntiles, codes_tiled, sf_tiled);
  return hipGetLastError();
}

hipError_t launch_mx_gemm(const MxGemmArgs& g, hipStream_t s) {
  const int B = (int)g.B, N = (int)g.N, K = (int)g.K;
  _Float16* y = reinterpret_cast<_Float16*>(g.y);
  if (B <= 32) {
    hipLaunchKernelGGL(mx_gemm_skinny, dim3((unsigned)(N / 32)), dim3(kMsWaves * 64), 0, s, g.a, g.as,
                       g.ag, g.a_group_rows, g.w, g.ws, g.wg, y, B, N, K);
    return hipGetLastError();
  }
  const int tiles_m = (B + kMwTile - 1) / kMwTile, tiles_n = (N + kMwTile - 1) / kMwTile;
  hipLaunchKernelGGL(mx_gemm_wide, dim3((unsigned)(tiles_m * tiles_n)), dim3(kMwThreads), 0, s, g.a,
                     g.as, g.ag, g.a_group_rows, g.w, g.ws, g.wg, y, B, N, K, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace nvfp4
