// qlin kernels for gfx950.  One wave owns one 64-row tile of W (lane = row)
// in the quantizer and the GEMV kernels; the GEMMs feed fp16 MFMA.
#pragma once

#include <type_traits>

#include "codes.h"

namespace qlin {

// -------------------------------------------------------------- utilities --
// Load the 64 fp16 values of (row, block j) of a row-major fp16 matrix.
__device__ __forceinline__ void load_row_block(const uint16_t* __restrict__ w16, int64_t ld,
                                               int row, int j, bool valid, float* w) {
  if (valid) {
    const uint4* p = reinterpret_cast<const uint4*>(w16 + (int64_t)row * ld + (int64_t)j * kBlock);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 v = p[i];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2 h = as_h2(u[e]);
        w[8 * i + 2 * e] = (float)h.x;
        w[8 * i + 2 * e + 1] = (float)h.y;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) w[i] = 0.f;
  }
}

// Scale and zero from a group's extremes (fp32 subtract, IEEE divide, fp16
// round-to-nearest-even, zero point from the stored scale, ties to even).
__device__ __forceinline__ void scale_zero(float mn, float mx, int qmax, uint16_t& s16bits,
                                           float& s, int& z) {
  const float s32 = __fdiv_rn(mx - mn, (float)qmax);
  const f16 s16 = (f16)s32;
  s = (float)s16;
  s16bits = __builtin_bit_cast(uint16_t, s16);
  z = 0;
  if (s != 0.f) {
    const float zr = __builtin_rintf(__fdiv_rn(-mn, s));
    z = (int)clampf(zr, 0.f, (float)qmax);
  } else {
    s16bits = 0;
  }
}

template <int BITS>
__device__ __forceinline__ void codes_and_store(const float* w, float s, int z,
                                                uint32_t* __restrict__ dst) {
  constexpr int qmax = (1 << BITS) - 1;
  const RtnParams p = rtn_params(s, z, qmax);
  float code[64];
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    float q0 = __builtin_rintf(w[c] * p.r);
    q0 = rtn_fix(w[c], q0, p);
    code[c] = clampf(q0, p.lo, p.hi) + (float)z;
  }
  uint32_t out[2 * BITS];
  pack_block<BITS>(code, out);
  if constexpr (BITS % 2 == 1) {
    // 2*BITS words, 8-byte aligned rows (3, 5, 7 bits)
    uint2* d2 = reinterpret_cast<uint2*>(dst);
#pragma unroll
    for (int i = 0; i < BITS; ++i) d2[i] = make_uint2(out[2 * i], out[2 * i + 1]);
  } else {
    uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
    for (int i = 0; i < BITS / 2; ++i)
      d4[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
  }
}

// ------------------------------------------------------------- quantizer --
// A launch quantizes a batch of up to kQuantBatch matrices (one bit width and
// group kind): the jobs travel in the kernel arguments, work items are
// numbered consecutively over the jobs (end[i] = items of jobs 0..i), and
// each work-group finds its job by a scan over the ends.
constexpr int kQuantBatch = 64;
// Widths with a packed layout (all of the lever's quantized widths).
template <int BITS>
constexpr bool kPackable = BITS >= 2 && BITS <= 8;
struct QuantJob {
  const uint16_t* w16;
  int64_t ld;
  uint32_t* codes;       // null: scale/zero only
  uint16_t* scale;
  uint8_t* zero;
  int n, kb;
};
struct QuantBatch {
  QuantJob job[kQuantBatch];
  int end[kQuantBatch];
  int count;
};

__device__ __forceinline__ int quant_job_of(const QuantBatch& b, int item, int& first) {
  int ji = 0;
  for (int i = 0; i + 1 < b.count; ++i)
    if (item >= b.end[i]) ji = i + 1;
  first = ji == 0 ? 0 : b.end[ji - 1];
  return ji;
}

// Group 64.  Work item = (tile, y) of a job, y = ceil(kb / WAVES) per tile;
// wave w handles K-block j = y*WAVES + w for the 64 rows of the tile.
template <int BITS, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_quantize_g64(const QuantBatch b) {
  constexpr int qmax = (1 << BITS) - 1;
  const int lane = lane_id(), wave = wave_id();
  int first;
  const QuantJob& q = b.job[quant_job_of(b, blockIdx.x, first)];
  const int ny = (q.kb + WAVES - 1) / WAVES;
  const int item = blockIdx.x - first;
  const int t = item / ny;
  const int j = (item % ny) * WAVES + wave;
  if (j >= q.kb) return;
  const int row = t * kTile + lane;
  float w[64];
  load_row_block(q.w16, q.ld, row, j, row < q.n, w);
  float mn = w[0], mx = w[0];
#pragma unroll
  for (int i = 1; i < 64; ++i) { mn = __builtin_fminf(mn, w[i]); mx = __builtin_fmaxf(mx, w[i]); }
  uint16_t sb; float s; int z;
  scale_zero(mn, mx, qmax, sb, s, z);
  const int64_t mi = ((int64_t)t * q.kb + j) * kTile + lane;
  q.scale[mi] = sb;
  q.zero[mi] = (uint8_t)z;
  if constexpr (kPackable<BITS>) {
    if (q.codes != nullptr) codes_and_store<BITS>(w, s, z, q.codes + mi * (2 * BITS));
  }
}

// One group per row.  Work item = tile; the WAVES waves split the K-blocks,
// the row extremes are combined through LDS, then each wave writes its blocks.
template <int BITS, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_quantize_row(const QuantBatch b) {
  constexpr int qmax = (1 << BITS) - 1;
  __shared__ float smn[WAVES][64], smx[WAVES][64];
  const int lane = lane_id(), wave = wave_id();
  int first;
  const QuantJob& q = b.job[quant_job_of(b, blockIdx.x, first)];
  const int t = blockIdx.x - first;
  const int kb = q.kb;
  const int row = t * kTile + lane;
  const bool valid = row < q.n;
  float mn = 0.f, mx = 0.f;
  bool empty = true;
  for (int j = wave; j < kb; j += WAVES) {
    float w[64];
    load_row_block(q.w16, q.ld, row, j, valid, w);
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      mn = empty ? w[i] : __builtin_fminf(mn, w[i]);
      mx = empty ? w[i] : __builtin_fmaxf(mx, w[i]);
      empty = false;
    }
  }
  smn[wave][lane] = empty ? __builtin_inff() : mn;
  smx[wave][lane] = empty ? -__builtin_inff() : mx;
  __syncthreads();
  mn = smn[0][lane]; mx = smx[0][lane];
#pragma unroll
  for (int i = 1; i < WAVES; ++i) { mn = __builtin_fminf(mn, smn[i][lane]); mx = __builtin_fmaxf(mx, smx[i][lane]); }
  uint16_t sb; float s; int z;
  scale_zero(mn, mx, qmax, sb, s, z);
  if (wave == 0) {
    q.scale[(int64_t)t * kTile + lane] = sb;
    q.zero[(int64_t)t * kTile + lane] = (uint8_t)z;
  }
  if constexpr (kPackable<BITS>) {
    if (q.codes == nullptr) return;
    for (int j = wave; j < kb; j += WAVES) {
      float w[64];
      load_row_block(q.w16, q.ld, row, j, valid, w);
      const int64_t bi = ((int64_t)t * kb + j) * kTile + lane;
      codes_and_store<BITS>(w, s, z, q.codes + bi * (2 * BITS));
    }
  }
}

// ---------------------------------------------------- split-K finishing --
// Every work-group of an output tile writes its partial sums to the
// workspace; the last one to arrive (ticket) adds the partials in split order,
// so the result does not depend on arrival order, and re-arms the ticket.
//
// Partials move between work-groups, which may sit on different XCDs with
// separate L2 caches, as device-scope atomic stores and loads (relaxed, agent
// scope: the store is written through to the device coherence point, the load
// reads from it).  A writer waits until all its stores are acknowledged
// (vmcnt = 0) before it takes its ticket, so the last work-group sees every
// partial.  This replaces an agent-scope release/acquire fence pair, whose L2
// write-back and invalidate cost ~0.2 us each and serialize per XCD when
// hundreds of work-groups finish together.
__device__ __forceinline__ void put_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float get_partial(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait for every store this wave issued to be acknowledged.  The signal
// fences keep the compiler from moving the atomics across the wait.
__device__ __forceinline__ void partials_written() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One wave: true for the last of `splits` arrivals at tickets[t] (after
// partials_written()); the winner re-arms the ticket.
__device__ __forceinline__ bool split_ticket(uint32_t* __restrict__ tickets, int t, int splits) {
  uint32_t prev = 0;
  if (lane_id() == 0)
    prev = __hip_atomic_fetch_add(&tickets[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __builtin_amdgcn_readfirstlane(prev);
  if (prev != (uint32_t)(splits - 1)) return false;
  if (lane_id() == 0)
    __hip_atomic_store(&tickets[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Sum of one output's split partials p[0], p[stride], ... in split order; the
// loads of up to 8 splits are in flight together (a load-add chain would pay
// one memory round trip per split).
__device__ __forceinline__ float sum_splits(const float* __restrict__ p, int64_t stride,
                                            int splits) {
  float acc = 0.f;
  for (int b = 0; b < splits; b += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = get_partial(p + (int64_t)min(b + i, splits - 1) * stride);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (b + i < splits) acc += v[i];
  }
  return acc;
}

// Scale of a block that may lie past the wave's range (its address clamped by
// the caller): the load is always issued, and the converted value multiplied
// by 1 or 0 where it is used.  A select would let the compiler move the load
// into a branch, where its conversion waits for it at once (vmcnt(0)) and
// serializes the blocks that were meant to be in flight together.
__device__ __forceinline__ float masked_scale(uint16_t raw, bool valid) {
  return h2f(raw) * (valid ? 1.f : 0.f);
}

// Keeps the compiler's scheduler from moving work across this point: placed
// after the loads of all blocks in flight, so that every load is issued before
// the first decode waits for its data.
__device__ __forceinline__ void loads_issued() { __builtin_amdgcn_sched_barrier(0); }

// -------------------------------------------------------- packed GEMV --
// One work-group per (tile, split); lane = row of the tile.  A wave issues the
// loads of up to U blocks before decoding any, so a short K range costs one
// memory round trip.  x is read with wave-uniform addresses (scalar loads,
// shared by all rows of the tile).
template <int BITS>
__device__ __forceinline__ void load_block_words(const uint32_t* __restrict__ blk, uint32_t* wd) {
  if constexpr (BITS % 2 == 1) {
    // 2*BITS words, 8-byte aligned rows (3, 5, 7 bits)
    const uint2* b2 = reinterpret_cast<const uint2*>(blk);
#pragma unroll
    for (int i = 0; i < BITS; ++i) { const uint2 v = b2[i]; wd[2 * i] = v.x; wd[2 * i + 1] = v.y; }
  } else {
    const uint4* b4 = reinterpret_cast<const uint4*>(blk);
#pragma unroll
    for (int i = 0; i < BITS / 2; ++i) {
      const uint4 v = b4[i];
      wd[4 * i] = v.x; wd[4 * i + 1] = v.y; wd[4 * i + 2] = v.z; wd[4 * i + 3] = v.w;
    }
  }
}

// DPP lane moves within rows of 16 lanes (row_mirror 0x140, row_half_mirror
// 0x141, quad permutations).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

// Sum over each row of 16 lanes, left in every lane of the row: pairs, quads,
// half rows, rows.  Each step adds a lane and its partner, so both get the
// same (commutative) sum and every lane of a row ends with one value.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<0xB1>(v);    // lane ^ 1
  v += dpp_f<0x4E>(v);    // lane ^ 2
  v += dpp_f<0x141>(v);   // mirror within 8 lanes: the other quad
  v += dpp_f<0x140>(v);   // mirror within 16 lanes: the other half row
  return v;
}

// The x sums of the U blocks jj[0..U-1] a wave works on (for the folded zero
// point): lane l reads U consecutive x of block l / (64/U) (one load, issued
// with the block loads), block_xsums_finish adds them within rows of 16 lanes
// and reads the row sums back as wave-uniform values.
template <int U>
struct XsumLoad {
  typename std::conditional<U == 4, uint2, typename std::conditional<U == 2, uint32_t, uint16_t>::type>::type v;
};

// Block u of the wave's round is jb + u * jstep, clamped below j1 (as the
// code loads clamp it).
template <int U>
__device__ __forceinline__ XsumLoad<U> block_xsums_load(const f16x2* __restrict__ x2, int jb,
                                                        int jstep, int j1, int lane) {
  constexpr int LPB = 64 / U;   // lanes per block
  const int u = lane / LPB, i = lane % LPB;
  const int j = min(jb + u * jstep, j1 - 1);
  const uint16_t* xp = reinterpret_cast<const uint16_t*>(x2) + (int64_t)j * 64 + i * U;
  XsumLoad<U> r;
  if constexpr (U == 4) r.v = *reinterpret_cast<const uint2*>(xp);
  else if constexpr (U == 2) r.v = *reinterpret_cast<const uint32_t*>(xp);
  else r.v = *xp;
  return r;
}

template <int U>
__device__ __forceinline__ void block_xsums_finish(const XsumLoad<U>& ld, float (&X)[U]) {
  const f16x2 one = {(f16)1.0f, (f16)1.0f};
  float s;
  if constexpr (U == 4)
    s = __builtin_amdgcn_fdot2(as_h2(ld.v.y), one,
                               __builtin_amdgcn_fdot2(as_h2(ld.v.x), one, 0.f, false), false);
  else if constexpr (U == 2) s = __builtin_amdgcn_fdot2(as_h2(ld.v), one, 0.f, false);
  else s = h2f(ld.v);
  s = row_sum16(s);
  auto rl = [&](int l) __attribute__((always_inline)) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), l));
  };
#pragma unroll
  for (int v = 0; v < U; ++v) {
    if constexpr (U == 4) X[v] = rl(16 * v);
    else if constexpr (U == 2) X[v] = rl(32 * v) + rl(32 * v + 16);
    else X[v] = (rl(0) + rl(16)) + (rl(32) + rl(48));
  }
}

// One wave's share of a tile's dot products, for NM matrices that share x
// (NM = 2: gate and up): K-blocks jfirst, jfirst + jstep, ... below j1, U at a
// time.  The loads of all U blocks of every matrix are issued first, without
// branches: a block past the range re-reads the last block of the range and
// gets scale 0.  The decode of block u then only waits for its own loads,
// while x of block u+1 is fetched (scalar loads) during block u's decode.
// The zero point is folded: block u adds s * (sum x q - z * X[u]), X[u] the
// block's x sum (block_xsums_*), and the codes are decoded as fp16 subnormals
// (block_xq).
// codes_t / scale_t / zero_t point at the tile's first block / entry.
template <int BITS, int U, int NM>
__device__ __forceinline__ void tile_dot(const uint32_t* const (&codes_t)[NM],
                                         const uint16_t* const (&scale_t)[NM],
                                         const uint8_t* const (&zero_t)[NM],
                                         const f16x2* __restrict__ x2, int G, int jfirst, int j1,
                                         int jstep, int lane, float (&acc)[NM]) {
  constexpr int WPB = 2 * BITS;
  for (int jb = jfirst; jb < j1; jb += jstep * U) {
    uint32_t wd[U][NM][WPB];
    uint16_t sr[U][NM];
    int z[U][NM], jj[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * jstep;
      jj[u] = j < j1 ? j : j1 - 1;
    }
    // the x sums' and the metadata loads first, then the codes: loads return
    // in order, so a block's decode and its scale/zero combine wait only for
    // its own codes
    const XsumLoad<U> xl = block_xsums_load<U>(x2, jb, jstep, j1, lane);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t mi = (int64_t)((G == 1) ? 0 : jj[u]) * kTile + lane;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        sr[u][m] = scale_t[m][mi];
        z[u][m] = zero_t[m][mi];
      }
    }
    loads_issued();
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < NM; ++m)
        load_block_words<BITS>(codes_t[m] + ((int64_t)jj[u] * kTile + lane) * WPB, wd[u][m]);
    loads_issued();
    float X[U];
    block_xsums_finish<U>(xl, X);
    f16x2 xc[32], xn[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) xc[i] = x2[(int64_t)jj[0] * 32 + i];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u + 1 < U) {
#pragma unroll
        for (int i = 0; i < 32; ++i) xn[i] = x2[(int64_t)jj[u + 1] * 32 + i];
      }
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const float t = __builtin_fmaf(block_xq<BITS>(wd[u][m], xc), 16777216.f,
                                       -(float)z[u][m] * X[u]);
        acc[m] = __builtin_fmaf(masked_scale(sr[u][m], jb + u * jstep < j1), t, acc[m]);
      }
      if (u + 1 < U) {
#pragma unroll
        for (int i = 0; i < 32; ++i) xc[i] = xn[i];
      }
    }
  }
}

// Up to kMaxMats packed matrices that share K (and x), launched together.
// Their tiles are numbered consecutively: matrix i owns launch tiles
// [tile_end[i-1], tile_end[i]).  With SWIGLU, matrices 0 (gate) and 1 (up)
// have the same n and launch tile t covers tile t of both.
constexpr int kMaxMats = 4;
struct GemvSet {
  const uint32_t* codes[kMaxMats];
  const uint16_t* scale[kMaxMats];
  const uint8_t* zero[kMaxMats];
  float* y[kMaxMats];
  int n[kMaxMats];
  int tile_end[kMaxMats];
  int count;
};

// silu(g) = g / (1 + exp(-g)) with the hardware reciprocal (1 ulp); g << 0
// gives 1/inf = 0 and so -0
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g));
}

// grid = (launch tiles, splits), block = WAVES waves; lane = row of the tile.
// The WAVES waves of split s take the K-blocks j0+w, j0+w+WAVES, ... of
// [j0, j1) (consecutive 128*bits-byte runs).  Plain: y = the tile's dot
// products.  SWIGLU: every wave does its blocks of the gate and the up tile
// (one x for both), and the output is h = silu(gate . x) * (up . x), in fp32
// (y[0]) and/or fp16 (h16, nearest even); either may be null.
template <int BITS, int WAVES, int U, bool SWIGLU>
__global__ __launch_bounds__(WAVES * 64) void k_gemv_packed(
    const GemvSet set, const f16x2* __restrict__ x2, float* __restrict__ part,
    uint32_t* __restrict__ tickets, int kb, int G, int splits, int kbps,
    uint16_t* __restrict__ h16) {
  constexpr int WPB = 2 * BITS;
  constexpr int NM = SWIGLU ? 2 : 1;                  // matrices per tile
  __shared__ float red[NM][WAVES][64];
  const int lane = lane_id(), wave = wave_id();
  const int sp = blockIdx.y;
  // this work-group's matrix (uniform selects, no indexing of the argument)
  const uint32_t* codes = set.codes[0];
  const uint16_t* scale = set.scale[0];
  const uint8_t* zero = set.zero[0];
  float* y = set.y[0];
  int n = set.n[0], tb = 0;
  if constexpr (!SWIGLU) {
#pragma unroll
    for (int i = 1; i < kMaxMats; ++i)
      if (i < set.count && (int)blockIdx.x >= set.tile_end[i - 1]) {
        codes = set.codes[i]; scale = set.scale[i]; zero = set.zero[i];
        y = set.y[i]; n = set.n[i]; tb = set.tile_end[i - 1];
      }
  }
  const int t = blockIdx.x - tb;
  const int64_t ct = (int64_t)t * kb * kTile * WPB, mt = (int64_t)t * G * kTile;
  const uint32_t* codes_t[NM];
  const uint16_t* scale_t[NM];
  const uint8_t* zero_t[NM];
  codes_t[0] = codes + ct; scale_t[0] = scale + mt; zero_t[0] = zero + mt;
  if constexpr (SWIGLU) {
    codes_t[NM - 1] = set.codes[1] + ct;
    scale_t[NM - 1] = set.scale[1] + mt;
    zero_t[NM - 1] = set.zero[1] + mt;
  }
  const int j0 = sp * kbps;
  const int j1 = min(kb, j0 + kbps);
  float acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = 0.f;
  tile_dot<BITS, U, NM>(codes_t, scale_t, zero_t, x2, G, j0 + wave, j1, WAVES, lane, acc);
#pragma unroll
  for (int m = 0; m < NM; ++m) red[m][wave][lane] = acc[m];
  lds_barrier();
  if (wave != 0) return;
  float tot[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    tot[m] = red[m][0][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) tot[m] += red[m][w][lane];
  }
  if (splits > 1) {
    // part[split][matrix][launch row]
    const int64_t np = (int64_t)gridDim.x * kTile;
    const int64_t grow = (int64_t)blockIdx.x * kTile + lane;
#pragma unroll
    for (int m = 0; m < NM; ++m) put_partial(part + ((int64_t)sp * NM + m) * np + grow, tot[m]);
    partials_written();
    if (!split_ticket(tickets, blockIdx.x, splits)) return;
#pragma unroll
    for (int m = 0; m < NM; ++m) tot[m] = sum_splits(part + m * np + grow, NM * np, splits);
  }
  const int row = t * kTile + lane;
  if (row >= n) return;
  if constexpr (SWIGLU) {
    const float h = silu(tot[0]) * tot[NM - 1];
    if (y != nullptr) y[row] = h;
    if (h16 != nullptr) h16[row] = __builtin_bit_cast(uint16_t, (f16)h);
  } else {
    y[row] = tot[0];
  }
}

// Work-groups go to the 8 XCDs (each with its own L2) round-robin by their
// flattened id.  This maps the flattened id to a grid position (x fastest)
// such that every XCD gets one contiguous range of positions, so that
// neighbouring positions (the parts of one tile, which share its scale and
// zero lines) are fetched into one L2.  A bijection of the grid onto itself.
constexpr int kXcds = 8;
__device__ __forceinline__ void xcd_grid_pos(int& x, int& y) {
  const int nx = gridDim.x, n = nx * gridDim.y;
  const int f = blockIdx.x + nx * blockIdx.y;
  const int per = n / kXcds, rem = n % kXcds, xcd = f % kXcds, local = f / kXcds;
  const int lin = xcd < rem ? xcd * (per + 1) + local
                            : rem * (per + 1) + (xcd - rem) * per + local;
  x = lin % nx;
  y = lin / nx;
}

// ------------------------------------------------ narrow packed GEMV --
// For launches of few tiles: a work-group covers 64/NG rows of a tile (grid.x =
// NG x launch tiles), so a small matrix is spread over NG times as many
// compute units as one work-group per tile would reach.  Lane = NG*r + g: row
// r of the work-group's rows and slice g of every 64-code block (codes
// (64/NG)*g onwards), so the lanes of a wave read one contiguous run of the
// block per instruction.  x differs between slices and is read with vector
// loads (128/NG bytes per lane and block; NG distinct addresses per wave).
template <int BITS, int NG>
constexpr int slice_words() {
  if constexpr (BITS >= 5 && BITS <= 7) {
    // the 4-bit plane's slice words, then the high plane's (one word for the
    // 1-bit plane)
    if constexpr (BITS == 5) return slice_words<4, NG>() + 1;
    else return slice_words<4, NG>() + slice_words<BITS - 4, NG>();
  } else {
    return BITS == 3 ? 2 : (NG == 4 ? BITS / 2 : (BITS == 2 ? 1 : BITS / 4));
  }
}
template <int BITS, int NG>
struct SliceWords {
  static constexpr int n = slice_words<BITS, NG>();
};

// The words holding slice g of one row's block (row_blk = the row's first word).
template <int BITS, int NG>
__device__ __forceinline__ void load_slice_words(const uint32_t* __restrict__ row_blk, int g,
                                                 uint32_t* wd) {
  constexpr int CPS = 64 / NG;                        // codes per slice
  if constexpr (BITS >= 5 && BITS <= 7) {
    constexpr int W4 = SliceWords<4, NG>::n;
    load_slice_words<4, NG>(row_blk, g, wd);
    if constexpr (BITS == 5) wd[W4] = row_blk[8 + (NG == 4 ? g >> 1 : g >> 2)];   // 32 codes/word
    else load_slice_words<BITS - 4, NG>(row_blk + 8, g, wd + W4);
  } else if constexpr (BITS == 3) {
    // the low-bit word of the slice's 16-code half-run, the run's third-bit word
    const int c0 = CPS * g, run = c0 >> 5, u = (c0 >> 4) & 1;
    wd[0] = row_blk[3 * run + u];
    wd[1] = row_blk[3 * run + 2];
  } else if constexpr (BITS == 2 && NG == 8) {
    wd[0] = row_blk[g >> 1];                          // 16 codes per word
  } else {
    constexpr int W = SliceWords<BITS, NG>::n;        // whole words
    if constexpr (W == 1) {
      wd[0] = row_blk[g];
    } else if constexpr (W == 2) {
      const uint2 v = reinterpret_cast<const uint2*>(row_blk)[g];
      wd[0] = v.x; wd[1] = v.y;
    } else {
      const uint4 v = reinterpret_cast<const uint4*>(row_blk)[g];
      wd[0] = v.x; wd[1] = v.y; wd[2] = v.z; wd[3] = v.w;
    }
  }
}

// 2- and 3-bit terms of 8 codes: the pairs (2p, 2p+1) of the 8, p = 0..3,
// come out of v under the mask of p with scale class S = 4^p; xs[p] is their
// x pair.  Returns their sum over the 8 codes of x_k * (q_k - z), unscaled.
__device__ __forceinline__ float low_bits8(uint32_t v, const f16x2* xs, int z, uint32_t kMagic) {
  float a[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t m = (3u << (2 * p)) | (3u << (16 + 2 * p));
    const f16x2 h = as_h2((v & m) | kMagic) - as_h2(zconst(z, 2 * p));
    a[p] = __builtin_amdgcn_fdot2(h, xs[p], 0.f, false);
  }
  return a[0] + a[1] * 0.25f + a[2] * 0.0625f + a[3] * 0.015625f;
}

// 3-bit: low bits L and third bits H (already aligned like the 2-bit fields).
__device__ __forceinline__ float three_bits8(uint32_t L, uint32_t H, const f16x2* xs, int z,
                                             uint32_t kMagic) {
  float a[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t m2 = (3u << (2 * p)) | (3u << (16 + 2 * p));
    const uint32_t m1 = (1u << (2 * p + 2)) | (1u << (2 * p + 18));
    const uint32_t t = (L & m2) | (H & ~m2);          // bit-field insert
    const f16x2 h = as_h2((t & (m2 | m1)) | kMagic) - as_h2(zconst(z, 2 * p));
    a[p] = __builtin_amdgcn_fdot2(h, xs[p], 0.f, false);
  }
  return a[0] + a[1] * 0.25f + a[2] * 0.0625f + a[3] * 0.015625f;
}

// 4-bit terms of the 8 codes of word v (x pairs xs[0..3]).
__device__ __forceinline__ float four_bits8(uint32_t v, const f16x2* xs, int z, uint32_t kMagic) {
  const f16x2 c1 = as_h2(zconst(z, 0)), c16 = as_h2(zconst(z, 4));
  const uint32_t vs = v >> 8;
  const float a0 = __builtin_amdgcn_fdot2(as_h2((v & 0x000F000Fu) | kMagic) - c1, xs[0], 0.f, false);
  const float b0 = __builtin_amdgcn_fdot2(as_h2((v & 0x00F000F0u) | kMagic) - c16, xs[1], 0.f, false);
  const float a1 = __builtin_amdgcn_fdot2(as_h2((vs & 0x000F000Fu) | kMagic) - c1, xs[2], 0.f, false);
  const float b1 = __builtin_amdgcn_fdot2(as_h2((vs & 0x00F000F0u) | kMagic) - c16, xs[3], 0.f, false);
  return (a0 + a1) + (b0 + b1) * 0.0625f;
}

// 8-bit terms of the 8 codes of words v, u (x pairs xs[0..3]).
__device__ __forceinline__ float eight_bits8(uint32_t v, uint32_t u, const f16x2* xs, int z,
                                             uint32_t kMagic) {
  const f16x2 c = as_h2(zconst(z, 0));
  const f16x2 h0 = as_h2(__builtin_amdgcn_perm(0x64646464u, v, 0x04020400u)) - c;
  const f16x2 h1 = as_h2(__builtin_amdgcn_perm(0x64646464u, v, 0x04030401u)) - c;
  const f16x2 g0 = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04020400u)) - c;
  const f16x2 g1 = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030401u)) - c;
  const float a0 = __builtin_amdgcn_fdot2(h0, xs[0], 0.f, false);
  const float b0 = __builtin_amdgcn_fdot2(h1, xs[1], 0.f, false);
  const float a1 = __builtin_amdgcn_fdot2(g0, xs[2], 0.f, false);
  const float b1 = __builtin_amdgcn_fdot2(g1, xs[3], 0.f, false);
  return (a0 + a1) + (b0 + b1);
}

// 1-bit plane: NP code pairs from bits 0..NP-1 of each half of v (shifted to
// the slice by the caller), scale class S = 2^p; z is 0 or 1.
template <int NP>
__device__ __forceinline__ float one_bits(uint32_t v, const f16x2* xs, int z, uint32_t kMagic) {
  // sum over p of dot_p / 2^p, evaluated as a Horner scheme in 1/2
  float acc = 0.f;
#pragma unroll
  for (int p = NP - 1; p >= 0; --p) {
    const uint32_t m = (1u << p) | (1u << (16 + p));
    const f16x2 h = as_h2((v & m) | kMagic) - as_h2(zconst(z, p));
    acc = __builtin_amdgcn_fdot2(h, xs[p], acc * 0.5f, false);
  }
  return acc;
}

// sum over the codes of slice g of x_k * (q_k - z), unscaled; xs = the
// slice's x pairs.  The decode of block_dot, restricted to the slice.  A
// slice of 16 codes is two 8-code halves; the second half of a 2- or 3-bit
// half-run sits 8 bits (low bits) / 1 bit (aligned third bits) higher.
template <int BITS, int NG>
__device__ __forceinline__ float slice_dot(const uint32_t* wd, const f16x2* xs, int z, int g,
                                           uint32_t kMagic) {
  if constexpr (BITS == 4) {
    if constexpr (NG == 4) return four_bits8(wd[0], xs, z, kMagic) + four_bits8(wd[1], xs + 4, z, kMagic);
    else return four_bits8(wd[0], xs, z, kMagic);
  } else if constexpr (BITS == 8) {
    if constexpr (NG == 4)
      return eight_bits8(wd[0], wd[1], xs, z, kMagic) + eight_bits8(wd[2], wd[3], xs + 4, z, kMagic);
    else return eight_bits8(wd[0], wd[1], xs, z, kMagic);
  } else if constexpr (BITS == 2) {
    if constexpr (NG == 4) {
      return low_bits8(wd[0], xs, z, kMagic) + low_bits8(wd[0] >> 8, xs + 4, z, kMagic);
    } else {
      return low_bits8(wd[0] >> (8 * (g & 1)), xs, z, kMagic);
    }
  } else if constexpr (BITS >= 5 && BITS <= 7) {
    // q - z = (lo - z % 16) + 16 * (hi - z / 16)
    constexpr int W4 = SliceWords<4, NG>::n;
    const float lo = slice_dot<4, NG>(wd, xs, z & 15, g, kMagic);
    float hi;
    if constexpr (BITS == 5) {
      // 1-bit plane: NG = 4 takes 8 pairs at bit 8*(g%2), NG = 8 four at 4*(g%4)
      if constexpr (NG == 4) hi = one_bits<8>(wd[W4] >> (8 * (g & 1)), xs, z >> 4, kMagic);
      else hi = one_bits<4>(wd[W4] >> (4 * (g & 3)), xs, z >> 4, kMagic);
    } else {
      hi = slice_dot<BITS - 4, NG>(wd + W4, xs, z >> 4, g, kMagic);
    }
    return lo + 16.f * hi;
  } else {  // BITS == 3
    const uint32_t H = wd[1];
    const int c0 = (64 / NG) * g;
    const uint32_t Hu = ((c0 >> 4) & 1) ? __builtin_amdgcn_alignbit(H, H, 8) : H;
    if constexpr (NG == 4) {
      return three_bits8(wd[0], Hu, xs, z, kMagic) + three_bits8(wd[0] >> 8, Hu >> 1, xs + 4, z, kMagic);
    } else {
      const bool hi = (c0 >> 3) & 1;
      return three_bits8(hi ? wd[0] >> 8 : wd[0], hi ? Hu >> 1 : Hu, xs, z, kMagic);
    }
  }
}

// Sum over the NG consecutive lanes of a row's slices, the same order for
// every row: pairs, then quads (DPP), then octets (swizzle).
template <int NG>
__device__ __forceinline__ float slice_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                             0xB1, 0xF, 0xF, false));  // [1,0,3,2]
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                             0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  if constexpr (NG == 8)
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                               0x1F | (4 << 10)));     // lane ^ 4
  return v;
}

// grid = (NG x launch tiles, splits), block = WAVES waves.  Work-group b
// covers rows RW*(b % NG) .. +RW-1 (RW = 64/NG) of launch tile b / NG; its
// waves take the K-blocks j0+w, j0+w+WAVES, ... of the split's range, U at a
// time, all loads of the U blocks issued before any decode.  Outputs, sets,
// SwiGLU pairs and split-K partials as in k_gemv_packed (partials per launch
// row, tickets per work-group).
template <int BITS, int NG, int WAVES, int U, bool SWIGLU>
__global__ __launch_bounds__(WAVES * 64) void k_gemv_narrow(
    const GemvSet set, const f16x2* __restrict__ x2, float* __restrict__ part,
    uint32_t* __restrict__ tickets, int kb, int G, int splits, int kbps,
    uint16_t* __restrict__ h16) {
  constexpr int WPB = 2 * BITS;
  constexpr int NM = SWIGLU ? 2 : 1;
  constexpr int RW = kTile / NG;                      // rows per work-group
  constexpr int SW = SliceWords<BITS, NG>::n;
  constexpr int XP = 32 / NG;                         // x pairs per slice
  __shared__ float red[NM][WAVES][RW];
  const uint32_t magic = vreg_const(kMagic);
  const int lane = lane_id(), wave = wave_id();
  const int r = lane / NG, g = lane % NG;
  int bx, sp;
  xcd_grid_pos(bx, sp);
  const int lt = bx / NG, part_i = bx % NG;
  const uint32_t* codes = set.codes[0];
  const uint16_t* scale = set.scale[0];
  const uint8_t* zero = set.zero[0];
  float* y = set.y[0];
  int n = set.n[0], tb = 0;
  if constexpr (!SWIGLU) {
#pragma unroll
    for (int i = 1; i < kMaxMats; ++i)
      if (i < set.count && lt >= set.tile_end[i - 1]) {
        codes = set.codes[i]; scale = set.scale[i]; zero = set.zero[i];
        y = set.y[i]; n = set.n[i]; tb = set.tile_end[i - 1];
      }
  }
  const int t = lt - tb;
  const int R = part_i * RW + r;                      // row within the tile
  const int64_t ct = (int64_t)t * kb * kTile * WPB, mt = (int64_t)t * G * kTile;
  const uint32_t* codes_t[NM];
  const uint16_t* scale_t[NM];
  const uint8_t* zero_t[NM];
  codes_t[0] = codes + ct; scale_t[0] = scale + mt; zero_t[0] = zero + mt;
  if constexpr (SWIGLU) {
    codes_t[NM - 1] = set.codes[1] + ct;
    scale_t[NM - 1] = set.scale[1] + mt;
    zero_t[NM - 1] = set.zero[1] + mt;
  }
  const int j0 = sp * kbps;
  const int j1 = min(kb, j0 + kbps);
  float acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = 0.f;
  for (int jb = j0 + wave; jb < j1; jb += WAVES * U) {
    uint32_t wd[U][NM][SW];
    uint16_t sr[U][NM];
    int z[U][NM];
    f16x2 xs[U][XP];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * WAVES;
      const int jj = j < j1 ? j : j1 - 1;     // past the range: re-read, scale 0
      const int64_t mi = (int64_t)((G == 1) ? 0 : jj) * kTile + R;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        load_slice_words<BITS, NG>(codes_t[m] + ((int64_t)jj * kTile + R) * WPB, g, wd[u][m]);
        sr[u][m] = scale_t[m][mi];
        z[u][m] = zero_t[m][mi];
      }
      const uint4* xp = reinterpret_cast<const uint4*>(x2 + (int64_t)jj * 32 + XP * g);
#pragma unroll
      for (int i = 0; i < XP / 4; ++i) {
        const uint4 xv = xp[i];
        xs[u][4 * i + 0] = as_h2(xv.x); xs[u][4 * i + 1] = as_h2(xv.y);
        xs[u][4 * i + 2] = as_h2(xv.z); xs[u][4 * i + 3] = as_h2(xv.w);
      }
    }
    if constexpr (U > 1) loads_issued();
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < NM; ++m)
        acc[m] = __builtin_fmaf(masked_scale(sr[u][m], jb + u * WAVES < j1),
                                slice_dot<BITS, NG>(wd[u][m], xs[u], z[u][m], g, magic), acc[m]);
  }
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    acc[m] = slice_sum<NG>(acc[m]);
    if (g == 0) red[m][wave][r] = acc[m];
  }
  lds_barrier();
  if (wave != 0 || lane >= RW) return;
  float tot[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    tot[m] = red[m][0][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) tot[m] += red[m][w][lane];
  }
  if (splits > 1) {
    // part[split][matrix][launch row], launch row = RW * position + lane
    const int64_t np = (int64_t)gridDim.x * RW;
    const int64_t grow = (int64_t)bx * RW + lane;
#pragma unroll
    for (int m = 0; m < NM; ++m) put_partial(part + ((int64_t)sp * NM + m) * np + grow, tot[m]);
    partials_written();
    if (!split_ticket(tickets, bx, splits)) return;
#pragma unroll
    for (int m = 0; m < NM; ++m) tot[m] = sum_splits(part + m * np + grow, NM * np, splits);
  }
  const int row = t * kTile + part_i * RW + lane;
  if (row >= n) return;
  if constexpr (SWIGLU) {
    const float h = silu(tot[0]) * tot[NM - 1];
    if (y != nullptr) y[row] = h;
    if (h16 != nullptr) h16[row] = __builtin_bit_cast(uint16_t, (f16)h);
  } else {
    y[row] = tot[0];
  }
}

// ------------------------------------------------------ fused RTN GEMV --
// Reads the fp16 masters, re-rounds every weight with the group's scale/zero
// as it is read (codes never stored), accumulates x * (q - z) per group and
// scales by s.  BITS == 16 is the unquantized control: x * w.
template <int BITS, int WAVES, int U>
__global__ __launch_bounds__(WAVES * 64) void k_gemv_fused(
    const uint16_t* __restrict__ w16, int64_t ld, const uint16_t* __restrict__ scale,
    const uint8_t* __restrict__ zero, const f16x2* __restrict__ x2, float* __restrict__ y,
    float* __restrict__ part, uint32_t* __restrict__ tickets,
    int n, int kb, int G, int splits, int kbps) {
  __shared__ float red[WAVES][64];
  const int lane = lane_id(), wave = wave_id();
  const int t = blockIdx.x, sp = blockIdx.y;
  const int row = t * kTile + lane;
  const int rrow = min(row, n - 1);
  const uint4* wr = reinterpret_cast<const uint4*>(w16 + (int64_t)rrow * ld);
  const int j0 = sp * kbps;
  const int j1 = min(kb, j0 + kbps);
  float yacc = 0.f;
  for (int jb = j0 + wave; jb < j1; jb += WAVES * U) {
    // as in k_gemv_packed: branch-free loads of all U blocks, x of the next
    // block fetched during the current block's work
    uint4 wvu[U][8];
    float su[U];
    int zu[U], jj[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * WAVES;
      jj[u] = j < j1 ? j : j1 - 1;
#pragma unroll
      for (int i = 0; i < 8; ++i) wvu[u][i] = wr[(int64_t)jj[u] * 8 + i];
      if constexpr (BITS != 16) {
        const int64_t mi = ((int64_t)t * G + ((G == 1) ? 0 : jj[u])) * kTile + lane;
        su[u] = masked_scale(scale[mi], j < j1);
        zu[u] = zero[mi];
      } else {
        su[u] = j < j1 ? 1.f : 0.f;
        zu[u] = 0;
      }
    }
    f16x2 xc[32], xn[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) xc[i] = x2[(int64_t)jj[0] * 32 + i];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u + 1 < U) {
#pragma unroll
        for (int i = 0; i < 32; ++i) xn[i] = x2[(int64_t)jj[u + 1] * 32 + i];
      }
      const uint4* wv = wvu[u];
      float a = 0.f, b = 0.f;
      if constexpr (BITS == 16) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a = __builtin_amdgcn_fdot2(as_h2(wv[i].x), xc[4 * i + 0], a, false);
          b = __builtin_amdgcn_fdot2(as_h2(wv[i].y), xc[4 * i + 1], b, false);
          a = __builtin_amdgcn_fdot2(as_h2(wv[i].z), xc[4 * i + 2], a, false);
          b = __builtin_amdgcn_fdot2(as_h2(wv[i].w), xc[4 * i + 3], b, false);
        }
      } else {
        constexpr int qmax = (1 << BITS) - 1;
        const RtnParams p = rtn_params(su[u], zu[u], qmax);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t uw[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
          float wf[8], q[8];
          bool tie = false;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f16x2 h = as_h2(uw[e]);
            wf[2 * e] = (float)h.x;
            wf[2 * e + 1] = (float)h.y;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            bool te;
            q[e] = rtn_raw(wf[e], p, te);
            tie |= te;
          }
          if (__builtin_amdgcn_ballot_w64(tie) != 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = rtn_fix(wf[e], q[e], p);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const auto pk = __builtin_amdgcn_cvt_pkrtz(clampf(q[2 * e], p.lo, p.hi),
                                                       clampf(q[2 * e + 1], p.lo, p.hi));
            const f16x2 h = __builtin_bit_cast(f16x2, pk);
            if (e & 1) b = __builtin_amdgcn_fdot2(h, xc[4 * i + e], b, false);
            else a = __builtin_amdgcn_fdot2(h, xc[4 * i + e], a, false);
          }
        }
      }
      yacc = __builtin_fmaf(su[u], a + b, yacc);
      if (u + 1 < U) {
#pragma unroll
        for (int i = 0; i < 32; ++i) xc[i] = xn[i];
      }
    }
  }
  red[wave][lane] = yacc;
  __syncthreads();
  if (wave != 0) return;
  float tot = red[0][lane];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) tot += red[w][lane];
  if (splits == 1) {
    if (row < n) y[row] = tot;
    return;
  }
  const int64_t np = (int64_t)gridDim.x * kTile;
  put_partial(part + (int64_t)sp * np + row, tot);
  partials_written();
  if (!split_ticket(tickets, t, splits)) return;
  const float acc = sum_splits(part + row, np, splits);
  if (row < n) y[row] = acc;
}

// Narrow form for launches of few tiles: a work-group covers 8 rows of a
// tile (grid.x = 8 x tiles); lane = 8*r + g takes weights 8g .. 8g+7 of row
// r's block, so a wave reads 8 whole 128-byte block rows per load.  Every
// weight is re-rounded exactly as in k_gemv_fused; the 8 lanes of a row add
// their sums in a fixed order.
template <int BITS, int WAVES, int U>
__global__ __launch_bounds__(WAVES * 64) void k_gemv_fused_narrow(
    const uint16_t* __restrict__ w16, int64_t ld, const uint16_t* __restrict__ scale,
    const uint8_t* __restrict__ zero, const f16x2* __restrict__ x2, float* __restrict__ y,
    float* __restrict__ part, uint32_t* __restrict__ tickets,
    int n, int kb, int G, int splits, int kbps) {
  constexpr int NG = 8, RW = kTile / NG;
  __shared__ float red[WAVES][RW];
  const int lane = lane_id(), wave = wave_id();
  const int r = lane / NG, g = lane % NG;
  const int bx = blockIdx.x, sp = blockIdx.y;
  const int t = bx / NG, part_i = bx % NG;
  const int R = part_i * RW + r;
  const int row = t * kTile + R;
  const int rrow = min(row, n - 1);
  const uint4* wr = reinterpret_cast<const uint4*>(w16 + (int64_t)rrow * ld) + g;
  const int j0 = sp * kbps;
  const int j1 = min(kb, j0 + kbps);
  float yacc = 0.f;
  for (int jb = j0 + wave; jb < j1; jb += WAVES * U) {
    uint4 wv[U], xv[U];
    uint16_t sr[U];
    int zu[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * WAVES;
      const int jj = j < j1 ? j : j1 - 1;      // past the range: re-read, scale 0
      wv[u] = wr[(int64_t)jj * 8];
      xv[u] = reinterpret_cast<const uint4*>(x2 + (int64_t)jj * 32)[g];
      if constexpr (BITS != 16) {
        const int64_t mi = ((int64_t)t * G + ((G == 1) ? 0 : jj)) * kTile + R;
        sr[u] = scale[mi];
        zu[u] = zero[mi];
      }
    }
    if constexpr (U > 1) loads_issued();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = jb + u * WAVES < j1;
      const uint32_t uw[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
      const f16x2 xs[4] = {as_h2(xv[u].x), as_h2(xv[u].y), as_h2(xv[u].z), as_h2(xv[u].w)};
      float a = 0.f, b = 0.f, s;
      if constexpr (BITS == 16) {
        s = valid ? 1.f : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (e & 1) b = __builtin_amdgcn_fdot2(as_h2(uw[e]), xs[e], b, false);
          else a = __builtin_amdgcn_fdot2(as_h2(uw[e]), xs[e], a, false);
        }
      } else {
        constexpr int qmax = (1 << BITS) - 1;
        s = masked_scale(sr[u], valid);
        const RtnParams p = rtn_params(s, zu[u], qmax);
        float wf[8], q[8];
        bool tie = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f16x2 h = as_h2(uw[e]);
          wf[2 * e] = (float)h.x;
          wf[2 * e + 1] = (float)h.y;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bool te;
          q[e] = rtn_raw(wf[e], p, te);
          tie |= te;
        }
        if (__builtin_amdgcn_ballot_w64(tie) != 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) q[e] = rtn_fix(wf[e], q[e], p);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const auto pk = __builtin_amdgcn_cvt_pkrtz(clampf(q[2 * e], p.lo, p.hi),
                                                     clampf(q[2 * e + 1], p.lo, p.hi));
          const f16x2 h = __builtin_bit_cast(f16x2, pk);
          if (e & 1) b = __builtin_amdgcn_fdot2(h, xs[e], b, false);
          else a = __builtin_amdgcn_fdot2(h, xs[e], a, false);
        }
      }
      yacc = __builtin_fmaf(s, a + b, yacc);
    }
  }
  yacc = slice_sum<NG>(yacc);
  if (g == 0) red[wave][r] = yacc;
  lds_barrier();
  if (wave != 0 || lane >= RW) return;
  float tot = red[0][lane];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) tot += red[w][lane];
  const int orow = t * kTile + part_i * RW + lane;
  if (splits > 1) {
    // part[split][launch row], launch row = RW * position + lane
    const int64_t np = (int64_t)gridDim.x * RW;
    const int64_t grow = (int64_t)bx * RW + lane;
    put_partial(part + (int64_t)sp * np + grow, tot);
    partials_written();
    if (!split_ticket(tickets, bx, splits)) return;
    tot = sum_splits(part + grow, np, splits);
  }
  if (orow < n) y[orow] = tot;
}

// ------------------------------------------------------ skinny GEMM (M<=16)
// v_mfma_f32_16x16x32_f16: A = X (16 rows, zero past m), B = W^T.  Lane
// (c = lane % 16, q = lane / 16) supplies row c and the 8 K-positions
// 16q + 8s .. +7 of the block for instruction s in {0, 1}; both operands use
// this same assignment of K positions, which therefore only permutes the sum.
// The output D[4q + r][c] of column group cg is Y[4q + r][tile*64 + 16cg + c].
template <int BITS>
__device__ __forceinline__ void load_quarter(const uint32_t* __restrict__ blk, int q, uint32_t* wl) {
  if constexpr (BITS == 4) {
    const uint2 v = reinterpret_cast<const uint2*>(blk)[q];
    wl[0] = v.x; wl[1] = v.y;
  } else if constexpr (BITS == 2) {
    wl[0] = blk[q];
  } else if constexpr (BITS == 8) {
    const uint4 v = reinterpret_cast<const uint4*>(blk)[q];
    wl[0] = v.x; wl[1] = v.y; wl[2] = v.z; wl[3] = v.w;
  } else {  // 3: low word 3*(q/2) + q%2, high word 3*(q/2) + 2
    const int run = q >> 1, u = q & 1;
    wl[0] = blk[3 * run + u];
    const uint32_t H = blk[3 * run + 2];
    wl[1] = u ? __builtin_amdgcn_alignbit(H, H, 8) : H;
  }
}

// The 8 codes of the lane's quarter for instruction s (0 or 1).
template <int BITS>
__device__ __forceinline__ f16x8 deq_quarter(const uint32_t* wl, int s, const Deq& d, uint32_t magic) {
  if constexpr (BITS == 4) {
    return deq_chunk4(wl[s], d, magic);
  } else if constexpr (BITS == 2) {
    return deq_chunk2(s ? (wl[0] >> 8) : wl[0], d, magic);
  } else if constexpr (BITS == 8) {
    return deq_chunk8(wl[2 * s], wl[2 * s + 1], d);
  } else {
    return deq_chunk3(s ? (wl[0] >> 8) : wl[0], s ? (wl[1] >> 1) : wl[1], d, magic);
  }
}

// Up to kMaxMats packed matrices that share K (and X), multiplied in one
// launch (q/k/v, or gate/up, of a prefill).  Launch columns are numbered
// consecutively over the matrices: matrix i owns columns [end[i-1], end[i])
// (a column is a 64-row tile for M <= 16, four tiles for the tiled GEMM).
struct GemmSet {
  const uint32_t* codes[kMaxMats];
  const uint16_t* scale[kMaxMats];
  const uint8_t* zero[kMaxMats];
  float* y[kMaxMats];
  int64_t ldy[kMaxMats];
  int n[kMaxMats];
  int end[kMaxMats];
  int count;
  uint16_t* h16;         // gate/up pairs: fp16 h (leading dimension ldy[0]), or null
};

struct GemmMat {
  const uint32_t* codes;
  const uint16_t* scale;
  const uint8_t* zero;
  float* y;
  int64_t ldy;
  int n, tiles, col;     // col: the launch column within the matrix
};

__device__ __forceinline__ GemmMat gemm_mat(const GemmSet& s, int x) {
  int i = 0;
  for (int k = 0; k + 1 < s.count; ++k)
    if (x >= s.end[k]) i = k + 1;
  GemmMat g;
  g.codes = s.codes[i];
  g.scale = s.scale[i];
  g.zero = s.zero[i];
  g.y = s.y[i];
  g.ldy = s.ldy[i];
  g.n = s.n[i];
  g.tiles = (g.n + kTile - 1) / kTile;
  g.col = x - (i == 0 ? 0 : s.end[i - 1]);
  return g;
}

// A wave's RB x 2 accumulator tiles of 32x32 (lane (c, h), element r: row
// m0 + 32rb + 8(r/4) + 4h + r%4, column t*64 + 32cb + c) stored into Y [m, ldy]
// of n columns.  A tile wholly inside Y takes no bounds checks and steps its
// row pointer by ldy.
template <int RB>
__device__ __forceinline__ void store_acc_tile(const f32x16 (&acc)[RB][2], float* __restrict__ y,
                                               int64_t ldy, int m, int n, int m0, int t, int c,
                                               int h) {
  float* ybase = y + (int64_t)(m0 + 4 * h) * ldy + t * kTile + c;
  if (m - m0 >= 32 * RB && (t + 1) * kTile <= n) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float* p = ybase + (int64_t)(32 * rb + 8 * q) * ldy;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[0] = acc[rb][0][4 * q + e];
          p[32] = acc[rb][1][4 * q + e];
          p += ldy;
        }
      }
    return;
  }
  const int mrem = m - m0 - 4 * h;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    if (t * kTile + 32 * cb + c >= n) continue;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dr = 32 * rb + 8 * (r >> 2) + (r & 3);
        if (dr < mrem) ybase[(int64_t)dr * ldy + 32 * cb] = acc[rb][cb][r];
      }
  }
}

template <int BITS, int WAVES, int U>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_skinny(
    const GemmSet set, const uint16_t* __restrict__ X, int64_t ldx, int m,
    float* __restrict__ part, uint32_t* __restrict__ tickets, int kb, int G, int splits,
    int kbps) {
  constexpr int WPB = 2 * BITS;
  constexpr int QW = (BITS == 3) ? 2 : BITS / 2;       // words held per quarter block
  __shared__ f32x4 red[WAVES][4][64];
  const uint32_t magic = vreg_const(kMagic);
  const int lane = lane_id(), wave = wave_id();
  const int c = lane & 15, q = lane >> 4;
  const GemmMat mat = gemm_mat(set, blockIdx.x);
  const uint32_t* __restrict__ codes = mat.codes;
  const uint16_t* __restrict__ scale = mat.scale;
  const uint8_t* __restrict__ zero = mat.zero;
  const int n = mat.n;
  const int t = mat.col, sp = blockIdx.y;
  const int tg = blockIdx.x;                 // launch tile (tickets, partials)
  const int j0 = sp * kbps;
  const int j1 = min(kb, j0 + kbps);
  f32x4 acc[4];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) acc[cg] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const bool xrow = c < m;
  const uint16_t* xr = X + (int64_t)(xrow ? c : 0) * ldx;
  // the fp16 range of the weight operand (maybe_wide): the work-group scans
  // its tile's scales over its K range in one round trip
  float fw[4] = {1.f, 1.f, 1.f, 1.f};
  {
    const int g0 = (G == 1) ? 0 : j0, ng = (G == 1) ? 1 : j1 - j0;
    const int tid = threadIdx.x;
    const uint16_t* st[1] = {scale + ((int64_t)t * G + g0) * kTile};
    uint32_t f8[1];
    wide_rows8<BITS, 1>(st, ng, tid, WAVES * 64, f8);
    if (__syncthreads_or(f8[0] != 0)) {
      // rare: OR the threads' row flags (thread t: rows 8 (t % 8) + e)
      __shared__ uint32_t fl[8];
      if (tid < 8) fl[tid] = 0;
      __syncthreads();
      if (f8[0] != 0) atomicOr(&fl[tid & 7], f8[0]);
      __syncthreads();
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        const int r = 16 * cg + c;
        if ((fl[r >> 3] >> (r & 7)) & 1u) fw[cg] = kWideScale;
      }
    }
  }
  for (int jb = j0 + wave; jb < j1; jb += WAVES * U) {
    uint4 xv[U][2];
    uint32_t wl[U][4][QW];
    float su[U][4];
    int zu[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * WAVES;
      if (j >= j1) continue;
      xv[u][0] = make_uint4(0, 0, 0, 0);
      xv[u][1] = make_uint4(0, 0, 0, 0);
      if (xrow) {
        const uint4* xp = reinterpret_cast<const uint4*>(xr + (int64_t)j * kBlock + 16 * q);
        xv[u][0] = xp[0];
        xv[u][1] = xp[1];
      }
      const int g = (G == 1) ? 0 : j;
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        const int r = 16 * cg + c;
        load_quarter<BITS>(codes + (((int64_t)t * kb + j) * kTile + r) * WPB, q, wl[u][cg]);
        const int64_t mi = ((int64_t)t * G + g) * kTile + r;
        su[u][cg] = h2f(scale[mi]);
        zu[u][cg] = zero[mi];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * WAVES;
      if (j >= j1) continue;
      const f16x8 a0 = u4_to_f16x8(xv[u][0]), a1 = u4_to_f16x8(xv[u][1]);
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        const Deq d = make_deq(su[u][cg] * fw[cg], zu[u][cg]);
        acc[cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, deq_quarter<BITS>(wl[u][cg], 0, d, magic),
                                                         acc[cg], 0, 0, 0);
        acc[cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, deq_quarter<BITS>(wl[u][cg], 1, d, magic),
                                                         acc[cg], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) red[wave][cg][lane] = acc[cg];
  __syncthreads();
  if (wave != 0) return;
  f32x4 tot[4];
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) {
    tot[cg] = red[0][cg][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) tot[cg] += red[w][cg][lane];
    tot[cg] *= unscale(fw[cg]);
  }
  const int64_t np = (int64_t)gridDim.x * kTile;
  if (splits > 1) {
    // part[split][16][np]
#pragma unroll
    for (int cg = 0; cg < 4; ++cg)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        put_partial(part + ((int64_t)sp * 16 + 4 * q + r) * np + tg * kTile + 16 * cg + c,
                    tot[cg][r]);
    partials_written();
    if (!split_ticket(tickets, tg, splits)) return;
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) tot[cg] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // split order; the 16 loads of one split are in flight together
    for (int s2 = 0; s2 < splits; ++s2) {
      float v[4][4];
#pragma unroll
      for (int cg = 0; cg < 4; ++cg)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v[cg][r] = get_partial(part + ((int64_t)s2 * 16 + 4 * q + r) * np + tg * kTile +
                                 16 * cg + c);
#pragma unroll
      for (int cg = 0; cg < 4; ++cg)
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[cg][r] += v[cg][r];
    }
  }
#pragma unroll
  for (int cg = 0; cg < 4; ++cg)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mrow = 4 * q + r, col = t * kTile + 16 * cg + c;
      if (mrow < m && col < n) mat.y[(int64_t)mrow * mat.ldy + col] = tot[cg][r];
    }
}

// ----------------------------------------------------- tiled GEMM (M>16) --
// v_mfma_f32_32x32x16_f16.  Work-group = 4 waves; wave w owns W tile
// blockIdx.x*4 + w (64 rows = two 32-column MFMA blocks), all MB rows of X.
// Register-staged form, used for 32-row X tiles (several work-groups per CU
// hide its load latency): X blocks go global -> registers -> LDS (fp16,
// double buffered, rows padded to 144 bytes); the weight operand is decoded
// straight from global memory into registers, so each code is read and
// decoded once per work-group.  Lane (c = lane % 32, h = lane / 32) supplies row c and the
// K positions 32h + 8s .. +7 of the block for instruction s in 0..3.
// D[8*(r/4) + 4*h + r%4][c] is acc register r.
constexpr int kLdsRow = 72;   // fp16 per padded LDS row

template <int BITS>
__device__ __forceinline__ void load_half(const uint32_t* __restrict__ blk, int h, uint32_t* wl) {
  if constexpr (BITS >= 5 && BITS <= 7) {
    // wl[0..3]: the 4-bit plane's half (words 4h..4h+3, read as two 8-byte
    // pairs: 5- and 7-bit rows are 8-byte aligned); then the high plane's half
    const uint2* b2 = reinterpret_cast<const uint2*>(blk) + 2 * h;
    const uint2 v = b2[0], u = b2[1];
    wl[0] = v.x; wl[1] = v.y; wl[2] = u.x; wl[3] = u.y;
    if constexpr (BITS == 5) wl[4] = blk[8 + h];
    else load_half<BITS - 4>(blk + 8, h, wl + 4);
  } else if constexpr (BITS == 4) {
    const uint4 v = reinterpret_cast<const uint4*>(blk)[h];
    wl[0] = v.x; wl[1] = v.y; wl[2] = v.z; wl[3] = v.w;
  } else if constexpr (BITS == 2) {
    const uint2 v = reinterpret_cast<const uint2*>(blk)[h];
    wl[0] = v.x; wl[1] = v.y;
  } else if constexpr (BITS == 8) {
    const uint4* b4 = reinterpret_cast<const uint4*>(blk) + 2 * h;
    const uint4 v = b4[0], u = b4[1];
    wl[0] = v.x; wl[1] = v.y; wl[2] = v.z; wl[3] = v.w;
    wl[4] = u.x; wl[5] = u.y; wl[6] = u.z; wl[7] = u.w;
  } else {
    wl[0] = blk[3 * h]; wl[1] = blk[3 * h + 1]; wl[2] = blk[3 * h + 2];
  }
}

template <int BITS>
__device__ __forceinline__ f16x8 deq_half(const uint32_t* wl, int s, const DeqT<BITS>& d,
                                          uint32_t magic) {
  if constexpr (BITS >= 5 && BITS <= 7) {
    f16x2 lo[4], hi[4];
    qz_chunk4(wl[s], d.lo, magic, lo);
    if constexpr (BITS == 5) {
      qz_chunk1(wl[4] >> (4 * s), d.hi, magic, hi);
    } else if constexpr (BITS == 6) {
      const uint32_t v = wl[4 + (s >> 1)];
      qz_chunk2((s & 1) ? (v >> 8) : v, d.hi, magic, hi);
    } else {
      const int u = s >> 1;
      const uint32_t L = wl[4 + u];
      const uint32_t Hu = u ? __builtin_amdgcn_alignbit(wl[6], wl[6], 8) : wl[6];
      qz_chunk3((s & 1) ? (L >> 8) : L, (s & 1) ? (Hu >> 1) : Hu, d.hi, magic, hi);
    }
    const f16x2 sixteen = {(f16)16.0f, (f16)16.0f};
#pragma unroll
    for (int p = 0; p < 4; ++p) lo[p] = __builtin_elementwise_fma(hi[p], sixteen, lo[p]);
    return scaled8(lo, d.lo.s);
  } else if constexpr (BITS == 4) {
    return deq_chunk4(wl[s], d, magic);
  } else if constexpr (BITS == 2) {
    const uint32_t v = wl[s >> 1];
    return deq_chunk2((s & 1) ? (v >> 8) : v, d, magic);
  } else if constexpr (BITS == 8) {
    return deq_chunk8(wl[2 * s], wl[2 * s + 1], d);
  } else {
    const int u = s >> 1;
    const uint32_t L = wl[u];
    const uint32_t Hu = u ? __builtin_amdgcn_alignbit(wl[2], wl[2], 8) : wl[2];
    return deq_chunk3((s & 1) ? (L >> 8) : L, (s & 1) ? (Hu >> 1) : Hu, d, magic);
  }
}

template <int BITS, int MB>
__global__ __launch_bounds__(256) void k_gemm_tiles(
    const GemmSet set, const uint16_t* __restrict__ X, int64_t ldx, int m, int kb, int G,
    int splits, int kbps, float* __restrict__ part, uint32_t* __restrict__ tickets) {
  constexpr int WPB = 2 * BITS;
  constexpr int HW = WPB / 2;               // words of a half block
  constexpr int RB = MB / 32;               // 32-row MFMA blocks of X
  constexpr int XCH = MB * 8 / 256;         // 16-byte X chunks per thread per block
  static_assert(XCH <= 8, "X staging covers at most 256 rows");
  __shared__ __attribute__((aligned(16))) f16 xs[2][MB][kLdsRow];
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = wave_id();
  const int c = lane & 31, h = lane >> 5;
  const GemmMat mat = gemm_mat(set, blockIdx.x);
  const uint32_t* __restrict__ codes = mat.codes;
  const uint16_t* __restrict__ scale = mat.scale;
  const uint8_t* __restrict__ zero = mat.zero;
  const int n = mat.n;
  const int t = mat.col * 4 + wave;
  const bool tvalid = t < mat.tiles;
  const int tt = tvalid ? t : 0;
  const int m0 = blockIdx.y * MB;
  const uint32_t magic = vreg_const(kMagic);
  // K-blocks [ja, ja + nk) of split blockIdx.z
  const int ja = blockIdx.z * kbps;
  const int nk = min(kb, ja + kbps) - ja;

  f32x16 acc[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;

  // Per-thread X chunk addresses.  Rows past m read row m0 instead: an X row
  // only feeds its own output row, which is never stored.  Likewise a wave
  // whose tile lies past n decodes tile 0 and stores nothing.
  const uint16_t* xsrc[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int ch = tid + 256 * i;
    const int row = ch >> 3, c8 = ch & 7;
    xsrc[i] = X + (int64_t)(m0 + row < m ? m0 + row : m0) * ldx + 8 * c8;
  }
  const uint32_t* wsrc[2];
  int64_t msrc[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int r = 32 * cb + c;
    wsrc[cb] = codes + ((int64_t)tt * kb * kTile + r) * WPB;
    msrc[cb] = (int64_t)tt * G * kTile + r;
  }
  // the fp16 range of the weight operand: scale factor of each column block
  // (set below, before the first decode) and whether any is scaled
  float fw[2];
  bool w_wide;
  u32x4 xv[2][XCH];
  uint32_t wl[2][2][HW];
  float sc[2][2];
  int zc[2][2];
  f16x8 bfrag[2][2][4];      // [register set][column block][slice]

  // Block data moves: issue (global -> registers, set p), land (registers ->
  // LDS buffer p and decoded B fragments of set p), mma (LDS buffer p and B
  // fragments of set p -> accumulators).  Set and buffer indices are
  // compile-time and the bodies are branch-free, so one block's decode can be
  // interleaved with the previous block's MFMAs.
  auto issue = [&](int jr, auto setc) __attribute__((always_inline)) {
    constexpr int P = decltype(setc)::value;
    const int j = ja + jr;
#pragma unroll
    for (int i = 0; i < XCH; ++i)
      xv[P][i] = *reinterpret_cast<const u32x4*>(xsrc[i] + (int64_t)j * kBlock);
    const int g = (G == 1) ? 0 : j;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      load_half<BITS>(wsrc[cb] + (int64_t)j * kTile * WPB, h, wl[P][cb]);
      sc[P][cb] = h2f(scale[msrc[cb] + (int64_t)g * kTile]);
      zc[P][cb] = zero[msrc[cb] + (int64_t)g * kTile];
    }
  };
  auto land_x = [&](auto setc, int i) __attribute__((always_inline)) {
    constexpr int P = decltype(setc)::value;
    const int ch = tid + 256 * i;
    const int row = ch >> 3, c8 = ch & 7;
    *reinterpret_cast<u32x4*>(&xs[P][row][8 * c8]) = xv[P][i];
  };
  // One K-slice of block P's MFMAs, then one slice of the next block's
  // decode (set Q) and X store: independent work placed between MFMAs so the
  // VALU and LDS work overlaps the 32-cycle matrix-core operations.
  auto step = [&](auto setc, auto nextc, bool decode_next) __attribute__((always_inline)) {
    constexpr int P = decltype(setc)::value;
    constexpr int Q = decltype(nextc)::value;
    DeqT<BITS> dn[2];
    if (decode_next) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) dn[cb] = make_deq_b<BITS>(sc[Q][cb] * fw[cb], zc[Q][cb]);
    }
    // A fragments of slice s4+1 are read from LDS while slice s4's MFMAs run.
    f16x8 a[2][RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      a[0][rb] = *reinterpret_cast<const f16x8*>(&xs[P][32 * rb + c][32 * h]);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      if (s4 < 3) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          a[(s4 + 1) & 1][rb] =
              *reinterpret_cast<const f16x8*>(&xs[P][32 * rb + c][32 * h + 8 * (s4 + 1)]);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[s4 & 1][rb], bfrag[P][cb][s4],
                                                               acc[rb][cb], 0, 0, 0);
      if (decode_next) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) bfrag[Q][cb][s4] = deq_half<BITS>(wl[Q][cb], s4, dn[cb], magic);
        if (s4 < XCH) land_x(nextc, s4);
        if (s4 + 4 < XCH) land_x(nextc, s4 + 4);
      }
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  // pipeline: block j computes while block j+1 is decoded and j+2 is loading;
  // prefetch indices are clamped to the last block (re-read, unused) so the
  // loop bodies have no branches.
  issue(0, S0{});
  issue(nk > 1 ? 1 : 0, S1{});
  // the fp16 range of the weight operand (maybe_wide): the wave scans its
  // tile's scales over the K range in one round trip, issued after the first
  // two blocks' loads so that the two round trips overlap
  {
    const int g0 = (G == 1) ? 0 : ja, ng = (G == 1) ? 1 : nk;
    const uint16_t* st[1] = {scale + ((int64_t)tt * G + g0) * kTile};
    uint32_t f8[1];
    wide_rows8<BITS, 1>(st, ng, lane, 64, f8);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) fw[cb] = wave_row_flag(f8[0], 32 * cb + c) ? kWideScale : 1.f;
    w_wide = __builtin_amdgcn_ballot_w64(f8[0] != 0) != 0;
  }

#pragma unroll
  for (int i = 0; i < XCH; ++i) land_x(S0{}, i);
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const DeqT<BITS> d = make_deq_b<BITS>(sc[0][cb] * fw[cb], zc[0][cb]);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) bfrag[0][cb][s4] = deq_half<BITS>(wl[0][cb], s4, d, magic);
  }
  __syncthreads();
  for (int j = 0;; j += 2) {
    step(S0{}, S1{}, true);           // block j; decode block j+1
    issue(min(j + 2, nk - 1), S0{});
    __syncthreads();
    if (j + 1 >= nk) break;
    step(S1{}, S0{}, true);           // block j+1; decode block j+2
    issue(min(j + 3, nk - 1), S1{});
    __syncthreads();
    if (j + 2 >= nk) break;
  }
  if (w_wide) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[rb][cb] *= unscale(fw[cb]);
  }

  if (splits > 1) {
    // The partial tile goes to the workspace in fragment order, [split][work-
    // group][fragment quad][thread] x 16 bytes, so every store and load moves
    // 4 KB of consecutive bytes per work-group; the last work-group of this
    // output tile to arrive adds the splits in order 0, 1, ... .
    constexpr int NQ = RB * 2 * 4;          // float4 quads per thread
    const int64_t wg = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    const int64_t groups = (int64_t)gridDim.x * gridDim.y;
    float* pw = part + ((blockIdx.z * groups + wg) * NQ * 256 + tid) * 4;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            put_partial(pw + ((rb * 2 + cb) * 4 + q) * 1024 + e, acc[rb][cb][4 * q + e]);
    partials_written();
    __syncthreads();
    __shared__ uint32_t s_last;
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(&tickets[wg], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == (uint32_t)(splits - 1);
      if (s_last) __hip_atomic_store(&tickets[wg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;
    const float* pr = part + (wg * NQ * 256 + tid) * 4;
    for (int s2 = 0; s2 < splits; ++s2) {
      f32x4 v[NQ];
#pragma unroll
      for (int i = 0; i < NQ; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[i][e] = get_partial(pr + ((int64_t)s2 * groups * NQ + i) * 1024 + e);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[rb][cb][4 * q + e] += v[(rb * 2 + cb) * 4 + q][e];
    }
  }

  if (!tvalid) return;
  store_acc_tile<RB>(acc, mat.y, mat.ldy, m, n, m0, t, c, h);
}

// ---------------------------------------- small-M GEMM (K split in the WG)
// For small M over few tiles: work-group = 32*RB rows of X x one 64-row W
// tile over its split's K range.  Its 4 waves take the K-blocks j0+w, j0+w+4, ...
// and issue the loads of up to U blocks (X A-fragments straight from global
// memory, codes, scales, zeros) before decoding any, so a short K range costs
// about one memory round trip; the 4 partial 32x64 tiles are then added in
// LDS in wave order.  Operand layout as in k_gemm_tiles (lane (c, h): X row
// 32rb + c / W row 32cb + c, K positions 32h + 8s .. +7 for instruction s).
// PAIR: the set is (gate, up) with equal n; each wave multiplies its X
// fragments by the same tile of both, the two tiles are reduced one after
// the other, and the output is h = silu(gate . x) * (up . x) in fp32 (y[0],
// if not null) and/or fp16 (set.h16), both with leading dimension ldy[0].
// DUAL: one matrix, and a work-group covers its tiles 2x and 2x + 1 (grid.x
// = tile pairs): each X fragment feeds twice the MFMAs, so a tall X tile over
// few tiles moves half the X bytes per MFMA through L1.
// CB = 1: a work-group covers one 32-row half of each tile (grid.x = half
// tiles, half = x mod 2), twice the work-groups for a grid too small to fill
// the chip.
template <int BITS, int U, int RB, bool PAIR = false, bool DUAL = false, int CB = 2,
          int WAVES = 4>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_ksplit(
    const GemmSet set, const uint16_t* __restrict__ X, int64_t ldx, int m, int kb, int G,
    int splits, int kbps, float* __restrict__ part, uint32_t* __restrict__ tickets) {
  constexpr int WPB = 2 * BITS;
  constexpr int HW = WPB / 2;                 // words of a half block
  constexpr int NE = RB * CB * 1024;         // elements of a wave's partial tile
  static_assert(CB == 1 || CB == 2, "column blocks per tile");
  static_assert(CB == 2 || !DUAL, "tile pairs take whole tiles");
  constexpr int NM = (PAIR || DUAL) ? 2 : 1; // tiles per work-group
  static_assert(!(PAIR && DUAL), "one of PAIR, DUAL");
  constexpr int NT = WAVES * 64;             // threads
  __shared__ float red[WAVES][NE];
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = wave_id();
  const int c = lane & 31, h = lane >> 5;
  const GemmMat mat = gemm_mat(set, blockIdx.x);
  // tile of each of the NM products (DUAL: a tile past the matrix re-reads
  // its last one and is not stored); column block of cb = cb0 + cb
  const int col = CB == 2 ? mat.col : mat.col >> 1;
  const int cb0 = CB == 2 ? 0 : mat.col & 1;
  int tm[NM], tl[NM];
#pragma unroll
  for (int mi = 0; mi < NM; ++mi) {
    tm[mi] = DUAL ? 2 * col + mi : col;
    tl[mi] = min(tm[mi], mat.tiles - 1);
  }
  const int m0 = blockIdx.y * 32 * RB;
  const uint32_t magic = vreg_const(kMagic);
  const int j0 = blockIdx.z * kbps;
  const int j1 = min(kb, j0 + kbps);
  // rows past m read row m0: an X row only feeds its own output row, never stored
  const uint16_t* xrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int xr = m0 + 32 * rb + c;
    xrow[rb] = X + (int64_t)(xr < m ? xr : m0) * ldx + 32 * h;
  }
  const uint32_t* wsrc[NM][CB];
  const uint16_t* ssrc[NM];
  const uint8_t* zsrc[NM];
#pragma unroll
  for (int mi = 0; mi < NM; ++mi) {
    const uint32_t* codes = PAIR ? set.codes[mi] : mat.codes;
    const int64_t mt = (int64_t)tl[mi] * G * kTile + c;
    ssrc[mi] = (PAIR ? set.scale[mi] : mat.scale) + mt;
    zsrc[mi] = (PAIR ? set.zero[mi] : mat.zero) + mt;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      wsrc[mi][cb] = codes + ((int64_t)tl[mi] * kb * kTile + 32 * (cb0 + cb) + c) * WPB;
  }
  f32x16 acc[NM][RB][CB];
#pragma unroll
  for (int mi = 0; mi < NM; ++mi)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][rb][cb][r] = 0.f;
  // The fp16 range of the weight operand (maybe_wide): a column whose
  // scales reach 65520 / qmax needs s * 2^-8 as its fp16 operand (and its
  // sums times 2^8).  The K loop decodes every column with s itself -- exact
  // for every other column, as a column's sums depend on its own operand
  // only -- and each thread keeps the largest |s| it loads for its columns
  // (smax, magnitude bits); after the loop the work-group ORs the flags, and a thread whose
  // column has such a scale computes that column's sums again with the
  // scaling (wide_dot; rare).  No scan of its own: scanning the scales
  // before the loop cost a memory round trip per launch (the Qwen3-8B M = 8
  // step 1.94 against 1.75 ms).
  uint32_t smax[NM][CB];
#pragma unroll
  for (int mi = 0; mi < NM; ++mi)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) smax[mi][cb] = 0;

  constexpr int step = WAVES * U;
  for (int jb = j0 + wave; jb < j1; jb += step) {
    f16x8 xa[U][RB][4];
    uint32_t wl[U][NM][CB][HW];
    uint16_t sr[U][NM][CB];
    int zc[U][NM][CB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + WAVES * u;
      const int jj = j < j1 ? j : j1 - 1;     // past the range: re-read, scale 0
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const f16x8* xp = reinterpret_cast<const f16x8*>(xrow[rb] + (int64_t)jj * kBlock);
#pragma unroll
        for (int s = 0; s < 4; ++s) xa[u][rb][s] = xp[s];
      }
      const int64_t g = (G == 1) ? 0 : jj;
#pragma unroll
      for (int mi = 0; mi < NM; ++mi)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          load_half<BITS>(wsrc[mi][cb] + (int64_t)jj * kTile * WPB, h, wl[u][mi][cb]);
          sr[u][mi][cb] = ssrc[mi][32 * (cb0 + cb) + g * kTile];
          zc[u][mi][cb] = zsrc[mi][32 * (cb0 + cb) + g * kTile];
        }
    }
    if constexpr (U > 1 || PAIR) loads_issued();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = jb + WAVES * u < j1;
#pragma unroll
      for (int mi = 0; mi < NM; ++mi)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          // (a block past the range gets scale 0; see masked_scale)
          const DeqT<BITS> d = make_deq_b<BITS>(
              h2f(sr[u][mi][cb]) * (valid ? 1.f : 0.f), zc[u][mi][cb]);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const f16x8 bf = deq_half<BITS>(wl[u][mi][cb], s, d, magic);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              acc[mi][rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xa[u][rb][s], bf,
                                                                       acc[mi][rb][cb], 0, 0, 0);
          }
        }
    }
    // the largest scale magnitude of this thread's columns (after the
    // decode, so that it does not change how the loads are scheduled)
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mi = 0; mi < NM; ++mi)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) smax[mi][cb] = max(smax[mi][cb], sr[u][mi][cb] & 0x7FFFu);
  }
  // The columns that need the operand scale: this thread's flags, OR-ed over
  // the work-group (bit c of wf[mi][cb]: column 32 (cb0 + cb) + c).
  uint32_t f = 0;
#pragma unroll
  for (int mi = 0; mi < NM; ++mi)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      if (maybe_wide<BITS>(h2f((uint16_t)smax[mi][cb]))) f |= 1u << (mi * CB + cb);
  bool wide[NM][CB];
#pragma unroll
  for (int mi = 0; mi < NM; ++mi)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) wide[mi][cb] = false;
  const bool any_wide = __syncthreads_or(f != 0);
  if (any_wide) {
    // rare
    __shared__ uint32_t wf[NM * CB];
    if (tid < NM * CB) wf[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NM * CB; ++q)
      if ((f >> q) & 1u) atomicOr(&wf[q], 1u << c);
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) wide[mi][cb] = (wf[mi * CB + cb] >> c) & 1u;
  }
  // The sums of matrix mi's column cl (0 .. 63 of its tile) for X row `row`
  // over this work-group's K range, with the operand scale: each weight as
  // the fp16 operand s 2^-8 (q - z) (one rounding of the exact product, as
  // the packed multiply forms it), times x, added in fp32; then times 2^8.
  auto wide_dot = [&](int mi, int row, int cl) {
    if (row >= m) return 0.f;
    const uint32_t* codes = PAIR ? set.codes[mi] : mat.codes;
    const uint16_t* scale = PAIR ? set.scale[mi] : mat.scale;
    const uint8_t* zero = PAIR ? set.zero[mi] : mat.zero;
    const uint16_t* xr = X + (int64_t)row * ldx;
    float sum = 0.f;
    for (int j = j0; j < j1; ++j) {
      const uint32_t* words = codes + (((int64_t)tl[mi] * kb + j) * kTile + cl) * WPB;
      const int64_t me = ((int64_t)tl[mi] * G + ((G == 1) ? 0 : j)) * kTile + cl;
      const float sj = h2f(scale[me]) * kWideScale;
      const int z = zero[me];
      for (int k = 0; k < kBlock; ++k) {
        const f16 w = (f16)(sj * (float)((int)code_at<BITS>(words, k) - z));
        sum += (float)w * h2f(xr[(int64_t)j * kBlock + k]);
      }
    }
    return sum * 256.f;
  };
  // element e = 1024 (CB rb + cb) + 64 r + lane of a wave's accumulators;
  // thread tid sums elements e = tid + NT i = lane + 64 (wave + WAVES i), so
  // (WAVES dividing 16) its block CB rb + cb = WAVES i / 16 is a constant and
  // its accumulator register r = (WAVES i) % 16 + wave is wave-uniform
  static_assert(NE % NT == 0 && 16 % WAVES == 0, "reduction split");
  constexpr int PT = NE / NT;                // elements per thread
  float v[NM][PT];
#pragma unroll
  for (int mi = 0; mi < NM; ++mi) {
    if (mi > 0) __syncthreads();             // the previous matrix's sums are read
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          red[wave][1024 * (CB * rb + cb) + 64 * r + lane] = acc[mi][rb][cb][r];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int e = tid + NT * i;
      float sum = red[0][e];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += red[w][e];   // wave order
      v[mi][i] = sum;
    }
    if (any_wide) {
      // (one copy of the rare loop, its result placed by an unrolled select)
#pragma nounroll
      for (int i = 0; i < PT; ++i) {
        const int rb = ((WAVES * i) >> 4) / CB, cb = ((WAVES * i) >> 4) % CB;
        const int r = ((WAVES * i) & 15) + wave;
        bool wc = false;
#pragma unroll
        for (int q = 0; q < CB; ++q) wc |= q == cb && wide[mi][q];
        if (!wc) continue;
        const float val = wide_dot(mi, m0 + 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3),
                                   32 * (cb0 + cb) + c);
#pragma unroll
        for (int q = 0; q < PT; ++q)
          if (q == i) v[mi][q] = val;
      }
    }
  }
  if (splits > 1) {
    // partials [split][work-group][matrix][element]; the last work-group of
    // this output tile to arrive adds the splits in order 0, 1, ...
    const int64_t wg = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    const int64_t groups = (int64_t)gridDim.x * gridDim.y;
    float* pw = part + (blockIdx.z * groups + wg) * NM * NE;
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
#pragma unroll
      for (int i = 0; i < PT; ++i) put_partial(pw + mi * NE + tid + NT * i, v[mi][i]);
    partials_written();
    __syncthreads();
    __shared__ uint32_t s_last;
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(&tickets[wg], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == (uint32_t)(splits - 1);
      if (s_last) __hip_atomic_store(&tickets[wg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
#pragma unroll
      for (int i = 0; i < PT; ++i)
        v[mi][i] = sum_splits(part + (wg * NM + mi) * NE + tid + NT * i, groups * NM * NE,
                              splits);
  }
  const int n = mat.n;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int rb = ((WAVES * i) >> 4) / CB, cb = ((WAVES * i) >> 4) % CB;
    const int r = ((WAVES * i) & 15) + wave;
    const int row = m0 + 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
    const int cl = 32 * (cb0 + cb) + c;
    if (row >= m) continue;
    if constexpr (PAIR) {
      const int col = tm[0] * kTile + cl;
      if (col >= n) continue;
      const int64_t o = (int64_t)row * mat.ldy + col;
      const float hv = silu(v[0][i]) * v[NM - 1][i];
      if (mat.y != nullptr) mat.y[o] = hv;
      if (set.h16 != nullptr) set.h16[o] = __builtin_bit_cast(uint16_t, (f16)hv);
    } else {
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) {
        const int col = tm[mi] * kTile + cl;
        if (col < n) mat.y[(int64_t)row * mat.ldy + col] = v[mi][i];
      }
    }
  }
}


// ------------------------------- GEMM, weights decoded once per work-group --
// Work-group = KG groups of 4 waves over 128 X rows x two 64-row W tiles
// (PAIR: tile t of gate and of up; otherwise tiles 2x and 2x + 1 of one matrix
// of the set, a tile past the matrix re-reading its last one and never
// stored).  Group g takes the K-blocks j0 + g, j0 + g + KG, ... of the
// work-group's range.  Per K-block, wave q of the group decodes column block q
// -- 32 W rows (32 (q % 2) + c of tile q / 2) x 64 K -- into the group's LDS
// buffers as the MFMA B fragments (lane (c, h), instruction s: K positions
// 32h + 8s .. +7), so each weight is decoded once per work-group; the group's
// 256 threads copy the block's 128 x 64 X tile into the same buffer with
// coalesced 16-byte loads (chunk k of row r at position k ^ (r % 8) of the
// row, so that these writes and the A-fragment reads fall on distinct
// banks); every wave of the group multiplies its 32 X rows (lane (c, h): X
// row 32q + c) by all four column blocks: 16 MFMAs per wave per K-block
// against one block decode.  The wave decodes its next block between the
// MFMAs of the current one, into the other of its group's two buffers: a wave
// that writes a buffer has passed the barrier that every wave reaches only
// after multiplying the block that buffer held before, so one barrier per
// step suffices.  The codes, scales, zeros and X chunks of the group's next
// D blocks are in flight meanwhile, in register slots (loads complete in
// order, so a wait for one load is a wait for every older one: everything a
// step waits for was requested D steps before).
// With KG = 2 each SIMD runs two instruction streams (one wave of each
// group); the groups meet at every step's barrier (a group with no block
// left in a step only takes part in the barrier) and finally add their sums
// through LDS, group 0's first; then group g finishes column half g of both
// tiles.
// The fp16 range of the operand as in k_gemm_ksplit: a decoding wave keeps
// its column's largest scale, and after the loop a flagged column's sums are
// computed again with the operand scale 2^-8.  Split K: partials per
// work-group in thread order, the last work-group of a tile adds the splits
// in order 0, 1, ...
template <int BITS, bool PAIR, int D, int KG>
__global__ __launch_bounds__(KG * 256) void k_gemm_wdec(
    const GemmSet set, const uint16_t* __restrict__ X, int64_t ldx, int m, int kb, int G,
    int splits, int kbps, float* __restrict__ part, uint32_t* __restrict__ tickets) {
  constexpr int WPB = 2 * BITS;
  constexpr int HW = WPB / 2;                // words of a half block
  static_assert(D == 2 || D == 4 || D == 8, "blocks in flight");
  static_assert(KG == 1 || KG == 2, "K groups");
  __shared__ f16x8 frag[KG][2][16][64];      // [group][buffer][4 column block + s][lane]
  __shared__ f16x8 xs[KG][2][128 * 8];       // [group][buffer][X row: 8 chunks of 16 bytes]
  __shared__ uint32_t wf[4];
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = wave_id();
  const int grp = wave >> 2, q = wave & 3;   // K group, wave within it
  const int c = lane & 31, h = lane >> 5;
  const GemmMat mat = gemm_mat(set, blockIdx.x);
  int tm[2], tl[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    tm[mi] = PAIR ? mat.col : 2 * mat.col + mi;
    tl[mi] = min(tm[mi], mat.tiles - 1);
  }
  const uint32_t magic = vreg_const(kMagic);
  const int j0 = blockIdx.z * kbps;
  const int j1 = min(kb, j0 + kbps);
  // this group's blocks: jg, jg + KG, ... (cnt of them); steps = the first
  // group's count, so that every wave meets the same barriers
  const int jg = j0 + grp;
  const int cnt = jg < j1 ? (j1 - jg + KG - 1) / KG : 0;
  const int steps = (j1 - j0 + KG - 1) / KG;
  // the column block this wave decodes: tile dm, rows 32 dcb ..
  const int dm = q >> 1, dcb = q & 1;
  const uint32_t* dcodes = PAIR ? (dm ? set.codes[1] : set.codes[0]) : mat.codes;
  const uint16_t* dscale = PAIR ? (dm ? set.scale[1] : set.scale[0]) : mat.scale;
  const uint8_t* dzero = PAIR ? (dm ? set.zero[1] : set.zero[0]) : mat.zero;
  const int dt = dm ? tl[1] : tl[0];
  const uint32_t* wsrc = dcodes + ((int64_t)dt * kb * kTile + 32 * dcb + c) * WPB;
  const int64_t mt = (int64_t)dt * G * kTile + 32 * dcb + c;
  const uint16_t* ssrc = dscale + mt;
  const uint8_t* zsrc = dzero + mt;
  // X staging: thread t of the group copies the 16-byte chunks xk = t % 8 of
  // rows t / 8 + 32i (i = 0..3) of the block's 128 x 64 X tile into LDS, where
  // chunk k of row r sits at position k ^ (r % 8) of the row, so that both
  // these writes and the A-fragment reads (lanes c = 0..7 of a wave: rows
  // r + c, one chunk each) fall on distinct banks; rows past m read row m0
  // (never stored)
  const int m0 = blockIdx.y * 128;
  const int t8 = (tid & 255) >> 3, xk = tid & 7;
  const uint16_t* xsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = m0 + t8 + 32 * i;
    xsrc[i] = X + (int64_t)(r < m ? r : m0) * ldx + 8 * xk;
  }
  const int xw = 8 * t8 + (xk ^ (t8 & 7));
  f16x8(*gfrag)[16][64] = frag[KG == 1 ? 0 : grp];
  f16x8(*gxs)[128 * 8] = xs[KG == 1 ? 0 : grp];

  uint32_t wl[D][HW];
  uint16_t sr[D];
  int zc[D];
  f16x8 xg[D][4];
  uint32_t smax = 0;
  // The group's block i (clamped to its last) into register slot u: this
  // thread's codes, scale and zero, and its four X chunks.  Both are requested
  // D steps ahead: loads complete in order, so a wait for one load is a wait
  // for every older one as well.
  auto request = [&](auto U, int i) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    const int jj = min(jg + KG * max(0, min(i, cnt - 1)), j1 - 1);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      xg[u][k] = *reinterpret_cast<const f16x8*>(xsrc[k] + (int64_t)jj * kBlock);
    load_half<BITS>(wsrc + (int64_t)jj * kTile * WPB, h, wl[u]);
    const int64_t g = (G == 1) ? 0 : jj;
    sr[u] = ssrc[g * kTile];
    zc[u] = zsrc[g * kTile];
  };
  // slot u's X chunks into the LDS buffer b
  auto store_x = [&](auto U, int b) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
#pragma unroll
    for (int k = 0; k < 4; ++k) gxs[b][xw + 256 * k] = xg[u][k];
  };
  auto deq_of = [&](auto U) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    smax = max(smax, (uint32_t)(sr[u] & 0x7FFFu));
    return make_deq_b<BITS>(h2f(sr[u]), zc[u]);
  };

  f32x16 acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[f][r] = 0.f;
  // prologue: the group's first D blocks of codes and the X of its first
  // block requested, its first block decoded into buffer 0, the codes of its
  // block D requested into that slot
  request(std::integral_constant<int, 0>(), 0);
  request(std::integral_constant<int, 1>(), 1);
  if constexpr (D > 2) {
    request(std::integral_constant<int, 2>(), 2);
    request(std::integral_constant<int, 3>(), 3);
  }
  if constexpr (D > 4) {
    request(std::integral_constant<int, 4>(), 4);
    request(std::integral_constant<int, 5>(), 5);
    request(std::integral_constant<int, 6>(), 6);
    request(std::integral_constant<int, 7>(), 7);
  }
  loads_issued();
  if (cnt > 0) {
    const DeqT<BITS> d = deq_of(std::integral_constant<int, 0>());
#pragma unroll
    for (int s = 0; s < 4; ++s)
      gfrag[0][4 * q + s][lane] = deq_half<BITS>(wl[0], s, d, magic);
  }
  store_x(std::integral_constant<int, 0>(), 0);
  request(std::integral_constant<int, 0>(), D);
  loads_issued();
  lds_barrier();
  // Step i (the group's block i: its X tile and B fragments in buffer i % 2):
  // the wave multiplies block i while it decodes block i + 1 (register slot
  // (i + 1) % D) into the other buffer, stores its X chunks of block i + 1
  // there, requests block i + 1 + D into that slot, and meets every wave at
  // the barrier.  `have`: block i exists;
  // `more`: block i + 1 exists; `sync`: step i + 1 exists.
  auto step = [&](auto U, int i, bool have, bool more, bool sync) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    constexpr int un = (u + 1) % D;
    const std::integral_constant<int, un> UN;
    f16x8(*fb)[64] = gfrag[i & 1];
    const f16x8* xb = gxs[i & 1] + 8 * (32 * q + c);
    f16x8(*fn)[64] = gfrag[(i + 1) & 1];
    DeqT<BITS> d;
    if (more) d = deq_of(UN);
    if (have) {
      f16x8 bq[2][4];
#pragma unroll
      for (int f = 0; f < 4; ++f) bq[0][f] = fb[4 * f][lane];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const f16x8 a = xb[(4 * h + s) ^ (c & 7)];
        if (s + 1 < 4) {
#pragma unroll
          for (int f = 0; f < 4; ++f) bq[(s + 1) & 1][f] = fb[4 * f + s + 1][lane];
        }
#pragma unroll
        for (int f = 0; f < 4; ++f)
          acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bq[s & 1][f], acc[f], 0, 0, 0);
        if (more) fn[4 * q + s][lane] = deq_half<BITS>(wl[un], s, d, magic);
      }
    }
    if (more) {
      store_x(UN, (i + 1) & 1);
      request(UN, i + 1 + D);
    }
    loads_issued();
    if (sync) lds_barrier();
  };
  // full rounds of D steps in which every group has its block and the next,
  // then the rest
  const int full = (KG == 1 ? cnt : min(cnt, (j1 - j0) / KG)) - 1;   // steps with `more` in all groups
  int i0 = 0;
  for (; i0 + D <= full; i0 += D) {
    step(std::integral_constant<int, 0>(), i0, true, true, true);
    step(std::integral_constant<int, 1>(), i0 + 1, true, true, true);
    if constexpr (D > 2) {
      step(std::integral_constant<int, 2>(), i0 + 2, true, true, true);
      step(std::integral_constant<int, 3>(), i0 + 3, true, true, true);
    }
    if constexpr (D > 4) {
      step(std::integral_constant<int, 4>(), i0 + 4, true, true, true);
      step(std::integral_constant<int, 5>(), i0 + 5, true, true, true);
      step(std::integral_constant<int, 6>(), i0 + 6, true, true, true);
      step(std::integral_constant<int, 7>(), i0 + 7, true, true, true);
    }
  }
  // the remaining steps i0 .. steps - 1 (fewer than 2D)
#pragma unroll
  for (int r = 0; r < 2 * D; ++r) {
    const int i = i0 + r;
    if (i >= steps) break;
    // (slot (i0 + r) % D = r % D: i0 is a multiple of D)
    auto go = [&](auto U) __attribute__((always_inline)) {
      step(U, i, i < cnt, i + 1 < cnt, i + 1 < steps);
    };
    switch (r % D) {
      case 0: go(std::integral_constant<int, 0>()); break;
      case 1: go(std::integral_constant<int, 1 % D>()); break;
      case 2: go(std::integral_constant<int, 2 % D>()); break;
      case 3: go(std::integral_constant<int, 3 % D>()); break;
      case 4: go(std::integral_constant<int, 4 % D>()); break;
      case 5: go(std::integral_constant<int, 5 % D>()); break;
      case 6: go(std::integral_constant<int, 6 % D>()); break;
      default: go(std::integral_constant<int, 7 % D>()); break;
    }
  }

  // Column blocks this thread finishes: all four (KG = 1), or half g of both
  // tiles (f = g, 2 + g) in group g, after the groups add their sums.
  auto keep = [&](int f) __attribute__((always_inline)) { return KG == 1 || (f & 1) == grp; };
  if constexpr (KG == 2) {
    // every wave is past its last multiply before the buffers are reused
    lds_barrier();
    float* red = reinterpret_cast<float*>(&frag[0][0][0][0]);   // [group][2][16][256]
    const int t = tid & 255;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (keep(f)) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((grp * 2 + (f >> 1)) * 16 + r) * 256 + t] = acc[f][r];
    }
    lds_barrier();
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (!keep(f)) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[f][r] += red[(((1 - grp) * 2 + (f >> 1)) * 16 + r) * 256 + t];
    }
  }

  // Columns that need the operand scale: bit c of wf[q] for column c of
  // column block q (found by the waves that decode it).
  const bool mine = maybe_wide<BITS>(h2f((uint16_t)smax));
  if (__syncthreads_or(mine)) {
    // rare
    if (tid < 4) wf[tid] = 0;
    __syncthreads();
    if (mine) atomicOr(&wf[q], 1u << c);
    __syncthreads();
    uint32_t fl[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) fl[f] = keep(f) ? wf[f] : 0u;
#pragma nounroll
    for (int i = 0; i < 64; ++i) {
      const int f = i >> 4, r = i & 15;
      const uint32_t ff = f == 0 ? fl[0] : f == 1 ? fl[1] : f == 2 ? fl[2] : fl[3];
      if (!((ff >> c) & 1u)) continue;
      const int row = m0 + 32 * q + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row >= m) continue;
      const int mi = f >> 1, cl = 32 * (f & 1) + c;
      const uint32_t* codes = PAIR ? (mi ? set.codes[1] : set.codes[0]) : mat.codes;
      const uint16_t* scale = PAIR ? (mi ? set.scale[1] : set.scale[0]) : mat.scale;
      const uint8_t* zero = PAIR ? (mi ? set.zero[1] : set.zero[0]) : mat.zero;
      const int t = mi ? tl[1] : tl[0];
      const uint16_t* xw = X + (int64_t)row * ldx;
      // each weight as the fp16 operand s 2^-8 (q - z), times x, added in
      // fp32, then times 2^8
      float sum = 0.f;
      for (int j = j0; j < j1; ++j) {
        const uint32_t* words = codes + (((int64_t)t * kb + j) * kTile + cl) * WPB;
        const int64_t me = ((int64_t)t * G + ((G == 1) ? 0 : j)) * kTile + cl;
        const float sj = h2f(scale[me]) * kWideScale;
        const int z = zero[me];
        for (int k = 0; k < kBlock; ++k) {
          const f16 w = (f16)(sj * (float)((int)code_at<BITS>(words, k) - z));
          sum += (float)w * h2f(xw[(int64_t)j * kBlock + k]);
        }
      }
      sum *= 256.f;
#pragma unroll
      for (int e = 0; e < 64; ++e)
        if (e == i) acc[e >> 4][e & 15] = sum;
    }
  }

  if (splits > 1) {
    // partials [split][work-group][4 column block + register][thread of the group]
    constexpr int NE = 4 * 16 * 256;
    const int t = tid & 255;
    const int64_t wg = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    const int64_t groups = (int64_t)gridDim.x * gridDim.y;
    float* pw = part + (blockIdx.z * groups + wg) * NE + t;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (!keep(f)) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) put_partial(pw + (f * 16 + r) * 256, acc[f][r]);
    }
    partials_written();
    __syncthreads();
    __shared__ uint32_t s_last;
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(&tickets[wg], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == (uint32_t)(splits - 1);
      if (s_last) __hip_atomic_store(&tickets[wg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    // one column block at a time, the loads of up to 8 splits in flight
    const float* pr = part + wg * NE + t;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (!keep(f)) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[f][r] = 0.f;
      for (int b = 0; b < splits; b += 8) {
        float v[8][16];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            v[i][r] = get_partial(pr + (int64_t)min(b + i, splits - 1) * groups * NE +
                                  (f * 16 + r) * 256);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (b + i < splits)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][r] += v[i][r];
      }
    }
  }

  // element r of column block f: row m0 + 32q + 8 (r / 4) + 4h + r % 4,
  // column 32 (f % 2) + c of tile tm[f / 2]
  const int n = mat.n;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = m0 + 32 * q + 8 * (r >> 2) + 4 * h + (r & 3);
    if (row >= m) continue;
    if constexpr (PAIR) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        if (!keep(cb)) continue;
        const int col = tm[0] * kTile + 32 * cb + c;
        if (col >= n) continue;
        const int64_t o = (int64_t)row * mat.ldy + col;
        const float hv = silu(acc[cb][r]) * acc[2 + cb][r];
        if (mat.y != nullptr) mat.y[o] = hv;
        if (set.h16 != nullptr) set.h16[o] = __builtin_bit_cast(uint16_t, (f16)hv);
      }
    } else {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if (!keep(f)) continue;
        const int col = tm[f >> 1] * kTile + 32 * (f & 1) + c;
        if (col < n) mat.y[(int64_t)row * mat.ldy + col] = acc[f][r];
      }
    }
  }
}


// ------------------------------------------------- embedding-row gather --
// Rows ids[i] of a packed weight, dequantized: out32 = s*(q - z) (exact in
// fp32), out16 = that value rounded to fp16 (nearest even).  One work-group
// per id; thread = 8 consecutive columns.  An id outside [0, n) gives a row of
// zeros.
template <int BITS>
__global__ __launch_bounds__(256) void k_embed_rows(
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scale,
    const uint8_t* __restrict__ zero, const int32_t* __restrict__ ids, int n, int kb, int G,
    uint16_t* __restrict__ out16, float* __restrict__ out32, int64_t ld_out) {
  constexpr int WPB = 2 * BITS;
  const int id = ids[blockIdx.x];
  const bool valid = id >= 0 && id < n;
  const int r = valid ? id : 0;
  const int t = r / kTile, rl = r % kTile;
  for (int c8 = threadIdx.x; c8 < kb * 8; c8 += 256) {
    const int j = c8 >> 3, c0 = (c8 & 7) * 8;
    const uint32_t* words = codes + (((int64_t)t * kb + j) * kTile + rl) * WPB;
    const int64_t mi = ((int64_t)t * G + ((G == 1) ? 0 : j)) * kTile + rl;
    const float s = valid ? h2f(scale[mi]) : 0.f;
    const int z = zero[mi];
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = s * (float)((int)code_at<BITS>(words, c0 + e) - z);
    const int64_t o = (int64_t)blockIdx.x * ld_out + 8 * c8;
    if (out32 != nullptr) {
      f32x4* d = reinterpret_cast<f32x4*>(out32 + o);
      d[0] = (f32x4){v[0], v[1], v[2], v[3]};
      d[1] = (f32x4){v[4], v[5], v[6], v[7]};
    }
    if (out16 != nullptr) {
      f16x8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (f16)v[e];
      *reinterpret_cast<f16x8*>(out16 + o) = h;
    }
  }
}

// ------------------------------------------ tiled GEMM, LDS-DMA pipeline --
// Same tiling and MFMA lane layout as k_gemm_tiles; the difference is how the
// operands arrive.  Every K-block's X tile (MB x 64 fp16), the four 64-row
// code blocks and their scales/zeros are copied global -> LDS by the
// direct-to-LDS loads of gfx950 (global_load_lds_dword[x4]), S blocks
// deep, into S separate LDS stages: no registers hold data in flight, so the
// loads of block j + S - 1 are issued while block j computes and the memory
// latency is hidden behind S - 1 blocks of MFMA work.  Each wave copies a
// quarter of the X tile and its own tile's codes and metadata.  The 16-byte
// chunks of X rows and of 4- and 8-bit code rows are XOR-swizzled in LDS (the
// direct-to-LDS loads pick their global source per lane accordingly) so that
// the fragment reads of 8 or 16 consecutive lanes touch distinct banks.
// f(std::integral_constant<int, I>) for I = B .. E-1, unrolled.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// One direct-to-LDS load of SZ bytes per lane: lane l's bytes land at
// lds + SZ * l (lds wave-uniform).
template <int SZ>
__device__ __forceinline__ void dma_to_lds(const void* src, void* lds) {
  typedef __attribute__((address_space(3))) void lds_void;
  static_assert(SZ == 4 || SZ == 16, "direct-to-LDS load size");
  if constexpr (SZ == 16) __builtin_amdgcn_global_load_lds(src, (lds_void*)lds, 16, 0, 0);
  else __builtin_amdgcn_global_load_lds(src, (lds_void*)lds, 4, 0, 0);
}

// LDS slot (16-byte chunk within the row) of X chunk c8 of row r: distinct
// for the 8 consecutive rows, and for the 8 even or 8 odd rows of 16
// consecutive rows, that one A-fragment read touches.
__device__ __forceinline__ int xswz(int r, int c8) { return c8 ^ (r & 7) ^ ((r >> 3) & 1); }

// Code rows of P = 2*BITS/4 chunks (4 bits: 2, 8 bits: 4): chunk e of row r
// sits in slot P*r + (e ^ cswz(r)); a B-fragment read of lanes c = 0..15
// (rows c, one chunk index each) then hits distinct banks.
template <int BITS>
__device__ __forceinline__ int cswz(int r) {
  if constexpr (BITS == 4) return ((r >> 2) ^ (r >> 3)) & 1;
  else if constexpr (BITS == 8) return ((r >> 1) ^ (r >> 2)) & 3;
  else return 0;
}
template <int BITS> constexpr bool kCodeSwz = BITS == 4 || BITS == 8;

template <int BITS, int MB>
struct GemmStage {
  f16 x[MB * 64];                    // X tile, swizzled 16-byte chunks
  uint32_t w[4][64 * 2 * BITS];      // codes of the four tiles' block, as in HBM
  uint32_t meta[4][64];              // per tile: 64 fp16 scales, then 64 uint8 zeros
};

// One LDS variable per stage (distinct objects let the compiler track which
// direct-to-LDS loads a read depends on).
template <int BITS, int MB, int I>
__device__ __forceinline__ GemmStage<BITS, MB>& gemm_stage() {
  __shared__ __attribute__((aligned(16))) GemmStage<BITS, MB> st;
  return st;
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt not waited on); gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Direct-to-LDS load pieces per wave for one tile's code block (64 rows x
// 2*BITS words): {bytes per lane, instructions}.  (The 3-byte-per-code
// block, 1536 bytes, goes as dwords.)
template <int BITS> struct WDma;
template <> struct WDma<2> { static constexpr int SZ = 16, N = 1; };
template <> struct WDma<3> { static constexpr int SZ = 4, N = 6; };
template <> struct WDma<4> { static constexpr int SZ = 16, N = 2; };
template <> struct WDma<8> { static constexpr int SZ = 16, N = 4; };
template <> struct WDma<5> { static constexpr int SZ = 4, N = 10; };
template <> struct WDma<6> { static constexpr int SZ = 16, N = 3; };
template <> struct WDma<7> { static constexpr int SZ = 4, N = 14; };

// PAIR: the set is (gate, up) with equal n, and a work-group covers two
// 64-row tiles of each: waves 0 and 1 multiply gate tiles 2x and 2x + 1,
// waves 2 and 3 the same tiles of up.  After the K loop each gate wave and
// the up wave of its tile swap halves of their accumulators through the
// (then idle) LDS stages, one 32-row block at a time: the gate wave finishes
// columns 0-31 of the tile, the up wave columns 32-63, each writing
// h = silu(g) * u in fp32 (y[0], if not null) and/or fp16 (set.h16),
// leading dimension ldy[0].
template <int BITS, int MB, int S, bool PAIR = false>
__global__ __launch_bounds__(256, 2) void k_gemm_lds(
    const GemmSet set, const uint16_t* __restrict__ X, int64_t ldx, int m, int kb, int G,
    int splits, int kbps, float* __restrict__ part, uint32_t* __restrict__ tickets) {
  constexpr int WPB = 2 * BITS;
  constexpr int RB = MB / 32;               // 32-row MFMA blocks of X
  constexpr int XQ = MB / 32;               // X pieces (16 B) per thread per block
  constexpr int NDMA = XQ + WDma<BITS>::N + 1;
  static_assert(S >= 2 && (S - 1) * NDMA < 64, "stages");
  static_assert(WDma<BITS>::SZ * 64 * WDma<BITS>::N == 64 * WPB * 4, "code block pieces");
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = wave_id();
  const int c = lane & 31, h = lane >> 5;
  const GemmMat mat = gemm_mat(set, blockIdx.x);
  const int mi = PAIR ? (wave >> 1) : 0;
  const uint32_t* __restrict__ codes = PAIR ? set.codes[mi] : mat.codes;
  const uint16_t* __restrict__ scale = PAIR ? set.scale[mi] : mat.scale;
  const uint8_t* __restrict__ zero = PAIR ? set.zero[mi] : mat.zero;
  const int n = mat.n;
  const int t = PAIR ? mat.col * 2 + (wave & 1) : mat.col * 4 + wave;
  const bool tvalid = t < mat.tiles;
  const int tt = tvalid ? t : 0;
  const int m0 = blockIdx.y * MB;
  const uint32_t magic = vreg_const(kMagic);
  const int ja = blockIdx.z * kbps;
  const int nk = min(kb, ja + kbps) - ja;

  // per-lane global sources of this lane's pieces (block 0 of the range)
  const char* xsrc[XQ];
#pragma unroll
  for (int i = 0; i < XQ; ++i) {
    const int q = tid + 256 * i;            // LDS position of the piece
    const int row = q >> 3, c8 = xswz(row, q & 7);
    const int xr = m0 + row < m ? m0 + row : m0;
    xsrc[i] = reinterpret_cast<const char*>(X + (int64_t)xr * ldx + 8 * c8);
  }
  const char* wsrc = reinterpret_cast<const char*>(codes + (int64_t)tt * kb * kTile * WPB);
  // source byte offset (within the code block) of this lane's piece i
  int woff[WDma<BITS>::N];
#pragma unroll
  for (int i = 0; i < WDma<BITS>::N; ++i) {
    const int slot = 64 * i + lane;
    if constexpr (kCodeSwz<BITS>) {
      constexpr int P = WPB / 4;
      const int r = slot / P;
      woff[i] = 16 * (P * r + ((slot % P) ^ cswz<BITS>(r)));
    } else {
      woff[i] = slot * WDma<BITS>::SZ;
    }
  }
  // metadata piece: lanes 0-31 two scales each, lanes 32-63 four zeros each
  // (lanes 48-63 repeat 32-47 into the unused upper quarter)
  const char* msrc = lane < 32
      ? reinterpret_cast<const char*>(scale + (int64_t)tt * G * kTile) + 4 * lane
      : reinterpret_cast<const char*>(zero + (int64_t)tt * G * kTile) + 4 * ((lane - 32) & 15);

  auto issue = [&](int j, auto stc) __attribute__((always_inline)) {
    constexpr int I = decltype(stc)::value;
    GemmStage<BITS, MB>& st = gemm_stage<BITS, MB, I>();
    const int jg = ja + j;
#pragma unroll
    for (int i = 0; i < XQ; ++i)
      dma_to_lds<16>(xsrc[i] + (int64_t)jg * kBlock * 2, st.x + (256 * i + 64 * wave) * 8);
#pragma unroll
    for (int i = 0; i < WDma<BITS>::N; ++i)
      dma_to_lds<WDma<BITS>::SZ>(wsrc + ((int64_t)jg * kTile * WPB) * 4 + woff[i],
                                 reinterpret_cast<char*>(st.w[wave]) + i * 64 * WDma<BITS>::SZ);
    const int64_t g = (G == 1) ? 0 : jg;
    dma_to_lds<4>(msrc + (lane < 32 ? g * kTile * 2 : g * kTile), st.meta[wave]);
  };

  f32x16 acc[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;
  // the fp16 range of the weight operand over the K range (maybe_wide): the
  // wave owns its columns; set after the prologue is issued (below), so the
  // scan's round trip overlaps the first blocks' loads
  float fw[2];
  bool w_wide;

  // Block j from stage I: decode this wave's B operand from the staged codes
  // slice by slice, interleaved with the MFMAs of the previous slice.
  auto compute = [&](auto stc) __attribute__((always_inline)) {
    constexpr int I = decltype(stc)::value;
    const GemmStage<BITS, MB>& st = gemm_stage<BITS, MB, I>();
    uint32_t wl[2][BITS];
    DeqT<BITS> d[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int r = 32 * cb + c;
      if constexpr (BITS == 4) {
        const uint4 v = reinterpret_cast<const uint4*>(st.w[wave])[2 * r + (h ^ cswz<4>(r))];
        wl[cb][0] = v.x; wl[cb][1] = v.y; wl[cb][2] = v.z; wl[cb][3] = v.w;
      } else if constexpr (BITS == 8) {
        const uint4* w4 = reinterpret_cast<const uint4*>(st.w[wave]) + 4 * r;
        const uint4 v = w4[(2 * h) ^ cswz<8>(r)], u = w4[(2 * h + 1) ^ cswz<8>(r)];
        wl[cb][0] = v.x; wl[cb][1] = v.y; wl[cb][2] = v.z; wl[cb][3] = v.w;
        wl[cb][4] = u.x; wl[cb][5] = u.y; wl[cb][6] = u.z; wl[cb][7] = u.w;
      } else {
        load_half<BITS>(st.w[wave] + r * WPB, h, wl[cb]);
      }
      const uint16_t sb = reinterpret_cast<const uint16_t*>(st.meta[wave])[r];
      const int zb = reinterpret_cast<const uint8_t*>(st.meta[wave])[128 + r];
      d[cb] = make_deq_b<BITS>(h2f(sb) * fw[cb], zb);
    }
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      f16x8 a[RB], b[2];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = 32 * rb + c, c8 = xswz(row, 4 * h + s4);
        a[rb] = *reinterpret_cast<const f16x8*>(st.x + row * 64 + 8 * c8);
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) b[cb] = deq_half<BITS>(wl[cb], s4, d[cb], magic);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[rb], b[cb], acc[rb][cb], 0, 0, 0);
    }
    // let the scheduler interleave the LDS operand reads with the MFMAs
    // (measured ~1 % on the 128-row pipeline)
    __builtin_amdgcn_iglp_opt(0);
  };

  // Wait until this wave's loads of block j are in LDS (rem = blocks issued
  // after it), then a barrier makes every wave's part visible; the stage
  // freed by block j-1 is refilled with block j+S-1 right after.
  auto wait_block = [&](int rem) __attribute__((always_inline)) {
    static_for<0, S - 1>([&](auto rc) __attribute__((always_inline)) {
      constexpr int R = decltype(rc)::value;
      if (rem == R) wait_vm<R * NDMA>();
    });
  };
  auto step = [&](int j, auto stc) __attribute__((always_inline)) {
    constexpr int I = decltype(stc)::value;
    wait_block(min(S - 2, nk - 1 - j));
    lds_barrier();
    if (j + S - 1 < nk) issue(j + S - 1, std::integral_constant<int, (I + S - 1) % S>{});
    compute(stc);
  };

  // prologue: blocks 0 .. S-2 into stages 0 .. S-2
  static_for<0, S - 1>([&](auto ic) __attribute__((always_inline)) {
    constexpr int I = decltype(ic)::value;
    if (I < nk) issue(I, ic);
  });
  // (the scan's loads complete after the prologue's: by the time its result
  // is used every load issued so far has landed, so the vmcnt waits of the
  // pipeline below still count only its own loads)
  {
    const int g0 = (G == 1) ? 0 : ja, ng = (G == 1) ? 1 : nk;
    const uint16_t* st[1] = {scale + ((int64_t)tt * G + g0) * kTile};
    uint32_t f8[1];
    wide_rows8<BITS, 1, 8>(st, ng, lane, 64, f8);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) fw[cb] = wave_row_flag(f8[0], 32 * cb + c) ? kWideScale : 1.f;
    w_wide = __builtin_amdgcn_ballot_w64(f8[0] != 0) != 0;
  }
  // the loop body covers S blocks, so every stage index is a constant
  for (int j = 0; j < nk; j += S) {
    static_for<0, S>([&](auto ic) __attribute__((always_inline)) {
      constexpr int I = decltype(ic)::value;
      if (j + I < nk) step(j + I, ic);
    });
  }
  if (w_wide) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[rb][cb] *= unscale(fw[cb]);
  }

  if (splits > 1) {
    // partial tile -> workspace in fragment order [split][work-group][quad]
    // [thread] x 16 bytes; the last work-group of the output tile to arrive
    // adds the splits in order 0, 1, ...
    constexpr int NQ = RB * 2 * 4;
    const int64_t wg = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    const int64_t groups = (int64_t)gridDim.x * gridDim.y;
    float* pw = part + ((blockIdx.z * groups + wg) * NQ * 256 + tid) * 4;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            put_partial(pw + ((rb * 2 + cb) * 4 + q) * 1024 + e, acc[rb][cb][4 * q + e]);
    partials_written();
    __syncthreads();
    __shared__ uint32_t s_last;
    if (tid == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(&tickets[wg], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == (uint32_t)(splits - 1);
      if (s_last) __hip_atomic_store(&tickets[wg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;
    const float* pr = part + (wg * NQ * 256 + tid) * 4;
    for (int s2 = 0; s2 < splits; ++s2) {
      // one 32-row block at a time: 8 quads in flight, not all NQ
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[i][e] = get_partial(pr + ((int64_t)s2 * groups * NQ + rb * 8 + i) * 1024 + e);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[rb][cb][4 * q + e] += v[cb * 4 + q][e];
      }
    }
  }

  // rows m0 + 32rb + 8(r/4) + 4h + r%4 of columns t*64 + 32cb + c
  const int64_t ldy = mat.ldy;
  const int mrem = m - m0 - 4 * h;
  if constexpr (PAIR) {
    // every wave has passed its last read of the stages (and every load into
    // them has landed) once all are at this barrier
    __syncthreads();
    const bool up_wave = wave >= 2;
    const int keep = up_wave ? 1 : 0;          // the column half this wave finishes
    // the pair's exchange area: [column half][r][lane], 8 KB
    float* xch = reinterpret_cast<float*>((wave & 1) ? (void*)&gemm_stage<BITS, MB, 1>()
                                                     : (void*)&gemm_stage<BITS, MB, 0>());
    const int col = t * kTile + 32 * keep + c;
    const int64_t obase = (int64_t)(m0 + 4 * h) * ldy + col;
    // a tile wholly inside H: no per-element bounds checks
    const bool full = m - m0 >= MB && (t + 1) * kTile <= n;
    float* const y32 = mat.y;
    uint16_t* const y16 = set.h16;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[((1 - keep) * 16 + r) * 64 + lane] = acc[rb][1 - keep][r];
      __syncthreads();
      if (tvalid && col < n) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int64_t o = obase + (int64_t)(32 * rb + 8 * q) * ldy;
#pragma unroll
          for (int e = 0; e < 4; ++e, o += ldy) {
            const int r = 4 * q + e;
            if (!full && 32 * rb + 8 * q + e >= mrem) continue;
            const float other = xch[(keep * 16 + r) * 64 + lane];
            const float mine = acc[rb][keep][r];
            const float hv = up_wave ? silu(other) * mine : silu(mine) * other;
            if (y32 != nullptr) y32[o] = hv;
            if (y16 != nullptr) y16[o] = __builtin_bit_cast(uint16_t, (f16)hv);
          }
        }
      }
      __syncthreads();
    }
    return;
  }
  if (!tvalid) return;
  store_acc_tile<RB>(acc, mat.y, ldy, m, n, m0, t, c, h);
}

}  // namespace qlin
