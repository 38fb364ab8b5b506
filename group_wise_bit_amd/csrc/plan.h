// Host-side launch plans shared by the C-ABI entry points and the kernel
// launchers (the launchers are instantiated per bit width in inst.hip, so that
// the widths compile in parallel).
#pragma once

#include "../../include/qlin.h"
#include "kernels.h"

namespace qlin {

inline int64_t tiles_of(int64_t n) { return (n + kTile - 1) / kTile; }

constexpr int kWaves = 4;                    // waves per work-group (GEMV, skinny GEMM)

// Workspace layout: a fixed region of arrival counters (one uint32 per tile,
// kCounterBytes, so calls of any shape can share one workspace without their
// partial sums ever landing on another call's counters), then the fp32
// partials.
constexpr int64_t kCounterBytes = 65536;

// Split of the K-blocks over work-groups for the tile-per-work-group kernels.
struct Split { int splits, kbps; };

// GEMV launch kinds: packed codes (single matrix or a set), a gate/up pair
// with the SwiGLU combination, fp16 masters re-rounded on the fly.
enum class GemvKind { kPacked, kPair, kFused };

// GEMV launch shape: work-groups of `rows` rows of one tile (64: a whole tile,
// lane = row; 16 / 8: 4 / 8 lanes per row over slices of each block) per K
// split; the waves of a work-group split the K-blocks of its split.  Each wave
// keeps up to `unroll` blocks in flight, so the work-group is sized to cover
// its K range in about one round of loads.
struct GemvCfg {
  int waves, splits, kbps, unroll;
  int rows;
};

// Packed GEMV launch over a set of matrices (shared K, bits, group).
struct PackedLaunch {
  GemvSet set;
  int tiles;          // launch tiles (grid.x)
  int kb, G;
  bool swiglu;
  uint16_t* h16;
};

// A GEMM launch over a set of matrices (shared K, bits, group; one X).
struct GemmPlan {
  GemmSet set;
  int64_t tiles;      // all 64-row tiles of the set
  int cols4;          // all work-group columns of four tiles (tiled GEMM)
  int kb, G, bits;
  int end_tiles[kMaxMats], end_cols4[kMaxMats];   // set.end in either unit
};

// Tiled-GEMM launch shape: work-group tile = MB rows of X x 256 rows of W
// (four 64-row tiles), gx = work-group columns; or (mb = 0 / 1) the K-split
// kernel, 32 or 64 rows of X x one 64-row tile, or x two adjacent tiles
// (dual), or x one 32-row half of a tile (half).  Measured on MI355X
// (graph-replayed launches over rotating cold weights, the Qwen2.5-0.5B and
// Qwen3-8B layer shapes and q/k/v, gate/up sets, M = 8..2048, int4): up to
// M = 256 the K-split kernel is 1.1-2x faster (all loads of a wave's K-blocks
// in flight at once; 64 X rows from 256 tiles up); half tiles double a grid
// too small to fill the chip, tile pairs halve the X bytes per MFMA of a
// large or tall one.  Above M = 256 a tall X tile pays only when the grid is
// large.
// mb = 0 / 1: k_gemm_ksplit with 32 / 64 X rows, gx in tiles (dual: in tile
// pairs; half: in 32-row halves of tiles)
// mb = 6: k_gemm_ksplit with 128 X rows (each wave's decoded fragment feeds
// four MFMA row blocks), over whole or half tiles, no tile pairs.
struct TilesCfg { int mb, gx, gy, splits, kbps; bool dual, half; };

constexpr int kMbKsplit128 = 6;
// mb = 8: k_gemm_wdec, 128 X rows x two tiles (a gate/up pair's tile t, or
// tiles 2x and 2x + 1 of one matrix: gx in tile pairs, pairable sets only),
// each weight decoded once per work-group into LDS
constexpr int kMbWdec = 8;
constexpr int kWdecRows = 128;
// the K-split kernel's forms and their X rows
inline bool is_ksplit(int mb) { return mb <= 1 || mb == kMbKsplit128; }
inline int ksplit_rows(int mb) { return mb == kMbKsplit128 ? 128 : 32 * (mb + 1); }

// Kernel launchers, one instantiation per bit width (inst.hip).
template <int B>
void launch_quant_batch(const QuantJob* jobs, int count, bool row, hipStream_t st);
template <int B>
void launch_gemv_packed(const PackedLaunch& L, const f16x2* x2, float* part, uint32_t* tick,
                        GemvCfg c, hipStream_t st);
template <int B>   // B = 2 .. 8, or 16 (the unquantized control)
void launch_gemv_fused(const qlin_weight* w, const f16x2* x2, float* y, float* part,
                       uint32_t* tick, GemvCfg c, hipStream_t st);
template <int B>   // B = 2, 3, 4, 8
void launch_gemm_skinny(const GemmPlan& p, const uint16_t* X, int64_t ldx, int m, float* part,
                        uint32_t* tick, Split sp, hipStream_t st);
template <int B>
void launch_gemm_tiles(const GemmPlan& p, const uint16_t* X, int64_t ldx, int m, TilesCfg c,
                       float* part, uint32_t* tick, hipStream_t st);
template <int B>
void launch_gemm_swiglu(const GemmSet& set, const uint16_t* X, int64_t ldx, int m, int kb, int G,
                        TilesCfg c, float* part, uint32_t* tick, hipStream_t st);
template <int B>
void launch_embed_rows(const uint32_t* codes, const uint16_t* scale, const uint8_t* zero,
                       const int32_t* ids, int count, int n, int kb, int G, uint16_t* out16,
                       float* out32, int64_t ld_out, hipStream_t st);

}  // namespace qlin
