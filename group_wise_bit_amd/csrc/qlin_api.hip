// qlin C ABI: argument validation (host only, no HIP call), launch-shape
// selection and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/qlin.h"
#include "../../include/qlin_tune.h"
#include "plan.h"

using namespace qlin;

namespace {

thread_local int g_last_hip_error = 0;

// Launch-shape overrides set through qlin_set_launch_override (sweeps and
// tests only): per family one word, bit 63 = set, then three 16-bit fields.
// One atomic load per call gives a consistent snapshot.
std::atomic<uint64_t> g_override[2];

bool launch_override(int family, int& a, int& b, int& c) {
  const uint64_t v = g_override[family].load(std::memory_order_relaxed);
  if ((v >> 63) == 0) return false;
  a = (int)(v & 0xFFFFu);
  b = (int)((v >> 16) & 0xFFFFu);
  c = (int)((v >> 32) & 0xFFFFu);
  return true;
}

constexpr int kMaxN = 1 << 24;
constexpr int kMaxK = 1 << 20;
constexpr int kMaxM = 1 << 20;
constexpr int kTargetGroups = 64;            // work-groups a split-K launch aims for
constexpr int kMinBlocksPerWave = 2;         // K-blocks per wave before splitting further

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range { uintptr_t lo, hi; };
inline Range range_of(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + (uintptr_t)(bytes > 0 ? bytes : 0)};
}
inline bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Widths with a packed-code layout, and every width of the lever (scale/zero
// precompute and the fused re-quantizing GEMV from fp16 masters): the same.
bool valid_bits(int bits) { return bits >= 2 && bits <= 8; }
bool lever_bits(int bits) { return bits >= 2 && bits <= 8; }

qlin_status check_nk(int32_t n, int32_t k) {
  if (n < 1 || n > kMaxN || k < kBlock || k > kMaxK || (k % kBlock) != 0) return QLIN_ERR_SHAPE;
  return QLIN_OK;
}

qlin_status check_group(int32_t group, int32_t k) {
  return (group == kBlock || group == k) ? QLIN_OK : QLIN_ERR_GROUP;
}

int64_t packed_bytes(int64_t n, int64_t k, int bits) {
  return tiles_of(n) * kTile * (k / kBlock) * 2 * bits * 4;
}
int64_t meta_entries(int64_t n, int64_t k, int group) {
  return tiles_of(n) * kTile * (group == k ? 1 : k / kBlock);
}

qlin_status hip_status(hipError_t e) {
  if (e == hipSuccess) return QLIN_OK;
  g_last_hip_error = (int)e;
  return QLIN_ERR_HIP;
}

// One check per process and device: the kernels are built for gfx950 only.
qlin_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { g_last_hip_error = (int)e; return QLIN_ERR_NO_DEVICE; }
  static thread_local int cached_dev = -1;
  static thread_local bool cached_ok = false;
  if (dev == cached_dev) return cached_ok ? QLIN_OK : QLIN_ERR_NO_DEVICE;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) { g_last_hip_error = (int)e; return QLIN_ERR_NO_DEVICE; }
  cached_dev = dev;
  cached_ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  return cached_ok ? QLIN_OK : QLIN_ERR_NO_DEVICE;
}

qlin_status check_weight(const qlin_weight* w, bool allow_master, bool allow16) {
  if (w == nullptr) return QLIN_ERR_NULL;
  qlin_status st = check_nk(w->n, w->k);
  if (st != QLIN_OK) return st;
  if (w->reserved != 0) return QLIN_ERR_FORMAT;
  if (w->format == QLIN_FMT_PACKED) {
    if (!valid_bits(w->bits)) return QLIN_ERR_BITS;
    if (w->ld != 0) return QLIN_ERR_SHAPE;
  } else if (w->format == QLIN_FMT_FP16_MASTER) {
    if (!allow_master) return QLIN_ERR_FORMAT;
    if (!(lever_bits(w->bits) || (allow16 && w->bits == 16))) return QLIN_ERR_BITS;
    if (w->ld < w->k) return QLIN_ERR_SHAPE;
    if (w->ld % 8 != 0) return QLIN_ERR_ALIGN;
  } else {
    return QLIN_ERR_FORMAT;
  }
  if (w->data == nullptr) return QLIN_ERR_NULL;
  if (!aligned16(w->data)) return QLIN_ERR_ALIGN;
  if (w->bits != 16) {
    st = check_group(w->group, w->k);
    if (st != QLIN_OK) return st;
    if (w->scale == nullptr || w->zero == nullptr) return QLIN_ERR_NULL;
    if (!aligned16(w->scale) || !aligned16(w->zero)) return QLIN_ERR_ALIGN;
  }
  return QLIN_OK;
}

int64_t weight_bytes(const qlin_weight* w) {
  if (w->format == QLIN_FMT_PACKED) return packed_bytes(w->n, w->k, w->bits);
  return ((int64_t)(w->n - 1) * w->ld + w->k) * 2;
}

bool output_overlaps_weight(const qlin_weight* w, Range out) {
  if (overlaps(out, range_of(w->data, weight_bytes(w)))) return true;
  if (w->bits != 16) {
    const int64_t me = meta_entries(w->n, w->k, w->group);
    if (overlaps(out, range_of(w->scale, me * 2))) return true;
    if (overlaps(out, range_of(w->zero, me))) return true;
  }
  return false;
}


constexpr int64_t kMaxSplitTiles = kCounterBytes / 4;

// Skinny-GEMM split: 4 waves per work-group, 2 K-blocks in flight per wave;
// K is split across work-groups only for few tiles and long K (each split
// costs an agent-scope release fence per work-group).
Split choose_split(int64_t tiles, int kb, int64_t ws_bytes, int64_t part_rows) {
  constexpr int kPerGroup = kWaves * kMinBlocksPerWave;
  int want = 1;
  if (tiles < 32 && kb >= 4 * kPerGroup) {
    want = (int)((kTargetGroups + tiles - 1) / tiles);
    if (want > kb / kPerGroup) want = kb / kPerGroup;
  }
  if (want < 1 || tiles > kMaxSplitTiles) want = 1;
  while (want > 1) {
    const int64_t need = kCounterBytes + (int64_t)want * part_rows * tiles * kTile * 4;
    if (need <= ws_bytes) break;
    --want;
  }
  const int kbps = (kb + want - 1) / want;
  const int splits = (kb + kbps - 1) / kbps;
  return Split{splits, kbps};
}

int64_t split_ws_bytes(int64_t tiles, int kb, int64_t part_rows) {
  const Split s = choose_split(tiles, kb, INT64_MAX, part_rows);
  if (s.splits <= 1) return 0;
  return kCounterBytes + (int64_t)s.splits * part_rows * tiles * kTile * 4;
}



GemvCfg gemv_config(int64_t tiles, int kb, GemvKind kind, int bits, int64_t ws_bytes) {
  // Measured on MI355X (graph-replayed launches over rotating cold weights;
  // bits 2, 3, 4, 8; the Qwen2.5-0.5B, Qwen3-0.6B and Qwen3-8B layer shapes,
  // q/k/v sets and gate/up pairs; fp16 masters for the fused kernel).  A
  // launch of few tiles is latency-bound and runs on as many compute units as
  // it has work-groups, while a K split costs ~1.3 us of partial-sum round
  // trips.  So the packed kernels narrow the work-group first (8 or 16 rows
  // over 8 / 4 slices of each block) while tiles x K-blocks <= 4096, and split
  // K when one wave would otherwise decode many blocks in sequence (long K
  // over up to 128 tiles).  Launches of many tiles use 4-wave work-groups, so that the tail
  // of the grid is short.  The fused kernel reads 2 bytes per weight and does
  // about 7 VALU ops per weight: 8-row work-groups up to 256 tiles (16 waves,
  // 8 for short K over many tiles), whole tiles beyond.
  const bool fused = kind == GemvKind::kFused, pair = kind == GemvKind::kPair;
  int waves = fused ? 8 : 16;
  int splits = 1;
  int rows = 64;
  if (fused) {
    if (tiles <= 256) {
      rows = 8;
      waves = (kb <= 16 && tiles >= 64) ? 8 : 16;
      if (kb >= 128) splits = kb / 64;
    }
  } else if (tiles > 256) {
    waves = 4;
  } else if (tiles > 128) {
    // whole tiles, 16 waves, no split at every width (3 bits took 8 waves x 4
    // splits until the zero point was folded; now the Qwen3-8B gate at int3
    // 7.85 -> 7.00 us and its gate/up pair 12.3 -> 11.9 us without the split)
  } else if (tiles * kb <= 4096) {
    // (a gate/up pair of 64+ tiles: 8-row, 8-wave work-groups; Qwen2.5-0.5B
    // gate/up 4.6 -> 4.4 us)
    rows = ((pair && tiles < 64) || (!pair && tiles >= 48)) ? 16 : 8;
    waves = ((pair && tiles < 64) || kb >= 32) ? 16 : 8;
    if (kb >= 128) splits = kb / 64;   // very long K over a few tiles
  } else if (tiles > 64 && kb < 128 && (bits == 2 || bits == 4) && !pair) {
    // 65-128 tiles over medium K at 2 and 4 bits: whole tiles, 16 waves, no
    // split (the Qwen3-8B q/k/v set, 96 tiles x 64 K-blocks: int4 6.23 ->
    // 5.68 us, int2 5.76 -> 5.55 us against four splits; int3 6.24 -> 6.62 us,
    // so 3 bits keeps the split)
  } else {
    splits = kb >= 128 ? kb / 64 : kb / 16;
  }
  if (splits > 16) splits = 16;
  if (splits > kb) splits = kb;
  if (splits < 1) splits = 1;
  // a launch-shape override (qlin_set_launch_override: waves, splits, rows;
  // sweeps and tests) replaces the choice
  {
    int w, sp, rw;
    if (launch_override(QLIN_TUNE_GEMV, w, sp, rw)) {
      waves = w;
      splits = sp < kb ? sp : kb;
      rows = rw;
    }
  }
  if (fused && rows == 16) rows = 8;   // the fused kernel comes in 64- and 8-row forms
  // split-K: one ticket per work-group of the launch's first split; partial
  // sums for every launch row (two per row for a gate/up pair)
  const int64_t part_rows = (pair ? 2 : 1) * tiles * kTile;
  if (tiles * (kTile / rows) > kMaxSplitTiles) splits = 1;
  while (splits > 1 && kCounterBytes + (int64_t)splits * part_rows * 4 > ws_bytes) --splits;
  const int kbps = (kb + splits - 1) / splits;
  // blocks kept in flight per wave: the wave's share of the split, up to 4
  // (packed; whole-tile gate/up pairs up to 4 bits), 2 (other gate/up pairs,
  // 8-row fused) or 1 (64-row fused)
  const int unroll = fused ? (rows == 64 ? 1 : 2) : (pair ? (rows == 64 && bits <= 4 ? 4 : 2) : 4);
  const int per_wave = (kbps + waves - 1) / waves;
  int u = 1;
  while (u < unroll && u < per_wave) u *= 2;
  return GemvCfg{waves, (kb + kbps - 1) / kbps, kbps, u, rows};
}

int64_t gemv_ws_bytes(int64_t tiles, int kb, GemvKind kind, int bits) {
  const GemvCfg c = gemv_config(tiles, kb, kind, bits, INT64_MAX);
  if (c.splits <= 1) return 0;
  return kCounterBytes + (int64_t)c.splits * (kind == GemvKind::kPair ? 2 : 1) * tiles * kTile * 4;
}



qlin_status run_quant(const QuantJob* jobs, int count, int bits, bool row, hipStream_t st) {
  switch (bits) {
    case 2: launch_quant_batch<2>(jobs, count, row, st); break;
    case 3: launch_quant_batch<3>(jobs, count, row, st); break;
    case 4: launch_quant_batch<4>(jobs, count, row, st); break;
    case 5: launch_quant_batch<5>(jobs, count, row, st); break;
    case 6: launch_quant_batch<6>(jobs, count, row, st); break;
    case 7: launch_quant_batch<7>(jobs, count, row, st); break;
    default: launch_quant_batch<8>(jobs, count, row, st); break;
  }
  return hip_status(hipGetLastError());
}

// Host checks of one quantization job; the ranges it reads and writes.
struct QuantRanges { Range in, codes, scale, zero; };

qlin_status check_quant_job(const uint16_t* w16, int64_t ld_w, int32_t n, int32_t k, int32_t bits,
                            int32_t group, const uint32_t* codes, const uint16_t* scale,
                            const uint8_t* zero, QuantRanges& r) {
  qlin_status st = check_nk(n, k);
  if (st != QLIN_OK) return st;
  if (!lever_bits(bits) || (codes != nullptr && !valid_bits(bits))) return QLIN_ERR_BITS;
  st = check_group(group, k);
  if (st != QLIN_OK) return st;
  if (w16 == nullptr || scale == nullptr || zero == nullptr) return QLIN_ERR_NULL;
  if (ld_w < k) return QLIN_ERR_SHAPE;
  if (ld_w % 8 != 0) return QLIN_ERR_ALIGN;
  if (!aligned16(w16) || !aligned16(scale) || !aligned16(zero) ||
      (codes != nullptr && !aligned16(codes)))
    return QLIN_ERR_ALIGN;
  r.in = range_of(w16, ((int64_t)(n - 1) * ld_w + k) * 2);
  const int64_t me = meta_entries(n, k, group);
  r.scale = range_of(scale, me * 2);
  r.zero = range_of(zero, me);
  r.codes = range_of(codes, codes != nullptr ? packed_bytes(n, k, bits) : 0);
  if (overlaps(r.in, r.scale) || overlaps(r.in, r.zero) || overlaps(r.scale, r.zero) ||
      overlaps(r.codes, r.in) || overlaps(r.codes, r.scale) || overlaps(r.codes, r.zero))
    return QLIN_ERR_ALIAS;
  return QLIN_OK;
}



PackedLaunch packed_launch(const qlin_weight* const* w, float* const* y, int count) {
  PackedLaunch L{};
  int64_t tiles = 0;
  for (int i = 0; i < count; ++i) {
    L.set.codes[i] = static_cast<const uint32_t*>(w[i]->data);
    L.set.scale[i] = w[i]->scale;
    L.set.zero[i] = w[i]->zero;
    L.set.y[i] = y[i];
    L.set.n[i] = w[i]->n;
    tiles += tiles_of(w[i]->n);
    L.set.tile_end[i] = (int)tiles;
  }
  L.set.count = count;
  L.tiles = (int)tiles;
  L.kb = w[0]->k / kBlock;
  L.G = (w[0]->group == w[0]->k) ? 1 : L.kb;
  L.swiglu = false;
  L.h16 = nullptr;
  return L;
}

qlin_status run_packed(const PackedLaunch& L, int bits, const uint16_t* x, void* workspace,
                       GemvCfg c, hipStream_t stream) {
  uint32_t* tick = static_cast<uint32_t*>(workspace);
  float* part = c.splits > 1
      ? reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes) : nullptr;
  const f16x2* x2 = reinterpret_cast<const f16x2*>(x);
  switch (bits) {
    case 2: launch_gemv_packed<2>(L, x2, part, tick, c, stream); break;
    case 3: launch_gemv_packed<3>(L, x2, part, tick, c, stream); break;
    case 4: launch_gemv_packed<4>(L, x2, part, tick, c, stream); break;
    case 5: launch_gemv_packed<5>(L, x2, part, tick, c, stream); break;
    case 6: launch_gemv_packed<6>(L, x2, part, tick, c, stream); break;
    case 7: launch_gemv_packed<7>(L, x2, part, tick, c, stream); break;
    default: launch_gemv_packed<8>(L, x2, part, tick, c, stream); break;
  }
  return hip_status(hipGetLastError());
}



GemmPlan gemm_plan(const qlin_weight* const* w, float* const* Y, const int64_t* ldy, int count,
                   bool skinny) {
  GemmPlan p{};
  int64_t tiles = 0, cols4 = 0;
  for (int i = 0; i < count; ++i) {
    p.set.codes[i] = static_cast<const uint32_t*>(w[i]->data);
    p.set.scale[i] = w[i]->scale;
    p.set.zero[i] = w[i]->zero;
    p.set.y[i] = Y[i];
    p.set.ldy[i] = ldy[i];
    p.set.n[i] = w[i]->n;
    const int64_t t = tiles_of(w[i]->n);
    tiles += t;
    cols4 += (t + 3) / 4;
    p.end_tiles[i] = (int)tiles;
    p.end_cols4[i] = (int)cols4;
    p.set.end[i] = (int)(skinny ? tiles : cols4);
  }
  p.set.count = count;
  p.tiles = tiles;
  p.cols4 = (int)cols4;
  p.kb = w[0]->k / kBlock;
  p.G = (w[0]->group == w[0]->k) ? 1 : p.kb;
  p.bits = w[0]->bits;
  return p;
}



// pairable: tile pairs stay within one matrix (one matrix, or every
// matrix of the set has an even tile count)
TilesCfg tiles_config(int64_t gx, int64_t tiles, int kb, int m, int count, bool pairable,
                      int bits, int64_t ws_bytes) {
  TilesCfg c;
  c.gx = (int)gx;
  c.dual = false;
  c.half = false;
  int want = 1;
  if (m <= 256 && (tiles < 256 || m <= 16)) {
    // the K-split kernel: one 64-row W tile x 32 X rows per work-group; for
    // M > 16, K is split across work-groups (at most 8 ways) only when the
    // grid is under 256 work-groups, keeping at least 8 K-blocks per split
    c.mb = 0;
    // a grid of under 128 work-groups runs over half tiles: twice the
    // work-groups, no partial-sum round trip (measured at M = 8 and 128:
    // Qwen2.5-0.5B q/k/v, o, down and Qwen3-8B k 15-25 % faster)
    const int64_t groups0 = tiles * ((m + 31) / 32);
    c.half = groups0 < 128;
    const int64_t groups = c.half ? 2 * groups0 : groups0;
    if (m <= 16) {
      // M <= 16 (measured at M = 8 on the Qwen2.5-0.5B and Qwen3-8B shapes):
      // a work-group's K range is one or two rounds of loads already, so a
      // split mostly adds its partial-sum round trip; split only launches of
      // under 64 work-groups, and very long K (about 48 K-blocks per split)
      if (groups < 64) {
        want = (int)((128 + groups - 1) / groups);
        if (want > 8) want = 8;
        if (want > kb / 8) want = kb / 8;
      } else if (kb >= 128) {
        // ... but no more work-groups than CUs: the Qwen3-8B down projection
        // (128 half-tile work-groups, 192 K-blocks) at M = 8 took 19.3 /
        // 18.3 / 16.3 / 18.5 us at 4 / 3 / 2 / 1 splits (int4; int2, int3,
        // int8 and M = 16 alike): two splits give 6 K-blocks per wave, four in
        // flight, one 16-wave work-group per CU
        want = kb / 48;
        const int64_t fill = groups < 256 ? 256 / groups : 1;
        if (want > fill) want = (int)fill;
        if (want > 8) want = 8;
      }
    } else if (groups < 256) {
      want = (int)((512 + groups - 1) / groups);
      if (want > 8) want = 8;
      if (want > kb / 8) want = kb / 8;
    }
  } else if (m <= 256) {
    c.mb = 1;                              // K-split kernel, 64 X rows
  }
  if (m > 16 && m <= 256 && pairable && kb >= 32 && tiles * ((m + 31) / 32) >= 384) {
    // a large grid of long-K work-groups: 32 X rows over tile pairs, each X
    // fragment feeding twice the MFMAs (Qwen3-8B int4 at M = 128: the gate/up
    // set 61 -> 49 us, the q/k/v set 25 -> 20 us, gate alone 36 -> 32 us;
    // the q/k/v set at 5 / 6 / 8 bits 31.2 / 31.7 / 30.0 -> 28.5 / 28.9 /
    // 25.0 us)
    c.mb = 0;
    c.half = false;
    c.dual = true;
    want = 1;
  } else if (m > 256) {
    // 128-row tiles when that already gives more work-groups than CUs (two
    // fit per CU), else 64 when that fills the chip; a smaller grid takes
    // the K-split kernel (64 X rows) for long K, 32-row tiles for short K
    // (also for sets, despite the idle waves of their partly filled
    // four-tile columns: Qwen2.5-0.5B q/k/v at M = 2048, 20.5 -> 16.6 us
    // against the K-split kernel over tile pairs)
    c.mb = 128;
    if ((int64_t)c.gx * ((m + 127) / 128) < 288) {
      c.mb = 64;
      if ((int64_t)c.gx * ((m + 63) / 64) < 256) c.mb = kb >= 32 ? 1 : 32;
    }
    // the K-split kernel over a tall M reads its X fragments through L1 for
    // every tile: over tile pairs each fragment feeds twice the MFMAs
    // (Qwen2.5-0.5B at M = 2048: down 52 -> 38 us, the q/k/v set 17.4 ->
    // 16.5 us)
    c.dual = c.mb <= 1;
  }
  if (m > 64 && m <= 256 && pairable && kb >= 128) {
    // very long K (the Qwen3-8B down projection, 4096 x 12288, at M = 128):
    // 128 X rows over tile pairs, each weight decoded once per work-group,
    // K split to about one work-group per CU (int4: 35.1 -> 32.9 us against
    // the K-split kernel; 8 splits 32.9, 4 splits 41.7 us)
    c.mb = kMbWdec;
    c.dual = c.half = false;
    const int64_t g = ((tiles + 1) / 2) * ((m + kWdecRows - 1) / kWdecRows);
    want = g >= 256 ? 1 : (int)((256 + g - 1) / g);
    if (want > 8) want = 8;
  }
  // a GEMM launch-shape override (form, splits; sweeps and tests) replaces
  // the choice: form 0 / 1 the K-split kernel with 32 / 64 X rows, 2 / 3 the
  // same with 64 / 32 X rows over tile pairs, 4 / 5 with 32 / 64 X rows over
  // half tiles, 6 / 7 with 128 X rows (whole / half tiles), 8 the
  // decode-once form
  {
    int mb, sp, unused;
    if (launch_override(QLIN_TUNE_GEMM, mb, sp, unused) && mb != 16) {
      c.mb = (mb == 6 || mb == 7) ? kMbKsplit128 : (mb == 2 || mb == 5) ? 1
             : (mb == 3 || mb == 4) ? 0 : mb;
      c.dual = mb == 2 || mb == 3;
      c.half = mb == 4 || mb == 5 || mb == 7;
      want = sp < kb ? sp : kb;
    }
  }
  if (!pairable) c.dual = false;       // tile pairs within one matrix only
  if (c.mb == kMbWdec && !pairable) c.mb = 0;
  if (want < 1) want = 1;
  const bool ks = is_ksplit(c.mb), wd = c.mb == kMbWdec;
  if (!ks) c.dual = c.half = false;
  if (c.mb == kMbKsplit128) c.dual = false;
  if (ks) c.gx = (int)(c.dual ? (tiles + 1) / 2 : c.half ? 2 * tiles : tiles);
  if (wd) c.gx = (int)((tiles + 1) / 2);
  const int rows = ks ? ksplit_rows(c.mb) : wd ? kWdecRows : c.mb;
  const int64_t wg_outputs =
      (int64_t)rows * (ks ? (c.dual ? 2 * kTile : c.half ? kTile / 2 : kTile)
                          : wd ? 2 * kTile : 256);
  c.gy = (m + rows - 1) / rows;
  if ((int64_t)c.gx * c.gy > kMaxSplitTiles) want = 1;
  while (want > 1 && kCounterBytes + (int64_t)want * c.gy * c.gx * wg_outputs * 4 > ws_bytes)
    --want;
  c.kbps = (kb + want - 1) / want;
  c.splits = (kb + c.kbps - 1) / c.kbps;
  return c;
}

int64_t tiles_ws_bytes(int64_t gx, int64_t tiles, int kb, int m, int count, bool pairable,
                       int bits) {
  const TilesCfg c = tiles_config(gx, tiles, kb, m, count, pairable, bits, INT64_MAX);
  if (c.splits <= 1) return 0;
  const int64_t wg_outputs =
      is_ksplit(c.mb) ? ksplit_rows(c.mb) * (c.dual ? 2 * kTile : c.half ? kTile / 2 : kTile)
      : c.mb == kMbWdec ? (int64_t)kWdecRows * 2 * kTile
                        : (int64_t)c.mb * 256;
  return kCounterBytes + (int64_t)c.splits * c.gy * c.gx * wg_outputs * 4;
}


constexpr int kSkinnyMaxM = 16;

// M <= 16: the K-split kernel (measured 1.1-2.5x faster than the skinny one
// on the Qwen2.5-0.5B and Qwen3-8B shapes at M = 8, int4; over half tiles it
// also beats it on long K over few tiles, where the skinny kernel's split
// used to be cheaper).  The GEMM override form 16 forces the skinny kernel,
// which exists for 2, 3, 4 and 8 bits only.
bool skinny_by_ksplit(int64_t tiles, int kb, int bits) {
  (void)tiles;
  (void)kb;
  if (bits >= 5 && bits <= 7) return true;
  int mb, sp, unused;
  if (launch_override(QLIN_TUNE_GEMM, mb, sp, unused) && mb == 16) return false;
  return true;
}


// Gate/up GEMM with the SwiGLU combination (one launch, h written once).
// mb as in TilesCfg: 0 / 1 the K-split kernel with 32 / 64 X rows and both
// matrices' tile t in each work-group (gx = tiles); 64 / 128 the LDS-DMA
// pipeline over two tiles of each matrix (gx = tiles / 2, rounded up).  The
// choice follows tiles_config for the equivalent two-matrix set.
TilesCfg swiglu_config(int64_t tiles, int kb, int m, int64_t ws_bytes) {
  TilesCfg c;
  c.dual = c.half = false;
  int want = 1;
  const int64_t cols2 = (tiles + 1) / 2;
  if (m <= 256) {
    c.mb = (2 * tiles < 256 || m <= 16) ? 0 : 1;
    if (c.mb == 0) {
      // under 256 pair work-groups: over half tiles (as many work-groups as
      // the two-matrix set has, each loading X once for both matrices;
      // measured at M = 8 and 128 on the Qwen2.5-0.5B, Qwen3-0.6B and
      // Qwen3-8B pairs; the Qwen2.5-0.5B pair at M = 128, 304 pair
      // work-groups, 12.7 over half tiles against 12.3 us over whole ones)
      const int64_t pairs = tiles * ((m + 31) / 32);
      c.half = pairs < 256;
      // splits counted as for the two-matrix set, with its rules
      const int64_t groups = 2 * pairs;
      if (m <= 16) {
        if (groups < 64) {
          want = (int)((128 + groups - 1) / groups);
          if (want > 8) want = 8;
          if (want > kb / 8) want = kb / 8;
        } else if (kb >= 128) {
          want = kb / 48;
          if (want > 8) want = 8;
        }
      } else if (groups < 256) {
        want = (int)((512 + groups - 1) / groups);
        if (want > 8) want = 8;
        if (want > kb / 8) want = kb / 8;
      }
    }
  } else {
    c.mb = 128;
    if (cols2 * ((m + 127) / 128) < 288) {
      c.mb = 64;
      if (cols2 * ((m + 63) / 64) < 256) c.mb = 1;
    }
  }
  if (m > 64 && m <= 256 && tiles * ((m + kWdecRows - 1) / kWdecRows) >= 128) {
    // many tiles over long K (the Qwen3-8B gate/up pair, 12288 x 4096, at
    // M = 128: 192 work-groups): 128 X rows x tile t of both matrices, each
    // weight decoded once per work-group (int4: 51.5 -> 47.2 us against the
    // K-split pair; a K split measured slower: 61.6 us at 2 splits)
    c.mb = kMbWdec;
    c.half = false;
    want = 1;
  }
  // a GEMM launch-shape override (form, splits) replaces the choice (form 32
  // runs as 64; 4 / 5: the K-split pair over half tiles with 32 / 64 X rows;
  // 8: the decode-once form)
  {
    int mb, sp, unused;
    if (launch_override(QLIN_TUNE_GEMM, mb, sp, unused) &&
        (mb <= 1 || (mb >= 4 && mb <= 8) || mb == 32 || mb == 64 || mb == 128)) {
      c.mb = mb == 32 ? 64 : mb == 4 ? 0 : mb == 5 ? 1 : (mb == 6 || mb == 7) ? kMbKsplit128 : mb;
      c.half = mb == 4 || mb == 5;
      want = sp < kb ? sp : kb;
    }
  }
  if (want < 1) want = 1;
  const bool ks = is_ksplit(c.mb), wd = c.mb == kMbWdec;
  if (!ks) c.half = false;
  if (c.mb == kMbKsplit128) c.half = true;     // two accumulator sets: half tiles only
  c.gx = (int)(ks ? (c.half ? 2 * tiles : tiles) : wd ? tiles : cols2);
  const int rows = ks ? ksplit_rows(c.mb) : wd ? kWdecRows : c.mb;
  const int64_t wg_outputs =
      (int64_t)rows * (ks ? (c.half ? kTile : 2 * kTile) : wd ? 2 * kTile : 256);
  c.gy = (m + rows - 1) / rows;
  if ((int64_t)c.gx * c.gy > kMaxSplitTiles) want = 1;
  while (want > 1 && kCounterBytes + (int64_t)want * c.gy * c.gx * wg_outputs * 4 > ws_bytes)
    --want;
  c.kbps = (kb + want - 1) / want;
  c.splits = (kb + c.kbps - 1) / c.kbps;
  return c;
}

int64_t swiglu_ws_bytes(int64_t tiles, int kb, int m) {
  const TilesCfg c = swiglu_config(tiles, kb, m, INT64_MAX);
  if (c.splits <= 1) return 0;
  const bool ks = is_ksplit(c.mb);
  const int64_t wg_outputs =
      ks ? ksplit_rows(c.mb) * (c.half ? kTile : 2 * kTile)
      : c.mb == kMbWdec ? (int64_t)kWdecRows * 2 * kTile
                        : (int64_t)c.mb * 256;
  return kCounterBytes + (int64_t)c.splits * c.gy * c.gx * wg_outputs * 4;
}


}  // namespace

// ------------------------------------------------ no-allocation GEMV --
// qlin_gemv_noalloc takes its split-K workspace from this file-scope device
// array instead of a caller's buffer.  Each GPU holds its own copy (device
// globals are per device) until the process ends; host code reaches it only
// through the address hipGetSymbolAddress returns on that device (the array's
// name in host code is not a device address).
constexpr int64_t kNoAllocScratchBytes = 1 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
qlin_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { g_last_hip_error = (int)e; return QLIN_ERR_NO_DEVICE; }
  if (dev < 0 || dev >= kMaxScratchDevices) return QLIN_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QLIN_OK;
}

// Zeroes the split-K arrival counters at the start of the scratch array (a
// kernel, not hipMemsetAsync, so that a captured call records no memset node).
__global__ __launch_bounds__(256) void k_clear_counters(uint32_t* __restrict__ c, int n) {
  for (int i = threadIdx.x + blockIdx.x * 256; i < n; i += gridDim.x * 256) c[i] = 0u;
}

// Checks shared by the multi-matrix GEMV entry points: `count` packed
// weights with one k, bits and group; outputs of `out_bytes[i]` bytes that
// overlap nothing else.
qlin_status check_set(const qlin_weight* w, int count, const uint16_t* x, void* const* outs,
                      const int64_t* out_bytes, int nouts, void* workspace,
                      int64_t workspace_bytes) {
  for (int i = 0; i < count; ++i) {
    const qlin_status st = check_weight(&w[i], false, false);
    if (st != QLIN_OK) return st;
    if (w[i].k != w[0].k) return QLIN_ERR_SHAPE;
    if (w[i].bits != w[0].bits || w[i].group != w[0].group) return QLIN_ERR_FORMAT;
  }
  if (x == nullptr) return QLIN_ERR_NULL;
  if (!aligned16(x)) return QLIN_ERR_ALIGN;
  if (workspace_bytes < 0) return QLIN_ERR_WORKSPACE;
  if (workspace != nullptr && !aligned16(workspace)) return QLIN_ERR_ALIGN;
  const Range rx = range_of(x, (int64_t)w[0].k * 2);
  const Range rw = range_of(workspace, workspace != nullptr ? workspace_bytes : 0);
  for (int i = 0; i < nouts; ++i) {
    if (outs[i] == nullptr) continue;
    if (!aligned16(outs[i])) return QLIN_ERR_ALIGN;
    const Range r = range_of(outs[i], out_bytes[i]);
    if (overlaps(r, rx) || overlaps(r, rw)) return QLIN_ERR_ALIAS;
    for (int j = 0; j < count; ++j)
      if (output_overlaps_weight(&w[j], r)) return QLIN_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (outs[j] != nullptr && overlaps(r, range_of(outs[j], out_bytes[j]))) return QLIN_ERR_ALIAS;
  }
  if (rw.hi > rw.lo) {
    if (overlaps(rw, rx)) return QLIN_ERR_ALIAS;
    for (int j = 0; j < count; ++j)
      if (output_overlaps_weight(&w[j], rw)) return QLIN_ERR_ALIAS;
  }
  return QLIN_OK;
}

int64_t set_tiles(const qlin_weight* w, int count) {
  int64_t t = 0;
  for (int i = 0; i < count; ++i) t += tiles_of(w[i].n);
  return t;
}

extern "C" {

const char* qlin_status_string(int status) {
  switch (status) {
    case QLIN_OK: return "QLIN_OK";
    case QLIN_ERR_NULL: return "QLIN_ERR_NULL: a required pointer is NULL";
    case QLIN_ERR_SHAPE: return "QLIN_ERR_SHAPE: size or pitch out of range";
    case QLIN_ERR_BITS: return "QLIN_ERR_BITS: unsupported bit width";
    case QLIN_ERR_GROUP: return "QLIN_ERR_GROUP: group must be 64 or k";
    case QLIN_ERR_ALIGN: return "QLIN_ERR_ALIGN: pointer or pitch misaligned";
    case QLIN_ERR_FORMAT: return "QLIN_ERR_FORMAT: weight format not allowed here";
    case QLIN_ERR_ALIAS: return "QLIN_ERR_ALIAS: output overlaps an input";
    case QLIN_ERR_WORKSPACE: return "QLIN_ERR_WORKSPACE: workspace too small";
    case QLIN_ERR_NO_DEVICE: return "QLIN_ERR_NO_DEVICE: no gfx950 device is current";
    case QLIN_ERR_HIP: return "QLIN_ERR_HIP: a HIP call failed";
    default: return "QLIN: unknown status";
  }
}

int qlin_last_hip_error(void) { return g_last_hip_error; }

int qlin_abi_version(void) { return 1; }

int64_t qlin_packed_bytes(int32_t n, int32_t k, int32_t bits) {
  if (check_nk(n, k) != QLIN_OK || !valid_bits(bits)) return 0;
  return packed_bytes(n, k, bits);
}

int64_t qlin_meta_entries(int32_t n, int32_t k, int32_t group) {
  if (check_nk(n, k) != QLIN_OK || check_group(group, k) != QLIN_OK) return 0;
  return meta_entries(n, k, group);
}

qlin_status qlin_quantize(const uint16_t* w16, int64_t ld_w, int32_t n, int32_t k, int32_t bits,
                          int32_t group, uint32_t* codes, uint16_t* scale, uint8_t* zero,
                          hipStream_t stream) {
  QuantRanges r;
  qlin_status st = check_quant_job(w16, ld_w, n, k, bits, group, codes, scale, zero, r);
  if (st != QLIN_OK) return st;
  st = check_device();
  if (st != QLIN_OK) return st;
  const QuantJob job{w16, ld_w, codes, scale, zero, n, k / kBlock};
  return run_quant(&job, 1, bits, group != kBlock, stream);
}

qlin_status qlin_quantize_batch(const qlin_quant_job* jobs, int32_t count, int32_t bits,
                                int32_t group, hipStream_t stream) {
  if (count < 0) return QLIN_ERR_SHAPE;
  if (count == 0) return QLIN_OK;
  if (jobs == nullptr) return QLIN_ERR_NULL;
  if (group != kBlock && group != 0) return QLIN_ERR_GROUP;
  std::vector<QuantRanges> rs((size_t)count);
  std::vector<QuantJob> qj((size_t)count);
  for (int i = 0; i < count; ++i) {
    const qlin_quant_job& j = jobs[i];
    qlin_status st = check_quant_job(j.w16, j.ld_w, j.n, j.k, bits, group == 0 ? j.k : kBlock,
                                     j.codes, j.scale, j.zero, rs[(size_t)i]);
    if (st != QLIN_OK) return st;
    qj[(size_t)i] = QuantJob{j.w16, j.ld_w, j.codes, j.scale, j.zero, j.n, j.k / kBlock};
  }
  // no job's outputs may overlap another job's inputs or outputs
  for (int i = 0; i < count; ++i)
    for (int j = 0; j < count; ++j) {
      if (i == j) continue;
      const QuantRanges& a = rs[(size_t)i];
      const QuantRanges& b = rs[(size_t)j];
      for (const Range& o : {a.codes, a.scale, a.zero})
        if (overlaps(o, b.in) || overlaps(o, b.codes) || overlaps(o, b.scale) || overlaps(o, b.zero))
          return QLIN_ERR_ALIAS;
    }
  qlin_status st = check_device();
  if (st != QLIN_OK) return st;
  return run_quant(qj.data(), count, bits, group == 0, stream);
}

int64_t qlin_gemv_workspace_bytes(const qlin_weight* w) {
  if (check_weight(w, true, true) != QLIN_OK) return 0;
  return gemv_ws_bytes(tiles_of(w->n), w->k / kBlock,
                       w->format == QLIN_FMT_PACKED ? GemvKind::kPacked : GemvKind::kFused, w->bits);
}

int64_t gemm_set_ws_bytes(const qlin_weight* w, int count, int32_t m) {
  if (w == nullptr || count < 1 || count > kMaxMats || m < 1 || m > kMaxM) return 0;
  int64_t tiles = 0, cols4 = 0;
  bool pairable = true;
  for (int i = 0; i < count; ++i) {
    if (check_weight(&w[i], false, false) != QLIN_OK || w[i].k != w[0].k) return 0;
    tiles += tiles_of(w[i].n);
    cols4 += (tiles_of(w[i].n) + 3) / 4;
    if (count > 1 && tiles_of(w[i].n) % 2 != 0) pairable = false;
  }
  if (m > kSkinnyMaxM || skinny_by_ksplit(tiles, w[0].k / kBlock, w[0].bits))
    return tiles_ws_bytes(cols4, tiles, w[0].k / kBlock, m, count, pairable, w[0].bits);
  return split_ws_bytes(tiles, w[0].k / kBlock, 16);
}

int64_t qlin_gemm_workspace_bytes(const qlin_weight* w, int32_t m) {
  return gemm_set_ws_bytes(w, 1, m);
}

int64_t qlin_gemm_multi_workspace_bytes(const qlin_weight* w, int32_t count, int32_t m) {
  return gemm_set_ws_bytes(w, count, m);
}

qlin_status qlin_gemv(const qlin_weight* w, const uint16_t* x, float* y, void* workspace,
                      int64_t workspace_bytes, hipStream_t stream) {
  qlin_status st = check_weight(w, true, true);
  if (st != QLIN_OK) return st;
  if (x == nullptr || y == nullptr) return QLIN_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return QLIN_ERR_ALIGN;
  if (workspace_bytes < 0) return QLIN_ERR_WORKSPACE;
  if (workspace == nullptr) workspace_bytes = 0;
  if (workspace != nullptr && !aligned16(workspace)) return QLIN_ERR_ALIGN;
  const Range ry = range_of(y, (int64_t)w->n * 4);
  if (overlaps(ry, range_of(x, (int64_t)w->k * 2)) || output_overlaps_weight(w, ry))
    return QLIN_ERR_ALIAS;
  if (workspace_bytes > 0) {
    const Range rw = range_of(workspace, workspace_bytes);
    if (overlaps(rw, ry) || overlaps(rw, range_of(x, (int64_t)w->k * 2)) ||
        output_overlaps_weight(w, rw))
      return QLIN_ERR_ALIAS;
  }
  st = check_device();
  if (st != QLIN_OK) return st;
  const int64_t tiles = tiles_of(w->n);
  const int kb = w->k / kBlock;
  const GemvCfg sp = gemv_config(
      tiles, kb, w->format == QLIN_FMT_PACKED ? GemvKind::kPacked : GemvKind::kFused, w->bits,
      workspace_bytes);
  if (w->format == QLIN_FMT_PACKED)
    return run_packed(packed_launch(&w, &y, 1), w->bits, x, workspace, sp, stream);
  uint32_t* tick = static_cast<uint32_t*>(workspace);
  float* part = sp.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes)
                              : nullptr;
  const f16x2* x2 = reinterpret_cast<const f16x2*>(x);
  {
    switch (w->bits) {
      case 2: launch_gemv_fused<2>(w, x2, y, part, tick, sp, stream); break;
      case 3: launch_gemv_fused<3>(w, x2, y, part, tick, sp, stream); break;
      case 4: launch_gemv_fused<4>(w, x2, y, part, tick, sp, stream); break;
      case 5: launch_gemv_fused<5>(w, x2, y, part, tick, sp, stream); break;
      case 6: launch_gemv_fused<6>(w, x2, y, part, tick, sp, stream); break;
      case 7: launch_gemv_fused<7>(w, x2, y, part, tick, sp, stream); break;
      case 8: launch_gemv_fused<8>(w, x2, y, part, tick, sp, stream); break;
      default: launch_gemv_fused<16>(w, x2, y, part, tick, sp, stream); break;
    }
  }
  return hip_status(hipGetLastError());
}

int64_t qlin_gemv_multi_workspace_bytes(const qlin_weight* w, int32_t count) {
  if (w == nullptr || count < 1 || count > kMaxMats) return 0;
  for (int i = 0; i < count; ++i)
    if (check_weight(&w[i], false, false) != QLIN_OK || w[i].k != w[0].k) return 0;
  return gemv_ws_bytes(set_tiles(w, count), w[0].k / kBlock, GemvKind::kPacked, w[0].bits);
}

qlin_status qlin_gemv_multi(const qlin_weight* w, int32_t count, const uint16_t* x,
                            float* const* y, void* workspace, int64_t workspace_bytes,
                            hipStream_t stream) {
  if (w == nullptr || y == nullptr) return QLIN_ERR_NULL;
  if (count < 1 || count > kMaxMats) return QLIN_ERR_SHAPE;
  void* outs[kMaxMats];
  int64_t out_bytes[kMaxMats];
  for (int i = 0; i < count; ++i) {
    if (y[i] == nullptr) return QLIN_ERR_NULL;
    outs[i] = y[i];
    out_bytes[i] = (int64_t)w[i].n * 4;
  }
  qlin_status st = check_set(w, count, x, outs, out_bytes, count, workspace, workspace_bytes);
  if (st != QLIN_OK) return st;
  if (workspace == nullptr) workspace_bytes = 0;
  st = check_device();
  if (st != QLIN_OK) return st;
  const qlin_weight* wp[kMaxMats];
  for (int i = 0; i < count; ++i) wp[i] = &w[i];
  const PackedLaunch L = packed_launch(wp, y, count);
  const GemvCfg c = gemv_config(L.tiles, L.kb, GemvKind::kPacked, w[0].bits, workspace_bytes);
  return run_packed(L, w[0].bits, x, workspace, c, stream);
}

int64_t qlin_gemv_swiglu_workspace_bytes(const qlin_weight* gate) {
  if (check_weight(gate, false, false) != QLIN_OK) return 0;
  return gemv_ws_bytes(tiles_of(gate->n), gate->k / kBlock, GemvKind::kPair, gate->bits);
}

qlin_status qlin_gemv_swiglu(const qlin_weight* gate, const qlin_weight* up, const uint16_t* x,
                             float* h, uint16_t* h16, void* workspace, int64_t workspace_bytes,
                             hipStream_t stream) {
  if (gate == nullptr || up == nullptr) return QLIN_ERR_NULL;
  if (h == nullptr && h16 == nullptr) return QLIN_ERR_NULL;
  const qlin_weight pair[2] = {*gate, *up};
  void* outs[2] = {h, h16};
  const int64_t out_bytes[2] = {(int64_t)gate->n * 4, (int64_t)gate->n * 2};
  qlin_status st = check_set(pair, 2, x, outs, out_bytes, 2, workspace, workspace_bytes);
  if (st != QLIN_OK) return st;
  if (up->n != gate->n) return QLIN_ERR_SHAPE;
  if (workspace == nullptr) workspace_bytes = 0;
  st = check_device();
  if (st != QLIN_OK) return st;
  const qlin_weight* wp[2] = {gate, up};
  float* ys[2] = {h, nullptr};
  PackedLaunch L = packed_launch(wp, ys, 2);
  L.tiles = (int)tiles_of(gate->n);
  L.swiglu = true;
  L.h16 = h16;
  const GemvCfg c = gemv_config(L.tiles, L.kb, GemvKind::kPair, gate->bits, workspace_bytes);
  return run_packed(L, gate->bits, x, workspace, c, stream);
}

qlin_status qlin_embed_rows(const qlin_weight* w, const int32_t* ids, int32_t count,
                            uint16_t* out16, float* out32, int64_t ld_out, hipStream_t stream) {
  qlin_status st = check_weight(w, false, false);
  if (st != QLIN_OK) return st;
  if (count < 0 || count > kMaxM || ld_out < w->k) return QLIN_ERR_SHAPE;
  if (count == 0) return QLIN_OK;
  if (ids == nullptr || (out16 == nullptr && out32 == nullptr)) return QLIN_ERR_NULL;
  if (ld_out % 8 != 0) return QLIN_ERR_ALIGN;
  if (!aligned16(out16) || !aligned16(out32)) return QLIN_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(ids) & 3u) != 0) return QLIN_ERR_ALIGN;
  const int64_t span = ((int64_t)(count - 1) * ld_out + w->k);
  const Range r16 = range_of(out16, out16 != nullptr ? span * 2 : 0);
  const Range r32 = range_of(out32, out32 != nullptr ? span * 4 : 0);
  const Range rid = range_of(ids, (int64_t)count * 4);
  if (overlaps(r16, r32) || overlaps(r16, rid) || overlaps(r32, rid) ||
      output_overlaps_weight(w, r16) || output_overlaps_weight(w, r32))
    return QLIN_ERR_ALIAS;
  st = check_device();
  if (st != QLIN_OK) return st;
  const int kb = w->k / kBlock;
  const int G = (w->group == w->k) ? 1 : kb;
  const uint32_t* codes = static_cast<const uint32_t*>(w->data);
  switch (w->bits) {
#define QLIN_EMBED(B)                                                                        \
    case B:                                                                                  \
      launch_embed_rows<B>(codes, w->scale, w->zero, ids, count, w->n, kb, G, out16, out32,  \
                           ld_out, stream);                                                  \
      break;
    QLIN_EMBED(2)
    QLIN_EMBED(3)
    QLIN_EMBED(4)
    QLIN_EMBED(5)
    QLIN_EMBED(6)
    QLIN_EMBED(7)
    QLIN_EMBED(8)
#undef QLIN_EMBED
    default: return QLIN_ERR_BITS;
  }
  return hip_status(hipGetLastError());
}

// Launches a checked GEMM plan (M <= 16: skinny kernel, else tiled).
qlin_status run_gemm(const GemmPlan& p, const uint16_t* X, int m, int64_t ld_x, void* workspace,
                     int64_t workspace_bytes, hipStream_t stream) {
  uint32_t* tick = static_cast<uint32_t*>(workspace);
  char* pbase = static_cast<char*>(workspace) + kCounterBytes;
  if (m <= kSkinnyMaxM && !skinny_by_ksplit(p.tiles, p.kb, p.bits)) {
    const Split sp = choose_split(p.tiles, p.kb, workspace_bytes, 16);
    float* part = sp.splits > 1 ? reinterpret_cast<float*>(pbase) : nullptr;
    switch (p.bits) {
      case 2: launch_gemm_skinny<2>(p, X, ld_x, m, part, tick, sp, stream); break;
      case 3: launch_gemm_skinny<3>(p, X, ld_x, m, part, tick, sp, stream); break;
      case 4: launch_gemm_skinny<4>(p, X, ld_x, m, part, tick, sp, stream); break;
      default: launch_gemm_skinny<8>(p, X, ld_x, m, part, tick, sp, stream); break;
    }
  } else {
    bool pairable = true;
    for (int i = 0; p.set.count > 1 && i < p.set.count; ++i)
      if ((p.end_tiles[i] - (i == 0 ? 0 : p.end_tiles[i - 1])) % 2 != 0) pairable = false;
    const TilesCfg c = tiles_config(p.cols4, p.tiles, p.kb, m, p.set.count, pairable, p.bits,
                                    workspace_bytes);
    float* part = c.splits > 1 ? reinterpret_cast<float*>(pbase) : nullptr;
    // launch columns of each matrix in the chosen kernel's unit: four-tile
    // columns for the tiled kernels (the K-split launcher sets its own)
    GemmPlan q = p;
    for (int i = 0; i < q.set.count; ++i) q.set.end[i] = c.mb >= 32 ? p.end_cols4[i] : p.end_tiles[i];
    switch (p.bits) {
      case 2: launch_gemm_tiles<2>(q, X, ld_x, m, c, part, tick, stream); break;
      case 3: launch_gemm_tiles<3>(q, X, ld_x, m, c, part, tick, stream); break;
      case 4: launch_gemm_tiles<4>(q, X, ld_x, m, c, part, tick, stream); break;
      case 5: launch_gemm_tiles<5>(q, X, ld_x, m, c, part, tick, stream); break;
      case 6: launch_gemm_tiles<6>(q, X, ld_x, m, c, part, tick, stream); break;
      case 7: launch_gemm_tiles<7>(q, X, ld_x, m, c, part, tick, stream); break;
      default: launch_gemm_tiles<8>(q, X, ld_x, m, c, part, tick, stream); break;
    }
  }
  return hip_status(hipGetLastError());
}

qlin_status qlin_gemm(const qlin_weight* w, const uint16_t* X, int32_t m, int64_t ld_x, float* Y,
                      int64_t ld_y, void* workspace, int64_t workspace_bytes,
                      hipStream_t stream) {
  return qlin_gemm_multi(w, 1, X, m, ld_x, &Y, &ld_y, workspace, workspace_bytes, stream);
}

qlin_status qlin_gemm_multi(const qlin_weight* w, int32_t count, const uint16_t* X, int32_t m,
                            int64_t ld_x, float* const* Y, const int64_t* ld_y, void* workspace,
                            int64_t workspace_bytes, hipStream_t stream) {
  if (w == nullptr || Y == nullptr || ld_y == nullptr) return QLIN_ERR_NULL;
  if (count < 1 || count > kMaxMats) return QLIN_ERR_SHAPE;
  for (int i = 0; i < count; ++i) {
    const qlin_status st = check_weight(&w[i], false, false);
    if (st != QLIN_OK) return st;
    if (w[i].k != w[0].k) return QLIN_ERR_SHAPE;
    if (w[i].bits != w[0].bits || w[i].group != w[0].group) return QLIN_ERR_FORMAT;
  }
  if (X == nullptr) return QLIN_ERR_NULL;
  if (m < 1 || m > kMaxM || ld_x < w[0].k) return QLIN_ERR_SHAPE;
  if (ld_x % 8 != 0 || !aligned16(X)) return QLIN_ERR_ALIGN;
  if (workspace_bytes < 0) return QLIN_ERR_WORKSPACE;
  if (workspace == nullptr) workspace_bytes = 0;
  if (workspace != nullptr && !aligned16(workspace)) return QLIN_ERR_ALIGN;
  const Range rX = range_of(X, ((int64_t)(m - 1) * ld_x + w[0].k) * 2);
  const Range rw = range_of(workspace, workspace_bytes);
  if (overlaps(rw, rX)) return QLIN_ERR_ALIAS;
  for (int i = 0; i < count; ++i) {
    if (output_overlaps_weight(&w[i], rw)) return QLIN_ERR_ALIAS;
    if (Y[i] == nullptr) return QLIN_ERR_NULL;
    if (ld_y[i] < w[i].n) return QLIN_ERR_SHAPE;
    if (!aligned16(Y[i])) return QLIN_ERR_ALIGN;
    const Range rY = range_of(Y[i], ((int64_t)(m - 1) * ld_y[i] + w[i].n) * 4);
    if (overlaps(rY, rX) || overlaps(rY, rw)) return QLIN_ERR_ALIAS;
    for (int j = 0; j < count; ++j)
      if (output_overlaps_weight(&w[j], rY)) return QLIN_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(rY, range_of(Y[j], ((int64_t)(m - 1) * ld_y[j] + w[j].n) * 4)))
        return QLIN_ERR_ALIAS;
  }
  const qlin_status st = check_device();
  if (st != QLIN_OK) return st;
  const qlin_weight* wp[kMaxMats];
  for (int i = 0; i < count; ++i) wp[i] = &w[i];
  const GemmPlan p = gemm_plan(wp, Y, ld_y, count, m <= kSkinnyMaxM);
  return run_gemm(p, X, m, ld_x, workspace, workspace_bytes, stream);
}

int64_t qlin_gemm_swiglu_workspace_bytes(const qlin_weight* gate, int32_t m) {
  if (check_weight(gate, false, false) != QLIN_OK || m < 1 || m > kMaxM) return 0;
  return swiglu_ws_bytes(tiles_of(gate->n), gate->k / kBlock, m);
}

qlin_status qlin_gemm_swiglu(const qlin_weight* gate, const qlin_weight* up, const uint16_t* X,
                             int32_t m, int64_t ld_x, float* H, uint16_t* H16, int64_t ld_h,
                             void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  if (gate == nullptr || up == nullptr || X == nullptr) return QLIN_ERR_NULL;
  if (H == nullptr && H16 == nullptr) return QLIN_ERR_NULL;
  const qlin_weight* wp[2] = {gate, up};
  for (int i = 0; i < 2; ++i) {
    const qlin_status st = check_weight(wp[i], false, false);
    if (st != QLIN_OK) return st;
  }
  if (up->k != gate->k || up->n != gate->n) return QLIN_ERR_SHAPE;
  if (up->bits != gate->bits || up->group != gate->group) return QLIN_ERR_FORMAT;
  const int n = gate->n, k = gate->k;
  if (m < 1 || m > kMaxM || ld_x < k || ld_h < n) return QLIN_ERR_SHAPE;
  if (ld_x % 8 != 0 || !aligned16(X) || !aligned16(H) || !aligned16(H16)) return QLIN_ERR_ALIGN;
  if (workspace_bytes < 0) return QLIN_ERR_WORKSPACE;
  if (workspace == nullptr) workspace_bytes = 0;
  if (workspace != nullptr && !aligned16(workspace)) return QLIN_ERR_ALIGN;
  const int64_t span = (int64_t)(m - 1) * ld_h + n;
  const Range rX = range_of(X, ((int64_t)(m - 1) * ld_x + k) * 2);
  const Range rw = range_of(workspace, workspace_bytes);
  const Range rH = range_of(H, H != nullptr ? span * 4 : 0);
  const Range rH16 = range_of(H16, H16 != nullptr ? span * 2 : 0);
  const Range outs[3] = {rw, rH, rH16};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], rX)) return QLIN_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], outs[j])) return QLIN_ERR_ALIAS;
    for (int j = 0; j < 2; ++j)
      if (output_overlaps_weight(wp[j], outs[i])) return QLIN_ERR_ALIAS;
  }
  const qlin_status st = check_device();
  if (st != QLIN_OK) return st;
  const int64_t tiles = tiles_of(n);
  const int kb = k / kBlock;
  const int G = (gate->group == k) ? 1 : kb;
  const TilesCfg c = swiglu_config(tiles, kb, m, workspace_bytes);
  GemmSet set{};
  for (int i = 0; i < 2; ++i) {
    set.codes[i] = static_cast<const uint32_t*>(wp[i]->data);
    set.scale[i] = wp[i]->scale;
    set.zero[i] = wp[i]->zero;
    set.n[i] = n;
    set.ldy[i] = ld_h;
  }
  set.y[0] = H;
  set.end[0] = c.gx;                 // every launch column is matrix 0's (the pair's)
  set.end[1] = c.gx;
  set.count = 2;
  set.h16 = H16;
  uint32_t* tick = static_cast<uint32_t*>(workspace);
  float* part = c.splits > 1
      ? reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes) : nullptr;
  switch (gate->bits) {
    case 2: launch_gemm_swiglu<2>(set, X, ld_x, m, kb, G, c, part, tick, stream); break;
    case 3: launch_gemm_swiglu<3>(set, X, ld_x, m, kb, G, c, part, tick, stream); break;
    case 4: launch_gemm_swiglu<4>(set, X, ld_x, m, kb, G, c, part, tick, stream); break;
    case 5: launch_gemm_swiglu<5>(set, X, ld_x, m, kb, G, c, part, tick, stream); break;
    case 6: launch_gemm_swiglu<6>(set, X, ld_x, m, kb, G, c, part, tick, stream); break;
    case 7: launch_gemm_swiglu<7>(set, X, ld_x, m, kb, G, c, part, tick, stream); break;
    default: launch_gemm_swiglu<8>(set, X, ld_x, m, kb, G, c, part, tick, stream); break;
  }
  return hip_status(hipGetLastError());
}

qlin_status qlin_set_launch_override(int32_t family, const int32_t* params) {
  if (family != QLIN_TUNE_GEMV && family != QLIN_TUNE_GEMM) return QLIN_ERR_SHAPE;
  if (params == nullptr) {
    g_override[family].store(0, std::memory_order_relaxed);
    return QLIN_OK;
  }
  const int a = params[0], b = params[1], c = family == QLIN_TUNE_GEMV ? params[2] : 0;
  if (b < 1 || b > 0xFFFF) return QLIN_ERR_SHAPE;
  if (family == QLIN_TUNE_GEMV) {
    if (!(a == 4 || a == 8 || a == 16) || !(c == 8 || c == 16 || c == 64)) return QLIN_ERR_SHAPE;
  } else if (!((a >= 0 && a <= 8) || a == 16 || a == 32 || a == 64 || a == 128)) {
    return QLIN_ERR_SHAPE;
  }
  g_override[family].store((1ull << 63) | (uint64_t)(uint32_t)a | ((uint64_t)(uint32_t)b << 16) |
                               ((uint64_t)(uint32_t)c << 32),
                           std::memory_order_relaxed);
  return QLIN_OK;
}

qlin_status qlin_gemv_noalloc(const qlin_weight* w, const uint16_t* x, float* y,
                              hipStream_t stream) {
  // host checks first (every error but QLIN_ERR_HIP / NO_DEVICE before any
  // HIP call), then the scratch array's address on this device
  qlin_status st = check_weight(w, true, true);
  if (st != QLIN_OK) return st;
  if (x == nullptr || y == nullptr) return QLIN_ERR_NULL;
  const int64_t need = qlin_gemv_workspace_bytes(w);
  if (need > kNoAllocScratchBytes) return QLIN_ERR_WORKSPACE;
  st = check_device();
  if (st != QLIN_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != QLIN_OK) return st;
  if (need > 0) {
    // the launch splits K: its arrival counters must start at zero (calls
    // leave them zero, but the array keeps whatever the last call left)
    hipLaunchKernelGGL(k_clear_counters, dim3(16), dim3(256), 0, stream,
                       static_cast<uint32_t*>(ws), (int)(kCounterBytes / 4));
    st = hip_status(hipGetLastError());
    if (st != QLIN_OK) return st;
  }
  return qlin_gemv(w, x, y, ws, need, stream);
}

}  // extern "C"
