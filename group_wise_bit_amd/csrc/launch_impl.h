// Kernel launchers: launch shapes -> hipLaunchKernelGGL, templated on the bit
// width.  Included only by inst.hip, which instantiates one width per object.
#pragma once

#include "plan.h"

namespace qlin {

// One launch per kQuantBatch jobs (same bits, same group kind).
template <int B>
void launch_quant_batch(const QuantJob* jobs, int count, bool row, hipStream_t st) {
  for (int c0 = 0; c0 < count; c0 += kQuantBatch) {
    QuantBatch qb;
    qb.count = count - c0 < kQuantBatch ? count - c0 : kQuantBatch;
    int items = 0;
    for (int i = 0; i < qb.count; ++i) {
      qb.job[i] = jobs[c0 + i];
      const int tiles = (int)tiles_of(qb.job[i].n);
      items += row ? tiles : tiles * ((qb.job[i].kb + kWaves - 1) / kWaves);
      qb.end[i] = items;
    }
    for (int i = qb.count; i < kQuantBatch; ++i) qb.end[i] = items;
    if (row)
      hipLaunchKernelGGL((k_quantize_row<B, kWaves>), dim3(items), dim3(kWaves * 64), 0, st, qb);
    else
      hipLaunchKernelGGL((k_quantize_g64<B, kWaves>), dim3(items), dim3(kWaves * 64), 0, st, qb);
  }
}

template <int B, int W, int U, bool SW>
void launch_gemv_packed_w(const PackedLaunch& L, const f16x2* x2, float* part, uint32_t* tick,
                          GemvCfg c, hipStream_t st) {
  if (c.rows == 16)
    hipLaunchKernelGGL((k_gemv_narrow<B, 4, W, U, SW>), dim3(4 * L.tiles, c.splits), dim3(W * 64),
                       0, st, L.set, x2, part, tick, L.kb, L.G, c.splits, c.kbps, L.h16);
  else if (c.rows == 8)
    hipLaunchKernelGGL((k_gemv_narrow<B, 8, W, U, SW>), dim3(8 * L.tiles, c.splits), dim3(W * 64),
                       0, st, L.set, x2, part, tick, L.kb, L.G, c.splits, c.kbps, L.h16);
  else
    hipLaunchKernelGGL((k_gemv_packed<B, W, U, SW>), dim3(L.tiles, c.splits), dim3(W * 64), 0, st,
                       L.set, x2, part, tick, L.kb, L.G, c.splits, c.kbps, L.h16);
}

template <int B, bool SW>
void launch_gemv_packed_s(const PackedLaunch& L, const f16x2* x2, float* part, uint32_t* tick,
                          GemvCfg c, hipStream_t st) {
  if (c.waves == 16) {
    if (c.unroll == 1) launch_gemv_packed_w<B, 16, 1, SW>(L, x2, part, tick, c, st);
    else if (c.unroll == 2) launch_gemv_packed_w<B, 16, 2, SW>(L, x2, part, tick, c, st);
    else launch_gemv_packed_w<B, 16, ((SW && B > 4) ? 2 : 4), SW>(L, x2, part, tick, c, st);
  } else if (c.waves == 8) {
    if (c.unroll == 1) launch_gemv_packed_w<B, 8, 1, SW>(L, x2, part, tick, c, st);
    else if (c.unroll == 2) launch_gemv_packed_w<B, 8, 2, SW>(L, x2, part, tick, c, st);
    else launch_gemv_packed_w<B, 8, ((SW && B > 4) ? 2 : 4), SW>(L, x2, part, tick, c, st);
  } else {
    if (c.unroll == 1) launch_gemv_packed_w<B, 4, 1, SW>(L, x2, part, tick, c, st);
    else if (c.unroll == 2) launch_gemv_packed_w<B, 4, 2, SW>(L, x2, part, tick, c, st);
    else launch_gemv_packed_w<B, 4, ((SW && B > 4) ? 2 : 4), SW>(L, x2, part, tick, c, st);
  }
}

template <int B>
void launch_gemv_packed(const PackedLaunch& L, const f16x2* x2, float* part, uint32_t* tick,
                        GemvCfg c, hipStream_t st) {
  if (L.swiglu) launch_gemv_packed_s<B, true>(L, x2, part, tick, c, st);
  else launch_gemv_packed_s<B, false>(L, x2, part, tick, c, st);
}

template <int B, int W, int U>
void launch_gemv_fused_w(const qlin_weight* w, const f16x2* x2, float* y, float* part,
                         uint32_t* tick, GemvCfg c, hipStream_t st) {
  const int kb = w->k / kBlock;
  const int G = (w->bits == 16 || w->group != w->k) ? kb : 1;
  dim3 grid((unsigned)tiles_of(w->n), c.splits);
  hipLaunchKernelGGL((k_gemv_fused<B, W, U>), grid, dim3(W * 64), 0, st,
                     static_cast<const uint16_t*>(w->data), w->ld, w->scale, w->zero, x2, y, part,
                     tick, w->n, kb, G, c.splits, c.kbps);
}

template <int B, int W, int U>
void launch_gemv_fused_narrow_w(const qlin_weight* w, const f16x2* x2, float* y, float* part,
                                uint32_t* tick, GemvCfg c, hipStream_t st) {
  const int kb = w->k / kBlock;
  const int G = (w->bits == 16 || w->group != w->k) ? kb : 1;
  dim3 grid((unsigned)(8 * tiles_of(w->n)), c.splits);
  hipLaunchKernelGGL((k_gemv_fused_narrow<B, W, U>), grid, dim3(W * 64), 0, st,
                     static_cast<const uint16_t*>(w->data), w->ld, w->scale, w->zero, x2, y, part,
                     tick, w->n, kb, G, c.splits, c.kbps);
}

// The 64-row fused kernel needs ~150 VGPRs: at most 8 waves (512 threads) per
// work-group.
template <int B>
void launch_gemv_fused(const qlin_weight* w, const f16x2* x2, float* y, float* part,
                       uint32_t* tick, GemvCfg c, hipStream_t st) {
  if (c.rows == 8) {
    if (c.waves == 16) {
      if (c.unroll == 1) launch_gemv_fused_narrow_w<B, 16, 1>(w, x2, y, part, tick, c, st);
      else launch_gemv_fused_narrow_w<B, 16, 2>(w, x2, y, part, tick, c, st);
    } else if (c.waves == 8) {
      if (c.unroll == 1) launch_gemv_fused_narrow_w<B, 8, 1>(w, x2, y, part, tick, c, st);
      else launch_gemv_fused_narrow_w<B, 8, 2>(w, x2, y, part, tick, c, st);
    } else {
      if (c.unroll == 1) launch_gemv_fused_narrow_w<B, 4, 1>(w, x2, y, part, tick, c, st);
      else launch_gemv_fused_narrow_w<B, 4, 2>(w, x2, y, part, tick, c, st);
    }
  } else if (c.waves >= 8) {
    launch_gemv_fused_w<B, 8, 1>(w, x2, y, part, tick, c, st);
  } else {
    launch_gemv_fused_w<B, 4, 1>(w, x2, y, part, tick, c, st);
  }
}

template <int B>
void launch_gemm_skinny(const GemmPlan& p, const uint16_t* X, int64_t ldx, int m, float* part,
                        uint32_t* tick, Split sp, hipStream_t st) {
  hipLaunchKernelGGL((k_gemm_skinny<B, kWaves, 2>), dim3((unsigned)p.tiles, sp.splits),
                     dim3(kWaves * 64), 0, st, p.set, X, ldx, m, part, tick, p.kb, p.G,
                     sp.splits, sp.kbps);
}

// MB = 32: the register-staged kernel (several work-groups per CU hide its
// load latency); MB = 64 / 128: the LDS-DMA pipeline, 4 / 3 stages deep
// (two work-groups per CU).
template <int B, int MB>
void launch_tiles_mb(const GemmPlan& p, const uint16_t* X, int64_t ldx, int m, TilesCfg c,
                     float* part, uint32_t* tick, hipStream_t st) {
  if constexpr (MB == 32)
    hipLaunchKernelGGL((k_gemm_tiles<B, MB>), dim3(c.gx, c.gy, c.splits), dim3(256), 0, st,
                       p.set, X, ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
  else
    hipLaunchKernelGGL((k_gemm_lds<B, MB, (MB == 128 ? 3 : 4)>), dim3(c.gx, c.gy, c.splits),
                       dim3(256), 0, st, p.set, X, ldx, m, p.kb, p.G, c.splits, c.kbps, part,
                       tick);
}

// Grids of no more work-groups than CUs, 32 X rows over whole tiles, long K:
// the work-group's waves split K further -- 8 waves with 4 blocks in flight
// each, or 16 with 2 for the widths whose decode costs more (3, 5, 6 bits;
// 7 would spill) -- so that each SIMD runs two or four instruction streams
// and one wave's decode goes beside another's MFMAs.  (Measured on the
// Qwen3-8B GEMMs at M = 128, against one wave per SIMD holding two sets of
// loads: the int4 step 4.29 -> 4.18 ms, int3 4.55 -> 4.40; o and down 7-10 %
// faster with 16 waves than with 8 at 3 and 5 bits, equal at 2, 4 and 8.)
// Returns whether it launched.
template <int B, int RB>
bool launch_ksplit_one_cu(bool want, dim3 grid, const GemmSet& set, const GemmPlan& p,
                          const uint16_t* X, int64_t ldx, int m, const TilesCfg& c, float* part,
                          uint32_t* tick, hipStream_t st) {
  if constexpr (RB == 1) {
    if (want) {
      if constexpr (B == 3 || B == 5 || B == 6)
        hipLaunchKernelGGL((k_gemm_ksplit<B, 2, 1, false, false, 2, 16>), grid, dim3(1024), 0,
                           st, set, X, ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
      else
        hipLaunchKernelGGL((k_gemm_ksplit<B, 4, 1, false, false, 2, 8>), grid, dim3(512), 0, st,
                           set, X, ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
      return true;
    }
  }
  return false;
}

template <int B, int RB>
void launch_gemm_ksplit_rb(const GemmSet& set, const GemmPlan& p, const uint16_t* X,
                           int64_t ldx, int m, TilesCfg c, float* part, uint32_t* tick,
                           hipStream_t st) {
  // blocks in flight per wave: the wave's share of the split, up to 4 (2 for
  // 64-row X tiles, whose X fragments take twice the registers)
  const int per_wave = (c.kbps + 3) / 4;
  const dim3 grid(c.gx, c.gy, c.splits);
  const bool one_per_cu = (int64_t)c.gx * c.gy * c.splits <= 256;
  if constexpr (RB == 4) {
    // 128 X rows: the X fragments of a block take 64 registers; two blocks
    // in flight per wave when the wave has them (one wave per SIMD, up to
    // 512 registers), whole or half tiles
    if (c.half) {
      if (per_wave >= 2)
        hipLaunchKernelGGL((k_gemm_ksplit<B, 2, 4, false, false, 1>), grid, dim3(256), 0, st,
                           set, X, ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
      else
        hipLaunchKernelGGL((k_gemm_ksplit<B, 1, 4, false, false, 1>), grid, dim3(256), 0, st,
                           set, X, ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
    } else {
      if (per_wave >= 2)
        hipLaunchKernelGGL((k_gemm_ksplit<B, 2, 4>), grid, dim3(256), 0, st, set, X, ldx, m,
                           p.kb, p.G, c.splits, c.kbps, part, tick);
      else
        hipLaunchKernelGGL((k_gemm_ksplit<B, 1, 4>), grid, dim3(256), 0, st, set, X, ldx, m,
                           p.kb, p.G, c.splits, c.kbps, part, tick);
    }
  } else {
  if (c.half && RB == 1 && m <= 16) {
    // M <= 16 over half tiles: 16 waves split K, as in the decode GEMV, so
    // that a work-group keeps up to 64 blocks in flight
    // (a 16-wave work-group caps a wave at 128 registers: four blocks in
    // flight fit up to 4 bits)
    const int per16 = (c.kbps + 15) / 16;
    const dim3 block(1024);
    bool done = false;
    if constexpr (B <= 4) {
      if (per16 >= 4) {
        hipLaunchKernelGGL((k_gemm_ksplit<B, 4, 1, false, false, 1, 16>), grid, block, 0, st,
                           set, X, ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
        done = true;
      }
    }
    if (done) {
    } else if (per16 >= 2)
      hipLaunchKernelGGL((k_gemm_ksplit<B, 2, 1, false, false, 1, 16>), grid, block, 0, st, set,
                         X, ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
    else
      hipLaunchKernelGGL((k_gemm_ksplit<B, 1, 1, false, false, 1, 16>), grid, block, 0, st, set,
                         X, ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
  } else if (c.half) {   // half tiles: half the codes and accumulators per wave
    if (per_wave >= 4 && RB == 1)
      hipLaunchKernelGGL((k_gemm_ksplit<B, 4, RB, false, false, 1>), grid, dim3(256), 0, st, set,
                         X, ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
    else if (per_wave >= 2)
      hipLaunchKernelGGL((k_gemm_ksplit<B, 2, RB, false, false, 1>), grid, dim3(256), 0, st, set,
                         X, ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
    else
      hipLaunchKernelGGL((k_gemm_ksplit<B, 1, RB, false, false, 1>), grid, dim3(256), 0, st, set,
                         X, ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
  } else if (c.dual) {   // tile pairs: two accumulator sets, so at most 2 blocks in flight
                         // (1 with 64 X rows, to keep 2 waves per SIMD, unless the grid
                         // has no more work-groups than CUs: one wave per SIMD anyway)
    bool done = false;
    // a grid of no more work-groups than CUs, 32 X rows: 8 waves split K, two
    // instruction streams per SIMD (the Qwen3-8B q/k/v set at M = 128: 20.4
    // us, against 24.4 with 16 waves of one block)
    if constexpr (RB == 1) {
      if (one_per_cu && per_wave >= 4) {
        hipLaunchKernelGGL((k_gemm_ksplit<B, 2, RB, false, true, 2, 8>), grid, dim3(512), 0, st,
                           set, X, ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
        done = true;
      }
    } else if constexpr (B != 5) {   // (64 X rows at 5 bits would spill)
      if (one_per_cu && per_wave >= 4) {
        hipLaunchKernelGGL((k_gemm_ksplit<B, 1, RB, false, true, 2, 8>), grid, dim3(512), 0, st,
                           set, X, ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
        done = true;
      }
    }
    if (done) {
    } else if ((RB == 1 || one_per_cu) && per_wave >= 2)
      hipLaunchKernelGGL((k_gemm_ksplit<B, 2, RB, false, true>), grid, dim3(256), 0, st, set, X,
                         ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
    else
      hipLaunchKernelGGL((k_gemm_ksplit<B, 1, RB, false, true>), grid, dim3(256), 0, st, set, X,
                         ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
  } else if (launch_ksplit_one_cu<B, RB>(one_per_cu && per_wave >= 8, grid, set, p, X, ldx, m,
                                          c, part, tick, st)) {
  } else if (per_wave >= 4 && RB == 1)
    hipLaunchKernelGGL((k_gemm_ksplit<B, 4, RB>), grid, dim3(256), 0, st, set, X, ldx, m, p.kb,
                       p.G, c.splits, c.kbps, part, tick);
  else if (per_wave >= 2)
    hipLaunchKernelGGL((k_gemm_ksplit<B, 2, RB>), grid, dim3(256), 0, st, set, X, ldx, m, p.kb,
                       p.G, c.splits, c.kbps, part, tick);
  else
    hipLaunchKernelGGL((k_gemm_ksplit<B, 1, RB>), grid, dim3(256), 0, st, set, X, ldx, m, p.kb,
                       p.G, c.splits, c.kbps, part, tick);
  }
}

template <int B>
void launch_gemm_ksplit(const GemmPlan& p, const uint16_t* X, int64_t ldx, int m, TilesCfg c,
                        float* part, uint32_t* tick, hipStream_t st) {
  GemmSet set = p.set;
  for (int i = 0; i < set.count; ++i)
    set.end[i] = c.dual   ? (p.end_tiles[i] + 1) / 2
                 : c.half ? 2 * p.end_tiles[i]
                          : p.end_tiles[i];
  if (c.mb == kMbKsplit128) launch_gemm_ksplit_rb<B, 4>(set, p, X, ldx, m, c, part, tick, st);
  else if (c.mb == 1) launch_gemm_ksplit_rb<B, 2>(set, p, X, ldx, m, c, part, tick, st);
  else launch_gemm_ksplit_rb<B, 1>(set, p, X, ldx, m, c, part, tick, st);
}

template <int B>
void launch_gemm_tiles(const GemmPlan& p, const uint16_t* X, int64_t ldx, int m, TilesCfg c,
                       float* part, uint32_t* tick, hipStream_t st) {
  if (c.mb == kMbWdec) {
    // launch columns are tile pairs within each matrix (pairable sets)
    GemmSet set = p.set;
    for (int i = 0; i < set.count; ++i) set.end[i] = (p.end_tiles[i] + 1) / 2;
    hipLaunchKernelGGL((k_gemm_wdec<B, false, 4, 2>), dim3(c.gx, c.gy, c.splits), dim3(512), 0, st,
                       set, X, ldx, m, p.kb, p.G, c.splits, c.kbps, part, tick);
  } else if (is_ksplit(c.mb)) launch_gemm_ksplit<B>(p, X, ldx, m, c, part, tick, st);
  else if (c.mb == 32) launch_tiles_mb<B, 32>(p, X, ldx, m, c, part, tick, st);
  else if (c.mb == 64) launch_tiles_mb<B, 64>(p, X, ldx, m, c, part, tick, st);
  else launch_tiles_mb<B, 128>(p, X, ldx, m, c, part, tick, st);
}

template <int B>
void launch_gemm_swiglu(const GemmSet& set, const uint16_t* X, int64_t ldx, int m, int kb, int G,
                        TilesCfg c, float* part, uint32_t* tick, hipStream_t st) {
  const dim3 grid(c.gx, c.gy, c.splits);
  if (c.mb == kMbWdec)
    hipLaunchKernelGGL((k_gemm_wdec<B, true, 4, 2>), grid, dim3(512), 0, st, set, X, ldx, m, kb, G,
                       c.splits, c.kbps, part, tick);
  else if (c.mb == 128)
    hipLaunchKernelGGL((k_gemm_lds<B, 128, 3, true>), grid, dim3(256), 0, st, set, X, ldx, m, kb,
                       G, c.splits, c.kbps, part, tick);
  else if (c.mb == 64)
    hipLaunchKernelGGL((k_gemm_lds<B, 64, 4, true>), grid, dim3(256), 0, st, set, X, ldx, m, kb,
                       G, c.splits, c.kbps, part, tick);
  else if (c.half) {   // half tiles of both matrices
    if (c.mb == kMbKsplit128 && (c.kbps + 3) / 4 >= 2)
      hipLaunchKernelGGL((k_gemm_ksplit<B, 2, 4, true, false, 1>), grid, dim3(256), 0, st, set,
                         X, ldx, m, kb, G, c.splits, c.kbps, part, tick);
    else if (c.mb == kMbKsplit128)
      hipLaunchKernelGGL((k_gemm_ksplit<B, 1, 4, true, false, 1>), grid, dim3(256), 0, st, set,
                         X, ldx, m, kb, G, c.splits, c.kbps, part, tick);
    else if (c.mb == 1)
      hipLaunchKernelGGL((k_gemm_ksplit<B, 1, 2, true, false, 1>), grid, dim3(256), 0, st, set,
                         X, ldx, m, kb, G, c.splits, c.kbps, part, tick);
    else if ((c.kbps + 3) / 4 >= 4)
      hipLaunchKernelGGL((k_gemm_ksplit<B, 4, 1, true, false, 1>), grid, dim3(256), 0, st, set,
                         X, ldx, m, kb, G, c.splits, c.kbps, part, tick);
    else if ((c.kbps + 3) / 4 >= 2)
      hipLaunchKernelGGL((k_gemm_ksplit<B, 2, 1, true, false, 1>), grid, dim3(256), 0, st, set,
                         X, ldx, m, kb, G, c.splits, c.kbps, part, tick);
    else
      hipLaunchKernelGGL((k_gemm_ksplit<B, 1, 1, true, false, 1>), grid, dim3(256), 0, st, set,
                         X, ldx, m, kb, G, c.splits, c.kbps, part, tick);
  } else if (c.mb == 1)
    hipLaunchKernelGGL((k_gemm_ksplit<B, 1, 2, true>), grid, dim3(256), 0, st, set, X, ldx, m,
                       kb, G, c.splits, c.kbps, part, tick);
  else if (B <= 4 && (c.kbps + 3) / 4 >= 4)   // (wider codes: 1 wave per SIMD at 4 blocks)
    hipLaunchKernelGGL((k_gemm_ksplit<B, (B <= 4 ? 4 : 2), 1, true>), grid, dim3(256), 0, st,
                       set, X, ldx, m, kb, G, c.splits, c.kbps, part, tick);
  else if ((c.kbps + 3) / 4 >= 2)
    hipLaunchKernelGGL((k_gemm_ksplit<B, 2, 1, true>), grid, dim3(256), 0, st, set, X, ldx, m,
                       kb, G, c.splits, c.kbps, part, tick);
  else
    hipLaunchKernelGGL((k_gemm_ksplit<B, 1, 1, true>), grid, dim3(256), 0, st, set, X, ldx, m,
                       kb, G, c.splits, c.kbps, part, tick);
}

template <int B>
void launch_embed_rows(const uint32_t* codes, const uint16_t* scale, const uint8_t* zero,
                       const int32_t* ids, int count, int n, int kb, int G, uint16_t* out16,
                       float* out32, int64_t ld_out, hipStream_t st) {
  hipLaunchKernelGGL((k_embed_rows<B>), dim3(count), dim3(256), 0, st, codes, scale, zero, ids,
                     n, kb, G, out16, out32, ld_out);
}

}  // namespace qlin
