// One bit width's kernel launchers (and so its kernels), compiled as its own
// object: build.py compiles this file once per width with
// -DQLIN_INST_BITS=<width> and -DQLIN_INST_PART=<0: GEMV and row gather;
// 1: GEMM; 2: the quantizer, built with -ffp-contract=off so that no a*b+c of
// its scale, zero-point and code arithmetic is fused into one rounding>, in
// parallel, and links the objects with qlin_api.hip.
#include "launch_impl.h"

#ifndef QLIN_INST_BITS
#error "QLIN_INST_BITS must be defined"
#endif
#ifndef QLIN_INST_PART
#error "QLIN_INST_PART must be defined"
#endif

namespace qlin {

constexpr int kB = QLIN_INST_BITS;

#if QLIN_INST_PART == 0
#if QLIN_INST_BITS == 16
template void launch_gemv_fused<16>(const qlin_weight*, const f16x2*, float*, float*, uint32_t*,
                                    GemvCfg, hipStream_t);
#else
template void launch_gemv_packed<kB>(const PackedLaunch&, const f16x2*, float*, uint32_t*,
                                     GemvCfg, hipStream_t);
template void launch_gemv_fused<kB>(const qlin_weight*, const f16x2*, float*, float*, uint32_t*,
                                    GemvCfg, hipStream_t);
template void launch_embed_rows<kB>(const uint32_t*, const uint16_t*, const uint8_t*,
                                    const int32_t*, int, int, int, int, uint16_t*, float*, int64_t,
                                    hipStream_t);
#endif
#elif QLIN_INST_PART == 1
template void launch_gemm_tiles<kB>(const GemmPlan&, const uint16_t*, int64_t, int, TilesCfg,
                                    float*, uint32_t*, hipStream_t);
template void launch_gemm_swiglu<kB>(const GemmSet&, const uint16_t*, int64_t, int, int, int,
                                     TilesCfg, float*, uint32_t*, hipStream_t);
#if QLIN_INST_BITS == 2 || QLIN_INST_BITS == 3 || QLIN_INST_BITS == 4 || QLIN_INST_BITS == 8
template void launch_gemm_skinny<kB>(const GemmPlan&, const uint16_t*, int64_t, int, float*,
                                     uint32_t*, Split, hipStream_t);
#endif
#else
template void launch_quant_batch<kB>(const QuantJob*, int, bool, hipStream_t);
#endif

}  // namespace qlin
