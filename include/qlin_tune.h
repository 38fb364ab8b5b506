/*
 * qlin launch-shape override: for launch-shape sweeps and for tests that must
 * reach every kernel form.  Not part of the production interface: a normal
 * caller never calls it, and then every launch shape is the library's own
 * choice for the call's sizes (a pure function of them).
 *
 * qlin_set_launch_override(family, params) makes every later call of that
 * family, from any thread, use the given shape instead; params = NULL restores
 * the library's choice.  Results differ only by the order of the fp32
 * summation that another split implies and stay within the same tolerance.
 * Setting it while other threads launch kernels is allowed (each call reads
 * one consistent snapshot) but makes their launch shape depend on timing.
 *
 *   QLIN_TUNE_GEMV: params[0] = waves per work-group (4, 8, 16), params[1] =
 *     K splits across work-groups (>= 1, capped at the K-blocks), params[2] =
 *     rows per work-group (64: whole tiles; 16 or 8: narrow work-groups).
 *   QLIN_TUNE_GEMM: params[0] = kernel form (0 / 1: K-split kernel with 32 /
 *     64 X rows; 2 / 3: the same with 64 / 32 X rows over tile pairs; 4 / 5:
 *     with 32 / 64 X rows over half tiles; 6 / 7: with 128 X rows over whole /
 *     half tiles (the SwiGLU pair always over half tiles); 8: 128 X rows x
 *     a tile pair (the SwiGLU pair: tile t of gate and of up), each weight
 *     decoded once per work-group (a set whose matrices do not all have an
 *     even tile count runs form 0 instead); 16: the skinny kernel at m <= 16;
 *     32 / 64 / 128: tiled kernels with that X-tile height), params[1] = K
 *     splits across work-groups (>= 1).
 * Returns QLIN_OK, or QLIN_ERR_SHAPE for an unknown family or a value out of
 * range.  Splits are still capped by the workspace the call provides.
 */
#ifndef QLIN_TUNE_H
#define QLIN_TUNE_H

#include <stdint.h>
#include "qlin.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { QLIN_TUNE_GEMV = 0, QLIN_TUNE_GEMM = 1 };

qlin_status qlin_set_launch_override(int32_t family, const int32_t* params);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_TUNE_H */
