/*
 * qlin -- fused dequantize-matmul over group-wise affine low-bit weights, for
 * AMD Instinct MI355X (gfx950).  C ABI; every entry point enqueues HIP kernels
 * on the caller's stream and returns without synchronizing.
 *
 * What is computed (the Bitcrush README, sections "The machine" and "Under the
 * hood"; the Enargeia page, section "Run it"):
 *   - W [n, k] holds n output rows; k is the reduction axis.  Along k, each row
 *     is cut into groups of 64 weights ("SMART"), or one group covers the whole
 *     row ("NAIVE", one scale per output channel).
 *   - Each group has an fp16 scale s and an integer zero point z, found by
 *     round-to-nearest from the group's min and max:
 *         s = fp16( fl32( fl32(max - min) / qmax ) ),  qmax = 2^bits - 1
 *         z = clamp( rint( fl32(-min / s) ), 0, qmax )
 *     and each weight's code is  q = clamp( rint( fl32(w / s) ) + z, 0, qmax ),
 *     rint rounding half-way cases to even.  A group whose stored scale is 0
 *     (all values equal) has z = 0 and all codes 0.
 *   - The matmul uses each code as the weight s * (q - z), formed in registers
 *     and never written to memory, and accumulates in fp32.
 *
 * Memory ownership: the caller allocates and frees every buffer (device memory
 * unless noted); the library allocates nothing and keeps no state apart from
 * the calling thread's last HIP error code.  All pointers must be 16-byte
 * aligned device pointers.  A call that fails validation returns an error
 * before touching the GPU.  Output buffers must not overlap any input.
 * Under HIP stream (graph) capture a call records its kernel launches with the
 * pointers it was given: every buffer a captured call addresses (codes,
 * scales, zeros, x, outputs, workspace) must stay allocated at the same
 * address for as long as the graph may be replayed.
 *
 * ---------------------------------------------------------------------------
 * Packed-code layout ("tiled"):
 *   Rows are taken in tiles of 64; the last tile is padded with rows whose
 *   codes, scales and zeros are 0.  k is cut into blocks of 64 codes (k must be
 *   a multiple of 64).  The 64 codes of row n, block j occupy 2*bits uint32
 *   words; blocks are stored tile-major, then block, then row within the tile:
 *       word offset = ((n / 64) * (k / 64) + j) * 64 * 2*bits + (n % 64) * 2*bits
 *   so one block of a whole tile (64 rows) is one contiguous 128*bits-byte run.
 *   Inside a block:
 *   - bits 2, 4, 8: word w holds codes c = w*(32/bits) + i, i = 0 .. 32/bits-1;
 *     even i fill the low 16 bits and odd i the high 16 bits, each half from
 *     its least significant bit up, in order of i:
 *         bit position of code i = 16*(i % 2) + bits*(i / 2).
 *   - bits 3: codes form two runs of 32 (run r = c / 32), each in three words.
 *     Words 3r and 3r+1 hold the low two bits of run codes 0..15 and 16..31 in
 *     the 2-bit arrangement above; word 3r+2 holds bit 2 of all 32 run codes:
 *     run code c' (0..31) with u = c'/16, i = c'%16, p = i/2, e = i%2 puts it
 *     at position  (p < 4 ? 2p + 2 : 2(p-4) + 3) + 16e,  plus 8 (mod 32) if u = 1.
 *   - bits 5, 6, 7 ("split planes"): words 0..7 hold bits 0..3 of the 64 codes
 *     in the 4-bit arrangement; words 8 .. 2*bits-1 hold bits 4 .. bits-1 as a
 *     (bits-4)-bit code in the 1-, 2- or 3-bit arrangement, where 1 bit
 *     follows the rule for bits 2, 4, 8 (word w: codes 32w + i at 16*(i%2) + i/2).
 *   With this arrangement, masking a word (or the word shifted right by 8)
 *   leaves two consecutive codes in the mantissas of two fp16 halves, so a
 *   pair of codes becomes a pair of fp16 values with one AND-OR.
 * Scale and zero tables use the same tiling: entry (n, g) of the [n, G] table
 * (G = k/64 for group 64, G = 1 for group k) is at ((n/64)*G + g)*64 + n%64.
 * Scales are fp16 bit patterns (uint16), zeros uint8.
 * ---------------------------------------------------------------------------
 */
#ifndef QLIN_H
#define QLIN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qlin_status {
  QLIN_OK = 0,
  QLIN_ERR_NULL = 1,        /* a required pointer is NULL                        */
  QLIN_ERR_SHAPE = 2,       /* n, k or m out of range, k % 64 != 0, pitch < row  */
  QLIN_ERR_BITS = 3,        /* bits not allowed for the call (see qlin_weight)      */
  QLIN_ERR_GROUP = 4,       /* group neither 64 nor k                            */
  QLIN_ERR_ALIGN = 5,       /* a pointer not 16-byte aligned, or a pitch not a
                               multiple of 8 elements                            */
  QLIN_ERR_FORMAT = 6,      /* unknown weight format, or format not allowed here  */
  QLIN_ERR_ALIAS = 7,       /* an output overlaps an input                       */
  QLIN_ERR_WORKSPACE = 8,   /* workspace too small for the chosen launch          */
  QLIN_ERR_NO_DEVICE = 9,   /* no gfx950 device is current                       */
  QLIN_ERR_HIP = 10         /* a HIP call failed; see qlin_last_hip_error()       */
} qlin_status;

enum {
  QLIN_FMT_PACKED = 0,      /* data = tiled packed codes (uint32)                 */
  QLIN_FMT_FP16_MASTER = 1  /* data = fp16 master weights [n, ld], row-major      */
};

/* A quantized weight matrix as seen by the matmul entry points. */
typedef struct qlin_weight {
  int32_t n;                /* output rows                                        */
  int32_t k;                /* reduction length, multiple of 64                   */
  int32_t bits;             /* PACKED: 2 .. 8.  FP16_MASTER: 2 .. 8, or 16 =
                               unquantized (the whole lever)                       */
  int32_t group;            /* 64, or k for one group per row                     */
  int32_t format;           /* QLIN_FMT_*                                         */
  int32_t reserved;         /* must be 0                                          */
  const void* data;         /* codes (PACKED) or fp16 masters (FP16_MASTER)       */
  int64_t ld;               /* FP16_MASTER: row pitch in elements (>= k, % 8 == 0);
                               PACKED: must be 0                                  */
  const uint16_t* scale;    /* tiled fp16 scales; unused (may be NULL) if bits=16 */
  const uint8_t* zero;      /* tiled uint8 zeros; unused (may be NULL) if bits=16 */
} qlin_weight;

/* Human-readable name of a status code (static string, never NULL). */
const char* qlin_status_string(int status);

/* The HIP error code behind the calling thread's last QLIN_ERR_HIP (0 if none). */
int qlin_last_hip_error(void);

/* ABI version of this header; bumped on any incompatible change. */
int qlin_abi_version(void);

/* Bytes of the packed code buffer of an [n, k] matrix at `bits` (0 if invalid). */
int64_t qlin_packed_bytes(int32_t n, int32_t k, int32_t bits);

/* Entries of each (tiled) scale and zero table (0 if invalid). */
int64_t qlin_meta_entries(int32_t n, int32_t k, int32_t group);

/*
 * Round-to-nearest quantization of fp16 master weights (per-group scale/zero
 * precompute, then codes).  Bitcrush README, "Under the hood": a scale/zero
 * precompute pass, then the group-wise affine rounding.
 *   w16      fp16 masters [n, ld_w] row-major, ld_w >= k, ld_w % 8 == 0.
 *   bits     2 .. 8 (every width has a packed layout).
 *   codes    packed codes out, qlin_packed_bytes(n, k, bits) bytes; pass NULL to
 *            compute only scale and zero (a change of bit width then needs no
 *            new codes: the fused matmul re-rounds on the fly).
 *   scale    out, qlin_meta_entries(n, k, group) fp16 bit patterns (tiled).
 *   zero     out, same number of uint8 entries (tiled).
 * Padding rows of the last tile are written as 0.  Bit-exact and deterministic.
 */
qlin_status qlin_quantize(const uint16_t* w16, int64_t ld_w, int32_t n, int32_t k,
                          int32_t bits, int32_t group, uint32_t* codes,
                          uint16_t* scale, uint8_t* zero, hipStream_t stream);

/*
 * Batched quantization (the Bitcrush README, "The machine" and "Under the
 * hood": a move of the bit-width lever re-quantizes every weight matrix of the
 * model from its fp16 master, on the GPU, without re-uploading anything):
 * qlin_quantize on each job, all jobs with the same bits and group kind,
 * group = 64 (per 64-group) or 0 (one group per row, i.e. group = k of each
 * job).  Jobs are launched 64 at a time (one kernel launch per 64 jobs);
 * results are identical to one qlin_quantize per job.  codes may be NULL in
 * any job (scale/zero only).  No job's outputs may overlap another job's
 * inputs or outputs (QLIN_ERR_ALIAS).  count = 0 is a no-op.
 */
typedef struct {
  const uint16_t* w16;   /* fp16 master [n, ld_w] */
  int64_t ld_w;
  int32_t n, k;
  uint32_t* codes;       /* NULL: scale/zero only */
  uint16_t* scale;
  uint8_t* zero;
} qlin_quant_job;

qlin_status qlin_quantize_batch(const qlin_quant_job* jobs, int32_t count, int32_t bits,
                                int32_t group, hipStream_t stream);

/*
 * Workspace needed by qlin_gemv / qlin_gemm for their split-K launches, at the
 * launch shape the library picks for this weight and m.  0 means the launch
 * needs none.  Layout: the first 65536 bytes hold uint32 arrival counters (one
 * per output tile of the launch: 64 rows of W for GEMV and m <= 16, 256 rows
 * of W x up to 128 rows of X for larger m), the rest fp32 partial sums.  The
 * counter region must be zero before first use (zero-fill the workspace
 * once); every call leaves it zero again and the partials are scratch, so
 * calls of different shapes may share one workspace as long as they do not
 * run at the same time.
 */
int64_t qlin_gemv_workspace_bytes(const qlin_weight* w);
int64_t qlin_gemm_workspace_bytes(const qlin_weight* w, int32_t m);

/*
 * Decode GEMV, M = 1:  y[n] = sum_k x[k] * s(q - z)   (fp32 out).
 * Enargeia, "Run it": every weight is read once per output word, unpacked in
 * registers.  Bitcrush, "Under the hood": with FP16_MASTER the codes are
 * recomputed from the fp16 masters as they are read (bits 2..8), or the plain
 * fp16 weights are used (bits 16, the top of the lever).
 *   x   fp16 [k];  y  fp32 [n].
 *   workspace may be NULL when qlin_gemv_workspace_bytes(w) is 0; a smaller or
 *   missing workspace makes the call use fewer, longer work items instead.
 * Deterministic: the same inputs give bitwise the same y.
 */
qlin_status qlin_gemv(const qlin_weight* w, const uint16_t* x, float* y,
                      void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * GEMM:  Y[m, n] = sum_k X[m, k] * s(q - z),  PACKED weights only.
 * X fp16 [m, ld_x] (ld_x >= k, % 8 == 0), Y fp32 [m, ld_y] (ld_y >= n).
 * X is used as given (fp16) and each dequantized weight s*(q - z) is its
 * exact value rounded once to fp16 (nearest even); both feed the fp16
 * matrix cores with fp32 accumulation (Enargeia, "Measured, not asserted":
 * prefill is the dense, tiled-matmul form of the same product).  fp16 rather
 * than bf16 operands: bf16 rounding of X and of the weights alone exceeds
 * 1e-3 * max_row sum |x w| at short reductions (k = 192), at the same
 * matrix-core rate.
 * Range: the fp16 operand holds every dequantized weight of masters with
 * |w| <= 49120 (2 bits), 57312 (3), 61408 (4), 63456 (5), 64480 (6),
 * 64992 (7), 65248 (8).  Beyond that a weight s * (q - z) can reach 65520,
 * past fp16's largest value; every finite master is still accepted: a
 * work-group (or wave) whose columns have a scale >= 65520 / (2^bits - 1)
 * decodes its operands with the scale times 2^-8 and multiplies its sums by
 * 2^8, so that Y stays finite and within the same tolerance (small weights
 * beside such large ones may then lose low bits to fp16 underflow).
 * Deterministic.  Workspace as for qlin_gemv.
 */
qlin_status qlin_gemm(const qlin_weight* w, const uint16_t* X, int32_t m, int64_t ld_x,
                      float* Y, int64_t ld_y, void* workspace, int64_t workspace_bytes,
                      hipStream_t stream);

/*
 * qlin_gemv without any allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same GEMV, same launch shapes and results as
 * qlin_gemv with a workspace of qlin_gemv_workspace_bytes(w), but the split-K
 * workspace is a static device array inside the library, 1 MiB (1048576
 * bytes) per GPU, held from the library's load until the process ends.  A
 * weight whose launch would need more (qlin_gemv_workspace_bytes(w) >
 * 1048576: a 16-way K split of 256 tiles, for example) returns
 * QLIN_ERR_WORKSPACE.  The first call on a device looks the array up
 * (hipGetSymbolAddress); a call whose launch splits K first clears the
 * array's arrival counters with a small kernel (no memset node, no
 * allocation).  Every call on one GPU shares that GPU's array: calls that
 * can run at the same time on one GPU (on different streams) race and must
 * not be issued; calls on one stream are ordered and safe.  Errors as for
 * qlin_gemv.
 */
qlin_status qlin_gemv_noalloc(const qlin_weight* w, const uint16_t* x, float* y,
                              hipStream_t stream);

/*
 * Several GEMMs that share X, in one launch (the prefill form of the decode
 * step's grouping: q, k and v, or gate and up, of a layer read the same
 * normalized activations):  Y_i = X . W_i^T,  i = 0 .. count-1, count <= 4.
 * w: `count` PACKED weights with the same k, bits and group; Y[i] fp32
 * [m, ld_y[i]] (ld_y[i] >= w[i].n).  Each Y_i is what qlin_gemm gives for
 * w[i] to the same tolerance.  Workspace sized by
 * qlin_gemm_multi_workspace_bytes(w, count, m).  Errors as for qlin_gemm,
 * plus count outside 1..4 or different k -> QLIN_ERR_SHAPE, different bits or
 * group -> QLIN_ERR_FORMAT.
 */
int64_t qlin_gemm_multi_workspace_bytes(const qlin_weight* w, int32_t count, int32_t m);
qlin_status qlin_gemm_multi(const qlin_weight* w, int32_t count, const uint16_t* X, int32_t m,
                            int64_t ld_x, float* const* Y, const int64_t* ld_y, void* workspace,
                            int64_t workspace_bytes, hipStream_t stream);

/*
 * Gated MLP input of a prefill in one launch: the prefill (M-row) form of
 * qlin_gemv_swiglu (the Bitcrush README, "Under the hood": the SwiGLU kernel
 * after the gate and up projections; the Enargeia page, "Measured, not
 * asserted": prefill is the tiled-matmul form of the same products):
 *     H[m, n] = silu(G[m, n]) * U[m, n],   G = X . gate^T,  U = X . up^T,
 *     silu(g) = g / (1 + exp(-g)),
 * with G and U formed as qlin_gemm forms Y (same operand rounding, fp32
 * accumulation) and never written to memory.  gate and up are PACKED weights
 * with the same n, k, bits and group.  X fp16 [m, ld_x] (ld_x >= k, % 8 == 0).
 * Outputs, either may be NULL (not both), leading dimension ld_h >= n for
 * both: H fp32 [m, ld_h]; H16 fp16 bit patterns [m, ld_h], H rounded to
 * nearest even (ready as the down projection's X when ld_h % 8 == 0).
 * Writes a quarter of the bytes of the two fp32 outputs of qlin_gemm_multi.
 * Deterministic.  Workspace as for qlin_gemm, sized by
 * qlin_gemm_swiglu_workspace_bytes(gate, m).  Errors: different n or k ->
 * QLIN_ERR_SHAPE, different bits or group -> QLIN_ERR_FORMAT, otherwise as
 * for qlin_gemm.
 */
int64_t qlin_gemm_swiglu_workspace_bytes(const qlin_weight* gate, int32_t m);
qlin_status qlin_gemm_swiglu(const qlin_weight* gate, const qlin_weight* up, const uint16_t* X,
                             int32_t m, int64_t ld_x, float* H, uint16_t* H16, int64_t ld_h,
                             void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * Several decode GEMVs that share x, in one launch (the Enargeia page, "One
 * decode step": the per-token dispatch list, where q, k and v, and gate and
 * up, each read the same normalized activation):
 *     y_i[n] = sum_k x[k] * s_i(q_i - z_i),   i = 0 .. count-1,  count <= 4.
 * w points to `count` PACKED weights with the same k, bits and group (n may
 * differ); y to `count` fp32 output pointers (y_i has w[i].n entries).  Each
 * y_i equals what qlin_gemv gives for w[i] to the same tolerance.
 * Workspace as for qlin_gemv, sized by qlin_gemv_multi_workspace_bytes.
 * Errors: count outside 1..4 -> QLIN_ERR_SHAPE; different k -> SHAPE; different
 * bits or group, or an FP16_MASTER weight -> QLIN_ERR_FORMAT.
 */
int64_t qlin_gemv_multi_workspace_bytes(const qlin_weight* w, int32_t count);
qlin_status qlin_gemv_multi(const qlin_weight* w, int32_t count, const uint16_t* x,
                            float* const* y, void* workspace, int64_t workspace_bytes,
                            hipStream_t stream);

/*
 * Gated MLP input of a decode step in one launch (the Bitcrush README, "Under
 * the hood": the SwiGLU kernel that follows the gate and up projections):
 *     h[n] = silu(g[n]) * u[n],   g = gate . x,  u = up . x,
 *     silu(g) = g / (1 + exp(-g)),
 * with g and u accumulated as in qlin_gemv and never written to memory.
 * gate and up are PACKED weights with the same n, k, bits and group.  h (fp32,
 * [n]) and h16 (fp16 bit patterns, [n], h rounded to nearest even, ready as
 * the next GEMV's x) are outputs; either may be NULL, not both.
 * Workspace sized by qlin_gemv_swiglu_workspace_bytes(gate).
 */
int64_t qlin_gemv_swiglu_workspace_bytes(const qlin_weight* gate);
qlin_status qlin_gemv_swiglu(const qlin_weight* gate, const qlin_weight* up, const uint16_t* x,
                             float* h, uint16_t* h16, void* workspace, int64_t workspace_bytes,
                             hipStream_t stream);

/*
 * Embedding-row gather from a packed weight (the Enargeia page, "Run it": the
 * tied token-embedding table, stored at 8 bits, serves both the input lookup
 * and the LM-head GEMV):
 *     out[i, :] = s(q - z) of row ids[i],   i = 0 .. count-1,
 * out32 exact in fp32, out16 the same values rounded to fp16 (nearest even:
 * ready as the first layer's input).  Either output may be NULL, not both;
 * both are [count, ld_out] row-major, ld_out >= k and a multiple of 8.
 * ids: int32 device array, 4-byte aligned.  An id outside [0, n) yields a row
 * of zeros (ids are not read on the host).  count = 0 is a no-op.
 * PACKED weights only (QLIN_ERR_FORMAT otherwise).
 */
qlin_status qlin_embed_rows(const qlin_weight* w, const int32_t* ids, int32_t count,
                            uint16_t* out16, float* out32, int64_t ld_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_H */
