// Code packing and unpacking for the tiled layout (see include/qlin.h), and the
// fp16 "magic number" decode: a code c OR-ed into the low mantissa bits of
// fp16 1024.0 reads as exactly 1024 + c, so one AND-OR per word turns two
// codes into an fp16 pair, and subtracting 1024 + z leaves q - z exactly.
#pragma once

#include "device_common.h"

#include <type_traits>

namespace qlin {

// ---------------------------------------------------------------- packing --
// 64 codes (0..qmax, held as floats) -> 2*BITS words of one block.
template <int BITS>
__device__ __forceinline__ void pack_block(const float* code, uint32_t* out) {
  if constexpr (BITS >= 5 && BITS <= 7) {
    // split planes: low 4 bits as a 4-bit block, the rest as a (BITS-4)-bit one
    float lo[64], hi[64];
#pragma unroll
    for (int c = 0; c < 64; ++c) {
      const uint32_t v = (uint32_t)code[c];
      lo[c] = (float)(v & 15u);
      hi[c] = (float)(v >> 4);
    }
    pack_block<4>(lo, out);
    pack_block<BITS - 4>(hi, out + 8);
  } else if constexpr (BITS == 3) {
#pragma unroll
    for (int run = 0; run < 2; ++run) {
      uint32_t lo0 = 0, lo1 = 0, hi = 0;
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        const uint32_t v = (uint32_t)code[32 * run + c];
        const int u = c >> 4, i = c & 15, p = i >> 1, e = i & 1;
        const int lpos = 16 * e + 2 * p;
        if (u == 0) lo0 |= (v & 3u) << lpos; else lo1 |= (v & 3u) << lpos;
        int hb = (p < 4 ? 2 * p + 2 : 2 * (p - 4) + 3) + 16 * e;
        if (u == 1) hb = (hb + 8) & 31;
        hi |= ((v >> 2) & 1u) << hb;
      }
      out[3 * run + 0] = lo0;
      out[3 * run + 1] = lo1;
      out[3 * run + 2] = hi;
    }
  } else {
    constexpr int per = 32 / BITS;
#pragma unroll
    for (int w = 0; w < 2 * BITS; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < per; ++i) {
        const uint32_t v = (uint32_t)code[w * per + i];
        word |= v << (16 * (i & 1) + BITS * (i >> 1));
      }
      out[w] = word;
    }
  }
}

// Code c (0..63) of one row's 64-code block, read back from the packed words
// (the inverse of pack_block, element by element).
template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t* words, int c) {
  if constexpr (BITS >= 5 && BITS <= 7) {
    return code_at<4>(words, c) | (code_at<BITS - 4>(words + 8, c) << 4);
  } else if constexpr (BITS == 3) {
    const int run = c >> 5, cr = c & 31;
    const int u = cr >> 4, i = cr & 15, p = i >> 1, e = i & 1;
    const uint32_t lo = (words[3 * run + u] >> (16 * e + 2 * p)) & 3u;
    int hb = (p < 4 ? 2 * p + 2 : 2 * (p - 4) + 3) + 16 * e;
    if (u == 1) hb = (hb + 8) & 31;
    return lo | (((words[3 * run + 2] >> hb) & 1u) << 2);
  } else {
    constexpr int per = 32 / BITS;
    const int w = c / per, i = c % per;
    return (words[w] >> (16 * (i & 1) + BITS * (i >> 1))) & ((1u << BITS) - 1u);
  }
}

// --------------------------------------------------- GEMV decode (fp16 pairs)
// Per (lane, block): the block's sum_k x_k * (q_k - z), unscaled, in fp32.
// Codes come out of a word scaled by S in {1, 4, 16, 64} (their bit offset in
// the half-word); (1024 + S*q) - (1024 + S*z) = S*(q - z) exactly in fp16, the
// dot product with an fp16 x pair is exact per product, and each scale class
// keeps its own fp32 accumulator, divided by S (exact) at the end.
__device__ __forceinline__ uint32_t zconst(int z, int shift) {
  return (0x6400u + ((uint32_t)z << shift)) * 0x00010001u;
}

template <int BITS>
__device__ __forceinline__ float block_dot(const uint32_t* wd, const f16x2* xb, int z, uint32_t kMagic);

// 1-bit plane (the high bit of 5-bit codes): word w holds codes 32w + i, bit
// p of each half pairs codes (2p, 2p+1) with scale class S = 2^(p mod 8);
// z is 0 or 1.
__device__ __forceinline__ float block_dot1(const uint32_t* wd, const f16x2* xb, int z,
                                            uint32_t kMagic) {
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t v = wd[w], vs = v >> 8;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t m = (1u << p) | (1u << (16 + p));
      const f16x2 c = as_h2(zconst(z, p));
      a[p] = __builtin_amdgcn_fdot2(as_h2((v & m) | kMagic) - c, xb[16 * w + p], a[p], false);
      a[p] = __builtin_amdgcn_fdot2(as_h2((vs & m) | kMagic) - c, xb[16 * w + 8 + p], a[p], false);
    }
  }
  return ((a[0] + a[1] * 0.5f) + (a[2] * 0.25f + a[3] * 0.125f)) +
         ((a[4] * 0.0625f + a[5] * 0.03125f) + (a[6] * 0.015625f + a[7] * 0.0078125f));
}

template <int BITS>
__device__ __forceinline__ float block_dot(const uint32_t* wd, const f16x2* xb, int z, uint32_t kMagic) {
  if constexpr (BITS >= 5 && BITS <= 7) {
    // q - z = (lo - z % 16) + 16 * (hi - z / 16) over the two planes (each
    // plane's zero fits its own magic constant)
    float hi;
    if constexpr (BITS == 5) hi = block_dot1(wd + 8, xb, z >> 4, kMagic);
    else hi = block_dot<BITS - 4>(wd + 8, xb, z >> 4, kMagic);
    return block_dot<4>(wd, xb, z & 15, kMagic) + 16.f * hi;
  } else if constexpr (BITS == 4) {
    const f16x2 c1 = as_h2(zconst(z, 0)), c16 = as_h2(zconst(z, 4));
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t v = wd[w], vs = v >> 8;
      const f16x2 h0 = as_h2((v & 0x000F000Fu) | kMagic) - c1;
      const f16x2 h1 = as_h2((v & 0x00F000F0u) | kMagic) - c16;
      const f16x2 h2 = as_h2((vs & 0x000F000Fu) | kMagic) - c1;
      const f16x2 h3 = as_h2((vs & 0x00F000F0u) | kMagic) - c16;
      a0 = __builtin_amdgcn_fdot2(h0, xb[4 * w + 0], a0, false);
      b0 = __builtin_amdgcn_fdot2(h1, xb[4 * w + 1], b0, false);
      a1 = __builtin_amdgcn_fdot2(h2, xb[4 * w + 2], a1, false);
      b1 = __builtin_amdgcn_fdot2(h3, xb[4 * w + 3], b1, false);
    }
    return (a0 + a1) + (b0 + b1) * 0.0625f;
  } else if constexpr (BITS == 2) {
    f16x2 c[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) c[p] = as_h2(zconst(z, 2 * p));
    float a[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t v = wd[w], vs = v >> 8;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t m = (3u << (2 * p)) | (3u << (16 + 2 * p));
        const f16x2 h = as_h2((v & m) | kMagic) - c[p];
        const f16x2 g = as_h2((vs & m) | kMagic) - c[p];
        a[p] = __builtin_amdgcn_fdot2(h, xb[8 * w + p], a[p], false);
        b[p] = __builtin_amdgcn_fdot2(g, xb[8 * w + 4 + p], b[p], false);
      }
    }
    return (a[0] + b[0]) + (a[1] + b[1]) * 0.25f + (a[2] + b[2]) * 0.0625f +
           (a[3] + b[3]) * 0.015625f;
  } else if constexpr (BITS == 3) {
    f16x2 c[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) c[p] = as_h2(zconst(z, 2 * p));
    float a[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int run = 0; run < 2; ++run) {
      const uint32_t H = wd[3 * run + 2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t L = wd[3 * run + u];
        const uint32_t Hu = u ? __builtin_amdgcn_alignbit(H, H, 8) : H;
        const uint32_t Ls = L >> 8, Hs = Hu >> 1;
        const int xo = 16 * run + 8 * u;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t m2 = (3u << (2 * p)) | (3u << (16 + 2 * p));
          const uint32_t m1 = (1u << (2 * p + 2)) | (1u << (2 * p + 18));
          // bit-field insert of L into H under m2, then keep the code bits
          const uint32_t tl = (L & m2) | (Hu & ~m2), ts = (Ls & m2) | (Hs & ~m2);
          const f16x2 h = as_h2((tl & (m2 | m1)) | kMagic) - c[p];
          const f16x2 g = as_h2((ts & (m2 | m1)) | kMagic) - c[p];
          a[p] = __builtin_amdgcn_fdot2(h, xb[xo + p], a[p], false);
          b[p] = __builtin_amdgcn_fdot2(g, xb[xo + 4 + p], b[p], false);
        }
      }
    }
    return (a[0] + b[0]) + (a[1] + b[1]) * 0.25f + (a[2] + b[2]) * 0.0625f +
           (a[3] + b[3]) * 0.015625f;
  } else {  // BITS == 8
    const f16x2 c = as_h2(zconst(z, 0));
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int w = 0; w < 16; w += 2) {
      const uint32_t v = wd[w], u = wd[w + 1];
      // bytes [b0, 0x64, b2, 0x64] and [b1, 0x64, b3, 0x64]
      const f16x2 h0 = as_h2(__builtin_amdgcn_perm(0x64646464u, v, 0x04020400u)) - c;
      const f16x2 h1 = as_h2(__builtin_amdgcn_perm(0x64646464u, v, 0x04030401u)) - c;
      const f16x2 g0 = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04020400u)) - c;
      const f16x2 g1 = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030401u)) - c;
      a0 = __builtin_amdgcn_fdot2(h0, xb[2 * w + 0], a0, false);
      b0 = __builtin_amdgcn_fdot2(h1, xb[2 * w + 1], b0, false);
      a1 = __builtin_amdgcn_fdot2(g0, xb[2 * w + 2], a1, false);
      b1 = __builtin_amdgcn_fdot2(g1, xb[2 * w + 3], b1, false);
    }
    return (a0 + a1) + (b0 + b1);
  }
}

// ------------------------------------- GEMV decode with the zero point folded
// sum_k x_k (q_k - z) = sum_k x_k q_k - z * sum_k x_k: the block's x sum is
// formed once per block and wave (block_xsums), so the per-pair subtraction
// of z goes away.  A code field masked out of a word, with nothing OR-ed in,
// is an fp16 subnormal: field F at bit offset b of a half-word reads as
// F * 2^(b - 24) exactly (for b + width <= 10).  One AND per code pair, one
// v_dot2 with the fp16 x pair (exact products, fp32 sums), and the classes'
// sums are combined with the exact powers of two.  block_xq returns
// sum_k x_k q_k * 2^-24 for the 64 codes of one row's block.
template <int BITS>
__device__ __forceinline__ float block_xq(const uint32_t* wd, const f16x2* xb);

// 1-bit plane: word w holds codes 32w + i at bit 16*(i % 2) + i/2.
__device__ __forceinline__ float block_xq1(const uint32_t* wd, const f16x2* xb) {
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t v = wd[w], vs = v >> 8;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t m = (1u << p) | (1u << (16 + p));
      a[p] = __builtin_amdgcn_fdot2(as_h2(v & m), xb[16 * w + p], a[p], false);
      a[p] = __builtin_amdgcn_fdot2(as_h2(vs & m), xb[16 * w + 8 + p], a[p], false);
    }
  }
  return ((a[0] + a[1] * 0.5f) + (a[2] * 0.25f + a[3] * 0.125f)) +
         ((a[4] * 0.0625f + a[5] * 0.03125f) + (a[6] * 0.015625f + a[7] * 0.0078125f));
}

template <int BITS>
__device__ __forceinline__ float block_xq(const uint32_t* wd, const f16x2* xb) {
  if constexpr (BITS >= 5 && BITS <= 7) {
    // q = lo + 16 hi over the two planes
    float hi;
    if constexpr (BITS == 5) hi = block_xq1(wd + 8, xb);
    else hi = block_xq<BITS - 4>(wd + 8, xb);
    return __builtin_fmaf(16.f, hi, block_xq<4>(wd, xb));
  } else if constexpr (BITS == 4) {
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t v = wd[w], vs = v >> 8;
      a0 = __builtin_amdgcn_fdot2(as_h2(v & 0x000F000Fu), xb[4 * w + 0], a0, false);
      b0 = __builtin_amdgcn_fdot2(as_h2(v & 0x00F000F0u), xb[4 * w + 1], b0, false);
      a1 = __builtin_amdgcn_fdot2(as_h2(vs & 0x000F000Fu), xb[4 * w + 2], a1, false);
      b1 = __builtin_amdgcn_fdot2(as_h2(vs & 0x00F000F0u), xb[4 * w + 3], b1, false);
    }
    return (a0 + a1) + (b0 + b1) * 0.0625f;
  } else if constexpr (BITS == 2) {
    float a[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t v = wd[w], vs = v >> 8;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t m = (3u << (2 * p)) | (3u << (16 + 2 * p));
        a[p] = __builtin_amdgcn_fdot2(as_h2(v & m), xb[8 * w + p], a[p], false);
        b[p] = __builtin_amdgcn_fdot2(as_h2(vs & m), xb[8 * w + 4 + p], b[p], false);
      }
    }
    return (a[0] + b[0]) + (a[1] + b[1]) * 0.25f + (a[2] + b[2]) * 0.0625f +
           (a[3] + b[3]) * 0.015625f;
  } else if constexpr (BITS == 3) {
    float a[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int run = 0; run < 2; ++run) {
      const uint32_t H = wd[3 * run + 2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t L = wd[3 * run + u];
        const uint32_t Hu = u ? __builtin_amdgcn_alignbit(H, H, 8) : H;
        const uint32_t Ls = L >> 8, Hs = Hu >> 1;
        const int xo = 16 * run + 8 * u;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t m2 = (3u << (2 * p)) | (3u << (16 + 2 * p));
          const uint32_t m1 = (1u << (2 * p + 2)) | (1u << (2 * p + 18));
          // the pair's low bits from L, its third bits from H: a 3-bit field
          // at offset 2p of each half
          const uint32_t tl = (L & m2) | (Hu & m1), ts = (Ls & m2) | (Hs & m1);
          a[p] = __builtin_amdgcn_fdot2(as_h2(tl), xb[xo + p], a[p], false);
          b[p] = __builtin_amdgcn_fdot2(as_h2(ts), xb[xo + 4 + p], b[p], false);
        }
      }
    }
    return (a[0] + b[0]) + (a[1] + b[1]) * 0.25f + (a[2] + b[2]) * 0.0625f +
           (a[3] + b[3]) * 0.015625f;
  } else {  // BITS == 8: each byte into the low byte of a half, high byte 0
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int w = 0; w < 16; w += 2) {
      const uint32_t v = wd[w], u = wd[w + 1];
      const f16x2 h0 = as_h2(__builtin_amdgcn_perm(0u, v, 0x0c020c00u));
      const f16x2 h1 = as_h2(__builtin_amdgcn_perm(0u, v, 0x0c030c01u));
      const f16x2 g0 = as_h2(__builtin_amdgcn_perm(0u, u, 0x0c020c00u));
      const f16x2 g1 = as_h2(__builtin_amdgcn_perm(0u, u, 0x0c030c01u));
      a0 = __builtin_amdgcn_fdot2(h0, xb[2 * w + 0], a0, false);
      b0 = __builtin_amdgcn_fdot2(h1, xb[2 * w + 1], b0, false);
      a1 = __builtin_amdgcn_fdot2(g0, xb[2 * w + 2], a1, false);
      b1 = __builtin_amdgcn_fdot2(g1, xb[2 * w + 3], b1, false);
    }
    return (a0 + a1) + (b0 + b1);
  }
}

// -------------------------------------------- MFMA operand decode (fp16 x 8)
// Eight consecutive codes of a block ("chunk") -> fp16 s * (q - z), rounded
// once to nearest even, in packed fp16 arithmetic.  The magic-number trick
// turns a pair of codes into fp16 1024 + S*q, S the code's place within its
// half-word (1, 4, 16, 64; 1, 2, 4, 8 for a 1-bit plane).  One packed fma by
// the exact power of two 1/S and by -(1024/S + z) gives q - z, an integer of
// at most 9 bits that fp16 holds exactly, so that fma rounds nothing; one
// packed multiply by s then rounds the exact product s * (q - z) once.  The
// result is the exact value rounded to fp16, as if formed in fp32 (where it
// is exact) and converted.
struct Deq {
  f16x2 s;        // (s, s)
  f16x2 inv[4];   // (1/S, 1/S)
  f16x2 c[4];     // (-(1024/S + z), same)
};

// S = 1, 4, 16, 64 (SH = 2) or S = 1, 2, 4, 8 (SH = 1, a 1-bit plane); z is
// a zero point, 0 .. 255.  -(1024 + z) is built as fp16 bits (exponent 10,
// mantissa z, sign set), and -(1024/S + z) = -(1024 + z) + (1024 - 1024/S)
// by one fp16 add, exact: both terms and the sum are integers below 2048.
template <int SH = 2>
__device__ __forceinline__ Deq make_deq(float s, int z) {
  Deq d;
  const f16 sh = (f16)s;                              // s is an fp16 value (or 0)
  d.s = (f16x2){sh, sh};
  const f16 c0 = __builtin_bit_cast(f16, (uint16_t)(0xE400u | (uint32_t)z));
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const f16 inv = (f16)(1.0f / (float)(1 << (SH * p)));
    const f16 c = p == 0 ? c0 : (f16)(c0 + (f16)(float)(1024 - (1024 >> (SH * p))));
    d.inv[p] = (f16x2){inv, inv};
    d.c[p] = (f16x2){c, c};
  }
  return d;
}

// q - z of a pair of codes, exact
__device__ __forceinline__ f16x2 qz_pair(uint32_t magic_pair, const Deq& d, int p) {
  return __builtin_elementwise_fma(as_h2(magic_pair), d.inv[p], d.c[p]);
}

__device__ __forceinline__ f16x8 scaled8(const f16x2* qz, f16x2 s) {
  f16x8 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const f16x2 w = qz[p] * s;
    r[2 * p] = w.x;
    r[2 * p + 1] = w.y;
  }
  return r;
}

// q - z of 8 codes, pairs in K order.
// int4: one word = 8 codes.  S=1 for (v & 0x000F000F), S=16 for (v & 0x00F000F0).
__device__ __forceinline__ void qz_chunk4(uint32_t v, const Deq& d, uint32_t kMagic, f16x2* o) {
  const uint32_t vs = v >> 8;
  o[0] = qz_pair((v & 0x000F000Fu) | kMagic, d, 0);
  o[1] = qz_pair((v & 0x00F000F0u) | kMagic, d, 2);
  o[2] = qz_pair((vs & 0x000F000Fu) | kMagic, d, 0);
  o[3] = qz_pair((vs & 0x00F000F0u) | kMagic, d, 2);
}

// int2: pairs 0..3 of v (the caller passes v >> 8 for the upper pairs).
__device__ __forceinline__ void qz_chunk2(uint32_t v, const Deq& d, uint32_t kMagic, f16x2* o) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t m = (3u << (2 * p)) | (3u << (16 + 2 * p));
    o[p] = qz_pair((v & m) | kMagic, d, p);
  }
}

// int3: low-bit word L (already shifted for the upper pairs) and high-bit word
// H (already rotated / shifted to line up with L).
__device__ __forceinline__ void qz_chunk3(uint32_t L, uint32_t H, const Deq& d, uint32_t kMagic,
                                          f16x2* o) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t m2 = (3u << (2 * p)) | (3u << (16 + 2 * p));
    const uint32_t m1 = (1u << (2 * p + 2)) | (1u << (2 * p + 18));
    const uint32_t t = (L & m2) | (H & ~m2);
    o[p] = qz_pair((t & (m2 | m1)) | kMagic, d, p);
  }
}

// 1-bit plane: bits 0..3 of each half of v (the caller shifts v to the chunk),
// S = 1, 2, 4, 8 (d from make_deq<1>).
__device__ __forceinline__ void qz_chunk1(uint32_t v, const Deq& d, uint32_t kMagic, f16x2* o) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t m = (1u << p) | (1u << (16 + p));
    o[p] = qz_pair((v & m) | kMagic, d, p);
  }
}

// int8: two words = 8 codes; the byte permute builds 1024 + q directly (S = 1).
__device__ __forceinline__ void qz_chunk8(uint32_t v, uint32_t u, const Deq& d, f16x2* o) {
  o[0] = qz_pair(__builtin_amdgcn_perm(0x64646464u, v, 0x04020400u), d, 0);
  o[1] = qz_pair(__builtin_amdgcn_perm(0x64646464u, v, 0x04030401u), d, 0);
  o[2] = qz_pair(__builtin_amdgcn_perm(0x64646464u, u, 0x04020400u), d, 0);
  o[3] = qz_pair(__builtin_amdgcn_perm(0x64646464u, u, 0x04030401u), d, 0);
}

__device__ __forceinline__ f16x8 deq_chunk4(uint32_t v, const Deq& d, uint32_t kMagic) {
  f16x2 o[4];
  qz_chunk4(v, d, kMagic, o);
  return scaled8(o, d.s);
}

__device__ __forceinline__ f16x8 deq_chunk2(uint32_t v, const Deq& d, uint32_t kMagic) {
  f16x2 o[4];
  qz_chunk2(v, d, kMagic, o);
  return scaled8(o, d.s);
}

__device__ __forceinline__ f16x8 deq_chunk3(uint32_t L, uint32_t H, const Deq& d, uint32_t kMagic) {
  f16x2 o[4];
  qz_chunk3(L, H, d, kMagic, o);
  return scaled8(o, d.s);
}

__device__ __forceinline__ f16x8 deq_chunk8(uint32_t v, uint32_t u, const Deq& d) {
  f16x2 o[4];
  qz_chunk8(v, u, d, o);
  return scaled8(o, d.s);
}

// 5-7 bits (split planes): q - z = (lo - z%16) + 16 (hi - z/16), both terms
// and the sum (|q - z| <= 127) exact in fp16; then one multiply by s.
struct Deq2 {
  Deq lo, hi;    // hi.s unused
};

template <int BITS>
using DeqT = typename std::conditional<(BITS >= 5 && BITS <= 7), Deq2, Deq>::type;

template <int BITS>
__device__ __forceinline__ DeqT<BITS> make_deq_b(float s, int z) {
  if constexpr (BITS >= 5 && BITS <= 7) {
    Deq2 d;
    d.lo = make_deq(s, z & 15);
    d.hi = BITS == 5 ? make_deq<1>(s, z >> 4) : make_deq(s, z >> 4);
    return d;
  } else {
    return make_deq(s, z);
  }
}

// The fp16 range of the matrix-core weight operand.  s * (q - z) rounded to
// fp16 is infinite once |s (q - z)| >= 65520, which finite fp16 masters of
// magnitude above 49120 (2 bits) ... 65248 (8 bits) can reach; that needs
// s >= 65520 / qmax.  A column with such a scale over the work-group's K
// range is decoded with s * 2^-8 throughout and its sums are scaled by 2^8
// at the end.  The tiled kernels find those columns before their first
// decode, by a scan of the scales over the K range (wide_rows8,
// wave_row_flag); the K-split kernel keeps each column's largest scale as
// its K loop loads them and computes a flagged column's sums again after
// the loop.  Both scalings are powers of two: the blocks that needed it keep
// exactly their rounding (s * 2^-8 >= 1, every nonzero operand normal);
// small weights elsewhere in that column may lose low bits to fp16
// underflow, far below the column's large products.  Columns of ordinary
// weights are untouched.
template <int BITS>
__device__ __forceinline__ bool maybe_wide(float s) {
  return s >= 65520.f / (float)((1 << BITS) - 1);
}

// The scan is one memory round trip: a tile's scales of ng consecutive
// groups are ng * 128 contiguous bytes (s_tile[i]: the first group's entry
// of row 0 of tile i).  Participant p of np (np a multiple of 8) loads the
// 16-byte chunks p, p + np, ... of each of the NT tiles -- rows 8 (p % 8) ..
// + 7 of one group each -- NB per tile at a time, all in flight together
// (NB * NT * 4 registers), and keeps their largest magnitudes; bit e of
// f[i]: row 8 (p % 8) + e of tile i has such a scale in one of those chunks.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
template <int BITS, int NT, int NB = 8>
__device__ __forceinline__ void wide_rows8(const uint16_t* const (&s_tile)[NT], int ng, int p,
                                           int np, uint32_t (&f)[NT]) {
  const int nch = ng * 8;
  u16x2 mx[NT][4];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) mx[i][q] = (u16x2){0, 0};
  for (int c0 = p; c0 < nch; c0 += NB * np) {
    uint4 v[NT][NB];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int ch = c0 + k * np;
        v[i][k] = ch < nch ? reinterpret_cast<const uint4*>(s_tile[i])[ch] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const uint32_t w[4] = {v[i][k].x, v[i][k].y, v[i][k].z, v[i][k].w};
#pragma unroll
        for (int q = 0; q < 4; ++q)   // magnitudes: the sign bit cleared
          mx[i][q] = __builtin_elementwise_max(mx[i][q],
                                               __builtin_bit_cast(u16x2, w[q] & 0x7FFF7FFFu));
      }
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    f[i] = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (maybe_wide<BITS>(h2f(mx[i][q][0]))) f[i] |= 1u << (2 * q);
      if (maybe_wide<BITS>(h2f(mx[i][q][1]))) f[i] |= 2u << (2 * q);
    }
  }
}

// Whether row r of the tile is flagged, given every lane's wide_rows8
// result (lane l: rows 8 (l % 8) + e); called by the whole wave.  Almost
// always no lane has a flag: one ballot.  Otherwise the lanes of equal
// l % 8 are OR-ed together and each lane reads its row's lane.
__device__ __forceinline__ bool wave_row_flag(uint32_t f8, int r) {
  if (__builtin_amdgcn_ballot_w64(f8 != 0) == 0) return false;
  f8 |= __shfl_xor(f8, 8);
  f8 |= __shfl_xor(f8, 16);
  f8 |= __shfl_xor(f8, 32);
  return (__shfl(f8, r >> 3) >> (r & 7)) & 1u;
}

constexpr float kWideScale = 0.00390625f;   // 2^-8
// the inverse of an operand scale (1 or 2^-8), exact
__device__ __forceinline__ float unscale(float f) { return f < 1.f ? 256.f : 1.f; }

// fp16 x 8 held in one uint4, as an MFMA operand.
__device__ __forceinline__ f16x8 u4_to_f16x8(uint4 v) { return __builtin_bit_cast(f16x8, v); }

}  // namespace qlin
