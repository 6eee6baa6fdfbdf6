// Device-side helpers for the gfx950 DBSA kernels: bf16 packing, RoPE angles,
// LDS tile layouts and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dbsa_internal.hpp"

namespace dbsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 bytes as a native vector (HIP's uint4 wrapper class blocks register promotion).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Masked scores are -inf; running maxima start at a finite floor so that a
// row whose first tiles are fully masked never forms (-inf) - (-inf).
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMaxFloor = -1.0e30f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even) packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// cos / sin of the RoPE angle p * w_i.  The angle is formed in revolutions and
// reduced to [0, 1) in double precision, then the hardware sine / cosine
// (input in revolutions, about 1.2e-7 absolute error) finish in single
// precision.  The reduction keeps the large-position error at the level of
// the final float rounding instead of p * eps.
__device__ __forceinline__ void rope_cs(int64_t pos, double rev, float& c, float& s) {
  double r = (double)pos * rev;
  r -= floor(r);
  float x = (float)r;
  s = __builtin_amdgcn_sinf(x);
  c = __builtin_amdgcn_cosf(x);
}

// One rotate-half pair (a, b) turned by the angle with cosine c and sine s.
// Written with explicit fused multiply-adds so that every kernel rounds the
// rotation identically (no context-dependent contraction).
__device__ __forceinline__ float rot_lo(float a, float b, float c, float s) {
  return __builtin_fmaf(a, c, -(b * s));
}
__device__ __forceinline__ float rot_hi(float a, float b, float c, float s) {
  return __builtin_fmaf(b, c, a * s);
}

// cos / sin of the 8 frequencies i0 .. i0+7 at one position.
__device__ __forceinline__ void rope_cs8(int64_t pos, const RopeFreq& f, int i0, float (&c)[8],
                                         float (&s)[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) rope_cs(pos, f.rev[i0 + r], c[r], s[r]);
}

// Rotate 8 rotate-half pairs held as two 16-byte bf16 chunks (first-half
// element r pairs with second-half element r) by precomputed angles, multiply
// by `scale` and round once to bf16.
__device__ __forceinline__ void rotate_chunk(u32x4& x1, u32x4& x2, const float (&c)[8],
                                             const float (&s)[8], float scale = 1.0f) {
  uint32_t a[4] = {x1.x, x1.y, x1.z, x1.w};
  uint32_t b[4] = {x2.x, x2.y, x2.z, x2.w};
  uint32_t oa[4], ob[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float c0 = c[2 * w], s0 = s[2 * w], c1 = c[2 * w + 1], s1 = s[2 * w + 1];
    const float a0 = bf16_lo(a[w]), a1 = bf16_hi(a[w]);
    const float b0 = bf16_lo(b[w]), b1 = bf16_hi(b[w]);
    oa[w] = pack_bf16x2(rot_lo(a0, b0, c0, s0) * scale, rot_lo(a1, b1, c1, s1) * scale);
    ob[w] = pack_bf16x2(rot_hi(a0, b0, c0, s0) * scale, rot_hi(a1, b1, c1, s1) * scale);
  }
  x1 = u32x4{oa[0], oa[1], oa[2], oa[3]};
  x2 = u32x4{ob[0], ob[1], ob[2], ob[3]};
}

// Rotation of one chunk pair at `pos` for frequencies i0 .. i0+7.
__device__ __forceinline__ void rope_rotate_chunk(u32x4& x1, u32x4& x2, int64_t pos,
                                                  const RopeFreq& f, int i0,
                                                  float scale = 1.0f) {
  float c[8], s[8];
  rope_cs8(pos, f, i0, c, s);
  rotate_chunk(x1, x2, c, s, scale);
}

// Eight probabilities of one MFMA result (registers B .. B+7) as a bf16 B operand.
template <int B>
__device__ __forceinline__ bf16x8 pack_p(const f32x16 s) {
  const u32x4 w = u32x4{pack_bf16x2(s[B + 0], s[B + 1]), pack_bf16x2(s[B + 2], s[B + 3]),
                             pack_bf16x2(s[B + 4], s[B + 5]), pack_bf16x2(s[B + 6], s[B + 7])};
  return __builtin_bit_cast(bf16x8, w);
}

// ---------------------------------------------------------------------------
// LDS tile layouts (bytes of one 64-key tile of one KV head).
//
// K tile: 64 rows (keys) x D bf16.  Row = D/8 chunks of 16 bytes; chunk c of
// row k sits at physical chunk c ^ swz(k) so that 16 lanes reading the same
// logical chunk of 16 consecutive rows hit 16 distinct bank groups.
//
// V^T tile: D rows (head dims) x 64 keys, 8 chunks of 16 bytes per row.  The
// keys inside each 16-key group are stored in the order in which the MFMA
// result layout hands out P (see vt_key_of_pos) so that one 16-byte read gives
// a lane the 8 keys it contracts over.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int k_chunk_phys(int row, int chunk) {
  if constexpr (D == 128) return chunk ^ (row & 15);
  else return chunk ^ ((row >> 1) & 7);
}
__device__ __forceinline__ int vt_chunk_phys(int drow, int chunk) {
  return chunk ^ ((drow >> 1) & 7);
}
// Key (0..15, within its 16-key group) stored at position p (0..15), and back.
__device__ __forceinline__ int vt_key_of_pos(int p) {
  return 8 * ((p & 7) >> 2) + 4 * (p >> 3) + (p & 3);
}
__device__ __forceinline__ int vt_pos_of_key(int k) {
  return 8 * ((k >> 2) & 1) + 4 * (k >> 3) + (k & 3);
}

// Workgroup order: the hardware hands consecutive workgroup ids to the 8 XCDs
// in turn.  Remap so that each XCD walks a contiguous range of logical work
// items (neighbouring query tiles of one KV head share K/V in that XCD's L2).
__device__ __forceinline__ int xcd_logical(int lin, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = lin & 7, i = lin >> 3;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Largest b in [0, n) with tab[b] <= t (tab ascending, tab[0] <= t).
__device__ __forceinline__ int upper_index(const int32_t* tab, int n, int t) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tab[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace dbsa
