// Device-side helpers for the gfx950 DBSA kernels: bf16 packing, RoPE angles,
// LDS tile layouts and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "dbsa_internal.hpp"

namespace dbsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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

// cos / sin of the sum of two angles from theirs (angle addition, explicit
// fused multiply-adds so every kernel rounds it identically).  bf16 K rows are
// rotated at position p = 64 t + r (t = p / 64, r = p % 64) as the sum of the
// angles at 64 t and at r: one angle per frequency is shared by a whole 64-row
// tile and one per row offset is fixed per thread, which replaces most of the
// per-element sine / cosine work (about 3e-7 absolute error in c and s).
__device__ __forceinline__ void angle_add(float ca, float sa, float cb, float sb, float& c,
                                          float& s) {
  c = __builtin_fmaf(ca, cb, -(sa * sb));
  s = __builtin_fmaf(sa, cb, ca * sb);
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


// RoPE angles of a workgroup's query rows through an LDS table: the rows of a
// 256-row workgroup hold only a few distinct positions (the G heads of a token
// share one), so each (position, frequency) cos / sin is computed once, by one
// thread, instead of once per row.  Table row j (position pos_of(j)) holds
// the D / 2 (cos, sin) pairs, padded by 16 bytes against bank conflicts.
template <int D>
struct AngleTable {
  static constexpr int H = D / 2;
  static constexpr int ROWB = H * 8 + 16;  // bytes per position
  // Fill rows 0 .. n_pos - 1 (all threads of the workgroup call this, in
  // whole wavefronts; the caller then synchronises the workgroup).  Entry e
  // is position e % n_pos, frequencies 8 (e / n_pos) .. + 7: with n_pos a
  // multiple of 64 the frequencies are the same across a wavefront, and are
  // read as scalars.
  template <typename PosOf, typename Freq>
  static __device__ __forceinline__ void fill(char* tab, int n_pos, int tid, int n_threads,
                                              PosOf&& pos_of, Freq&& freq) {
    for (int e = tid; e < n_pos * (H / 8); e += n_threads) {
      const int j = e % n_pos;
      int f0 = (e / n_pos) * 8;
      if (n_pos % 64 == 0) f0 = __builtin_amdgcn_readfirstlane(f0);
      const int64_t p = pos_of(j);
      f32x4* dst = reinterpret_cast<f32x4*>(tab + j * ROWB + f0 * 8);
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        float c0, s0, c1, s1;
        rope_cs(p, freq(f0 + i), c0, s0);
        rope_cs(p, freq(f0 + i + 1), c1, s1);
        dst[i / 2] = f32x4{c0, s0, c1, s1};
      }
    }
  }
  // cos / sin of frequencies f0 .. f0 + 7 at table row j.
  static __device__ __forceinline__ void read8(const char* tab, int j, int f0, float (&c)[8],
                                               float (&s)[8]) {
    const f32x4* src = reinterpret_cast<const f32x4*>(tab + j * ROWB + f0 * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 w = src[i];
      c[2 * i] = w[0];
      s[2 * i] = w[1];
      c[2 * i + 1] = w[2];
      s[2 * i + 1] = w[3];
    }
  }
};

// ---------------------------------------------------------------------------
// Tile layouts (one 64-key tile of one KV head), both [64 keys][D] bf16:
//   K tile  rotated keys; read as the A operand of S^T = K Q^T (16 bytes/lane).
//   V tile  values in their natural layout; read with ds_read_b64_tr_b16 so
//           each lane receives 4 keys of one head dim (the A operand of
//           O^T = V^T P^T) without any transpose pass.
// Rows are split in 16-byte chunks and chunk c of row r is stored at chunk
// c ^ swz(r), chosen so the lanes of one read hit distinct bank groups.  K
// tiles of the prefill are written by the pack step as exactly this LDS image;
// V tiles (and Stage-2 K tiles) are staged straight from the token-major
// tensors with per-lane source addresses that realise the same placement.
// ---------------------------------------------------------------------------
template <int D>
struct TileGeom {
  static constexpr int ROW = D * 2;                 // row bytes (K and V)
  static constexpr int KBYTES = kKeyTile * ROW;
  static constexpr int VBYTES = kKeyTile * ROW;
  static constexpr int STAGE = KBYTES + VBYTES;     // one LDS stage (K + V)
  static constexpr int TU4 = kKeyTile * D / 8;      // 16-byte chunks per tile matrix
  static constexpr int KCR = D / 8;                 // chunks per row
  static constexpr int KROW = ROW;
  // K rows: 16 lanes read one logical chunk of 16 consecutive rows.
  static __device__ __forceinline__ int k_phys(int row, int c) {
    if constexpr (D == 128) return c ^ (row & 15);
    else return c ^ ((row >> 1) & 7);
  }
  // V rows: a 16-lane transposed read covers 4 consecutive rows x 32 bytes;
  // the 4 rows land in 4 different 64-byte groups.
  static __device__ __forceinline__ int v_phys(int row, int c) {
    if constexpr (D == 128) return c ^ (4 * (row & 3));
    else return c ^ (4 * (row & 1));
  }
};

// This lane's value and its partner's 32 lanes away, ordered (lower lane's,
// upper lane's) in both lanes, by one v_permlane32_swap: a vector
// instruction, where a shuffle would be an LDS permute queued behind the tile
// reads of the other wavefront on the SIMD.
__device__ __forceinline__ f32x2 pair_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float max_xor32(float x) {
  const f32x2 h = pair_xor32(x);
  return __builtin_fmaxf(h[0], h[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const f32x2 h = pair_xor32(x);
  return h[0] + h[1];
}

// ---------------------------------------------------------------------------
// Flash-attention state of one lane pair (one query row) and the per-tile step.
//
// Lane l of a wavefront owns query row l % 32; half h = l / 32 holds keys
// (i/4)*8 + 4h + i%4 (+32 for the second MFMA) of each 64-key tile, i.e. the
// S^T = K Q^T result layout of v_mfma_f32_32x32x16_bf16.  O^T += V^T P^T
// keeps the output in the same row-per-lane layout: o[m][i] is head dim
// m*32 + (i/4)*8 + 4h + i%4.
//
// Scores carry scale * log2(e) (folded into Q) and are produced relative to
// the running reference m (the MFMA accumulator starts at -m).  The reference
// is raised only when a score exceeds it by more than kLazy (2^8 headroom for
// P), so the O rescale runs once or twice per row instead of every tile.
// ---------------------------------------------------------------------------
constexpr float kLazy = 8.0f;

// Placed first in the body of a rarely taken, wave-uniform branch: a volatile
// asm cannot be speculated, so the compiler keeps a real branch instead of
// if-converting the body into selects that every tile would then execute (the
// element mask of partly visible tiles and the softmax reference raise).
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>): a loop
// whose index is a compile-time constant in the body (register-array index).
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedDsRead = 0x100, kSchedTrans = 0x400;

// A 16-float MFMA accumulator with every element x, built from 64-bit pairs
// (the compiler is free to lower it to moves or copies; in the prefill loop
// this form measured about 1% faster than per-element initialisation).
__device__ __forceinline__ f32x16 splat16(float x) {
  typedef double f64x8 __attribute__((ext_vector_type(8)));
  const double d = __builtin_bit_cast(double, f32x2{x, x});
  const f64x8 v = {d, d, d, d, d, d, d, d};
  return __builtin_bit_cast(f32x16, v);
}

// The vector work of one tile (mask, maximum, exponentials, packing, row sum)
// is a chain of dependent instructions whose latency a single wavefront cannot
// hide; the tile loop therefore interleaves it, instruction group by group,
// with matrix work that does not depend on it:
//   pv_head  O += V^T P^T of the previous tile, with the mask and row maximum
//            of the current tile (and the rare reference raise after it);
//   exp_next P = 2^S of the current tile, its bf16 packing and row sum, with
//            the next tile's S^T = K Q^T (accumulators started at -m, the
//            reference just settled).
template <int D>
struct Flash {
  static constexpr int KS = D / 16;  // k-steps over the head dim
  static constexpr int OT = D / 32;  // O^T row tiles
  static constexpr int NPV = 4 * OT;  // P V products per tile (4 k-steps of 16 keys x OT)
  using Gm = TileGeom<D>;
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  f32x16 o[OT];
  float m, l;
  bool have;

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int t = 0; t < OT; ++t) o[t] = f32x16{};
    m = 0.0f;
    l = 0.0f;
    have = false;
  }

  // A operand of P V product j (k-step kk = j / OT, O^T rows 32t, t = j % OT):
  // two transposed reads of the natural V tile, keys 16kk + 4h + 0..3 and
  // 16kk + 8 + 4h + 0..3 at head dim 32t + col -- the key order in which the
  // S^T result layout hands out P (see exp_next).
  __device__ __forceinline__ bf16x8 vfrag(const char* st_v, const int (&vbase)[OT], int j) const {
    const char* a0 = st_v + vbase[j % OT] + (16 * (j / OT)) * Gm::ROW;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(a0 + 8 * Gm::ROW));
    const s16x8 v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v8);
  }
  // K fragment of k-step ks, rows h*32 .. +31 of the tile.
  __device__ __forceinline__ bf16x8 kfrag(const char* st_k, const int (&koff)[KS], int ks, int h) const {
    return *reinterpret_cast<const bf16x8*>(st_k + koff[ks] + h * 32 * Gm::KROW);
  }

  // S^T of one tile relative to the current reference m (no interleaving).
  __device__ __forceinline__ void scores(const char* st_k, const int (&koff)[KS],
                                         const bf16x8 (&qb)[KS], f32x16& s0, f32x16& s1) const {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = -m;
      s1[i] = -m;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(st_k, koff, ks, 0), qb[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(st_k, koff, ks, 1), qb[ks], s1, 0, 0, 0);
    }
  }

  // O^T += V^T P^T of one tile (no interleaving).
  __device__ __forceinline__ void pv(const char* st_v, const int (&vbase)[OT], const bf16x8 (&p)[4]) {
#pragma unroll
    for (int j = 0; j < NPV; ++j)
      o[j % OT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag(st_v, vbase, j), p[j / OT],
                                                          o[j % OT], 0, 0, 0);
  }

  struct NoHook {
    __device__ __forceinline__ void operator()(int) const {}
  };
  // Mask (when `mask`: key kr of the tile is kept iff vis(kr)), row maximum
  // and the rare reference raise (rescaling o and l); leaves s = S - m.  When
  // PV, the previous tile's O^T += V^T P^T (V from st_v, probabilities p) is
  // issued in NPV groups, fenced against the scheduler: group j holds P V
  // product j (its fragments were read two groups earlier), one step of the
  // maximum tree and hook(j) (the caller's tile requests, if any).
  template <bool PV, typename Vis, typename Hook = NoHook>
  __device__ __forceinline__ void pv_head(const char* st_v, const int (&vbase)[OT],
                                          const bf16x8 (&p)[4], f32x16& s0, f32x16& s1, bool mask,
                                          Vis vis, Hook hook = Hook{}) {
    if (mask) {
      keep_branch();
      const int hh = (threadIdx.x >> 5) & 1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kr = (i >> 2) * 8 + hh * 4 + (i & 3);
        s0[i] = vis(kr) ? s0[i] : kNegInf;
        s1[i] = vis(kr + 32) ? s1[i] : kNegInf;
      }
    }
    float mq[8];
    // Maximum-tree step j: pairs of four scores for j < 8, then the tree.
    auto max_step = [&](int j) {
      if (j < 8) {
        mq[j] = __builtin_fmaxf(__builtin_fmaxf(s0[2 * j], s0[2 * j + 1]),
                                __builtin_fmaxf(s1[2 * j], s1[2 * j + 1]));
      } else if (j < 12) {
        mq[j - 8] = __builtin_fmaxf(mq[j - 8], mq[j - 4]);
      } else if (j < 14) {
        mq[j - 12] = __builtin_fmaxf(mq[j - 12], mq[j - 10]);
      } else if (j == 14) {
        mq[0] = __builtin_fmaxf(mq[0], mq[1]);
      }
    };
    if constexpr (PV) {
      bf16x8 va[3];
      va[0] = vfrag(st_v, vbase, 0);
      va[1] = vfrag(st_v, vbase, 1);
      // The other wavefront of the SIMD is then in its softmax half: issue
      // these matrix instructions first (measured 1-3% faster).
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int j = 0; j < NPV; ++j) {
        if (j + 2 < NPV) va[(j + 2) % 3] = vfrag(st_v, vbase, j + 2);
        o[j % OT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j % 3], p[j / OT], o[j % OT], 0, 0, 0);
        max_step(j);
        hook(j);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int j = NPV; j < 15; ++j) max_step(j);
    } else {
#pragma unroll
      for (int j = 0; j < 15; ++j) max_step(j);
    }
    const float mx = max_xor32(mq[0]);
    const bool need = mx > kLazy || (!have && mx > kNegInf);
    if (__builtin_amdgcn_ballot_w64(need)) {
      keep_branch();
      const float delta = need ? mx : 0.0f;
      const float alpha = have ? __builtin_amdgcn_exp2f(-delta) : 0.0f;
      m += delta;
      have = have || mx > kNegInf;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] -= delta;
        s1[i] -= delta;
      }
#pragma unroll
      for (int t = 0; t < OT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
    }
  }

  // P = 2^s packed to bf16 into p, row sum added to l; the next tile's
  // S^T = K Q^T - m (K from st_k) goes to n0 / n1.  Issued in KS groups,
  // fenced against the scheduler.  The first half of the groups holds the
  // exponentials of s0 and the MFMAs of n1 (key rows 32..63), the second half
  // those of s1 and n0 (key rows 0..31), so n0 can take the registers of s0;
  // each group also packs and sums the pairs whose exponentials the group
  // before it issued.
  __device__ __forceinline__ void exp_next(const char* st_k, const int (&koff)[KS],
                                           const bf16x8 (&qb)[KS], f32x16& s0, f32x16& s1,
                                           bf16x8 (&p)[4], f32x16& n0, f32x16& n1) {
    static_assert(KS == 8 || KS == 4, "head dim 128 or 64");
    constexpr int H = KS / 2;    // groups per half
    constexpr int PPG = 8 / H;   // score pairs of one half per group
    uint32_t w0[8], w1[8];
    // Row sum of the probabilities as they enter P V (rounded to bf16), two
    // bf16 per v_dot2 against (1, 1), in two chains.
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float la = 0.0f, lb = 0.0f;
    auto fin0 = [&](int u) {
      w0[u] = pack_bf16x2(s0[2 * u], s0[2 * u + 1]);
      la = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0[u]), ones, la, false);
    };
    auto fin1 = [&](int u) {
      w1[u] = pack_bf16x2(s1[2 * u], s1[2 * u + 1]);
      lb = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1[u]), ones, lb, false);
    };
    // Group x: MFMAs of k-steps 2x, 2x + 1 of one accumulator.
    bf16x8 ka[2][2];
    auto kread = [&](int x, int h, int b) {
      ka[b][0] = kfrag(st_k, koff, (2 * x) % KS, h);
      ka[b][1] = kfrag(st_k, koff, (2 * x + 1) % KS, h);
    };
    n1 = splat16(-m);
    kread(0, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < KS; ++x) {
      const bool second = x >= H;
      if (x + 1 < KS) kread(x + 1, x + 1 >= H ? 0 : 1, (x + 1) & 1);
      if (x == H) {
        n0 = splat16(-m);
      }
      const int k0 = (2 * x) % KS, k1 = (2 * x + 1) % KS;
      if (!second) {
        n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[x & 1][0], qb[k0], n1, 0, 0, 0);
      } else {
        n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[x & 1][0], qb[k0], n0, 0, 0, 0);
      }
      const int xh = second ? x - H : x;
#pragma unroll
      for (int e = 0; e < PPG; ++e) {
        const int pr = xh * PPG + e;
        if (!second) {
          s0[2 * pr] = __builtin_amdgcn_exp2f(s0[2 * pr]);
          s0[2 * pr + 1] = __builtin_amdgcn_exp2f(s0[2 * pr + 1]);
        } else {
          s1[2 * pr] = __builtin_amdgcn_exp2f(s1[2 * pr]);
          s1[2 * pr + 1] = __builtin_amdgcn_exp2f(s1[2 * pr + 1]);
        }
      }
      if (!second) {
        n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[x & 1][1], qb[k1], n1, 0, 0, 0);
      } else {
        n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[x & 1][1], qb[k1], n0, 0, 0, 0);
      }
      if (x > 0)
#pragma unroll
        for (int e = 0; e < PPG; ++e) {
          const int xp = x - 1;
          if (xp < H) fin0((xp) * PPG + e);
          else fin1((xp - H) * PPG + e);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 0; e < PPG; ++e) fin1((H - 1) * PPG + e);
    l += la + lb;
    p[0] = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w0[2], w0[3]});
    p[1] = __builtin_bit_cast(bf16x8, u32x4{w0[4], w0[5], w0[6], w0[7]});
    p[2] = __builtin_bit_cast(bf16x8, u32x4{w1[0], w1[1], w1[2], w1[3]});
    p[3] = __builtin_bit_cast(bf16x8, u32x4{w1[4], w1[5], w1[6], w1[7]});
  }

  // Row sum over both lane halves (call once, all lanes).
  __device__ __forceinline__ float total() const { return sum_xor32(l); }
};

// This lane's fragment offsets inside a tile (see Flash::kfrag / vfrag).
// koff[ks]: K row col, logical chunk 2ks + hh, from the K tile start.
// vbase[t]: from the V tile start, the address this lane presents to the
// transposed V read for O^T rows 32t..: row 4h + q (q = (lane % 16) / 4),
// head dims 32t + 16 ((lane / 16) % 2) + 4 (lane % 4).
template <int D>
__device__ __forceinline__ void lane_offsets(int lane, int (&koff)[D / 16], int (&vbase)[D / 32]) {
  using Gm = TileGeom<D>;
  const int col = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = col * Gm::ROW + Gm::k_phys(col, 2 * ks + hh) * 16;
  const int q = (lane & 15) >> 2, b = (lane >> 4) & 1;
  const int row = 4 * hh + q;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    const int elem = 32 * t + 16 * b + 4 * (lane & 3);
    vbase[t] = row * Gm::ROW + Gm::v_phys(row, elem >> 3) * 16 + (elem & 7) * 2;
  }
}

// Asynchronous copy of `chunks` 16-byte chunks (a multiple of 64 per wave
// step) from global memory to LDS, bypassing registers: wavefront w moves
// chunks [64 i, 64 i + 64) for i = w, w + nw, ...; lane L lands at +16 L.
// Direct global->LDS load of 16 bytes per lane: lane L's bytes land at
// lds_dst + 16 L (lds_dst wave-uniform).  Written as inline asm on purpose:
// for the builtin form the compiler cannot tell ring stages apart and puts a
// wait for every in-flight tile load before later transposing LDS reads,
// which would drain the prefetch ring each tile.  The callers order LDS
// accesses themselves (explicit vmcnt waits, then a barrier).  M0 holds the
// LDS base (set by the compiler from the operand); one wait state separates
// its write from the load.
__device__ __forceinline__ void dma16(const void* gsrc, const void* lds_dst) {
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)lds_dst));
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gsrc), "{m0}"(base)
      : "memory");
}

// The same with a wave-uniform base address (in scalar registers) and a
// 32-bit per-lane byte offset: the per-lane 64-bit address arithmetic of
// dma16 disappears when the offsets stay fixed across tiles.
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, const void* lds_dst) {
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)lds_dst));
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "{m0}"(base)
      : "memory");
}

__device__ __forceinline__ void copy_to_lds(const u32x4* src, char* dst, int chunks, int wave,
                                            int nw, int lane) {
  for (int i = wave; i * 64 < chunks; i += nw) dma16(src + i * 64 + lane, dst + i * 1024);
}

// s_waitcnt immediate: vmcnt bits 3:0 and 15:14, expcnt 6:4 (7 = no wait),
// lgkmcnt 11:8 (15 = no wait).
template <int VM, int LGKM>
__device__ __forceinline__ void waitcnt() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

// Wait until at most n of this wave's vector-memory loads are outstanding
// (wave-uniform n >= 0; values above 12 other than 16, 24 and 32 wait for
// fewer, which is always safe); loads complete in issue order, so this waits
// for all but the n most recent.  LGKM0 additionally waits for this wave's
// LDS operations.
template <bool LGKM0 = false>
__device__ __forceinline__ void wait_vm(int n) {
  constexpr int L = LGKM0 ? 0 : 15;
  switch (n) {
    case 1: waitcnt<1, L>(); break;
    case 2: waitcnt<2, L>(); break;
    case 3: waitcnt<3, L>(); break;
    case 4: waitcnt<4, L>(); break;
    case 5: waitcnt<5, L>(); break;
    case 6: waitcnt<6, L>(); break;
    case 7: waitcnt<7, L>(); break;
    case 8: waitcnt<8, L>(); break;
    case 9: waitcnt<9, L>(); break;
    case 10: waitcnt<10, L>(); break;
    case 11: waitcnt<11, L>(); break;
    case 12: case 13: case 14: case 15: waitcnt<12, L>(); break;
    case 16: case 17: case 18: case 19: case 20: case 21: case 22: case 23: waitcnt<16, L>(); break;
    case 24: case 25: case 26: case 27: case 28: case 29: case 30: case 31: waitcnt<24, L>(); break;
    default: if (n >= 32) waitcnt<32, L>(); else waitcnt<0, L>(); break;
  }
}

// Workgroup barrier without a memory fence (no implied vmcnt(0) wait): the
// caller waits for exactly the loads it needs.  The signal fences keep the
// compiler from moving memory operations across it.
__device__ __forceinline__ void barrier_nofence() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------------------
// The software-pipelined tile walk of the 256-row kernels (the prefill and the
// shared-block Stage-2 kernel), after flash_walk_start.  K tiles and V tiles have separate LDS rings
// of four stages (tile t in stage t % 4), filled by the caller's load_k /
// load_v (direct global -> LDS loads, two tiles at a time).  Iteration i
// computes the softmax of tile i, P V of tile i - 1 and the scores of tile
// i + 1 (reading K of tile i + 1, V of tile i - 1).  V fragments are read at
// vread + stage * VBYTES + vbase[..]: the kernels pass the start of their LDS
// block and keep the V ring's offset in vbase.  Even iterations start
// with a barrier: every load requested two iterations earlier has landed
// (each wave waits for its own, the barrier for all), and the stages of K
// tiles i - 1, i and V tiles i - 3, i - 2 are refilled for the next two
// iterations; odd iterations run without one, so the two wavefronts of a SIMD
// can drift apart.  The refill requests go out in four parts spread over the
// P V group of the even iteration: issued together right after the barrier,
// the 64 direct loads of a workgroup queued at the memory unit and every wave
// waited there (about 15% of the walk, measured), the two waves of a SIMD at
// the same time.  The loop is unrolled over the four stages: every LDS
// fragment address is then the lane's base plus a constant, and the score
// registers alternate instead of being copied.  The last iteration also
// computes scores of a stale K stage; they are never used.  Leaves O, m, l
// in fl.
// ---------------------------------------------------------------------------
// The first loads of the walk (K of tiles 0, 1, 2 and V of tile 0); the
// kernels issue them before loading and rotating Q so the two overlap.
template <typename LoadK, typename LoadV>
__device__ __forceinline__ void flash_walk_start(const int n_tiles, LoadK&& load_k, LoadV&& load_v) {
  for (int i = 0; i < 3 && i < n_tiles; ++i) load_k(i);
  load_v(0);
}

template <int D, typename LoadK, typename LoadV, typename FullOf, typename VisOf>
__device__ __forceinline__ void flash_walk(Flash<D>& fl, char* const kring, char* const vread,
                                           const int n_tiles, const int (&koff)[D / 16],
                                           const int (&vbase)[D / 32],
                                           const bf16x8 (&qb)[D / 16], LoadK&& load_k,
                                           LoadV&& load_v, FullOf&& full_of, VisOf&& vis_of) {
  using Gm = TileGeom<D>;
  static_assert(kPrefillStages == 4, "two tiles in use and two in flight per ring");
  const auto request = [&](int i) {
    if (i + 3 < n_tiles) load_k(i + 3);
    if (i + 4 < n_tiles) load_k(i + 4);
    if (i + 1 < n_tiles) load_v(i + 1);
    if (i + 2 < n_tiles) load_v(i + 2);
  };
  const auto sync = [&](int i) {
    wait_vm(0);
    barrier_nofence();
    request(i);
  };
  const auto sync_only = [&]() {
    wait_vm(0);
    barrier_nofence();
  };
  // The requests of even iteration i, one part every quarter of its P V group.
  constexpr int ST = Flash<D>::NPV / 4;
  const auto spread_request = [&](int i) {
    return [&, i](int j) {
      if (j == 0) {
        if (i + 3 < n_tiles) load_k(i + 3);
      } else if (j == ST) {
        if (i + 4 < n_tiles) load_k(i + 4);
      } else if (j == 2 * ST) {
        if (i + 1 < n_tiles) load_v(i + 1);
      } else if (j == 3 * ST) {
        if (i + 2 < n_tiles) load_v(i + 2);
      }
    };
  };
  const auto ks = [&](int st) { return kring + st * Gm::KBYTES; };
  const auto vs = [&](int st) { return vread + st * Gm::VBYTES; };
  // Prologue: K of tiles 0, 1, 2 and V of tile 0 (issued by
  // flash_walk_start), all landed before the scores of tile 0.
  wait_vm(0);
  barrier_nofence();
  f32x16 s0, s1, n0, n1;
  bf16x8 pr[4];
  fl.scores(ks(0), koff, qb, s0, s1);
  sync(0);
  fl.template pv_head<false>(vs(0), vbase, pr, s0, s1, !full_of(0), vis_of(0));
  fl.exp_next(ks(1), koff, qb, s0, s1, pr, n0, n1);
  for (int i = 1; i < n_tiles; i += 4) {
    fl.template pv_head<true>(vs(0), vbase, pr, n0, n1, !full_of(i), vis_of(i));
    fl.exp_next(ks(2), koff, qb, n0, n1, pr, s0, s1);
    if (i + 1 >= n_tiles) break;
    sync_only();
    fl.template pv_head<true>(vs(1), vbase, pr, s0, s1, !full_of(i + 1), vis_of(i + 1),
                              spread_request(i + 1));
    fl.exp_next(ks(3), koff, qb, s0, s1, pr, n0, n1);
    if (i + 2 >= n_tiles) break;
    fl.template pv_head<true>(vs(2), vbase, pr, n0, n1, !full_of(i + 2), vis_of(i + 2));
    fl.exp_next(ks(0), koff, qb, n0, n1, pr, s0, s1);
    if (i + 3 >= n_tiles) break;
    sync_only();
    fl.template pv_head<true>(vs(3), vbase, pr, s0, s1, !full_of(i + 3), vis_of(i + 3),
                              spread_request(i + 3));
    fl.exp_next(ks(1), koff, qb, s0, s1, pr, n0, n1);
  }
  // P V of the last tile (its V may have been requested by the last barrier).
  wait_vm(0);
  barrier_nofence();
  fl.pv(vs((n_tiles - 1) % kPrefillStages), vbase, pr);
}

// Work queue of a persistent grid (about one workgroup per compute unit):
// items [0, n) are cut into 8 consecutive ranges, one per XCD (neighbouring
// items share K/V in that XCD's L2), each with a counter in `queue` that the
// kernel launched before zeroed.  A workgroup takes the next item of its own
// XCD's range and, once that is used up, of the other ranges in turn, so XCDs
// that run faster (their clocks differ) finish the work of slower ones, and no
// compute unit waits on the hardware dispatcher between items.  Called by one
// thread; -1 when every range is used up.
__device__ __forceinline__ int queue_claim(uint32_t* queue, int n) {
  const int qq = n >> 3, qr = n & 7;
  const int x0 = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 7;  // XCC_ID
  for (int d = 0; d < 8; ++d) {
    const int x = (x0 + d) & 7;
    const int size = qq + (x < qr ? 1 : 0);
    if (size == 0) continue;
    const int i = (int)atomicAdd(queue + x, 1u);
    if (i < size) return (x < qr ? x * (qq + 1) : qr * (qq + 1) + (x - qr) * qq) + i;
  }
  return -1;
}

// The item loop of a persistent grid: run(item, k) handles round k's item;
// its thread 0 stores the item of round k + 1 in s_next[(k + 1) & 1] (claimed
// early, so the claim's latency hides behind the round).  Every wave reads
// s_next[k & 1] before the round's barriers, so the round-(k + 1) slot is
// free when thread 0 writes it; the barrier after each round also frees the
// LDS for the next round's first tile requests.  (Callers build with machine
// loop-invariant code motion off: hoisted out of this loop, constants and
// addresses would stay live across the whole walk and spill registers.)
template <typename Run>
__device__ __forceinline__ void queue_loop(uint32_t* queue, int n, int* s_next, Run&& run) {
  if (threadIdx.x == 0) s_next[0] = queue_claim(queue, n);
  __syncthreads();
  for (int k = 0;; ++k) {
    const int item = s_next[k & 1];
    if (item < 0) break;
    run(item, k);
    __syncthreads();
  }
}

// Workgroup order: the hardware hands consecutive workgroup ids to the 8 XCDs
// in turn.  Remap so that each XCD walks a contiguous range of logical work
// items (neighbouring query tiles of one KV head share K/V in that XCD's L2).
__device__ __forceinline__ int xcd_logical(int lin, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = lin & 7, i = lin >> 3;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// int32 table carried in the kernel arguments at byte offset `off` of the
// argument block: read in place through the kernarg segment pointer (indexing
// the by-value argument would make the compiler copy it to private memory).
__device__ __forceinline__ const int32_t* kernarg_ints(size_t off) {
  return reinterpret_cast<const int32_t*>((const char*)__builtin_amdgcn_kernarg_segment_ptr() + off);
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
