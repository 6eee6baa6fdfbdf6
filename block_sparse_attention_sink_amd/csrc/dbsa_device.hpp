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


// ---------------------------------------------------------------------------
// Tile layouts (one 64-key tile of one KV head).
//
//   K tile   [64 keys][D] bf16, rotated                 (KBYTES)
//   V^T tile [D][64 keys] bf16; inside each 16-key group the keys are stored
//            in the order the MFMA result layout hands out P (vt_key_of_pos),
//            so one 16-byte read gives a lane the 8 keys it contracts over.
// Rows are split in 16-byte chunks and chunk c of row r is stored at chunk
// c ^ swz(r): 16 lanes reading the same logical chunk of 16 consecutive rows
// then hit 16 distinct bank groups.  The global tile images written by the
// pack step are byte-for-byte the LDS images, so staging is a linear copy.
// ---------------------------------------------------------------------------
template <int D>
struct TileGeom {
  static constexpr int KROW = D * 2;                // K row bytes
  static constexpr int VROW = kKeyTile * 2;         // V^T row bytes (128)
  static constexpr int KBYTES = kKeyTile * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;     // one LDS stage (K + V^T)
  static constexpr int TU4 = kKeyTile * D / 8;      // 16-byte chunks per tile matrix
  static constexpr int KCR = D / 8;                 // chunks per K row
  static __device__ __forceinline__ int k_phys(int row, int c) {
    if constexpr (D == 128) return c ^ (row & 15);
    else return c ^ ((row >> 1) & 7);
  }
  static __device__ __forceinline__ int v_phys(int row, int c) { return c ^ ((row >> 1) & 7); }
};

// Key (0..15, within its 16-key group) stored at position p (0..15), and back.
__device__ __forceinline__ int vt_key_of_pos(int p) {
  return 8 * ((p & 7) >> 2) + 4 * (p >> 3) + (p & 3);
}
__device__ __forceinline__ int vt_pos_of_key(int k) {
  return 8 * ((k >> 2) & 1) + 4 * (k >> 3) + (k & 3);
}

// Eight probabilities of one MFMA result (registers B .. B+7) as a bf16 B operand.
template <int B>
__device__ __forceinline__ bf16x8 pack_p(const f32x16 s) {
  const u32x4 w = u32x4{pack_bf16x2(s[B + 0], s[B + 1]), pack_bf16x2(s[B + 2], s[B + 3]),
                        pack_bf16x2(s[B + 4], s[B + 5]), pack_bf16x2(s[B + 6], s[B + 7])};
  return __builtin_bit_cast(bf16x8, w);
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

template <int D>
struct Flash {
  static constexpr int KS = D / 16;  // k-steps over the head dim
  static constexpr int OT = D / 32;  // O^T row tiles
  using Gm = TileGeom<D>;
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

  // S^T of one tile relative to the current reference m (K fragments from LDS).
  __device__ __forceinline__ void scores(const char* st, const int (&koff)[KS],
                                         const bf16x8 (&qb)[KS], f32x16& s0, f32x16& s1) const {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = -m;
      s1[i] = -m;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ka0 = *reinterpret_cast<const bf16x8*>(st + koff[ks]);
      const bf16x8 ka1 = *reinterpret_cast<const bf16x8*>(st + koff[ks] + 32 * Gm::KROW);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0, qb[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1, qb[ks], s1, 0, 0, 0);
    }
  }

  // Mask (when `mask`: key kr of the tile is kept iff vis(kr)), row maximum and
  // the rare reference raise (rescaling o and l).  Leaves s = S - m.
  template <typename Vis>
  __device__ __forceinline__ void head(f32x16& s0, f32x16& s1, bool mask, Vis vis) {
    if (mask) {
      const int hh = (threadIdx.x >> 5) & 1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kr = (i >> 2) * 8 + hh * 4 + (i & 3);
        s0[i] = vis(kr) ? s0[i] : kNegInf;
        s1[i] = vis(kr + 32) ? s1[i] : kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s0[i], s1[i]));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    const bool need = mx > kLazy || (!have && mx > kNegInf);
    if (__builtin_amdgcn_ballot_w64(need)) {
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

  // P = 2^s packed to bf16, row sum added to l.  When NEXT, the S^T MFMAs of
  // the next tile (K fragments from st_next) are issued interleaved with this
  // VALU work, so the wave's instruction stream alternates matrix and vector
  // instructions; the next tile's scores use the reference m just settled.
  template <bool NEXT>
  __device__ __forceinline__ void probs(f32x16& s0, f32x16& s1, bf16x8 (&p)[4],
                                        const char* st_next, const int (&koff)[KS],
                                        const bf16x8 (&qb)[KS], f32x16& n0, f32x16& n1) {
    if constexpr (NEXT) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        n0[i] = -m;
        n1[i] = -m;
      }
    }
    // 8 rounds: 2 next-tile MFMAs (one k-step) + 4 exponentials each.
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if constexpr (NEXT) {
        if (r < KS) {
          const bf16x8 ka0 = *reinterpret_cast<const bf16x8*>(st_next + koff[r]);
          const bf16x8 ka1 =
              *reinterpret_cast<const bf16x8*>(st_next + koff[r] + 32 * Gm::KROW);
          n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0, qb[r], n0, 0, 0, 0);
          n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1, qb[r], n1, 0, 0, 0);
        }
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 2 * r + e;
        s0[i] = __builtin_amdgcn_exp2f(s0[i]);
        s1[i] = __builtin_amdgcn_exp2f(s1[i]);
      }
      if constexpr (NEXT) {
        if (r < KS) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // 2 VALU
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // 2 VALU
        }
      }
    }
    p[0] = pack_p<0>(s0);
    p[1] = pack_p<8>(s0);
    p[2] = pack_p<0>(s1);
    p[3] = pack_p<8>(s1);
    float ra = 0.0f, rb = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ra += s0[i];
      rb += s1[i];
    }
    l += ra + rb;
  }

  // O^T += V^T P^T (V^T fragments from LDS); k-step outer, OT independent chains.
  __device__ __forceinline__ void pv(const char* st, const int (&voff)[4], const bf16x8 (&p)[4]) {
    bf16x8 vf[4 * OT];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int t = 0; t < OT; ++t)
        vf[kk * OT + t] = *reinterpret_cast<const bf16x8*>(st + voff[kk] + t * 32 * Gm::VROW);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int t = 0; t < OT; ++t)
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kk * OT + t], p[kk], o[t], 0, 0, 0);
  }

  // One whole tile without cross-tile pipelining.
  template <typename Vis>
  __device__ __forceinline__ void tile(const char* st, const int (&koff)[KS],
                                       const int (&voff)[4], const bf16x8 (&qb)[KS], bool mask,
                                       Vis vis) {
    f32x16 s0, s1, n0, n1;
    bf16x8 p[4];
    scores(st, koff, qb, s0, s1);
    head(s0, s1, mask, vis);
    probs<false>(s0, s1, p, st, koff, qb, n0, n1);
    pv(st, voff, p);
  }

  // Row sum over both lane halves (call once, all lanes).
  __device__ __forceinline__ float total() const { return l + __shfl_xor(l, 32); }
};

// This lane's fragment offsets inside a stage (see Flash::tile).
template <int D>
__device__ __forceinline__ void lane_offsets(int col, int hh, int (&koff)[D / 16], int (&voff)[4]) {
  using Gm = TileGeom<D>;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = col * Gm::KROW + Gm::k_phys(col, 2 * ks + hh) * 16;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    voff[kk] = Gm::KBYTES + col * Gm::VROW + Gm::v_phys(col, 2 * kk + hh) * 16;
}

// Asynchronous copy of `chunks` 16-byte chunks (a multiple of 64 per wave
// step) from global memory to LDS, bypassing registers: wavefront w moves
// chunks [64 i, 64 i + 64) for i = w, w + nw, ...; lane L lands at +16 L.
__device__ __forceinline__ void copy_to_lds(const u32x4* src, char* dst, int chunks, int wave,
                                            int nw, int lane) {
  for (int i = wave; i * 64 < chunks; i += nw)
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(src + i * 64 + lane),
        (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, 0, 0);
}

// Wait until at most n of this wave's vector-memory loads are outstanding
// (n: 0..15, wave-uniform).  Loads complete in issue order, so this waits for
// all but the n most recent.
__device__ __forceinline__ void wait_vm(int n) {
  // s_waitcnt immediate: vmcnt in bits 3:0, expcnt 6:4 (7 = no wait), lgkmcnt 11:8 (15).
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
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
