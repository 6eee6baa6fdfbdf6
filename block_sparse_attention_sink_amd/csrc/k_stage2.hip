// Stage 2 of DBSA on gfx950: per-query dynamic inference.
//
// [Notes, Method > Stage 2]: the cached (unrotated) K/V of the retrieved
// blocks, anchor first, are concatenated; RoPE is re-applied at the new
// sequential positions; the query tokens attend to all of it and then decode
// autoregressively.
//
// Kernels
//   k_gather_bf16 / k_gather_f32   materialise the gathered, re-rotated K and
//                                  the gathered V (HBM-bound copy + rotate).
//   k_new_kv_f32                   rotate the new tokens' K at their positions
//                                  and append K/V to the row's context buffer
//                                  (float32 path; bf16 does it in k_query_bf16).
//   k_query_bf16<D, RW, KW>        split-K flash attention of the packed
//                                  (token, head-in-group) rows of one KV head
//                                  over a segment list, 32 rows per attention
//                                  wavefront on the software-pipelined prefill
//                                  core, RW row wavefronts, each doubled into
//                                  two key halves when KW = 2 (pool blocks and
//                                  new tokens are rotated while staged; new
//                                  tokens are also appended to the context
//                                  buffer).
//   k_combine                      log-sum-exp merge of the split partials.
//   k_query_f32                    float32 rows (one wavefront per row).
#include "dbsa_device.hpp"

namespace dbsa {

// ---------------------------------------------------------------------------
// Gather + re-RoPE (materialised).
// ---------------------------------------------------------------------------
// bf16: positions p = 64 t + r are rotated by the angle sum of 64 t (shared by
// the block's tokens, which all lie in one 64-aligned tile) and r, exactly as
// the query kernel rotates pool rows, so both paths round identically.
template <int D>
__global__ __launch_bounds__(256) void k_gather_bf16(GatherArgs a) {
  constexpr int CP = D / 16, H = D / 2;
  constexpr int TOK = 256 / CP;
  static_assert(kKeyTile % TOK == 0, "a block's tokens share one 64-row tile");
  __shared__ float tile_c[H], tile_s[H];
  const int b = blockIdx.y;
  const int u = blockIdx.x * TOK + threadIdx.x / CP;
  const int c = threadIdx.x % CP;
  if (threadIdx.x < H) {
    const int64_t base = (int64_t)(blockIdx.x * TOK) & ~(int64_t)(kKeyTile - 1);
    rope_cs(base, a.freq.rev[threadIdx.x], tile_c[threadIdx.x], tile_s[threadIdx.x]);
  }
  __syncthreads();
  const int32_t* tab = a.n_inline ? kernarg_ints(offsetof(GatherArgs, inl)) : a.tab;
  const int32_t* st = tab + (int64_t)b * (a.n_ids + 1);
  if (u >= st[a.n_ids]) return;
  const int i = upper_index(st, a.n_ids, u);
  const int32_t* srcs = tab + (int64_t)a.batch * (a.n_ids + 1);
  const int64_t src_tok = srcs[(int64_t)b * a.n_ids + i] + (u - st[i]);
  float cs[8], sn[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    float cr, sr;
    rope_cs(u & (kKeyTile - 1), a.freq.rev[8 * c + r], cr, sr);
    angle_add(tile_c[8 * c + r], tile_s[8 * c + r], cr, sr, cs[r], sn[r]);
  }
  const u32x4* kp = reinterpret_cast<const u32x4*>(a.k_pool);
  const u32x4* vp = reinterpret_cast<const u32x4*>(a.v_pool);
  u32x4* ko = reinterpret_cast<u32x4*>(a.k_out);
  u32x4* vo = reinterpret_cast<u32x4*>(a.v_out);
  constexpr int CR = D / 8;
  auto head = [&](int g) __attribute__((always_inline)) {
    const int64_t src = (src_tok * a.hkv + g) * CR;
    const int64_t dst = (((int64_t)b * a.cap + u) * a.hkv + g) * CR;
    u32x4 k1 = kp[src + c], k2 = kp[src + c + CP];
    const u32x4 v1 = vp[src + c], v2 = vp[src + c + CP];
    rotate_chunk(k1, k2, cs, sn);
    ko[dst + c] = k1;
    ko[dst + c + CP] = k2;
    vo[dst + c] = v1;
    vo[dst + c + CP] = v2;
  };
  // Many KV heads: four heads' loads in flight per thread (measured 8%
  // faster with 32 heads; with 8 heads the plain loop is faster).
  if (a.hkv >= 16) {
#pragma unroll 4
    for (int g = 0; g < a.hkv; ++g) head(g);
  } else {
    for (int g = 0; g < a.hkv; ++g) head(g);
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_gather_f32(GatherArgs a) {
  constexpr int H = D / 2;
  const int b = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (token, pair)
  const int u = (int)(idx / H), i = (int)(idx % H);
  const int32_t* tab = a.n_inline ? kernarg_ints(offsetof(GatherArgs, inl)) : a.tab;
  const int32_t* st = tab + (int64_t)b * (a.n_ids + 1);
  if (u >= st[a.n_ids]) return;
  const int s = upper_index(st, a.n_ids, u);
  const int32_t* srcs = tab + (int64_t)a.batch * (a.n_ids + 1);
  const int64_t src_tok = srcs[(int64_t)b * a.n_ids + s] + (u - st[s]);
  float c, sn;
  rope_cs(u, a.freq.rev[i], c, sn);
  const float* kp = static_cast<const float*>(a.k_pool);
  const float* vp = static_cast<const float*>(a.v_pool);
  float* ko = static_cast<float*>(a.k_out);
  float* vo = static_cast<float*>(a.v_out);
  for (int g = 0; g < a.hkv; ++g) {
    const int64_t src = (src_tok * a.hkv + g) * D;
    const int64_t dst = (((int64_t)b * a.cap + u) * a.hkv + g) * D;
    const float x1 = kp[src + i], x2 = kp[src + i + H];
    ko[dst + i] = rot_lo(x1, x2, c, sn);
    ko[dst + i + H] = rot_hi(x1, x2, c, sn);
    vo[dst + i] = vp[src + i];
    vo[dst + i + H] = vp[src + i + H];
  }
}

// ---------------------------------------------------------------------------
// New tokens: rotate K at its position, append K/V to the context buffer.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_new_kv_f32(NewKVArgs a) {
  constexpr int H = D / 2;
  const int r = blockIdx.x, b = blockIdx.y;
  const int64_t pos = (int64_t)a.pos0[b] + r;
  const int64_t row = (int64_t)a.dst_row[b] + r;
  for (int u = threadIdx.x; u < a.hkv * H; u += blockDim.x) {
    const int g = u / H, i = u % H;
    const int64_t src = (((int64_t)b * a.n_new + r) * a.hkv + g) * D;
    const int64_t dst = (((int64_t)b * a.cap + row) * a.hkv + g) * D;
    const float* kp = static_cast<const float*>(a.k_new);
    const float* vp = static_cast<const float*>(a.v_new);
    float c, s;
    rope_cs(pos, a.freq.rev[i], c, s);
    float* ko = static_cast<float*>(a.k_dst);
    float* vo = static_cast<float*>(a.v_dst);
    const float x1 = kp[src + i], x2 = kp[src + i + H];
    ko[dst + i] = rot_lo(x1, x2, c, s);
    ko[dst + i + H] = rot_hi(x1, x2, c, s);
    vo[dst + i] = vp[src + i];
    vo[dst + i + H] = vp[src + i + H];
  }
}

// ---------------------------------------------------------------------------
// Segment tables: in the kernel arguments (read through the kernarg segment
// pointer, so no private copy is made) or in device memory.
// ---------------------------------------------------------------------------
__device__ __forceinline__ const int32_t* seg_block(const QueryArgs& a) {
  return a.n_inline ? kernarg_ints(offsetof(QueryArgs, inl)) : a.meta;
}

// ---------------------------------------------------------------------------
// The flash core on one half of every 64-key tile (keys 32h .. 32h + 31):
// two wavefronts share a row set, each running this on its own half with its
// own (m, l, O), merged once at the end.  Same lane layout, pipeline split
// (pv_head / exp_next) and lazy reference as the full-tile core; half the
// MFMAs and exponentials per wavefront and tile.
// ---------------------------------------------------------------------------
template <int D>
struct FlashHalf {
  static constexpr int KS = D / 16;
  static constexpr int OT = D / 32;
  static constexpr int NPV = 2 * OT;  // P V products per half tile (2 k-steps of 16 keys x OT)
  using Gm = TileGeom<D>;
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  f32x16 o[OT];
  float m, l;
  bool have;
  int h;  // key half (wave-uniform)

  __device__ __forceinline__ void init(int half) {
#pragma unroll
    for (int t = 0; t < OT; ++t) o[t] = f32x16{};
    m = 0.0f;
    l = 0.0f;
    have = false;
    h = half;
  }
  // V^T fragment of P V product j of this half: k-step 2h + j / OT.
  __device__ __forceinline__ bf16x8 vfrag(const char* st_v, const int (&vbase)[OT], int j) const {
    const char* a0 = st_v + vbase[j % OT] + (16 * (2 * h + j / OT)) * Gm::ROW;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(a0 + 8 * Gm::ROW));
    const s16x8 v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v8);
  }
  __device__ __forceinline__ bf16x8 kfrag(const char* st_k, const int (&koff)[KS], int ks) const {
    return *reinterpret_cast<const bf16x8*>(st_k + koff[ks] + h * 32 * Gm::KROW);
  }
  __device__ __forceinline__ void scores(const char* st_k, const int (&koff)[KS],
                                         const bf16x8 (&qb)[KS], f32x16& s) const {
    s = splat16(-m);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(st_k, koff, ks), qb[ks], s, 0, 0, 0);
  }
  __device__ __forceinline__ void pv(const char* st_v, const int (&vbase)[OT], const bf16x8 (&p)[2]) {
#pragma unroll
    for (int j = 0; j < NPV; ++j)
      o[j % OT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag(st_v, vbase, j), p[j / OT],
                                                          o[j % OT], 0, 0, 0);
  }
  // Mask, row maximum (16 scores a lane), rare reference raise; the previous
  // half tile's P V interleaved with the maximum tree.
  template <bool PV, typename Vis>
  __device__ __forceinline__ void pv_head(const char* st_v, const int (&vbase)[OT],
                                          const bf16x8 (&p)[2], f32x16& s, bool mask, Vis vis) {
    if (mask) {
      keep_branch();
      const int hh = (threadIdx.x >> 5) & 1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kr = 32 * h + (i >> 2) * 8 + hh * 4 + (i & 3);
        s[i] = vis(kr) ? s[i] : kNegInf;
      }
    }
    float mq[8];
    auto max_step = [&](int j) {
      if (j < 8) {
        mq[j] = __builtin_fmaxf(s[2 * j], s[2 * j + 1]);
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
#pragma unroll
      for (int j = 0; j < NPV; ++j) {
        if (j + 2 < NPV) va[(j + 2) % 3] = vfrag(st_v, vbase, j + 2);
        o[j % OT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j % 3], p[j / OT], o[j % OT], 0, 0, 0);
        max_step(2 * j);
        max_step(2 * j + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 2 * NPV; j < 15; ++j) max_step(j);
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
      for (int i = 0; i < 16; ++i) s[i] -= delta;
#pragma unroll
      for (int t = 0; t < OT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
    }
  }
  // P = 2^s packed to bf16 into p, row sum into l; the next half tile's
  // scores (relative to m) into n, in KS / 2 fenced groups of two MFMAs.
  __device__ __forceinline__ void exp_next(const char* st_k, const int (&koff)[KS],
                                           const bf16x8 (&qb)[KS], f32x16& s, bf16x8 (&p)[2],
                                           f32x16& n) {
    static_assert(KS == 8 || KS == 4, "head dim 128 or 64");
    constexpr int NG = KS / 2;
    constexpr int PPG = 8 / NG;  // score pairs per group
    uint32_t w[8];
    float sq[8];
    auto fin = [&](int u) {
      w[u] = pack_bf16x2(s[2 * u], s[2 * u + 1]);
      sq[u] = s[2 * u] + s[2 * u + 1];
    };
    bf16x8 ka[2][2];
    auto kread = [&](int x, int b) {
      ka[b][0] = kfrag(st_k, koff, 2 * x);
      ka[b][1] = kfrag(st_k, koff, 2 * x + 1);
    };
    n = splat16(-m);
    kread(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < NG; ++x) {
      if (x + 1 < NG) kread(x + 1, (x + 1) & 1);
      n = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[x & 1][0], qb[2 * x], n, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < PPG; ++e) {
        const int pr = x * PPG + e;
        s[2 * pr] = __builtin_amdgcn_exp2f(s[2 * pr]);
        s[2 * pr + 1] = __builtin_amdgcn_exp2f(s[2 * pr + 1]);
      }
      n = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[x & 1][1], qb[2 * x + 1], n, 0, 0, 0);
      if (x > 0)
#pragma unroll
        for (int e = 0; e < PPG; ++e) fin((x - 1) * PPG + e);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 0; e < PPG; ++e) fin((NG - 1) * PPG + e);
#pragma unroll
    for (int w2 = 4; w2 > 0; w2 >>= 1)
#pragma unroll
      for (int k = 0; k < w2; ++k) sq[k] += sq[k + w2];
    l += sq[0];
    p[0] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
    p[1] = __builtin_bit_cast(bf16x8, u32x4{w[4], w[5], w[6], w[7]});
  }
  __device__ __forceinline__ float total() const { return sum_xor32(l); }
};

// ---------------------------------------------------------------------------
// Query attention, bf16 MFMA, split-K over the context.
//
// Rows = (query token, head in GQA group) packed per KV head.  Workgroup =
// RW attention wavefronts of 32 packed rows each (the software-pipelined
// Flash core of the prefill, on v_mfma_f32_32x32x16_bf16) plus
// kQueryLoaders loader wavefronts, one of each kind per SIMD: a 32-row
// attention wavefront needs half of a SIMD's registers.  With KW = 2 (at
// most 64 rows) every row wavefront has a twin on the other half of each
// key tile, so all four SIMDs run attention; the twins merge their (m, l, O)
// through LDS after the last tile.  Iteration i of the
// attention computes the softmax of tile i, P V of tile i - 1 and the scores
// of tile i + 1, so it reads K of tile i + 1 and V of tile i - 1; meanwhile
// the loaders store K and V of tile i + 2 (K ring of two LDS stages, V ring
// of four).  Each loader thread owns two (row, chunk pair) items of every
// tile: it follows its rows through the segment list in registers, keeps
// every tile's K and V in registers kQueryLead tiles ahead of its store (the
// compiler counts these loads, so every store waits for exactly its own
// tile) and rotates K at the row's virtual position on the way to LDS (row
// angles in registers, the tile's angles from a small table).  New tokens
// (their rotated K and their V) also go to the context buffer.
// ---------------------------------------------------------------------------
template <int D, int RW, int KW>
__global__ __launch_bounds__(64 * (RW * KW + kQueryLoaders), 1) void k_query_bf16(QueryArgs a) {
  using Gm = TileGeom<D>;
  static_assert(KW == 1 || (KW == 2 && RW <= 2), "key halves for at most 64 rows");
  constexpr int NWA = RW * KW;  // attention wavefronts
  constexpr int NL = kQueryLoaders, NW = NWA + NL;
  constexpr int KS = D / 16, OT = D / 32, CP = D / 16, CR = D / 8, H = D / 2;
  constexpr int P = kQueryLead;
  constexpr int NT = 8;  // tile-angle table slots
  static_assert(NT >= P + 2 && (NT & (NT - 1)) == 0, "angle table ring");
  constexpr int ITEMS = kKeyTile * CP / (64 * NL);  // (row, chunk pair) items per loader thread
  static_assert(ITEMS >= 1 && ITEMS * 64 * NL == kKeyTile * CP, "items split evenly");
  constexpr int NVS = 4;  // V stages
  __shared__ __align__(16) char kring[2 * Gm::KBYTES];
  __shared__ __align__(16) char vring[NVS * Gm::VBYTES];
  __shared__ __align__(16) f32x2 rot_a[NT][kMaxHalf];  // cos / sin of w_i * u0 per tile
  __shared__ int32_t seg_start[kMaxSegments + 1], seg_src[kMaxSegments], seg_buf[kMaxSegments];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool loader = wave >= NWA;
  const int hh = lane >> 5, col = lane & 31;
  // Work item (split, KV head g, row group rg, batch row b).  With several
  // row groups, those of one (split, head, batch row) take consecutive
  // workgroup slots of one XCD (ids 8 apart: the hardware deals consecutive
  // ids to the 8 XCDs in turn), so they run side by side and can share the
  // tile reads through that XCD's L2.
  const int R = a.row_groups, W = a.n_split * a.hkv * a.batch;
  const int lin = blockIdx.x;
  const int rg = R > 1 ? (lin >> 3) % R : 0;
  const int w = R > 1 ? (lin / (8 * R)) * 8 + (lin & 7) : lin;
  if (w >= W) return;  // padding of the last group of 8 (before any barrier)
  const int g = w % a.hkv, split = (w / a.hkv) % a.n_split, b = w / (a.hkv * a.n_split);
  const int G = a.hq / a.hkv;
  const int way = wave / RW;  // key half (KW == 2) of an attention wavefront
  const int rho = rg * (32 * RW) + (wave % RW) * 32 + col;
  const bool live = !loader && rho < a.rows;
  const int r = live ? rho / G : 0;
  const int head = g * G + (live ? rho - (rho / G) * G : 0);
  const int32_t* tab = seg_block(a);
  const int pos0 = tab[a.seg.o_pos0 + b];
  const int dst0 = tab[a.seg.o_dst + b];
  const int qpos = pos0 + r;
  // Rotation offset of the row: keys and queries turn at virtual position + rot.
  const int rot = a.seg.o_rot >= 0 ? tab[a.seg.o_rot + b] : 0;

  const int nseg = tab[a.seg.o_nseg + b];
  {
    const int32_t* st = tab + a.seg.o_start + b * a.seg.stride;
    const int32_t* sr = tab + a.seg.o_src + b * a.seg.stride;
    const int32_t* sb = tab + a.seg.o_buf + b * a.seg.stride;
    for (int i = tid; i <= nseg; i += 64 * NW) {
      seg_start[i] = st[i];
      if (i < nseg) {
        seg_src[i] = sr[i];
        seg_buf[i] = sb[i];
      }
    }
  }
  __syncthreads();  // segment table visible

  const int T = seg_start[nseg];
  const int n_tiles = (T + kKeyTile - 1) / kKeyTile;
  const int it0 = split * a.tiles_per_split;
  const int cnt = max(0, min(it0 + a.tiles_per_split, n_tiles) - it0);

  if (loader) {
    const int ltid = tid - 64 * NWA;
    if (cnt == 0) {
      barrier_nofence();
      if constexpr (KW == 2) barrier_nofence();  // (the key halves' merge)
      return;
    }
    // Item k of this thread: row ltid / CP + k * 64 / ITEMS, chunks c and
    // c + CP (the two halves RoPE pairs up).  Rows past the split's last
    // key (the look-ahead past its last tile) repeat that key: they are
    // never used, and so cost no traffic beyond the split's own keys.
    const int c = ltid % CP;
    const int tend = min(T, (it0 + cnt) * kKeyTile);
    const uint64_t kb0 = reinterpret_cast<uint64_t>(a.k_pool), vb0 = reinterpret_cast<uint64_t>(a.v_pool);
    const uint64_t kb1 = reinterpret_cast<uint64_t>(a.k_ctx), vb1 = reinterpret_cast<uint64_t>(a.v_ctx);
    const uint64_t kb2 = reinterpret_cast<uint64_t>(a.k_new), vb2 = reinterpret_cast<uint64_t>(a.v_new);
    const int64_t tok0_1 = (int64_t)b * a.cap, tok0_2 = (int64_t)b * a.n_new;
    const double fa = a.freq.rev[lane % H];  // first loader wavefront: tile angle of frequency `lane`
    int rows[ITEMS], ko1[ITEMS], ko2[ITEMS], vo1[ITEMS], vo2[ITEMS];
    // Segment followed by each item's row: index and end, and the row
    // address (K, and V - K) and flags of position 0 in that segment's
    // coordinates, so that a tile only adds u * row stride.
    const int64_t rstride = (int64_t)a.hkv * D * 2;  // bytes per token row
    int sidx[ITEMS], send[ITEMS], fbase[ITEMS];
    uint64_t kaddr0[ITEMS], vdelta[ITEMS];
    auto enter = [&](auto kk, int sg) __attribute__((always_inline)) {
      constexpr int k = decltype(kk)::value;
      sidx[k] = sg;
      send[k] = seg_start[sg + 1];
      const int buf = seg_buf[sg];
      const int64_t sbase = (int64_t)seg_src[sg] - seg_start[sg];  // token = sbase + u
      // Branch-free select of the source (a pointer select here is
      // otherwise lowered to a lookup table in scratch memory).
      const uint64_t m0 = buf == 0 ? ~0ull : 0ull, m1 = buf == 1 ? ~0ull : 0ull;
      const uint64_t m2 = ~(m0 | m1);
      const uint64_t kb = (kb0 & m0) | (kb1 & m1) | (kb2 & m2);
      const uint64_t vb = (vb0 & m0) | (vb1 & m1) | (vb2 & m2);
      const int64_t trow0 = (buf == 0 ? 0 : buf == 1 ? tok0_1 : tok0_2) + sbase;
      kaddr0[k] = kb + static_cast<uint64_t>(trow0 * rstride + (int64_t)g * D * 2);
      vdelta[k] = vb - kb;
      // 4 * (context-buffer row - u) + (new << 1) + rotate
      fbase[k] = (int)((((uint32_t)dst0 + (uint32_t)sbase) << 2) | (buf == 2 ? 2u : 0u) |
                       (buf != 1 ? 1u : 0u));
    };
    float rb_c[ITEMS][8], rb_s[ITEMS][8];  // angles of the row offset
    static_for<ITEMS>([&](auto kk) __attribute__((always_inline)) {
      constexpr int k = decltype(kk)::value;
      const int row = ltid / CP + k * (kKeyTile / ITEMS);
      rows[k] = row;
      ko1[k] = row * Gm::ROW + Gm::k_phys(row, c) * 16;
      ko2[k] = row * Gm::ROW + Gm::k_phys(row, c + CP) * 16;
      vo1[k] = row * Gm::ROW + Gm::v_phys(row, c) * 16;
      vo2[k] = row * Gm::ROW + Gm::v_phys(row, c + CP) * 16;
      enter(kk, upper_index(seg_start, nseg, min(it0 * kKeyTile + row, tend - 1)));
#pragma unroll
      for (int i = 0; i < 8; ++i) rope_cs(row, a.freq.rev[8 * c + i], rb_c[k][i], rb_s[k][i]);
    });
    const bool writer = rg == 0;  // one row group writes the new tokens back
    typedef const __attribute__((address_space(1))) u32x4* gptr;  // global, not flat, loads
    u32x4 kr[P][ITEMS][2], vr[P][ITEMS][2];
    int fl[P][ITEMS];  // per tile and item: 4 * context-buffer row + (new << 1) + rotate
    // Loads of tile t into register set S (tiles past the split repeat its
    // last row, so the loads never need a branch); the first loader
    // wavefront also writes the tile's angles.
    auto issue = [&](auto set, int t) __attribute__((always_inline)) {
      constexpr int S = decltype(set)::value;
      static_for<ITEMS>([&](auto kk) __attribute__((always_inline)) {
        constexpr int k = decltype(kk)::value;
        const int u_real = (it0 + t) * kKeyTile + rows[k];
        const int u = min(u_real, tend - 1);
        while (u >= send[k]) enter(kk, sidx[k] + 1);
        const uint64_t ka = kaddr0[k] + static_cast<uint64_t>((int64_t)u * rstride);
        const gptr kp = reinterpret_cast<gptr>(ka);
        const gptr vp = reinterpret_cast<gptr>(ka + vdelta[k]);
        kr[S][k][0] = kp[c];
        kr[S][k][1] = kp[c + CP];
        vr[S][k][0] = vp[c];
        vr[S][k][1] = vp[c + CP];
        fl[S][k] = u_real < tend ? (int)((uint32_t)fbase[k] + ((uint32_t)u << 2)) : 0;
      });
      if (wave == NWA && lane < H) {
        float cs, sn;
        rope_cs((int64_t)(it0 + t) * kKeyTile + rot, fa, cs, sn);
        rot_a[t & (NT - 1)][lane] = f32x2{cs, sn};
      }
    };
    // Tile t from register set S: rotate K at u0 + row, store K and V into
    // the tile's stages; new tokens also go to the context buffer.
    auto store = [&](auto set, int t) __attribute__((always_inline)) {
      constexpr int S = decltype(set)::value;
      char* sk = kring + (t & 1) * Gm::KBYTES;
      char* sv = vring + (t & (NVS - 1)) * Gm::VBYTES;
      const f32x4* ap = reinterpret_cast<const f32x4*>(&rot_a[t & (NT - 1)][8 * c]);
      f32x4 av[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) av[h] = ap[h];  // the same 8 frequencies for every item
#pragma unroll
      for (int k = 0; k < ITEMS; ++k) {
        u32x4 x1 = kr[S][k][0], x2 = kr[S][k][1];
        const int f = fl[S][k];
        if (f & 1) {
          uint32_t wa[4] = {x1.x, x1.y, x1.z, x1.w}, wb[4] = {x2.x, x2.y, x2.z, x2.w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            float c0, s0, c1, s1;
            angle_add(av[h][0], av[h][1], rb_c[k][2 * h], rb_s[k][2 * h], c0, s0);
            angle_add(av[h][2], av[h][3], rb_c[k][2 * h + 1], rb_s[k][2 * h + 1], c1, s1);
            const float a0 = bf16_lo(wa[h]), a1 = bf16_hi(wa[h]);
            const float b0 = bf16_lo(wb[h]), b1 = bf16_hi(wb[h]);
            wa[h] = pack_bf16x2(rot_lo(a0, b0, c0, s0), rot_lo(a1, b1, c1, s1));
            wb[h] = pack_bf16x2(rot_hi(a0, b0, c0, s0), rot_hi(a1, b1, c1, s1));
          }
          x1 = u32x4{wa[0], wa[1], wa[2], wa[3]};
          x2 = u32x4{wb[0], wb[1], wb[2], wb[3]};
        }
        *reinterpret_cast<u32x4*>(sk + ko1[k]) = x1;
        *reinterpret_cast<u32x4*>(sk + ko2[k]) = x2;
        *reinterpret_cast<u32x4*>(sv + vo1[k]) = vr[S][k][0];
        *reinterpret_cast<u32x4*>(sv + vo2[k]) = vr[S][k][1];
        if ((f & 2) && writer) {
          keep_branch();
          const int64_t d = (((int64_t)b * a.cap + ((uint32_t)f >> 2)) * a.hkv + g) * CR;
          u32x4* ko = static_cast<u32x4*>(a.k_ctx);
          u32x4* vo = static_cast<u32x4*>(a.v_ctx);
          ko[d + c] = x1;
          ko[d + c + CP] = x2;
          vo[d + c] = vr[S][k][0];
          vo[d + c + CP] = vr[S][k][1];
        }
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // Barriers shared with the attention wavefronts: after tiles 0 and 1
    // are stored, after the scores of tile 0, then one per iteration.
    static_for<P>([&](auto t) __attribute__((always_inline)) { issue(t, (int)decltype(t)::value); });
    waitcnt<63, 0>();
    barrier_nofence();  // tile angles of tiles 0 .. P - 1 visible
    store(I0{}, 0);
    store(I1{}, 1);
    issue(I0{}, P);
    waitcnt<63, 0>();
    barrier_nofence();
    barrier_nofence();
    // Iteration i (K of tile i + 1 and V of tile i - 1 in use): request tile
    // i + 1 + P into the register set tile i + 1 left, store tile i + 2.
    // Whole groups of P iterations run without branches around the loads
    // (tiles stored past the split go to stages no product uses).
    auto step = [&](auto t, int i) __attribute__((always_inline)) {
      constexpr int S = decltype(t)::value;
      issue(std::integral_constant<int, (S + 1) % P>{}, i + 1 + P);
      store(std::integral_constant<int, (S + 2) % P>{}, i + 2);
      waitcnt<63, 0>();
      barrier_nofence();
    };
    int l0 = 0;
    for (; l0 + P <= cnt; l0 += P)
      static_for<P>([&](auto t) __attribute__((always_inline)) { step(t, l0 + (int)decltype(t)::value); });
    static_for<P>([&](auto t) __attribute__((always_inline)) {
      if (l0 + (int)decltype(t)::value < cnt) step(t, l0 + (int)decltype(t)::value);
    });
    if constexpr (KW == 2) barrier_nofence();  // (the key halves' merge)
    return;
  }

  // Attention wavefront: rows rho of the group; Q rotated at its position.
  bf16x8 qb[KS];
  {
    u32x4 raw[KS];
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.q) + (((int64_t)b * a.n_new + r) * a.hq + head) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) raw[ks] = live ? qp[2 * ks + hh] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks)
      rope_rotate_chunk(raw[ks], raw[ks + KS / 2], (int64_t)qpos + rot, a.freq, 16 * ks + 8 * hh,
                        a.q_scale);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
  }
  int koff[KS], vbase[OT];
  lane_offsets<D>(lane, koff, vbase);
  const auto kst = [&](int i) { return kring + (i & 1) * Gm::KBYTES; };
  const auto vst = [&](int i) { return vring + (i & (NVS - 1)) * Gm::VBYTES; };
  // Only tiles reaching past the first query token can hide keys from a row
  // (causal among the new tokens; rows past the context are all masked).
  const auto mask_of = [&](int i) { return (it0 + i) * kKeyTile + kKeyTile - 1 > pos0; };
  const auto vis_of = [&](int i) {
    const int lim = qpos - (it0 + i) * kKeyTile;
    return [=](int kr) { return kr <= lim; };
  };
  std::conditional_t<KW == 1, Flash<D>, FlashHalf<D>> fl;
  if constexpr (KW == 1) fl.init();
  else fl.init(way);
  if (cnt == 0) {
    barrier_nofence();
  } else if constexpr (KW == 1) {
    barrier_nofence();  // (the loaders' tile angles)
    barrier_nofence();  // tiles 0 and 1 stored
    f32x16 s0, s1, n0, n1;
    bf16x8 pr[4];
    fl.scores(kst(0), koff, qb, s0, s1);
    waitcnt<0, 0>();
    barrier_nofence();
    fl.template pv_head<false>(vst(0), vbase, pr, s0, s1, mask_of(0), vis_of(0));
    fl.exp_next(kst(1), koff, qb, s0, s1, pr, n0, n1);
    // Two iterations per trip so the score registers alternate.
    for (int i = 1; i < cnt; i += 2) {
      waitcnt<0, 0>();
      barrier_nofence();
      fl.template pv_head<true>(vst(i - 1), vbase, pr, n0, n1, mask_of(i), vis_of(i));
      fl.exp_next(kst(i + 1), koff, qb, n0, n1, pr, s0, s1);
      if (i + 1 >= cnt) break;
      waitcnt<0, 0>();
      barrier_nofence();
      fl.template pv_head<true>(vst(i), vbase, pr, s0, s1, mask_of(i + 1), vis_of(i + 1));
      fl.exp_next(kst(i + 2), koff, qb, s0, s1, pr, n0, n1);
    }
    waitcnt<0, 0>();
    barrier_nofence();
    fl.pv(vst(cnt - 1), vbase, pr);
  } else {
    // The same schedule on this wavefront's half of every tile.
    barrier_nofence();
    barrier_nofence();
    f32x16 s, n;
    bf16x8 pr[2];
    fl.scores(kst(0), koff, qb, s);
    waitcnt<0, 0>();
    barrier_nofence();
    fl.template pv_head<false>(vst(0), vbase, pr, s, mask_of(0), vis_of(0));
    fl.exp_next(kst(1), koff, qb, s, pr, n);
    for (int i = 1; i < cnt; i += 2) {
      waitcnt<0, 0>();
      barrier_nofence();
      fl.template pv_head<true>(vst(i - 1), vbase, pr, n, mask_of(i), vis_of(i));
      fl.exp_next(kst(i + 1), koff, qb, n, pr, s);
      if (i + 1 >= cnt) break;
      waitcnt<0, 0>();
      barrier_nofence();
      fl.template pv_head<true>(vst(i), vbase, pr, s, mask_of(i + 1), vis_of(i + 1));
      fl.exp_next(kst(i + 2), koff, qb, s, pr, n);
    }
    waitcnt<0, 0>();
    barrier_nofence();
    fl.pv(vst(cnt - 1), vbase, pr);
  }
  if constexpr (KW == 2) {
    // Merge the second key half into the first, lane by lane (the same row
    // and head dims), through the K ring and the angle table: both are idle
    // once the last barrier has passed.
    float* xo = reinterpret_cast<float*>(kring) + (wave % RW) * (16 * OT * 64) + lane;
    float* xm = reinterpret_cast<float*>(&rot_a[0][0]) + (wave % RW) * (3 * 64) + lane;
    static_assert(RW * 16 * OT * 64 * 4 <= 2 * Gm::KBYTES && RW * 3 * 64 * 4 <= sizeof(rot_a),
                  "merge buffers fit the idle LDS");
    if (way == 1) {
#pragma unroll
      for (int t = 0; t < OT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) xo[(t * 16 + i) * 64] = fl.o[t][i];
      xm[0] = fl.m;
      xm[64] = fl.l;
      xm[128] = fl.have ? 1.0f : 0.0f;
    }
    __syncthreads();
    if (way == 1) return;
    const bool h0 = fl.have, h1 = xm[128] != 0.0f;
    const float m1 = xm[64 * 0], l1 = xm[64];
    const float mm = h0 && h1 ? __builtin_fmaxf(fl.m, m1) : (h0 ? fl.m : m1);
    const float a0 = h0 ? __builtin_amdgcn_exp2f(fl.m - mm) : 0.0f;
    const float a1 = h1 ? __builtin_amdgcn_exp2f(m1 - mm) : 0.0f;
#pragma unroll
    for (int t = 0; t < OT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) fl.o[t][i] = fl.o[t][i] * a0 + xo[(t * 16 + i) * 64] * a1;
    fl.m = mm;
    fl.l = fl.l * a0 + l1 * a1;
    fl.have = h0 || h1;
  }
  const float lsum = fl.total();
  if (!live) return;
  if (a.part_o == nullptr) {
    const float inv = 1.0f / lsum;
    uint16_t* op = static_cast<uint16_t*>(a.o) + (((int64_t)b * a.n_new + r) * a.hq + head) * D;
#pragma unroll
    for (int m = 0; m < OT; ++m)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = m * 32 + q4 * 8 + hh * 4;
        const u32x2 w = {pack_bf16x2(fl.o[m][4 * q4 + 0] * inv, fl.o[m][4 * q4 + 1] * inv),
                         pack_bf16x2(fl.o[m][4 * q4 + 2] * inv, fl.o[m][4 * q4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d) = w;
      }
  } else {
    const int64_t prow = (((int64_t)b * a.hkv + g) * a.n_split + split) * a.rows + rho;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int m = 0; m < OT; ++m)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = m * 32 + q4 * 8 + hh * 4;
        *reinterpret_cast<f32x4*>(po + d) = f32x4{fl.o[m][4 * q4 + 0], fl.o[m][4 * q4 + 1],
                                                  fl.o[m][4 * q4 + 2], fl.o[m][4 * q4 + 3]};
      }
    if (hh == 0) {
      a.part_ml[prow * 2 + 0] = fl.m;
      a.part_ml[prow * 2 + 1] = lsum;
    }
  }
}

// ---------------------------------------------------------------------------
// Merge split partials: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over
// the splits that saw a key (l_s > 0).  One thread per 4 head dims; the
// partials of 8 splits are loaded at once and merged online batch by batch.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  constexpr int TPR = D / 4, RPB = 256 / TPR, SB = 8;
  const int rho = blockIdx.x * RPB + threadIdx.x / TPR, d4 = threadIdx.x % TPR;
  const int g = blockIdx.y, b = blockIdx.z;
  if (rho >= a.rows) return;
  const int G = a.hq / a.hkv;
  const int r = rho / G, head = g * G + rho % G;
  const int64_t base = ((int64_t)b * a.hkv + g) * a.n_split;
  float M = kNegInf, L = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < a.n_split; s0 += SB) {
    float m[SB], l[SB];
    f32x4 o[SB];
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const bool in = s0 + i < a.n_split;
      const int64_t prow = (base + s0 + i) * a.rows + rho;
      // (m, l) as one float pair.  (__builtin_bit_cast of a vector element
      // compiles to element 0 here, so no bit casts of lanes.)
      const f32x2 ml = in ? *reinterpret_cast<const f32x2*>(a.part_ml + prow * 2) : f32x2{0.0f, 0.0f};
      m[i] = ml[0];
      l[i] = ml[1];
      o[i] = in ? *reinterpret_cast<const f32x4*>(a.part_o + prow * D + 4 * d4) : f32x4{};
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < SB; ++i) Mb = l[i] > 0.0f ? fmaxf(Mb, m[i]) : Mb;
    const float sc = L > 0.0f ? __builtin_amdgcn_exp2f(M - Mb) : 0.0f;
    L *= sc;
    acc *= sc;
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const float w = l[i] > 0.0f ? __builtin_amdgcn_exp2f(m[i] - Mb) : 0.0f;
      L += w * l[i];
      acc += w * o[i];
    }
    M = Mb;
  }
  const float inv = 1.0f / L;
  const int64_t od = (((int64_t)b * a.n_new + r) * a.hq + head) * D + 4 * d4;
  if constexpr (BF16) {
    const u32x2 w = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.o) + od) = w;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + od) = acc * inv;
  }
}

// ---------------------------------------------------------------------------
// Merge of the shared-block schedule: per packed row, the n_ids block
// partials (O / l in bf16, lambda = m + log2 l) and the n_split partials of
// the tail / new-token pass (unnormalised O, m, l):
//   O = (sum_i 2^(lambda_i - M) O_i + sum_s 2^(m_s - M) O_s)
//       / (sum_i 2^(lambda_i - M) + sum_s 2^(m_s - M) l_s),
// M the largest exponent among them.  16 threads per row, 8 head dims each;
// the block partials are read once, 8 at a time, past the caches (8 in
// flight instead of 4: 163 -> 143 us on the 32-layer pool batch).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_merge(MergeArgs a) {
  constexpr int TPR = D / 8, RPB = 256 / TPR, U = 8;
  const int rho = blockIdx.x * RPB + threadIdx.x / TPR, c = threadIdx.x % TPR;
  const int g = blockIdx.y, b = blockIdx.z;
  if (rho >= a.rq) return;
  const int G = a.hq / a.hkv;
  const int r = rho / G, head = g * G + rho % G;
  const int64_t pb = ((int64_t)b * a.hkv + g) * a.n_ids;      // block partial rows
  const int64_t tb = ((int64_t)b * a.hkv + g) * a.n_split;    // tail partial rows
  // One pass, online: the running maximum M only moves up; when it does, the
  // sums so far are rescaled.  U partials are loaded before they are used.
  float M = kNegInf, L = 0.0f, acc[8] = {};
  auto add = [&](float lam, float wl, const float (&x)[8]) {
    if (lam > M) {
      const float sc = __builtin_amdgcn_exp2f(M - lam);
      L *= sc;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] *= sc;
      M = lam;
    }
    const float w = __builtin_amdgcn_exp2f(lam - M);
    L = __builtin_fmaf(w, wl, L);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_fmaf(w, x[k], acc[k]);
  };
  for (int i0 = 0; i0 < a.n_ids; i0 += U) {
    float lam[U];
    u32x4 xs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(i0 + u, a.n_ids - 1);
      const int64_t row = (pb + i) * a.rq + rho;
      lam[u] = i0 + u < a.n_ids ? a.part_lam[row] : kNegInf;
      xs[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.part_o + row * D + 8 * c));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u >= a.n_ids) break;
      const uint32_t w4[4] = {xs[u].x, xs[u].y, xs[u].z, xs[u].w};
      float x[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = bf16_lo(w4[k]);
        x[2 * k + 1] = bf16_hi(w4[k]);
      }
      add(lam[u], 1.0f, x);  // O / l with weight 2^(m + log2 l)
    }
  }
  for (int s = 0; s < a.n_split; ++s) {
    const int64_t row = (tb + s) * a.rq + rho;
    const f32x2 ml = *reinterpret_cast<const f32x2*>(a.tail_ml + row * 2);
    if (!(ml[1] > 0.0f)) continue;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(a.tail_o + row * D + 8 * c);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(a.tail_o + row * D + 8 * c + 4);
    const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    add(ml[0], ml[1], x);  // unnormalised O with weight 2^m, sum l
  }
  const float inv = 1.0f / L;
  const u32x4 out = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                     pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o) +
                            (((int64_t)b * a.n_new + r) * a.hq + head) * D + 8 * c) = out;
}

// ---------------------------------------------------------------------------
// float32 query rows: one wavefront per (batch, token, head), one key per lane.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_query_f32(QueryArgs a) {
  constexpr int H = D / 2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.z;
  const int idx = blockIdx.x * 4 + wave;  // (token, head)
  if (idx >= a.n_new * a.hq) return;      // no block-level synchronisation below
  const int r = idx / a.hq, head = idx % a.hq;
  const int g = head / (a.hq / a.hkv);
  const int32_t* tab = seg_block(a);
  const int qpos = tab[a.seg.o_pos0 + b] + r;
  const int rot = a.seg.o_rot >= 0 ? tab[a.seg.o_rot + b] : 0;
  const float* q = static_cast<const float*>(a.q) + (((int64_t)b * a.n_new + r) * a.hq + head) * D;
  float qr[D];
#pragma unroll
  for (int i = 0; i < H; ++i) {
    float c, s;
    rope_cs((int64_t)qpos + rot, a.freq.rev[i], c, s);
    qr[i] = rot_lo(q[i], q[i + H], c, s) * a.q_scale;
    qr[i + H] = rot_hi(q[i], q[i + H], c, s) * a.q_scale;
  }
  const int nseg = tab[a.seg.o_nseg + b];
  const int32_t* sst = tab + a.seg.o_start + b * a.seg.stride;
  const int32_t* ssrc = tab + a.seg.o_src + b * a.seg.stride;
  const int32_t* sbuf = tab + a.seg.o_buf + b * a.seg.stride;
  const float* kpool = static_cast<const float*>(a.k_pool);
  const float* vpool = static_cast<const float*>(a.v_pool);
  const float* kctx = static_cast<const float*>(a.k_ctx);
  const float* vctx = static_cast<const float*>(a.v_ctx);
  float m_run = kMaxFloor, l_run = 0.0f, acc0 = 0.0f, acc1 = 0.0f;
  const int end = qpos + 1;
  for (int base = 0; base < end; base += 64) {
    const int u = base + lane;
    float sc = kNegInf;
    const float* vrow = nullptr;
    if (u < end) {
      const int s = upper_index(sst, nseg, u);
      const int64_t tok = ssrc[s] + (u - sst[s]);
      const float* krow;
      const bool rot_row = sbuf[s] == 0;
      if (rot_row) {
        krow = kpool + (tok * a.hkv + g) * D;
        vrow = vpool + (tok * a.hkv + g) * D;
      } else {
        const int64_t row = (((int64_t)b * a.cap + tok) * a.hkv + g) * D;
        krow = kctx + row;
        vrow = vctx + row;
      }
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        float x1 = krow[i], x2 = krow[i + H];
        if (rot_row) {
          float c, sn;
          rope_cs((int64_t)u + rot, a.freq.rev[i], c, sn);
          const float y1 = rot_lo(x1, x2, c, sn), y2 = rot_hi(x1, x2, c, sn);
          x1 = y1;
          x2 = y2;
        }
        dot += qr[i] * x1 + qr[i + H] * x2;
      }
      sc = dot;
    }
    float mx = sc;
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float p = __builtin_amdgcn_exp2f(sc - m_new);
    float ps = p;
    for (int o = 32; o > 0; o >>= 1) ps += __shfl_xor(ps, o);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    acc0 *= alpha;
    acc1 *= alpha;
    const int n = min(64, end - base);
    const uint64_t vaddr = reinterpret_cast<uint64_t>(vrow);
    for (int kk = 0; kk < n; ++kk) {
      const float pk = __shfl(p, kk);
      const uint64_t va = (uint64_t)__shfl((long long)vaddr, kk);
      const float* vr = reinterpret_cast<const float*>(va);
      if (lane < D) acc0 += pk * vr[lane];
      if (lane + 64 < D) acc1 += pk * vr[lane + 64];
    }
  }
  float* o = static_cast<float*>(a.o) + (((int64_t)b * a.n_new + r) * a.hq + head) * D;
  if (lane < D) o[lane] = acc0 / l_run;
  if (lane + 64 < D) o[lane + 64] = acc1 / l_run;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_gather(const GatherArgs& a, int batch, int head_dim, int dtype,
                         hipStream_t stream) {
  if (dtype == 1) {
    const int64_t units = (int64_t)a.max_len * (head_dim / 2);
    const dim3 grid((unsigned)((units + 255) / 256), batch);
    if (head_dim == 128) hipLaunchKernelGGL(k_gather_f32<128>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(k_gather_f32<64>, grid, dim3(256), 0, stream, a);
  } else {
    const int tok = 256 / (head_dim / 16);
    const dim3 grid((a.max_len + tok - 1) / tok, batch);
    if (head_dim == 128) hipLaunchKernelGGL(k_gather_bf16<128>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(k_gather_bf16<64>, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_new_kv(const NewKVArgs& a, int batch, int head_dim, int dtype,
                         hipStream_t stream) {
  const dim3 grid(a.n_new, batch);
  if (dtype != 1) return hipErrorInvalidValue;  // bf16 appends inside k_query_bf16
  if (head_dim == 128) hipLaunchKernelGGL(k_new_kv_f32<128>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(k_new_kv_f32<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D>
static void launch_query_d(const QueryArgs& a, dim3 grid, hipStream_t stream) {
  const int w = a.n_split * a.hkv * grid.z;
  grid = dim3(a.row_groups > 1 ? (w + 7) / 8 * 8 * a.row_groups : w);
  constexpr int L = 64 * kQueryLoaders;
  if (a.key_ways == 2) {
    if (a.row_waves == 1) hipLaunchKernelGGL((k_query_bf16<D, 1, 2>), grid, dim3(L + 128), 0, stream, a);
    else hipLaunchKernelGGL((k_query_bf16<D, 2, 2>), grid, dim3(L + 256), 0, stream, a);
    return;
  }
  switch (a.row_waves) {
    case 1: hipLaunchKernelGGL((k_query_bf16<D, 1, 1>), grid, dim3(L + 64), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((k_query_bf16<D, 2, 1>), grid, dim3(L + 128), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((k_query_bf16<D, 3, 1>), grid, dim3(L + 192), 0, stream, a); break;
    default: hipLaunchKernelGGL((k_query_bf16<D, 4, 1>), grid, dim3(L + 256), 0, stream, a); break;
  }
}

hipError_t launch_query(const QueryArgs& a, int batch, int head_dim, int dtype,
                        hipStream_t stream) {
  if (dtype == 1) {
    const dim3 grid((a.n_new * a.hq + 3) / 4, 1, batch);
    if (head_dim == 128) hipLaunchKernelGGL(k_query_f32<128>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(k_query_f32<64>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (a.row_waves < 1 || a.row_waves > 4 || a.key_ways < 1 || a.key_ways > 2 ||
      (a.key_ways == 2 && (a.row_waves > 2 || a.row_groups != 1)))
    return hipErrorInvalidValue;
  const dim3 grid(a.n_split, a.hkv * a.row_groups, batch);
  if (head_dim == 128) launch_query_d<128>(a, grid, stream);
  else launch_query_d<64>(a, grid, stream);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, int batch, int head_dim, hipStream_t stream) {
  const int rpb = 256 / (head_dim / 8);
  const dim3 grid((a.rq + rpb - 1) / rpb, a.hkv, batch);
  if (head_dim == 128) hipLaunchKernelGGL(k_merge<128>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(k_merge<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int batch, int head_dim, int dtype,
                          hipStream_t stream) {
  const int rpb = 256 / (head_dim / 4);
  const dim3 grid((a.rows + rpb - 1) / rpb, a.hkv, batch);
  if (head_dim == 128) {
    if (dtype == 1) hipLaunchKernelGGL((k_combine<128, false>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((k_combine<128, true>), grid, dim3(256), 0, stream, a);
  } else {
    if (dtype == 1) hipLaunchKernelGGL((k_combine<64, false>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((k_combine<64, true>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dbsa
