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
//   k_query_bf16<D, RWW, KSPL>     split-K flash attention of the packed
//                                  (token, head-in-group) rows of one KV head
//                                  over a segment list (pool blocks and new
//                                  tokens are rotated while staged; new tokens
//                                  are also appended to the context buffer).
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
  const int32_t* st = a.start + (int64_t)b * (a.n_ids + 1);
  if (u >= st[a.n_ids]) return;
  const int i = upper_index(st, a.n_ids, u);
  const int64_t src_tok = a.src[(int64_t)b * a.n_ids + i] + (u - st[i]);
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
  for (int g = 0; g < a.hkv; ++g) {
    const int64_t src = (src_tok * a.hkv + g) * CR;
    const int64_t dst = (((int64_t)b * a.cap + u) * a.hkv + g) * CR;
    u32x4 k1 = kp[src + c], k2 = kp[src + c + CP];
    const u32x4 v1 = vp[src + c], v2 = vp[src + c + CP];
    rotate_chunk(k1, k2, cs, sn);
    ko[dst + c] = k1;
    ko[dst + c + CP] = k2;
    vo[dst + c] = v1;
    vo[dst + c + CP] = v2;
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_gather_f32(GatherArgs a) {
  constexpr int H = D / 2;
  const int b = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (token, pair)
  const int u = (int)(idx / H), i = (int)(idx % H);
  const int32_t* st = a.start + (int64_t)b * (a.n_ids + 1);
  if (u >= st[a.n_ids]) return;
  const int s = upper_index(st, a.n_ids, u);
  const int64_t src_tok = a.src[(int64_t)b * a.n_ids + s] + (u - st[s]);
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
  if (a.n_inline)
    return reinterpret_cast<const int32_t*>((const char*)__builtin_amdgcn_kernarg_segment_ptr() +
                                            offsetof(QueryArgs, inl));
  return a.meta;
}

// ---------------------------------------------------------------------------
// Query attention, bf16 MFMA, split-K over the context.
//
// Workgroup = RWW x KSPL wavefronts over 16 RWW packed rows (row = token * G +
// head in group) of one KV head and one key split: 16 rows per wavefront on
// v_mfma_f32_16x16x32_bf16 (see Flash16), and with KSPL = 2 the two halves of
// every 64-key tile go to two wavefronts with their own softmax state, merged
// through LDS at the end (twice the wavefronts per SIMD to hide the latency
// of one tile's dependent MFMA / shuffle / LDS chain).  Each tile is staged by
// direct global->LDS loads through a ring of 4 stages, three tiles ahead:
// per tile, wavefront 0 first resolves every row's source (segment lookup in
// LDS) into a small address table, then all wavefronts issue the loads.
// Rows from the pool or from the new tokens arrive unrotated and are rotated
// in LDS at their virtual position before the tile is used; the first row
// group also writes the new tokens' rotated K and their V to the context
// buffer (each new token lies in exactly one tile of one split).
// ---------------------------------------------------------------------------
template <int D, int RWW, int KSPL>
__global__ __launch_bounds__(64 * (RWW * KSPL + kQueryLoaders)) void k_query_bf16(QueryArgs a) {
  using Gm = TileGeom<D>;
  // RWW x KSPL attention wavefronts, then NL loader wavefronts that plan,
  // load and rotate the tiles ahead of the attention.
  constexpr int NWA = RWW * KSPL, NL = kQueryLoaders, NW = NWA + NL, KH = kKeyTile / KSPL;
  constexpr int KS = D / 32, OT = D / 16, CP = D / 16, CR = D / 8;
  constexpr int RW = 16;  // rows per wavefront
  constexpr int NST = 4;
  constexpr int INSTR = Gm::TU4 / 64;  // 1 KiB loads per matrix per tile
  constexpr int LPW = 2 * INSTR / NL;  // loads per loader wave per tile
  static_assert((2 * INSTR) % NL == 0, "loads must split evenly over the loader waves");
  static_assert((64 * NL) % CP == 0, "each loader thread keeps one chunk pair");
  constexpr uint8_t kRot = 1, kNew = 2;
  constexpr int H = D / 2;
  // Rotation work items (row, chunk pair) per thread; each thread keeps the
  // angles of its fixed row offsets in registers when it has at most two.
  constexpr int IPT = (kKeyTile * CP + 64 * NL - 1) / (64 * NL);
  constexpr bool KEEP_B = IPT <= 2;
  __shared__ __align__(16) char lds[NST * Gm::STAGE];
  __shared__ __align__(16) f32x2 rot_a[NST][kMaxHalf];  // cos / sin of w_i * u0 per stage
  __shared__ int32_t seg_start[kMaxSegments + 1], seg_src[kMaxSegments], seg_buf[kMaxSegments];
  __shared__ uint64_t row_k[NST][kKeyTile], row_v[NST][kKeyTile];
  __shared__ int32_t row_dst[NST][kKeyTile];
  __shared__ uint8_t row_flag[NST][kKeyTile];
  __shared__ uint8_t tile_flag[2 * NST];  // indexed by tile % 8 (see plan)

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool loader = wave >= NWA;
  const int ltid = tid - 64 * NWA;  // thread index among the loaders
  const int rw = wave % RWW, kh = loader ? 0 : wave / RWW;  // row wavefront, key half
  const int q16 = (lane >> 4) & 3, r16 = lane & 15;
  const int split = blockIdx.x;
  const int g = blockIdx.y % a.hkv, rg = blockIdx.y / a.hkv, b = blockIdx.z;
  const int G = a.hq / a.hkv;
  const int wrow0 = rg * (RW * RWW) + rw * RW;
  const bool wave_live = !loader && wrow0 < a.rows;
  const int rho = wrow0 + r16;
  const bool live = !loader && rho < a.rows;
  const int r = live ? rho / G : 0;
  const int head = g * G + (live ? rho - (rho / G) * G : 0);
  const int32_t* tab = seg_block(a);
  const int pos0 = tab[a.seg.o_pos0 + b];
  const int dst0 = tab[a.seg.o_dst + b];
  const int qpos = pos0 + r;

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

  bf16x8 qb[KS];
  {
    u32x4 raw[KS];
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.q) + (((int64_t)b * a.n_new + r) * a.hq + head) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) raw[ks] = live ? qp[4 * ks + q16] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks)
      rope_rotate_chunk(raw[ks], raw[ks + KS / 2], qpos, a.freq, 32 * ks + 8 * q16, a.q_scale);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
  }
  __syncthreads();  // segment table visible; Q loads retired

  const int T = seg_start[nseg];
  const int n_tiles = (T + kKeyTile - 1) / kKeyTile;
  const int it0 = split * a.tiles_per_split;
  const int cnt = max(0, min(it0 + a.tiles_per_split, n_tiles) - it0);

  // Per-source base addresses (bf16 elements -> bytes) and row strides.
  const uint64_t kb0 = reinterpret_cast<uint64_t>(a.k_pool), vb0 = reinterpret_cast<uint64_t>(a.v_pool);
  const uint64_t kb1 = reinterpret_cast<uint64_t>(a.k_ctx), vb1 = reinterpret_cast<uint64_t>(a.v_ctx);
  const uint64_t kb2 = reinterpret_cast<uint64_t>(a.k_new), vb2 = reinterpret_cast<uint64_t>(a.v_new);
  const int64_t tok0_1 = (int64_t)b * a.cap, tok0_2 = (int64_t)b * a.n_new;

  const double fa = a.freq.rev[lane % H];  // loader wavefront 0: tile angle of frequency `lane`
  // Row sources of local tile li (wavefront 0, one row per lane).  The tile
  // flags are double-buffered over 8 tiles: a slow wavefront may still read
  // tile li-1's flag while tile li+3's is being written.
  // Row sources of local tile li (loader wavefront 0, one row per lane).
  // The tile flags are double-buffered over 8 tiles: a slow wavefront may
  // still read tile li-1's flag while tile li+3's is being written.  The
  // tiles are planned in order, so each lane follows its row's segment
  // forward from the previous tile instead of searching for it.
  int s_cur = -1;
  auto plan = [&](int li) {
    if (wave == NWA) {
      const int u_real = (it0 + li) * kKeyTile + lane;
      const bool real = u_real < T;
      const int u = min(u_real, T - 1);  // rows past the context repeat the last row (masked)
      if (s_cur < 0) {
        s_cur = upper_index(seg_start, nseg, u);
      } else {
        while (s_cur + 1 < nseg && seg_start[s_cur + 1] <= u) ++s_cur;
      }
      const int s = s_cur;
      const int64_t tok = seg_src[s] + (u - seg_start[s]);
      const int buf = seg_buf[s];
      // Branch-free select of the source (a pointer select here is otherwise
      // lowered to a lookup table in scratch memory).
      const uint64_t m0 = buf == 0 ? ~0ull : 0ull, m1 = buf == 1 ? ~0ull : 0ull;
      const uint64_t m2 = ~(m0 | m1);
      const int64_t trow = (buf == 0 ? 0 : buf == 1 ? tok0_1 : tok0_2) + tok;
      const uint64_t off = 2ull * static_cast<uint64_t>((trow * a.hkv + g) * D);
      const int slot = li % NST;
      row_k[slot][lane] = ((kb0 & m0) | (kb1 & m1) | (kb2 & m2)) + off;
      row_v[slot][lane] = ((vb0 & m0) | (vb1 & m1) | (vb2 & m2)) + off;
      const uint8_t f = real ? (buf != 1 ? kRot : 0) | (buf == 2 ? kNew : 0) : 0;
      row_flag[slot][lane] = f;
      row_dst[slot][lane] = dst0 + (int)tok;
      if (lane < H) {
        float c, sn;
        rope_cs((int64_t)(it0 + li) * kKeyTile, fa, c, sn);
        rot_a[slot][lane] = f32x2{c, sn};
      }
      const uint64_t any_rot = __builtin_amdgcn_ballot_w64(f & kRot);
      const uint64_t any_new = __builtin_amdgcn_ballot_w64(f & kNew);
      if (lane == 0) tile_flag[li & (2 * NST - 1)] = (any_rot ? kRot : 0) | (any_new ? kNew : 0);
    }
  };
  // Loads of local tile li into its stage (all waves).
  auto load = [&](int li) {
    const int slot = li % NST;
    char* st = lds + slot * Gm::STAGE;
    const uint16_t* src[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int i = (wave - NWA) + j * NL;  // 0 .. 2*INSTR-1
      const int mat = i / INSTR, ii = i - mat * INSTR;
      const int off = ii * 1024 + lane * 16;
      const int row = off / Gm::ROW, p = (off % Gm::ROW) >> 4;
      const int c = mat == 0 ? Gm::k_phys(row, p) : Gm::v_phys(row, p);
      src[j] = reinterpret_cast<const uint16_t*>(mat == 0 ? row_k[slot][row] : row_v[slot][row]) +
               c * 8;
    }
    // All table reads first, then the loads back to back.
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int i = (wave - NWA) + j * NL;
      const int mat = i / INSTR, ii = i - mat * INSTR;
      dma16(src[j], st + mat * Gm::KBYTES + ii * 1024);
    }
  };

  Flash16<D> fl;
  fl.init();
  int koff[KS], vbase[OT];
  lane_offsets16<D>(lane, kh * KH, koff, vbase);
  // The in-LDS rotation handles chunk pair tid % CP of its rows: its 8
  // frequencies, and the angles of its fixed row offsets, live in registers
  // (no per-lane kernel-argument loads in the loop, whose vector-memory
  // counter is reserved for the tile loads).
  double fr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) fr[i] = a.freq.rev[8 * (ltid % CP) + i];
  float rb_c[KEEP_B ? IPT : 1][8], rb_s[KEEP_B ? IPT : 1][8];
  if constexpr (KEEP_B) {
#pragma unroll
    for (int k = 0; k < IPT; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rope_cs(((ltid + k * 64 * NL) / CP) & (kKeyTile - 1), fr[i], rb_c[k][i], rb_s[k][i]);
  }
  const bool writer = rg == 0;  // one row group writes the new tokens back

  // RoPE at the virtual position for pool rows and new tokens of local tile
  // li, in LDS; the new tokens' rotated K (from registers) and V go to the
  // context buffer.  Runs one tile ahead of the attention (see the loop).
  auto rotate = [&](int li) {
    const int slot = li % NST;
    if (!(tile_flag[li & (2 * NST - 1)] & kRot)) return;
    char* st = lds + slot * Gm::STAGE;
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int uidx = ltid + k * 64 * NL;
      if (uidx >= kKeyTile * CP) break;
      const int row = uidx / CP, c = uidx - row * CP;
      const uint8_t f = row_flag[slot][row];
      if (!(f & kRot)) continue;
      u32x4* k1 = reinterpret_cast<u32x4*>(st + row * Gm::ROW + Gm::k_phys(row, c) * 16);
      u32x4* k2 = reinterpret_cast<u32x4*>(st + row * Gm::ROW + Gm::k_phys(row, c + CP) * 16);
      u32x4 x1 = *k1, x2 = *k2;
      // angle(u0 + row) = angle(u0) (tile table) + angle(row) (registers).
      float cs[8], sn[8];
      const f32x4* ap = reinterpret_cast<const f32x4*>(&rot_a[slot][8 * c]);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const f32x4 av = ap[h];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int i = 2 * h + e;
          float cb, sb;
          if constexpr (KEEP_B) {
            cb = rb_c[k][i];
            sb = rb_s[k][i];
          } else {
            rope_cs(row, fr[i], cb, sb);
          }
          angle_add(av[2 * e], av[2 * e + 1], cb, sb, cs[i], sn[i]);
        }
      }
      rotate_chunk(x1, x2, cs, sn);
      *k1 = x1;
      *k2 = x2;
      if ((f & kNew) && writer) {
        const int64_t d = (((int64_t)b * a.cap + row_dst[slot][row]) * a.hkv + g) * CR;
        u32x4* ko = static_cast<u32x4*>(a.k_ctx);
        u32x4* vo = static_cast<u32x4*>(a.v_ctx);
        const char* vs = st + Gm::KBYTES + row * Gm::ROW;
        ko[d + c] = x1;
        ko[d + c + CP] = x2;
        vo[d + c] = *reinterpret_cast<const u32x4*>(vs + Gm::v_phys(row, c) * 16);
        vo[d + c + CP] = *reinterpret_cast<const u32x4*>(vs + Gm::v_phys(row, c + CP) * 16);
      }
    }
  };

  // Loader and attention wavefronts run separate loops (so their loop state
  // can share registers) that meet at the same barriers: one per tile, after
  // which the loaders request tile li+3 into the stage tile li-1 left and
  // rotate tile li+1 while the attention wavefronts use tile li.
  if (loader) {
    for (int li = 0; li < NST - 1 && li < cnt; ++li) plan(li);
    waitcnt<0, 0>();
    barrier_nofence();
    for (int li = 0; li < NST - 1 && li < cnt; ++li) load(li);
    if (cnt > 0) {
      wait_vm<true>(LPW * min(NST - 2, cnt - 1));  // tile 0 landed
      barrier_nofence();
      rotate(0);
    }
    for (int li = 0; li < cnt; ++li) {
      if (li + NST - 1 < cnt) plan(li + NST - 1);
      // Tile li+1 landed (only tile li+2's loads may fly; the rotation's LDS
      // writes are done too); the barrier publishes tile li's rotation and
      // the new address table, and frees tile li-1's stage for the refill.
      wait_vm<true>(LPW * max(0, min(NST - 3, cnt - 2 - li)));
      barrier_nofence();
      if (li + NST - 1 < cnt) load(li + NST - 1);
      if (li + 1 < cnt) rotate(li + 1);
    }
    if constexpr (KSPL == 2) {  // the attention wavefronts' merge below
      __syncthreads();
      __syncthreads();
    }
    return;
  }
  waitcnt<0, 0>();
  barrier_nofence();
  if (cnt > 0) barrier_nofence();
  for (int li = 0; li < cnt; ++li) {
    waitcnt<0, 0>();  // this wavefront's reads of tile li-1 are done
    barrier_nofence();
    if (wave_live) {
      const int k0 = (it0 + li) * kKeyTile + kh * KH;
      const int lim = qpos - k0;  // keys kr <= lim are visible (causal over new tokens)
      fl.template tile<KH>(lds + (li % NST) * Gm::STAGE, koff, vbase, qb, k0 + KH - 1 > pos0,
                           [=](int kr) { return kr <= lim; });
    }
  }
  (void)CR;

  float lsum = fl.total();
  if constexpr (KSPL == 2) {
    // Second key half -> LDS (the ring is free once every wavefront is past
    // its last tile); the first half merges: weights 2^(m_h - M) over halves
    // that saw a key.
    __syncthreads();
    float* xo = reinterpret_cast<float*>(lds) + rw * (OT * 256 + 32);
    if (kh == 1) {
#pragma unroll
      for (int t = 0; t < OT; ++t) *reinterpret_cast<f32x4*>(xo + (t * 64 + lane) * 4) = fl.o[t];
      if (q16 == 0) {
        xo[OT * 256 + 2 * r16] = fl.m;
        xo[OT * 256 + 2 * r16 + 1] = lsum;
      }
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = xo[OT * 256 + 2 * r16], l1 = xo[OT * 256 + 2 * r16 + 1];
    const bool h0 = lsum > 0.0f, h1 = l1 > 0.0f;
    const float M = h0 && h1 ? fmaxf(fl.m, m1) : h1 ? m1 : fl.m;
    const float w0 = h0 ? __builtin_amdgcn_exp2f(fl.m - M) : 0.0f;
    const float w1 = h1 ? __builtin_amdgcn_exp2f(m1 - M) : 0.0f;
#pragma unroll
    for (int t = 0; t < OT; ++t) {
      const f32x4 o1 = *reinterpret_cast<const f32x4*>(xo + (t * 64 + lane) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) fl.o[t][i] = w0 * fl.o[t][i] + w1 * o1[i];
    }
    fl.m = M;
    lsum = w0 * lsum + w1 * l1;
  }
  if (!live) return;
  if (a.n_split == 1) {
    const float inv = 1.0f / lsum;
    uint16_t* op = static_cast<uint16_t*>(a.o) + (((int64_t)b * a.n_new + r) * a.hq + head) * D;
#pragma unroll
    for (int t = 0; t < OT; ++t) {
      const int d = 16 * t + 4 * q16;
      const u32x2 w = {pack_bf16x2(fl.o[t][0] * inv, fl.o[t][1] * inv),
                       pack_bf16x2(fl.o[t][2] * inv, fl.o[t][3] * inv)};
      *reinterpret_cast<u32x2*>(op + d) = w;
    }
  } else {
    const int64_t prow = (((int64_t)b * a.hkv + g) * a.n_split + split) * a.rows + rho;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int t = 0; t < OT; ++t) *reinterpret_cast<f32x4*>(po + 16 * t + 4 * q16) = fl.o[t];
    if (q16 == 0) {
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
  const float* q = static_cast<const float*>(a.q) + (((int64_t)b * a.n_new + r) * a.hq + head) * D;
  float qr[D];
#pragma unroll
  for (int i = 0; i < H; ++i) {
    float c, s;
    rope_cs(qpos, a.freq.rev[i], c, s);
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
      const bool rot = sbuf[s] == 0;
      if (rot) {
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
        if (rot) {
          float c, sn;
          rope_cs(u, a.freq.rev[i], c, sn);
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
  switch (a.row_waves) {
    case 1: hipLaunchKernelGGL((k_query_bf16<D, 1, 2>), grid, dim3(64 * (2 + kQueryLoaders)), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((k_query_bf16<D, 2, 2>), grid, dim3(64 * (4 + kQueryLoaders)), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((k_query_bf16<D, 4, 2>), grid, dim3(64 * (8 + kQueryLoaders)), 0, stream, a); break;
    default: hipLaunchKernelGGL((k_query_bf16<D, 8, 1>), grid, dim3(64 * (8 + kQueryLoaders)), 0, stream, a); break;
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
  if (a.row_waves != 1 && a.row_waves != 2 && a.row_waves != 4 && a.row_waves != 8)
    return hipErrorInvalidValue;
  const dim3 grid(a.n_split, a.hkv * a.row_groups, batch);
  if (head_dim == 128) launch_query_d<128>(a, grid, stream);
  else launch_query_d<64>(a, grid, stream);
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
