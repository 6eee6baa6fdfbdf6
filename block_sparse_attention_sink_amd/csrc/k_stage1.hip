// Stage 1 of DBSA on gfx950: block-sparse streaming prefill.
//
// [Notes, Method > Stage 1]: block i attends to the anchor block (sink), to the
// previous j blocks and causally to itself; tokens sit at sequential
// positions; K/V are kept unrotated.  The page's implementation skips masked
// blocks; here the skipping is by construction: each query tile walks only
// the 64-key tiles that meet its visible key intervals.
//
// Kernels
//   k_pack_bf16     rotate K once per key tile and transpose V, writing each
//                   tile as the exact LDS byte image the prefill consumes.
//   k_prefill_bf16  flash attention on bf16 MFMA (v_mfma_f32_32x32x16_bf16):
//                   S^T = K Q^T and O^T += V^T P^T so that every softmax row
//                   statistic lives in one lane pair; online softmax in exp2.
//   k_rows_f32      one wavefront per (row, head) in float32 for the f32
//                   dtype (no MFMA; small correctness-grade problems).
#include "dbsa_device.hpp"

namespace dbsa {

// ---------------------------------------------------------------------------
// K rotation into tile images (the LDS byte images, see TileGeom).  One
// workgroup per (key tile slot, KV head); keys past the pool are zero.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64 * (D / 16)) void k_pack_bf16(PackArgs a) {
  using Gm = TileGeom<D>;
  constexpr int CP = D / 16;  // chunk pairs per key row (first half / second half)
  constexpr int CR = D / 8;   // 16-byte chunks per key row
  const int slot = blockIdx.x, g = blockIdx.y;
  if (a.queue != nullptr && slot == 0 && g == 0 && threadIdx.x < 8) a.queue[threadIdx.x] = 0u;
  const int kt = slot < a.sink_tiles ? slot : a.win_tile0 + (slot - a.sink_tiles);
  const int tid = threadIdx.x, key = tid / CP, c = tid % CP;
  const int64_t tok = (int64_t)kt * kKeyTile + key;
  u32x4 k1 = u32x4{0u, 0u, 0u, 0u}, k2 = k1;
  if (tok < a.n_tokens) {
    const u32x4* kp = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.k) +
                                                     (tok * a.hkv + g) * D);
    k1 = kp[c];
    k2 = kp[c + CP];
    rope_rotate_chunk(k1, k2, tok, a.freq, 8 * c);
  }
  u32x4* ko = reinterpret_cast<u32x4*>(a.k_tiles) + ((int64_t)g * a.n_slots + slot) * (64 * CR);
  ko[key * CR + Gm::k_phys(key, c)] = k1;
  ko[key * CR + Gm::k_phys(key, c + CP)] = k2;
}

// ---------------------------------------------------------------------------
// Block-sparse flash prefill, bf16 in / bf16 out, fp32 accumulation.
//
// Workgroup = 8 wavefronts = 256 query rows (256 / P tokens x P query heads
// of one KV head, below); each wave owns 32 rows (lane layout: see Flash).  The workgroup walks the
// 64-key tiles that meet its rows' visible intervals.  K tiles and V tiles
// have separate LDS rings of 4 stages, filled by direct global->LDS loads
// two tiles at a time (see the loop).
// ---------------------------------------------------------------------------
template <int D, bool SPLIT>
__global__ __launch_bounds__(64 * kPrefillWaves, 1) void k_prefill_bf16(PrefillArgs a) {
  using Gm = TileGeom<D>;
  constexpr int KS = D / 16;
  constexpr int NS = kPrefillStages;
  static_assert(NS == 4, "two tiles in use and two in flight per ring");
  __shared__ __align__(16) char lds[NS * (Gm::KBYTES + Gm::VBYTES)];
  char* const kring = lds;
  char* const vring = lds + NS * Gm::KBYTES;

  __shared__ int s_next[2];  // items of the next two rounds (written by thread 0)
  const int tid = threadIdx.x;

  // Logical work item: (kv head g, query tile qt, key split, group of P =
  // 2^pack_log2 query heads of g).  The workgroup's 256 rows are 256 / P
  // tokens x P heads: wave w takes head w % P of the group for tokens
  // 32 (w / P) .. + 31, so one LDS K/V tile serves P heads.  Without SPLIT
  // the walk is whole (n_split == 1), and the split bookkeeping compiles away.
  const int G = a.hq / a.hkv;
  const int pl = a.pack_log2, P = 1 << pl;
  const int HS = G >> pl;  // head groups per KV head
  const int nsp = SPLIT ? a.n_split : 1;
  const int per_g = a.n_qtiles * nsp * HS;

  // Without SPLIT the grid is persistent and takes its items from the work
  // queue a.queue (see queue_claim).
  const int n_items = per_g * a.hkv;

  // One work item (round k); thread 0 leaves the item it claims for the
  // next round in s_next[(k + 1) & 1].
  const auto run = [&](const int lam, const int k) {
  // (The lane index and the argument block pass through empty asm
  // statements so that nothing derived from them is hoisted out of the item
  // loop: kept live across items, those values would not fit the registers.)
  int tix = tid;
  asm volatile("" : "+v"(tix));
  auto kargs = (const __attribute__((address_space(4))) PrefillArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kargs));
  const auto& a = *kargs;
  const int wave = tix >> 6, lane = tix & 63;
  const int hh = lane >> 5, col = lane & 31;
  const int g = lam / per_g;
  const int rem = lam - g * per_g;
  const int qt = rem / (nsp * HS);
  const int rem2 = rem - qt * (nsp * HS);
  const int split = SPLIT ? rem2 / HS : 0;
  const int hsub = rem2 - split * HS;
  const int hig = (hsub << pl) + (wave & (P - 1));
  const int head = g * G + hig;
  const int tw = kPrefillRows >> pl;  // tokens per workgroup
  const int r0 = a.row0 + qt * tw;
  const int r1 = min(r0 + tw, a.row1);
  const int wrow = (wave >> pl) * kRowsPerWave;  // this wave's first token, from r0
  const int t = r0 + wrow + col;

  // Q first: its address needs only the row and the head, so its latency
  // overlaps the block lookups and the first tile requests below.
  u32x4 raw[KS];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.q) + ((int64_t)(min(t, r1 - 1) - a.q_row0) * a.hq + head) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) raw[ks] = qp[2 * ks + hh];
  }

  // Visible key intervals [Notes, Method > Stage 1, item 2]:
  // row t sees [lo(t), t] with lo(t) = start of block max(blk(t) - j, 0),
  // plus the anchor block [0, sink_end) when the sink is on.
  const int nb = a.n_blocks;
  // blk(x) = number of block starts off[1 .. nb - 1] at or before x.  The
  // rows of the workgroup lie in blocks b_first = blk(r0) .. b_last =
  // blk(r1 - 1), usually one or two.  With the table in the kernel arguments
  // (at most 511 blocks) every lane compares 8 entries and ballots count
  // them, and the other reads are scalar loads that wait for nothing else;
  // a table in device memory is searched.  (Readfirstlane tells the compiler
  // that these values are workgroup-uniform, which keeps them, and the tile
  // addresses built from them, in scalar registers.)
  int sink_end, lo_first, lo_last, lo_t;
  const auto lookup = [&](auto off, int b_first, int b_last) {
    b_first = __builtin_amdgcn_readfirstlane(b_first);
    b_last = __builtin_amdgcn_readfirstlane(b_last);
    sink_end = __builtin_amdgcn_readfirstlane(a.sink ? off[1] : 0);
    lo_first = __builtin_amdgcn_readfirstlane(off[max(b_first - a.j, 0)]);
    lo_last = __builtin_amdgcn_readfirstlane(off[max(b_last - a.j, 0)]);
    lo_t = lo_first;
    for (int bb = b_first + 1; bb <= b_last; ++bb)
      if (__builtin_amdgcn_readfirstlane(off[bb]) <= t)
        lo_t = __builtin_amdgcn_readfirstlane(off[max(bb - a.j, 0)]);
  };
  if (a.n_inline) {
    const auto off = reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
        (const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr() +
        offsetof(PrefillArgs, inl));
    int e[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) e[k] = off[8 * lane + k];
    int c0 = 0, c1 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int idx = 8 * lane + k;
      const bool in = idx >= 1 && idx < nb;
      c0 += __builtin_popcountll(__builtin_amdgcn_ballot_w64(in && e[k] <= r0));
      c1 += __builtin_popcountll(__builtin_amdgcn_ballot_w64(in && e[k] <= r1 - 1));
    }
    lookup(off, c0, c1);
  } else {
    lookup(a.offsets, upper_index(a.offsets, nb, r0), upper_index(a.offsets, nb, r1 - 1));
  }
  const int win0 = lo_first / kKeyTile;
  const int win1 = (r1 + kKeyTile - 1) / kKeyTile;
  int nsink = 0;
  if (a.sink && lo_last > 0) nsink = min((sink_end + kKeyTile - 1) / kKeyTile, win0);
  const int n_all = nsink + (win1 - win0);
  // This workgroup's part of the walk: tiles [it_lo, it_lo + n_tiles).
  const int per_split = SPLIT ? (n_all + nsp - 1) / nsp : n_all;
  const int it_lo = SPLIT ? min(split * per_split, n_all) : 0;
  const int n_tiles = SPLIT ? min(per_split, n_all - it_lo) : n_all;

  const u32x4* kbase = reinterpret_cast<const u32x4*>(a.k_tiles) + (int64_t)g * a.n_slots * Gm::TU4;
  const uint16_t* vsrc = static_cast<const uint16_t*>(a.v);
  auto tile_of = [&](int it) {
    if constexpr (SPLIT) it += it_lo;
    return it < nsink ? it : win0 + (it - nsink);
  };
  auto slot_of = [&](int kt) {
    return kt < a.sink_tiles ? kt : a.sink_tiles + (kt - a.win_tile0);
  };
  // Tile loads without registers: the K image is a linear copy; V rows come
  // straight from the token-major tensor, each lane fetching the chunk that
  // belongs at its LDS position.  Wave w moves the 1 KiB pieces w, w + 8, ...
  // of each matrix.
  constexpr int NPW = Gm::TU4 / 64 / kPrefillWaves;
  static_assert(NPW * 64 * kPrefillWaves == Gm::TU4, "tile pieces split evenly over the waves");
  // Per-lane offsets (32-bit, to keep registers free): K in 16-byte chunks
  // from the head's first tile image, V in elements from the first key tile.
  int kl[NPW], vo[NPW];
#pragma unroll
  for (int jj = 0; jj < NPW; ++jj) {
    const int i = wave + jj * kPrefillWaves;
    kl[jj] = i * 64 + lane;
    const int o16 = i * 1024 + lane * 16;
    const int row = o16 / Gm::ROW;
    vo[jj] = (row * a.hkv + g) * D + Gm::v_phys(row, (o16 % Gm::ROW) >> 4) * 8;
  }
  // The wave index as a scalar keeps the LDS destinations (M0) scalar.
  const int wsc = __builtin_amdgcn_readfirstlane(wave);
  const int64_t vtile = (int64_t)kKeyTile * a.hkv * D;  // elements per key tile of V
  auto load_k = [&](int it) {
    char* st = kring + (it % NS) * Gm::KBYTES;
    const u32x4* kt = kbase + (int64_t)slot_of(tile_of(it)) * Gm::TU4;
#pragma unroll
    for (int jj = 0; jj < NPW; ++jj)
      dma16s(16u * kl[jj], kt, st + (wsc + jj * kPrefillWaves) * 1024);
  };
  auto load_v = [&](int it) {
    char* st = vring + (it % NS) * Gm::VBYTES;
    const int kt = tile_of(it);
    if ((kt + 1) * kKeyTile <= a.n_keys) {
      const uint16_t* vt = vsrc + kt * vtile;
#pragma unroll
      for (int jj = 0; jj < NPW; ++jj)
        dma16s(2u * vo[jj], vt, st + (wsc + jj * kPrefillWaves) * 1024);
    } else {  // last, partial key tile: rows past the keys repeat the last key (masked)
#pragma unroll
      for (int jj = 0; jj < NPW; ++jj) {
        const int o16 = (wave + jj * kPrefillWaves) * 1024 + lane * 16;
        const int row = o16 / Gm::ROW;
        const int64_t tok = min(kt * kKeyTile + row, a.n_keys - 1);
        dma16(vsrc + (tok * a.hkv + g) * D + Gm::v_phys(row, (o16 % Gm::ROW) >> 4) * 8,
              st + (wsc + jj * kPrefillWaves) * 1024);
      }
    }
  };
  if (SPLIT && n_tiles <= 0) {  // no keys in this part of the walk: an empty partial
    const int trow = t - a.row0;
    if (t < r1 && hh == 0) {
      const int64_t prow = ((int64_t)g * a.n_split + split) * ((int64_t)(a.row1 - a.row0) * G) +
                           (int64_t)trow * G + hig;
      a.part_ml[prow * 2 + 0] = 0.0f;
      a.part_ml[prow * 2 + 1] = 0.0f;
    }
    return;
  }
  // Q has landed (the table lookups waited for it, or had the time to): the
  // compiler, which does not count the tile requests, then places no wait
  // for Q after them.
  waitcnt<0, 15>();
  flash_walk_start(n_tiles, load_k, load_v);
  if constexpr (!SPLIT)
    if (tid == 0) s_next[(k + 1) & 1] = queue_claim(a.queue, n_items);

  // Q: rotate at position t, fold scale * log2(e), round once to bf16.
  bf16x8 qb[KS];
  {
    if (t >= r1) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) raw[ks] = u32x4{0u, 0u, 0u, 0u};
    }
    // (The two lane halves' frequencies are read as scalars and selected:
    // a per-lane index would make them vector loads queued behind the tile
    // requests above.  Their address passes through an empty asm statement
    // so the loads stay here instead of being hoisted out of the item loop,
    // where they would be live across it.)
    auto frev = reinterpret_cast<const __attribute__((address_space(4))) double*>(
        (const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr() +
        offsetof(PrefillArgs, freq) + offsetof(RopeFreq, rev));
    asm volatile("" : "+s"(frev));
    using AT = AngleTable<D>;
    // With several heads per token (64 tokens of 4 heads) the workgroup's tw
    // positions go through an LDS table in V stages 1-3 (untouched until the
    // walk's first requests): one cos / sin per (token, frequency) instead of
    // one per row.  Uniform condition.
    if (tw % 64 == 0 && tw * AT::ROWB <= 3 * Gm::VBYTES) {
      char* const tab = vring + Gm::VBYTES;
      AT::fill(tab, tw, tix, 64 * kPrefillWaves, [&](int j) -> int64_t { return r0 + j; },
               [&](int f) { return (double)frev[f]; });
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks) {
        float c[8], sn[8];
        AT::read8(tab, wrow + col, 16 * ks + 8 * hh, c, sn);
        rotate_chunk(raw[ks], raw[ks + KS / 2], c, sn, a.q_scale);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks) {
        float c[8], sn[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          double f0 = frev[16 * ks + r], f1 = frev[16 * ks + 8 + r];
          asm volatile("" : "+s"(f0), "+s"(f1));  // (kept as two scalar loads)
          rope_cs(t, hh ? f1 : f0, c[r], sn[r]);
        }
        rotate_chunk(raw[ks], raw[ks + KS / 2], c, sn, a.q_scale);
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
  }

  Flash<D> fl;
  fl.init();

  int koff[KS], vbase[D / 32];
  lane_offsets<D>(lane, koff, vbase);
  // The V ring's offset goes into the lane's bases, and the walk addresses V
  // fragments from the start of the LDS block: every V read then takes its
  // stage and step as an immediate offset (the ring starts 64 KiB in, past
  // the reach of that offset field, and the address additions would
  // otherwise be redone every tile).
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    vbase[t] += static_cast<int>(vring - lds);
    asm volatile("" : "+v"(vbase[t]));
  }

  // Element mask only on tiles some row cannot fully see.
  const auto full_of = [&](int it) {
    const int k0 = tile_of(it) * kKeyTile;
    return (k0 + kKeyTile - 1 <= r0) && (k0 >= lo_last || (a.sink && k0 + kKeyTile <= sink_end));
  };
  const auto vis_of = [&](int it) {
    const int k0 = tile_of(it) * kKeyTile;
    const int tt = t - k0, lt = lo_t - k0, se = sink_end - k0;
    return [=](int kr) { return kr <= tt && (kr >= lt || kr < se); };
  };
  flash_walk<D>(fl, kring, lds, n_tiles, koff, vbase, qb, load_k, load_v, full_of, vis_of);

  const float lsum = fl.total();
  if constexpr (SPLIT) {
    // Split walk: unnormalised O and (m, l) of the row for k_combine.
    if (t >= r1) return;
    const int64_t prow = ((int64_t)g * a.n_split + split) * ((int64_t)(a.row1 - a.row0) * G) +
                         (int64_t)(t - a.row0) * G + hig;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(po + m * 32 + q4 * 8 + hh * 4) =
            f32x4{fl.o[m][4 * q4 + 0], fl.o[m][4 * q4 + 1], fl.o[m][4 * q4 + 2], fl.o[m][4 * q4 + 3]};
    if (hh == 0) {
      a.part_ml[prow * 2 + 0] = fl.m;
      a.part_ml[prow * 2 + 1] = lsum;
    }
    return;
  }

  // O = O / l in bf16, staged row by row in the wave's part of the K ring
  // (idle once the last barrier has passed: every K read and K load of the
  // walk is done) so that whole 16-byte chunks of a row go out together;
  // chunks are XOR-swizzled by row against LDS bank conflicts.
  const float inv = t < r1 ? 1.0f / lsum : 0.0f;
  constexpr int CPR = D / 8;  // 16-byte chunks per output row
  char* const ost = kring + wave * (kRowsPerWave * Gm::ROW);
  static_assert(kPrefillWaves * kRowsPerWave * Gm::ROW <= NS * Gm::KBYTES, "O fits the K ring");
#pragma unroll
  for (int m = 0; m < D / 32; ++m)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const u32x2 w = {pack_bf16x2(fl.o[m][4 * q4 + 0] * inv, fl.o[m][4 * q4 + 1] * inv),
                       pack_bf16x2(fl.o[m][4 * q4 + 2] * inv, fl.o[m][4 * q4 + 3] * inv)};
      const int ch = (m * 4 + q4) ^ (col & (CPR - 1));  // head dims 8 (m * 4 + q4) .. + 7
      *reinterpret_cast<u32x2*>(ost + col * Gm::ROW + ch * 16 + hh * 8) = w;
    }
  constexpr int RPI = 64 / CPR;  // rows per store instruction
#pragma unroll
  for (int i = 0; i < kRowsPerWave / RPI; ++i) {
    const int rr = i * RPI + lane / CPR, ch = lane % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ost + rr * Gm::ROW + (ch ^ (rr & (CPR - 1))) * 16);
    const int trow = r0 + wrow + rr;
    if (trow < r1)
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o) +
                                ((int64_t)(trow - a.q_row0) * a.hq + head) * D + ch * 8) = v;
  }
  };

  if constexpr (SPLIT) run(xcd_logical(blockIdx.x, gridDim.x), 0);
  else queue_loop(a.queue, n_items, s_next, run);
}

// ---------------------------------------------------------------------------
// float32 prefill: one wavefront per (row, head), one key per lane.
// k / v are the unrotated f32 pool; keys are rotated on the fly.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void rows_f32_chunk(const float (&qr)[D], const float* k,
                                               const float* v, int64_t key_stride,
                                               int s0, int s1, float& m_run, float& l_run,
                                               float (&acc)[2], const RopeFreq& f, int lane) {
  constexpr int H = D / 2;
  for (int base = s0; base < s1; base += 64) {
    const int s = base + lane;
    float sc = kNegInf;
    if (s < s1) {
      const float* kr = k + (int64_t)s * key_stride;
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        float c, sn;
        rope_cs(s, f.rev[i], c, sn);
        const float x1 = kr[i], x2 = kr[i + H];
        dot += qr[i] * rot_lo(x1, x2, c, sn) + qr[i + H] * rot_hi(x1, x2, c, sn);
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
    acc[0] *= alpha;
    acc[1] *= alpha;
    const int n = min(64, s1 - base);
    for (int kk = 0; kk < n; ++kk) {
      const float pk = __shfl(p, kk);
      const float* vr = v + (int64_t)(base + kk) * key_stride;
      if (lane < D) acc[0] += pk * vr[lane];
      if (lane + 64 < D) acc[1] += pk * vr[lane + 64];
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_rows_f32(PrefillArgs a) {
  constexpr int H = D / 2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = a.row0 + blockIdx.x * 4 + wave;
  const int head = blockIdx.y;
  if (t >= a.row1) return;  // no block-level synchronisation below
  const int g = head / (a.hq / a.hkv);
  const float* q = static_cast<const float*>(a.q) + ((int64_t)(t - a.q_row0) * a.hq + head) * D;
  float qr[D];
#pragma unroll
  for (int i = 0; i < H; ++i) {
    float c, s;
    rope_cs(t, a.freq.rev[i], c, s);
    qr[i] = rot_lo(q[i], q[i + H], c, s) * a.q_scale;
    qr[i + H] = rot_hi(q[i], q[i + H], c, s) * a.q_scale;
  }
  const int32_t* off = a.n_inline ? kernarg_ints(offsetof(PrefillArgs, inl)) : a.offsets;
  const int sink_end = a.sink ? off[1] : 0;
  const int lo_t = off[max(upper_index(off, a.n_blocks, t) - a.j, 0)];
  const float* k = static_cast<const float*>(a.k_tiles) + (int64_t)g * D;
  const float* v = static_cast<const float*>(a.v) + (int64_t)g * D;
  const int64_t stride = (int64_t)a.hkv * D;
  float m_run = kMaxFloor, l_run = 0.0f, acc[2] = {0.0f, 0.0f};
  if (a.sink && lo_t > 0) rows_f32_chunk<D>(qr, k, v, stride, 0, sink_end, m_run, l_run, acc, a.freq, lane);
  rows_f32_chunk<D>(qr, k, v, stride, lo_t, t + 1, m_run, l_run, acc, a.freq, lane);
  float* o = static_cast<float*>(a.o) + ((int64_t)(t - a.q_row0) * a.hq + head) * D;
  if (lane < D) o[lane] = acc[0] / l_run;
  if (lane + 64 < D) o[lane + 64] = acc[1] / l_run;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_pack(const PackArgs& a, int head_dim, int dtype, hipStream_t stream) {
  (void)dtype;
  const dim3 grid(a.n_slots, a.hkv);
  if (head_dim == 128)
    hipLaunchKernelGGL(k_pack_bf16<128>, grid, dim3(64 * 8), 0, stream, a);
  else
    hipLaunchKernelGGL(k_pack_bf16<64>, grid, dim3(64 * 4), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int dtype, hipStream_t stream) {
  if (dtype == 1) {  // float32
    const dim3 grid((a.row1 - a.row0 + 3) / 4, a.hq);
    if (head_dim == 128)
      hipLaunchKernelGGL(k_rows_f32<128>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(k_rows_f32<64>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const int items = a.n_qtiles * (a.hq >> a.pack_log2) * a.n_split;
  const dim3 grid(a.n_split > 1 ? items : std::min(items, a.n_workers));
  const dim3 block(64 * kPrefillWaves);
  if (a.n_split > 1) {
    if (head_dim == 128) hipLaunchKernelGGL((k_prefill_bf16<128, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_prefill_bf16<64, true>), grid, block, 0, stream, a);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((k_prefill_bf16<128, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_prefill_bf16<64, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dbsa
