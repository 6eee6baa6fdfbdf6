// Stage 2 of DBSA for a batch of queries with block loads shared across the
// queries that chose each block [Notes, Method > Stage 2, items 1-4].
//
// Query q places its selected blocks one after another at positions
// 0 .. T'_q - 1 and its query tokens after them.  A score depends only on the
// difference of the two positions RoPE turns by, so instead of rotating every
// block's keys at each query's placement, the keys are rotated once at their
// pool positions and each query's rows turn by the placement shift
//   position(token r) - placement start of block b + pool start of block b.
// One K/V tile of block b in LDS then serves the rows of every query that
// selected b; each (query, block) pair leaves a partial softmax, merged later
// with the query's tail / new-token pass (k_merge).
//
// Kernels
//   k_pack_shared_bf16   rotate the K tiles of every selected block at their
//                        pool positions into LDS byte images (one slot per
//                        (block, tile); a tile shared by two blocks is packed
//                        for each).
//   k_shared_bf16        flash attention of 256 packed rows (query, token,
//                        head in GQA group) over one block's tiles: the
//                        software-pipelined core of the prefill on
//                        v_mfma_f32_32x32x16_bf16; writes O / l (bf16) and
//                        m + log2 l per row.  A persistent grid that takes
//                        its items from a work queue (zeroed by the pack).
#include "dbsa_device.hpp"

namespace dbsa {

namespace {

struct SharedTab {
  const int32_t* off;
  const int32_t* bstart;
  const int32_t* istart;
  const int32_t* pairs;
  const int32_t* kslot;
  const int32_t* ublk;
  const int32_t* uslot;
};

template <typename Tables>  // (SharedTables, in any address space)
__device__ __forceinline__ SharedTab shared_tab(const int32_t* tab, const Tables& t) {
  return SharedTab{tab + t.o_off,   tab + t.o_bstart, tab + t.o_istart, tab + t.o_pairs,
                   tab + t.o_kslot, tab + t.o_ublk,   tab + t.o_uslot};
}

}  // namespace

// ---------------------------------------------------------------------------
// K tiles of the selected blocks, rotated at pool positions.  Tiles are
// relative to each block: tile i of block b holds its tokens off[b] + 64 i ..
// + 63 (zero past the block), so only a block's last tile is partial.  One
// workgroup per (slot, KV head); slot s belongs to used block u (uslot[u] <= s
// < uslot[u + 1]) and is its tile i = s - uslot[u].
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64 * (D / 16)) void k_pack_shared_bf16(SharedPackArgs a) {
  using Gm = TileGeom<D>;
  constexpr int CP = D / 16, CR = D / 8;
  const SharedTab tb = shared_tab(a.tab, a.t);
  const int slot = blockIdx.x, g = blockIdx.y;
  if (slot == 0 && g == 0 && threadIdx.x < kPrefillQueueWords) a.queue[threadIdx.x] = 0u;
  const int u = upper_index(tb.uslot, a.t.n_used, slot);
  const int b = tb.ublk[u];
  const int tid = threadIdx.x, key = tid / CP, c = tid % CP;
  const int64_t tok = (int64_t)tb.off[b] + (int64_t)(slot - tb.uslot[u]) * kKeyTile + key;
  u32x4 k1 = u32x4{0u, 0u, 0u, 0u}, k2 = k1;
  if (tok < tb.off[b + 1]) {
    const u32x4* kp = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.k) +
                                                     (tok * a.hkv + g) * D);
    k1 = kp[c];
    k2 = kp[c + CP];
    rope_rotate_chunk(k1, k2, tok, a.freq, 8 * c);
  }
  u32x4* ko = reinterpret_cast<u32x4*>(a.k_tiles) + ((int64_t)g * a.t.n_slots + slot) * (64 * CR);
  ko[key * CR + Gm::k_phys(key, c)] = k1;
  ko[key * CR + Gm::k_phys(key, c + CP)] = k2;
}

// ---------------------------------------------------------------------------
// Shared-block attention.  Workgroup = 8 wavefronts x 32 packed rows of the
// pairs (query, slot) that selected block b, chunk `chunk` of them; the
// workgroup walks the block's 64-key tiles (tokens off[b] + 64 i ..), the
// last one masked to the block.  Same LDS rings, loads and pipeline as
// k_prefill_bf16.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64 * kPrefillWaves, 1) void k_shared_bf16(SharedArgs a) {
  using Gm = TileGeom<D>;
  constexpr int KS = D / 16;
  constexpr int NS = kPrefillStages;
  static_assert(NS == 4, "two tiles in use and two in flight per ring");
  __shared__ __align__(16) char lds[NS * (Gm::KBYTES + Gm::VBYTES)];
  char* const kring = lds;
  char* const vring = lds + NS * Gm::KBYTES;

  __shared__ int s_next[2];
  const int n_all = a.t.n_items * a.hkv;

  // Work item lam = (kv head g, item); items are ordered by block, so each
  // XCD's range of the work queue walks consecutive chunks of one block (its
  // K/V tiles stay in that L2).  Round k of the persistent loop.
  const auto run = [&](const int lam, const int k) {
  // (The lane index and the argument block pass through empty asm
  // statements so that nothing derived from them is hoisted out of the item
  // loop: kept live across items, those values would not fit the registers.)
  int tix = threadIdx.x;
  asm volatile("" : "+v"(tix));
  auto kargs = (const __attribute__((address_space(4))) SharedArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kargs));
  const auto& a = *kargs;
  const int tid = tix, wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5, col = lane & 31;
  const SharedTab tb = shared_tab(a.tab, a.t);
  const int g = lam / a.t.n_items;
  const int item = lam - g * a.t.n_items;
  // The item's block: istart is ascending from istart[0] = 0, so blk = the
  // number of b in [1, n_blocks) with istart[b] <= item, counted 128 entries
  // at a time with ballots (one load latency for up to 128 blocks, instead of
  // a chain of dependent loads).
  int blk = 0;
  for (int b0 = 0; b0 < a.t.n_blocks; b0 += 128) {
    const int ba = b0 + lane, bb = b0 + 64 + lane;
    const int ia = ba < a.t.n_blocks ? tb.istart[ba] : INT32_MAX;
    const int ib = bb < a.t.n_blocks ? tb.istart[bb] : INT32_MAX;
    blk += __builtin_popcountll(__builtin_amdgcn_ballot_w64(ba >= 1 && ia <= item)) +
           __builtin_popcountll(__builtin_amdgcn_ballot_w64(ib <= item));
  }
  blk = __builtin_amdgcn_readfirstlane(blk);
  const int chunk = item - __builtin_amdgcn_readfirstlane(tb.istart[blk]);
  const int p0 = __builtin_amdgcn_readfirstlane(tb.bstart[blk]);
  const int n_rows = (__builtin_amdgcn_readfirstlane(tb.bstart[blk + 1]) - p0) * a.rq;
  const int key0 = __builtin_amdgcn_readfirstlane(tb.off[blk]);
  const int key1 = __builtin_amdgcn_readfirstlane(tb.off[blk + 1]);
  const int slot0 = __builtin_amdgcn_readfirstlane(tb.kslot[blk]);
  const int n_tiles = (key1 - key0 + kKeyTile - 1) / kKeyTile;

  // This lane's row: pair (batch row qb, slot of blk in its ids), token r,
  // head in group h (the pair itself is read after the first tile requests).
  const int G = a.hq / a.hkv;
  const int rho = chunk * kPrefillRows + wave * kRowsPerWave + col;
  const bool live = rho < n_rows;
  const int pr = live ? rho / a.rq : 0;
  const int rr = live ? rho - pr * a.rq : 0;
  const int r = rr / G;
  const int head = g * G + (rr - r * G);

  const u32x4* kbase = reinterpret_cast<const u32x4*>(a.k_tiles) +
                       ((int64_t)g * a.t.n_slots + slot0) * Gm::TU4;
  const uint16_t* vsrc = static_cast<const uint16_t*>(a.v);
  constexpr int NPW = Gm::TU4 / 64 / kPrefillWaves;
  static_assert(NPW * 64 * kPrefillWaves == Gm::TU4, "tile pieces split evenly over the waves");
  int kl[NPW], vo[NPW];
#pragma unroll
  for (int jj = 0; jj < NPW; ++jj) {
    const int i = wave + jj * kPrefillWaves;
    kl[jj] = i * 64 + lane;
    const int o16 = i * 1024 + lane * 16;
    const int row = o16 / Gm::ROW;
    vo[jj] = (row * a.hkv + g) * D + Gm::v_phys(row, (o16 % Gm::ROW) >> 4) * 8;
  }
  const int wsc = __builtin_amdgcn_readfirstlane(wave);
  auto load_k = [&](int it) {
    char* st = kring + (it % NS) * Gm::KBYTES;
    const u32x4* kt = kbase + (int64_t)it * Gm::TU4;
#pragma unroll
    for (int jj = 0; jj < NPW; ++jj)
      dma16s(16u * kl[jj], kt, st + (wsc + jj * kPrefillWaves) * 1024);
  };
  auto load_v = [&](int it) {
    char* st = vring + (it % NS) * Gm::VBYTES;
    const int k0 = key0 + it * kKeyTile;
    if (k0 + kKeyTile <= a.n_tokens) {  // (rows past the block are masked)
      const uint16_t* vt = vsrc + (int64_t)k0 * a.hkv * D;
#pragma unroll
      for (int jj = 0; jj < NPW; ++jj)
        dma16s(2u * vo[jj], vt, st + (wsc + jj * kPrefillWaves) * 1024);
    } else {  // end of the pool: rows past it repeat its last key (masked)
#pragma unroll
      for (int jj = 0; jj < NPW; ++jj) {
        const int o16 = (wave + jj * kPrefillWaves) * 1024 + lane * 16;
        const int row = o16 / Gm::ROW;
        const int64_t tok = min(k0 + row, a.n_tokens - 1);
        dma16(vsrc + (tok * a.hkv + g) * D + Gm::v_phys(row, (o16 % Gm::ROW) >> 4) * 8,
              st + (wsc + jj * kPrefillWaves) * 1024);
      }
    }
  };
  flash_walk_start(n_tiles, load_k, load_v);
  if (tid == 0) s_next[(k + 1) & 1] = queue_claim(a.queue, n_all);
  const int qi = tb.pairs[2 * (p0 + pr)];
  const int shift = tb.pairs[2 * (p0 + pr) + 1];
  const int qb = qi >> 16, qslot = qi & 0xffff;

  // Q of the row, rotated at its position relative to the block's pool
  // placement, scale * log2(e) folded in, rounded once to bf16.
  bf16x8 qb8[KS];
  {
    u32x4 raw[KS];
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.q) + (((int64_t)qb * a.n_new + r) * a.hq + head) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) raw[ks] = live ? qp[2 * ks + hh] : u32x4{0u, 0u, 0u, 0u};
    auto frev = reinterpret_cast<const __attribute__((address_space(4))) double*>(
        (const __attribute__((address_space(4))) char*)kargs + offsetof(SharedArgs, freq) +
        offsetof(RopeFreq, rev));
    using AT = AngleTable<D>;
    // The G rows of one (pair, token) share a position: with G >= 4 the
    // workgroup's 256 / G positions go through an LDS table in V stages 1-3
    // (untouched until the walk's first requests), one cos / sin per
    // (position, frequency).  Uniform condition.
    if (G >= 4 && (kPrefillRows / G) * AT::ROWB <= 3 * Gm::VBYTES) {
      char* const tab = vring + Gm::VBYTES;
      AT::fill(tab, kPrefillRows / G, tid, 64 * kPrefillWaves,
               [&](int j) -> int64_t {
                 const int rj = chunk * kPrefillRows + j * G;  // first row of position j
                 if (rj >= n_rows) return 0;
                 const int prj = rj / a.rq;
                 return (int64_t)tb.pairs[2 * (p0 + prj) + 1] + (rj - prj * a.rq) / G;
               },
               [&](int f) { return (double)frev[f]; });
      __syncthreads();
      const int jl = (wave * kRowsPerWave + col) / G;
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks) {
        float c[8], sn[8];
        AT::read8(tab, jl, 16 * ks + 8 * hh, c, sn);
        rotate_chunk(raw[ks], raw[ks + KS / 2], c, sn, a.q_scale);
      }
    } else {
      // (The two lane halves' frequencies are scalar loads, selected per lane.)
#pragma unroll
      for (int ks = 0; ks < KS / 2; ++ks) {
        float c[8], sn[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          double f0 = frev[16 * ks + i], f1 = frev[16 * ks + 8 + i];
          asm volatile("" : "+s"(f0), "+s"(f1));  // (kept as two scalar loads)
          rope_cs((int64_t)shift + r, hh ? f1 : f0, c[i], sn[i]);
        }
        rotate_chunk(raw[ks], raw[ks + KS / 2], c, sn, a.q_scale);
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb8[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
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

  // Every row sees the whole block: only its last tile, which may reach
  // past it, needs the element mask.
  const auto full_of = [&](int it) { return key0 + (it + 1) * kKeyTile <= key1; };
  const auto vis_of = [&](int it) {
    const int hi = key1 - (key0 + it * kKeyTile);
    return [=](int kr) { return kr < hi; };
  };
  flash_walk<D>(fl, kring, lds, n_tiles, koff, vbase, qb8, load_k, load_v, full_of, vis_of);

  // O / l in bf16 and lambda = m + log2(l), staged row by row through the
  // wave's part of the (idle) K ring so whole 16-byte chunks go out.
  const float lsum = fl.total();
  const float inv = live ? 1.0f / lsum : 0.0f;
  const int64_t prow = (((int64_t)qb * a.hkv + g) * a.n_ids + qslot) * a.rq + rr;
  if (live && hh == 0) a.part_lam[prow] = fl.m + __builtin_amdgcn_logf(lsum);
  constexpr int CPR = D / 8;
  char* const ost = kring + wave * (kRowsPerWave * Gm::ROW);
  static_assert(kPrefillWaves * kRowsPerWave * Gm::ROW <= NS * Gm::KBYTES, "O fits the K ring");
#pragma unroll
  for (int m = 0; m < D / 32; ++m)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const u32x2 w = {pack_bf16x2(fl.o[m][4 * q4 + 0] * inv, fl.o[m][4 * q4 + 1] * inv),
                       pack_bf16x2(fl.o[m][4 * q4 + 2] * inv, fl.o[m][4 * q4 + 3] * inv)};
      const int ch = (m * 4 + q4) ^ (col & (CPR - 1));
      *reinterpret_cast<u32x2*>(ost + col * Gm::ROW + ch * 16 + hh * 8) = w;
    }
  // Destination of each staged row: row rr_w of the wave belongs to lane
  // rr_w, which has its (query, slot) pair in registers (the rows of one wave
  // may span two pairs).
  constexpr int RPI = 64 / CPR;
#pragma unroll
  for (int i = 0; i < kRowsPerWave / RPI; ++i) {
    const int rr_w = i * RPI + lane / CPR, ch = lane % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ost + rr_w * Gm::ROW + (ch ^ (rr_w & (CPR - 1))) * 16);
    const int rho_s = chunk * kPrefillRows + wave * kRowsPerWave + rr_w;
    const int qi_s = __shfl(qi, rr_w);
    if (rho_s < n_rows) {
      const int pr_s = rho_s / a.rq;
      const int64_t row = (((int64_t)(qi_s >> 16) * a.hkv + g) * a.n_ids + (qi_s & 0xffff)) * a.rq +
                          (rho_s - pr_s * a.rq);
      *reinterpret_cast<u32x4*>(a.part_o + row * D + ch * 8) = v;
    }
  }
  };
  queue_loop(a.queue, n_all, s_next, run);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_shared_pack(const SharedPackArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid(a.t.n_slots, a.hkv);
  if (head_dim == 128)
    hipLaunchKernelGGL(k_pack_shared_bf16<128>, grid, dim3(64 * 8), 0, stream, a);
  else
    hipLaunchKernelGGL(k_pack_shared_bf16<64>, grid, dim3(64 * 4), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_shared(const SharedArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid(std::min(a.t.n_items * a.hkv, a.n_workers));
  if (head_dim == 128)
    hipLaunchKernelGGL(k_shared_bf16<128>, grid, dim3(64 * kPrefillWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(k_shared_bf16<64>, grid, dim3(64 * kPrefillWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dbsa
