// Stage 1 of DBSA on gfx950: block-sparse streaming prefill.
//
// [Notes, Method > Stage 1]: block i attends to the anchor block (sink), to the
// previous j blocks and causally to itself; tokens sit at sequential
// positions; K/V are kept unrotated.  The page's implementation skips masked
// blocks; here the skipping is by construction: each 128-row query tile walks
// only the 64-key tiles that meet its visible key intervals.
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
// Workgroup = 8 wavefronts = 256 query rows of one query head; wave w owns
// rows r0 + 32w .. +31 (lane layout: see Flash).  The workgroup walks the
// 64-key tiles that meet its rows' visible intervals.  K tiles and V tiles
// have separate LDS rings of 4 stages, filled by direct global->LDS loads
// two tiles at a time (see the loop).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64 * kPrefillWaves, 1) void k_prefill_bf16(PrefillArgs a) {
  using Gm = TileGeom<D>;
  constexpr int KS = D / 16;
  constexpr int NS = kPrefillStages;
  static_assert(NS == 4, "two tiles in use and two in flight per ring");
  __shared__ __align__(16) char lds[NS * (Gm::KBYTES + Gm::VBYTES)];
  char* const kring = lds;
  char* const vring = lds + NS * Gm::KBYTES;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5, col = lane & 31;

  // Logical work item: (kv head g, query tile qt, query head within the group).
  const int G = a.hq / a.hkv;
  const int lam = xcd_logical(blockIdx.x, gridDim.x);
  const int per_g = a.n_qtiles * G;
  const int g = lam / per_g;
  const int rem = lam - g * per_g;
  const int qt = rem / G;
  const int head = g * G + (rem - qt * G);
  const int r0 = a.row0 + qt * kPrefillRows;
  const int r1 = min(r0 + kPrefillRows, a.row1);
  const int t = r0 + wave * kRowsPerWave + col;

  // Visible key intervals [Notes, Method > Stage 1, item 2]:
  // row t sees [lo(t), t] with lo(t) = start of block max(blk(t) - j, 0),
  // plus the anchor block [0, sink_end) when the sink is on.
  const int32_t* off = a.offsets;
  const int nb = a.n_blocks;
  const int sink_end = a.sink ? off[1] : 0;
  const int lo_t = off[max(upper_index(off, nb, min(t, r1 - 1)) - a.j, 0)];
  const int lo_first = off[max(upper_index(off, nb, r0) - a.j, 0)];
  const int lo_last = off[max(upper_index(off, nb, r1 - 1) - a.j, 0)];
  const int win0 = lo_first / kKeyTile;
  const int win1 = (r1 + kKeyTile - 1) / kKeyTile;
  int nsink = 0;
  if (a.sink && lo_last > 0) nsink = min((sink_end + kKeyTile - 1) / kKeyTile, win0);
  const int n_tiles = nsink + (win1 - win0);

  // Q: rotate at position t, fold scale * log2(e), round once to bf16.
  bf16x8 qb[KS];
  {
    u32x4 raw[KS];
    const bool live = t < r1;
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.q) + ((int64_t)(t - a.q_row0) * a.hq + head) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) raw[ks] = live ? qp[2 * ks + hh] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks)
      rope_rotate_chunk(raw[ks], raw[ks + KS / 2], t, a.freq, 16 * ks + 8 * hh, a.q_scale);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
  }

  Flash<D> fl;
  fl.init();

  const u32x4* kbase = reinterpret_cast<const u32x4*>(a.k_tiles) + (int64_t)g * a.n_slots * Gm::TU4;
  const uint16_t* vsrc = static_cast<const uint16_t*>(a.v);
  auto tile_of = [&](int it) { return it < nsink ? it : win0 + (it - nsink); };
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
  // Requests of (even) iteration i: K of tiles i + 3 and i + 4 and V of
  // tiles i + 1 and i + 2, each when it exists.
  auto request = [&](int i) {
    if (i + 3 < n_tiles) load_k(i + 3);
    if (i + 4 < n_tiles) load_k(i + 4);
    if (i + 1 < n_tiles) load_v(i + 1);
    if (i + 2 < n_tiles) load_v(i + 2);
  };
  int koff[KS], vbase[D / 32];
  lane_offsets<D>(lane, koff, vbase);

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
  const auto kst = [&](int it) { return kring + (it % NS) * Gm::KBYTES; };
  const auto vst = [&](int it) { return vring + (it % NS) * Gm::VBYTES; };

  // Prologue: K of tiles 0, 1, 2 and V of tile 0, all landed before the
  // scores of tile 0.
  for (int i = 0; i < 3 && i < n_tiles; ++i) load_k(i);
  load_v(0);
  wait_vm(0);
  barrier_nofence();
  f32x16 s0, s1, n0, n1;
  bf16x8 pr[4];
  fl.scores(kst(0), koff, qb, s0, s1);
  // Iteration i computes the softmax of tile i, P V of tile i - 1 and the
  // scores of tile i + 1 (reading K of tile i + 1, V of tile i - 1).  Even
  // iterations start with a barrier: every load requested two iterations
  // earlier has landed (each wave waits for its own, the barrier for all),
  // and the stages of K tiles i - 1, i and V tiles i - 3, i - 2, which
  // iterations up to i - 1 read, are refilled for the next two iterations.
  // Odd iterations run without a barrier, so the two wavefronts of a SIMD
  // can drift apart.  The last iteration also computes scores, of a stale K
  // stage; they are never used.
  const auto sync = [&](int i) {
    wait_vm(0);
    barrier_nofence();
    request(i);
  };
  sync(0);
  fl.template pv_head<false>(vst(0), vbase, pr, s0, s1, !full_of(0), vis_of(0));
  fl.exp_next(kst(1), koff, qb, s0, s1, pr, n0, n1);
  // Two iterations per trip (odd, then even) so the score registers
  // alternate instead of being copied.
  for (int i = 1; i < n_tiles; i += 2) {
    fl.template pv_head<true>(vst(i - 1), vbase, pr, n0, n1, !full_of(i), vis_of(i));
    fl.exp_next(kst(i + 1), koff, qb, n0, n1, pr, s0, s1);
    if (i + 1 >= n_tiles) break;
    sync(i + 1);
    fl.template pv_head<true>(vst(i), vbase, pr, s0, s1, !full_of(i + 1), vis_of(i + 1));
    fl.exp_next(kst(i + 2), koff, qb, s0, s1, pr, n0, n1);
  }
  // P V of the last tile (its V may have been requested by the last barrier).
  wait_vm(0);
  barrier_nofence();
  fl.pv(vst(n_tiles - 1), vbase, pr);

  // O = O / l in bf16, staged row by row in the wave's part of the K ring
  // (idle once the last barrier has passed: every K read and K load of the
  // walk is done) so that whole 16-byte chunks of a row go out together;
  // chunks are XOR-swizzled by row against LDS bank conflicts.
  const float lsum = fl.total();
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
    const int trow = r0 + wave * kRowsPerWave + rr;
    if (trow < r1)
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o) +
                                ((int64_t)(trow - a.q_row0) * a.hq + head) * D + ch * 8) = v;
  }
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
  const int32_t* off = a.offsets;
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
  const dim3 grid(a.n_qtiles * a.hq);
  if (head_dim == 128)
    hipLaunchKernelGGL(k_prefill_bf16<128>, grid, dim3(64 * kPrefillWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(k_prefill_bf16<64>, grid, dim3(64 * kPrefillWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dbsa
