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
// K rotation into tile images (the LDS byte images, see TileGeom).
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
// 64-key tiles that meet its rows' visible intervals through a ring of 4 LDS
// stages filled by direct global->LDS loads, 3 tiles ahead of the compute.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64 * kPrefillWaves, 1) void k_prefill_bf16(PrefillArgs a) {
  using Gm = TileGeom<D>;
  constexpr int KS = D / 16;
  constexpr int NST = kPrefillStages;
  constexpr int LPW = 2 * Gm::TU4 / 64 / kPrefillWaves;  // loads per wave per tile
  __shared__ __align__(16) char lds[NST * Gm::STAGE];

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
  // Stage tile `it` into LDS stage `buf` without registers: the K image is a
  // linear copy; V rows come straight from the token-major tensor, each lane
  // fetching the chunk that belongs at its LDS position.
  auto load = [&](int it, int buf) {
    const int kt = tile_of(it);
    char* st = lds + buf * Gm::STAGE;
    copy_to_lds(kbase + (int64_t)slot_of(kt) * Gm::TU4, st, Gm::TU4, wave, kPrefillWaves, lane);
    for (int i = wave; i * 64 < Gm::TU4; i += kPrefillWaves) {
      const int off = i * 1024 + lane * 16;
      const int row = off / Gm::ROW, c = Gm::v_phys(row, (off % Gm::ROW) >> 4);
      const int64_t tok = min(kt * kKeyTile + row, a.n_keys - 1);
      dma16(vsrc + (tok * a.hkv + g) * D + c * 8, st + Gm::KBYTES + i * 1024);
    }
  };
  int koff[KS], vbase[D / 32];
  lane_offsets<D>(lane, koff, vbase);

  // Ring of NST stages: tile it+NST-1 is requested while tile it is computed.
  for (int p = 0; p < NST - 1 && p < n_tiles; ++p) load(p, p);
  for (int it = 0; it < n_tiles; ++it) {
    // Tile `it` has landed once at most the loads of the tiles after it
    // (issued earlier) are still outstanding; the barrier then also certifies
    // that every wave is done with the stage refilled below.
    wait_vm(LPW * min(NST - 2, n_tiles - 1 - it));
    barrier_nofence();
    if (it + NST - 1 < n_tiles) load(it + NST - 1, (it + NST - 1) % NST);
    const int k0 = tile_of(it) * kKeyTile;
    // Element mask only on tiles some row cannot fully see.
    const bool full = (k0 + kKeyTile - 1 <= r0) &&
                      (k0 >= lo_last || (a.sink && k0 + kKeyTile <= sink_end));
    const int tt = t - k0, lt = lo_t - k0, se = sink_end - k0;
    fl.tile(lds + (it % NST) * Gm::STAGE, koff, vbase, qb, !full,
            [=](int kr) { return kr <= tt && (kr >= lt || kr < se); });
  }

  const float lsum = fl.total();
  if (t < r1) {
    const float inv = 1.0f / lsum;
    uint16_t* op = static_cast<uint16_t*>(a.o) + ((int64_t)(t - a.q_row0) * a.hq + head) * D;
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = m * 32 + q4 * 8 + hh * 4;
        const u32x2 w = {pack_bf16x2(fl.o[m][4 * q4 + 0] * inv, fl.o[m][4 * q4 + 1] * inv),
                         pack_bf16x2(fl.o[m][4 * q4 + 2] * inv, fl.o[m][4 * q4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d) = w;
      }
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
