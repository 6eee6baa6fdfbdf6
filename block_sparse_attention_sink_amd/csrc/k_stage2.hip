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
//   k_new_kv_bf16 / k_new_kv_f32   rotate the new tokens' K at their positions
//                                  and append K/V to the row's context buffer.
//   k_query_bf16<D, FUSED>         split-K flash attention of the packed
//                                  (token, head-in-group) rows of one KV head
//                                  over a segment list; FUSED reads pool blocks
//                                  directly and rotates K while staging it.
//   k_combine                      log-sum-exp merge of the split partials.
//   k_query_f32                    float32 rows (one wavefront per row).
#include "dbsa_device.hpp"

namespace dbsa {

// ---------------------------------------------------------------------------
// Gather + re-RoPE (materialised).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_gather_bf16(GatherArgs a) {
  constexpr int CP = D / 16;
  constexpr int TOK = 256 / CP;
  const int b = blockIdx.y;
  const int u = blockIdx.x * TOK + threadIdx.x / CP;
  const int c = threadIdx.x % CP;
  const int32_t* st = a.start + (int64_t)b * (a.n_ids + 1);
  if (u >= st[a.n_ids]) return;
  const int i = upper_index(st, a.n_ids, u);
  const int64_t src_tok = a.src[(int64_t)b * a.n_ids + i] + (u - st[i]);
  float cs[8], sn[8];
  rope_cs8(u, a.freq, 8 * c, cs, sn);
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
__global__ __launch_bounds__(256) void k_new_kv_bf16(NewKVArgs a) {
  constexpr int CP = D / 16, CR = D / 8;
  const int r = blockIdx.x, b = blockIdx.y;
  const int64_t pos = (int64_t)a.pos0[b] + r;
  const int64_t row = (int64_t)a.dst_row[b] + r;
  for (int u = threadIdx.x; u < a.hkv * CP; u += blockDim.x) {
    const int g = u / CP, c = u % CP;
    const int64_t src = ((((int64_t)b * a.n_new + r) * a.hkv) + g) * CR;
    const int64_t dst = (((int64_t)b * a.cap + row) * a.hkv + g) * CR;
    const u32x4* kp = reinterpret_cast<const u32x4*>(a.k_new);
    const u32x4* vp = reinterpret_cast<const u32x4*>(a.v_new);
    u32x4 k1 = kp[src + c], k2 = kp[src + c + CP];
    rope_rotate_chunk(k1, k2, pos, a.freq, 8 * c);
    u32x4* ko = reinterpret_cast<u32x4*>(a.k_dst);
    u32x4* vo = reinterpret_cast<u32x4*>(a.v_dst);
    ko[dst + c] = k1;
    ko[dst + c + CP] = k2;
    vo[dst + c] = vp[src + c];
    vo[dst + c + CP] = vp[src + c + CP];
  }
}

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
// Query attention, bf16 MFMA, split-K over the context.
//
// Workgroup = 8 wavefronts over 256 packed rows (row = token * G + head in
// group) of one KV head; every wavefront also stages its share of each 64-key
// K/V tile.  Lane layout and the softmax follow the prefill kernel.
// ---------------------------------------------------------------------------
template <int D, bool FUSED>
__global__ __launch_bounds__(512) void k_query_bf16(QueryArgs a) {
  using Gm = TileGeom<D>;
  constexpr int KS = D / 16, CP = D / 16;
  constexpr int UNITS = 64 * CP;         // (key, chunk pair) units per tile
  constexpr int UPT = (UNITS + 511) / 512;
  __shared__ __align__(16) char lds[2 * Gm::STAGE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5, col = lane & 31;
  const int split = blockIdx.x;
  const int g = blockIdx.y % a.hkv, rg = blockIdx.y / a.hkv, b = blockIdx.z;
  const int G = a.hq / a.hkv;
  const int wrow0 = rg * 256 + wave * kRowsPerWave;
  const bool wave_live = wrow0 < a.rows;
  const int rho = wrow0 + col;
  const bool live = rho < a.rows;
  const int r = live ? rho / G : 0;
  const int head = g * G + (live ? rho - (rho / G) * G : 0);
  const int pos0 = a.pos0[b];
  const int qpos = pos0 + r;

  const int nseg = a.seg.nseg[b];
  const int32_t* sst = a.seg.start + (int64_t)b * a.seg.seg_stride;
  const int32_t* ssrc = a.seg.src + (int64_t)b * a.seg.seg_stride;
  const int32_t* sbuf = a.seg.buf + (int64_t)b * a.seg.seg_stride;
  const int T = sst[nseg];
  const int n_tiles = (T + kKeyTile - 1) / kKeyTile;
  const int it0 = split * a.tiles_per_split;
  const int it1 = min(it0 + a.tiles_per_split, n_tiles);

  bf16x8 qb[KS];
  {
    u32x4 raw[KS];
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.q) + (((int64_t)b * a.n_new + r) * a.hq + head) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) raw[ks] = live ? qp[2 * ks + hh] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks)
      rope_rotate_chunk(raw[ks], raw[ks + KS / 2], qpos, a.freq, 16 * ks + 8 * hh, a.q_scale);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
  }

  const uint16_t* kpool = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* vpool = static_cast<const uint16_t*>(a.v_pool);
  const uint16_t* kctx = static_cast<const uint16_t*>(a.k_ctx);
  const uint16_t* vctx = static_cast<const uint16_t*>(a.v_ctx);

  // Staging registers of one tile: this thread's (key, chunk pair) units.
  u32x4 k1[UPT], k2[UPT], v1[UPT], v2[UPT];
  int upos[UPT];
  bool urot[UPT];

  auto fetch = [&](int it) {
    const int u0 = it * kKeyTile;
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
      const int unit = tid + 512 * x;
      const int key = unit / CP, c = unit - key * CP;
      const int u = u0 + key;
      upos[x] = u;
      urot[x] = false;
      k1[x] = k2[x] = v1[x] = v2[x] = u32x4{0u, 0u, 0u, 0u};
      if (unit < UNITS && u < T) {
        const int s = upper_index(sst, nseg, u);
        const int64_t tok = ssrc[s] + (u - sst[s]);
        const uint16_t* kr;
        const uint16_t* vr;
        if (FUSED && sbuf[s] == 0) {
          kr = kpool + (tok * a.hkv + g) * D;
          vr = vpool + (tok * a.hkv + g) * D;
          urot[x] = true;
        } else {
          const int64_t row = (((int64_t)b * a.cap + tok) * a.hkv + g) * D;
          kr = kctx + row;
          vr = vctx + row;
        }
        const u32x4* kq = reinterpret_cast<const u32x4*>(kr);
        const u32x4* vq = reinterpret_cast<const u32x4*>(vr);
        k1[x] = kq[c];
        k2[x] = kq[c + CP];
        v1[x] = vq[c];
        v2[x] = vq[c + CP];
      }
    }
  };
  // Rotate (pool tokens), then write K rows and V^T columns into a stage.
  auto stage = [&](int buf) {
    char* st = lds + buf * Gm::STAGE;
#pragma unroll
    for (int x = 0; x < UPT; ++x) {
      const int unit = tid + 512 * x;
      if (unit >= UNITS) continue;
      const int key = unit / CP, c = unit - key * CP;
      if (FUSED && urot[x]) rope_rotate_chunk(k1[x], k2[x], upos[x], a.freq, 8 * c);
      *reinterpret_cast<u32x4*>(st + key * Gm::KROW + Gm::k_phys(key, c) * 16) = k1[x];
      *reinterpret_cast<u32x4*>(st + key * Gm::KROW + Gm::k_phys(key, c + CP) * 16) = k2[x];
      // V^T: head dim d of this key goes to row d, chunk ch, element e.
      const int p = vt_pos_of_key(key & 15);
      const int ch = 2 * (key >> 4) + (p >> 3), e = p & 7;
      char* vt = st + Gm::KBYTES + e * 2;
      const uint32_t w1[4] = {v1[x].x, v1[x].y, v1[x].z, v1[x].w};
      const uint32_t w2[4] = {v2[x].x, v2[x].y, v2[x].z, v2[x].w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int d1 = 8 * c + q, d2 = D / 2 + 8 * c + q;
        *reinterpret_cast<uint16_t*>(vt + d1 * Gm::VROW + Gm::v_phys(d1, ch) * 16) =
            (uint16_t)(q & 1 ? w1[q >> 1] >> 16 : w1[q >> 1]);
        *reinterpret_cast<uint16_t*>(vt + d2 * Gm::VROW + Gm::v_phys(d2, ch) * 16) =
            (uint16_t)(q & 1 ? w2[q >> 1] >> 16 : w2[q >> 1]);
      }
    }
  };

  Flash<D> fl;
  fl.init();
  int koff[KS], voff[4];
  lane_offsets<D>(col, hh, koff, voff);

  if (it0 < it1) {
    fetch(it0);
    stage(0);
  }
  __syncthreads();
  for (int it = it0; it < it1; ++it) {
    const int cur = (it - it0) & 1;
    if (it + 1 < it1) fetch(it + 1);
    if (wave_live) {
      const char* st = lds + cur * Gm::STAGE;
      const int u0 = it * kKeyTile;
      const int lim = qpos - u0;  // keys kr <= lim are visible (causal over new tokens)
      fl.tile(st, koff, voff, qb, u0 + kKeyTile - 1 > pos0, [=](int kr) { return kr <= lim; });
    }
    if (it + 1 < it1) stage(cur ^ 1);
    __syncthreads();
  }

  if (!live) return;
  const float lsum = fl.total();
  if (a.n_split == 1) {
    const float inv = 1.0f / lsum;
    uint16_t* op = static_cast<uint16_t*>(a.o) + (((int64_t)b * a.n_new + r) * a.hq + head) * D;
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
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
    for (int m = 0; m < D / 32; ++m)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = m * 32 + q4 * 8 + hh * 4;
        *reinterpret_cast<f32x4*>(po + d) =
            f32x4{fl.o[m][4 * q4 + 0], fl.o[m][4 * q4 + 1], fl.o[m][4 * q4 + 2],
                  fl.o[m][4 * q4 + 3]};
      }
    if (hh == 0) {
      a.part_ml[prow * 2 + 0] = fl.m;
      a.part_ml[prow * 2 + 1] = lsum;
    }
  }
}

// ---------------------------------------------------------------------------
// Merge split partials: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(D) void k_combine(CombineArgs a) {
  const int rho = blockIdx.x, g = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const int G = a.hq / a.hkv;
  const int r = rho / G, head = g * G + rho % G;
  const int64_t base = ((int64_t)b * a.hkv + g) * a.n_split;
  // Reference = largest split reference among splits that saw a key; splits
  // with no keys (l = 0) contribute nothing.
  float M = kNegInf;
  for (int s = 0; s < a.n_split; ++s) {
    const int64_t prow = (base + s) * a.rows + rho;
    if (a.part_ml[prow * 2 + 1] > 0.0f) M = fmaxf(M, a.part_ml[prow * 2]);
  }
  float L = 0.0f, acc = 0.0f;
  for (int s = 0; s < a.n_split; ++s) {
    const int64_t prow = (base + s) * a.rows + rho;
    if (!(a.part_ml[prow * 2 + 1] > 0.0f)) continue;
    const float w = __builtin_amdgcn_exp2f(a.part_ml[prow * 2] - M);
    L += w * a.part_ml[prow * 2 + 1];
    acc += w * a.part_o[prow * D + d];
  }
  const int64_t o = (((int64_t)b * a.n_new + r) * a.hq + head) * D + d;
  if (BF16) static_cast<uint16_t*>(a.o)[o] = to_bf16(acc / L);
  else static_cast<float*>(a.o)[o] = acc / L;
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
  const int qpos = a.pos0[b] + r;
  const float* q = static_cast<const float*>(a.q) + (((int64_t)b * a.n_new + r) * a.hq + head) * D;
  float qr[D];
#pragma unroll
  for (int i = 0; i < H; ++i) {
    float c, s;
    rope_cs(qpos, a.freq.rev[i], c, s);
    qr[i] = rot_lo(q[i], q[i + H], c, s) * a.q_scale;
    qr[i + H] = rot_hi(q[i], q[i + H], c, s) * a.q_scale;
  }
  const int nseg = a.seg.nseg[b];
  const int32_t* sst = a.seg.start + (int64_t)b * a.seg.seg_stride;
  const int32_t* ssrc = a.seg.src + (int64_t)b * a.seg.seg_stride;
  const int32_t* sbuf = a.seg.buf + (int64_t)b * a.seg.seg_stride;
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
  if (dtype == 1) {
    if (head_dim == 128) hipLaunchKernelGGL(k_new_kv_f32<128>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(k_new_kv_f32<64>, grid, dim3(256), 0, stream, a);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL(k_new_kv_bf16<128>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(k_new_kv_bf16<64>, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_query(const QueryArgs& a, int batch, int head_dim, int dtype,
                        hipStream_t stream) {
  if (dtype == 1) {
    const dim3 grid((a.n_new * a.hq + 3) / 4, 1, batch);
    if (head_dim == 128) hipLaunchKernelGGL(k_query_f32<128>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(k_query_f32<64>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const bool fused = a.k_pool != nullptr;
  const dim3 grid(a.n_split, a.hkv * a.row_groups, batch);
  if (head_dim == 128) {
    if (fused) hipLaunchKernelGGL((k_query_bf16<128, true>), grid, dim3(512), 0, stream, a);
    else hipLaunchKernelGGL((k_query_bf16<128, false>), grid, dim3(512), 0, stream, a);
  } else {
    if (fused) hipLaunchKernelGGL((k_query_bf16<64, true>), grid, dim3(512), 0, stream, a);
    else hipLaunchKernelGGL((k_query_bf16<64, false>), grid, dim3(512), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int batch, int head_dim, int dtype,
                          hipStream_t stream) {
  const dim3 grid(a.rows, a.hkv, batch);
  if (head_dim == 128) {
    if (dtype == 1) hipLaunchKernelGGL((k_combine<128, false>), grid, dim3(128), 0, stream, a);
    else hipLaunchKernelGGL((k_combine<128, true>), grid, dim3(128), 0, stream, a);
  } else {
    if (dtype == 1) hipLaunchKernelGGL((k_combine<64, false>), grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL((k_combine<64, true>), grid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dbsa
