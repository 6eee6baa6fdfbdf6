// Host side of the DBSA library: argument checks, planning, workspace layout,
// per-call tables and kernel launches behind the C ABI in dbsa.h.
//
// Method: "Efficient Many-Shot In-Context Learning with Dynamic Block-Sparse
// Attention" (paper-notes page, ACL 2025), cited as [Notes, section].
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "dbsa.h"
#include "dbsa_internal.hpp"

namespace dbsa {
namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DBSA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// Argument checks (pure host code, no HIP calls).
// ---------------------------------------------------------------------------
int check_attn(const dbsa_attn_t* a) {
  if (!a) return fail(DBSA_EINVAL, "attn is NULL");
  if (a->n_q_heads < 1 || a->n_kv_heads < 1)
    return fail(DBSA_EINVAL, "head counts must be >= 1 (got %d q, %d kv)", a->n_q_heads,
                a->n_kv_heads);
  if (a->n_q_heads % a->n_kv_heads != 0)
    return fail(DBSA_EUNSUPPORTED, "n_q_heads %d is not a multiple of n_kv_heads %d",
                a->n_q_heads, a->n_kv_heads);
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(DBSA_EUNSUPPORTED, "head_dim %d not supported (64 or 128)", a->head_dim);
  if (a->dtype != DBSA_BF16 && a->dtype != DBSA_F32)
    return fail(DBSA_EUNSUPPORTED, "dtype %d not supported", a->dtype);
  if (!(a->rope_theta > 0.0) || !std::isfinite(a->rope_theta))
    return fail(DBSA_EINVAL, "rope_theta must be finite and > 0");
  if (!std::isfinite(a->softmax_scale)) return fail(DBSA_EINVAL, "softmax_scale not finite");
  if (a->rope_inv_freq)
    for (int i = 0; i < a->head_dim / 2; ++i)
      if (!(a->rope_inv_freq[i] >= 0.0) || !std::isfinite(a->rope_inv_freq[i]))
        return fail(DBSA_EINVAL, "rope_inv_freq[%d] must be finite and >= 0", i);
  return DBSA_OK;
}

// Block offsets [Notes, Method > Stage 1, item 1]; also checks the blocks.
int check_blocks(const dbsa_blocks_t* b, std::vector<int32_t>& off) {
  if (!b) return fail(DBSA_EINVAL, "blocks is NULL");
  if (b->n_blocks < 1) return fail(DBSA_EINVAL, "n_blocks must be >= 1 (got %d)", b->n_blocks);
  if (!b->block_lens) return fail(DBSA_EINVAL, "block_lens is NULL");
  if (b->sink != 0 && b->sink != 1) return fail(DBSA_EINVAL, "sink must be 0 or 1");
  if (b->j < 0) return fail(DBSA_EINVAL, "j must be >= 0 (got %d)", b->j);
  off.assign((size_t)b->n_blocks + 1, 0);
  int64_t total = 0;
  for (int i = 0; i < b->n_blocks; ++i) {
    if (b->block_lens[i] < 1)
      return fail(DBSA_EINVAL, "block %d has length %d (must be >= 1)", i, b->block_lens[i]);
    total += b->block_lens[i];
    if (total >= (int64_t(1) << 31) - 1024)
      return fail(DBSA_EINVAL, "pool too long (>= 2^31 tokens)");
    off[i + 1] = (int32_t)total;
  }
  return DBSA_OK;
}

// Selected ids [Notes, Method > Stage 2, items 1-2]: anchor first, distinct, in range.
int check_ids(const int32_t* ids, int32_t n_ids, int32_t batch, int32_t n_blocks) {
  if (!ids) return fail(DBSA_EINVAL, "ids is NULL");
  if (batch < 1) return fail(DBSA_EINVAL, "batch must be >= 1");
  if (n_ids < 1) return fail(DBSA_EINVAL, "n_ids must be >= 1");
  std::vector<char> seen((size_t)n_blocks);
  for (int b = 0; b < batch; ++b) {
    std::fill(seen.begin(), seen.end(), 0);
    const int32_t* row = ids + (int64_t)b * n_ids;
    if (row[0] != 0)
      return fail(DBSA_EINVAL, "ids row %d starts with %d: the anchor block 0 must come first", b,
                  row[0]);
    for (int i = 0; i < n_ids; ++i) {
      if (row[i] < 0 || row[i] >= n_blocks)
        return fail(DBSA_EINVAL, "ids[%d][%d] = %d out of range [0, %d)", b, i, row[i], n_blocks);
      if (seen[row[i]]) return fail(DBSA_EINVAL, "ids row %d repeats block %d", b, row[i]);
      seen[row[i]] = 1;
    }
  }
  return DBSA_OK;
}

RopeFreq make_freq(const dbsa_attn_t* a) {
  RopeFreq f;
  const int half = a->head_dim / 2;
  for (int i = 0; i < kMaxHalf; ++i) {
    const double w = i >= half ? 0.0
                     : a->rope_inv_freq ? a->rope_inv_freq[i]
                                        : std::pow(a->rope_theta, -2.0 * i / a->head_dim);
    f.rev[i] = w / (2.0 * M_PI);
  }
  return f;
}

float q_scale_of(const dbsa_attn_t* a) {
  const double s = a->softmax_scale > 0.0f ? a->softmax_scale : 1.0 / std::sqrt((double)a->head_dim);
  return (float)(s * 1.4426950408889634);
}

size_t elem_bytes(const dbsa_attn_t* a) { return a->dtype == DBSA_F32 ? 4 : 2; }

// ---------------------------------------------------------------------------
// Per-call tables that do not fit the kernel arguments: written into the
// workspace by k_upload launches on the caller's stream (kUploadInts ints per
// launch).  Nothing is staged in host memory and the host never waits.
// ---------------------------------------------------------------------------
constexpr size_t kMaxTableBytes = size_t(1) << 20;

int upload_ints(const int32_t* src, size_t n, void* dst, hipStream_t s) {
  for (size_t i = 0; i < n; i += kUploadInts) {
    UploadArgs ua;
    ua.dst = static_cast<int32_t*>(dst) + i;
    ua.n = (int32_t)std::min<size_t>(kUploadInts, n - i);
    std::memcpy(ua.v, src + i, (size_t)ua.n * sizeof(int32_t));
    const hipError_t e = launch_upload(ua, s);
    if (e != hipSuccess) return hip_fail(e, "launch upload");
  }
  return DBSA_OK;
}

// ---------------------------------------------------------------------------
// Stage 1 planning.
// ---------------------------------------------------------------------------
struct Stage1Plan {
  std::vector<int32_t> off;  // offsets of all blocks (incl. an appended block)
  int32_t n_tokens = 0;      // keys available (pool + appended block)
  int32_t row0 = 0, row1 = 0;
  int32_t sink_tiles = 0, win_tile0 = 0, win_tile1 = 0, n_slots = 0;
  int32_t n_split = 1;       // key splits per query tile (short walks: appends)
  int32_t pack_log2 = 0;     // query heads of a KV head per workgroup (log2), bf16
  // workspace layout
  size_t off_meta = 0, off_k = 0, off_po = 0, off_ml = 0, off_queue = 0, total = 0;
  size_t meta_bytes = 0;
};

// Key tiles a set of rows can see: the window [lo, end) of the rows' block
// plus the anchor; for a whole-pool prefill that is every tile.
void stage1_layout(const dbsa_attn_t* a, Stage1Plan& p, bool whole_pool, int sink, int j) {
  const int nb = (int)p.off.size() - 1;
  if (whole_pool) {
    p.sink_tiles = 0;
    p.win_tile0 = 0;
  } else {
    // rows are the last block (index nb - 1)
    const int lo = p.off[std::max(nb - 1 - j, 0)];
    p.win_tile0 = lo / kKeyTile;
    p.sink_tiles = (sink && lo > 0) ? std::min<int>((int)cdiv(p.off[1], kKeyTile), p.win_tile0) : 0;
  }
  p.win_tile1 = (int32_t)cdiv(p.n_tokens, kKeyTile);
  p.n_slots = p.sink_tiles + (p.win_tile1 - p.win_tile0);
  // GQA: up to kPrefillPackHeads query heads of one KV head share a
  // workgroup and each K/V tile it stages (256 rows = tokens x heads).
  p.pack_log2 = 0;
  if (a->dtype == DBSA_BF16) {
    const int G = a->n_q_heads / a->n_kv_heads;
    while ((2 << p.pack_log2) <= std::min(G, kPrefillPackHeads) && G % (2 << p.pack_log2) == 0)
      ++p.pack_log2;
  }
  // A short walk over few query tiles (an append) would leave most compute
  // units idle: cut its key tiles into parts, one workgroup each, aiming at
  // 256 workgroups and keeping at least 16 tiles per part.
  p.n_split = 1;
  if (!whole_pool && a->dtype == DBSA_BF16) {
    const int64_t wgs = cdiv(p.row1 - p.row0, kPrefillRows >> p.pack_log2) *
                        (a->n_q_heads >> p.pack_log2);
    const int64_t by_len = std::max<int64_t>(1, p.n_slots / 16);
    p.n_split = (int32_t)std::min<int64_t>({cdiv(256, wgs), by_len, 8});
  }
  p.meta_bytes = p.off.size() * sizeof(int32_t);
  p.off_meta = 0;
  size_t cur = align_up(p.meta_bytes);
  if (a->dtype == DBSA_BF16) {
    const size_t tile = (size_t)kKeyTile * a->head_dim * 2;
    p.off_k = cur;
    cur = align_up(cur + (size_t)a->n_kv_heads * p.n_slots * tile);
  }
  if (a->dtype == DBSA_BF16 && p.n_split == 1) {
    p.off_queue = cur;
    cur = align_up(cur + kPrefillQueueWords * sizeof(uint32_t));
  }
  if (p.n_split > 1) {
    const size_t prow = (size_t)p.n_split * (p.row1 - p.row0) * a->n_q_heads;
    p.off_po = cur;
    cur = align_up(cur + prow * a->head_dim * sizeof(float));
    p.off_ml = cur;
    cur = align_up(cur + prow * 2 * sizeof(float));
  }
  p.total = cur;
}

// Workgroups of a persistent grid: one per compute unit of the current
// device (each fills one).
int compute_units(int32_t* n) {
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "compute unit count");
  *n = std::max(n_cu, 1);
  return DBSA_OK;
}

int launch_stage1(const dbsa_attn_t* a, const dbsa_blocks_t* blk, const Stage1Plan& p,
                  const void* q, int32_t q_row0, const void* k, const void* v, void* o,
                  void* ws, hipStream_t s, bool upload_table = true) {
  char* w = static_cast<char*>(ws);
  // Block offsets: in the kernel arguments when they fit, else uploaded once
  // (layers after the first reuse the uploaded table).
  const bool inl = p.off.size() <= (size_t)kInlineInts;
  if (!inl && upload_table) {
    const int rc = upload_ints(p.off.data(), p.off.size(), w + p.off_meta, s);
    if (rc) return rc;
  }
  const RopeFreq freq = make_freq(a);
  PrefillArgs pa;
  pa.n_inline = inl ? (int32_t)p.off.size() : 0;
  if (inl) std::memcpy(pa.inl, p.off.data(), p.off.size() * sizeof(int32_t));
  pa.q = q;
  pa.o = o;
  pa.offsets = reinterpret_cast<const int32_t*>(w + p.off_meta);
  pa.n_blocks = (int32_t)p.off.size() - 1;
  pa.sink = blk->sink;
  pa.j = blk->j;
  pa.row0 = p.row0;
  pa.row1 = p.row1;
  pa.q_row0 = q_row0;
  pa.hq = a->n_q_heads;
  pa.hkv = a->n_kv_heads;
  pa.pack_log2 = p.pack_log2;
  pa.n_qtiles = (int32_t)cdiv(p.row1 - p.row0, kPrefillRows >> p.pack_log2);
  pa.n_keys = p.n_tokens;
  pa.v = v;
  pa.sink_tiles = p.sink_tiles;
  pa.win_tile0 = p.win_tile0;
  pa.n_slots = p.n_slots;
  pa.q_scale = q_scale_of(a);
  pa.freq = freq;
  pa.n_split = p.n_split;
  pa.part_o = p.n_split > 1 ? reinterpret_cast<float*>(w + p.off_po) : nullptr;
  pa.part_ml = p.n_split > 1 ? reinterpret_cast<float*>(w + p.off_ml) : nullptr;
  pa.queue = (a->dtype == DBSA_BF16 && p.n_split == 1) ? reinterpret_cast<uint32_t*>(w + p.off_queue)
                                                        : nullptr;
  pa.n_workers = 0;
  if (pa.queue != nullptr) {
    const int rc = compute_units(&pa.n_workers);
    if (rc) return rc;
  }
  if (a->dtype == DBSA_BF16) {
    PackArgs ka;
    ka.k = k;
    ka.k_tiles = w + p.off_k;
    ka.n_tokens = p.n_tokens;
    ka.hkv = a->n_kv_heads;
    ka.sink_tiles = p.sink_tiles;
    ka.win_tile0 = p.win_tile0;
    ka.win_tile1 = p.win_tile1;
    ka.n_slots = p.n_slots;
    ka.freq = freq;
    ka.queue = pa.queue;
    hipError_t e = launch_pack(ka, a->head_dim, a->dtype, s);
    if (e != hipSuccess) return hip_fail(e, "launch k_pack");
    pa.k_tiles = ka.k_tiles;
  } else {
    pa.k_tiles = k;  // f32 rows kernel reads the unrotated pool directly
  }
  hipError_t e = launch_prefill(pa, a->head_dim, a->dtype, s);
  if (e != hipSuccess) return hip_fail(e, "launch prefill");
  if (p.n_split > 1) {  // merge the key splits: rows = (new token, head in group)
    CombineArgs ca;
    ca.part_o = pa.part_o;
    ca.part_ml = pa.part_ml;
    ca.o = o;
    ca.n_new = p.row1 - p.row0;
    ca.hq = a->n_q_heads;
    ca.hkv = a->n_kv_heads;
    ca.rows = (p.row1 - p.row0) * (a->n_q_heads / a->n_kv_heads);
    ca.n_split = p.n_split;
    e = launch_combine(ca, 1, a->head_dim, a->dtype, s);
    if (e != hipSuccess) return hip_fail(e, "launch combine");
  }
  return DBSA_OK;
}

// ---------------------------------------------------------------------------
// Stage 2 planning.
// ---------------------------------------------------------------------------
struct SegPlan {
  std::vector<int32_t> tables;  // start | src | buf | nseg | pos0 | dst_row [| rot]
  int32_t stride = 0;
  size_t o_start = 0, o_src = 0, o_buf = 0, o_nseg = 0, o_pos0 = 0, o_dst = 0;  // int32 index
  int32_t o_rot = -1;           // index of the rotation offsets, -1: none
};

struct QueryPlan {
  int32_t rows = 0, row_waves = 4, key_ways = 1, row_groups = 0, n_split = 1, tiles_per_split = 1;
  bool partials = false;  // rows leave partials (merged by k_combine or k_merge) instead of O
  size_t off_meta = 0, off_po = 0, off_ml = 0, total = 0, meta_bytes = 0;
};

void query_split(const dbsa_attn_t* a, int32_t batch, int32_t n_new, int64_t max_ctx,
                 QueryPlan& qp) {
  const int G = a->n_q_heads / a->n_kv_heads;
  qp.rows = n_new * G;
  // 32 packed rows per attention wavefront, at most 4 per workgroup, the rows
  // spread evenly over the fewest row groups.
  qp.row_groups = (int32_t)cdiv(qp.rows, 128);
  qp.row_waves = (int32_t)cdiv(cdiv(qp.rows, qp.row_groups), 32);
  // Up to 64 rows: two wavefronts per 32 rows, each on one half of every key
  // tile, so that the matrix cores of all four SIMDs take part.
  qp.key_ways = qp.rows <= 64 ? 2 : 1;
  const int64_t n_tiles = std::max<int64_t>(1, cdiv(max_ctx, kKeyTile));
  qp.n_split = 1;
  qp.tiles_per_split = (int32_t)n_tiles;
  if (a->dtype == DBSA_BF16) {
    // One workgroup per CU fits (the LDS ring is 128 KiB): aim for ~256 of
    // them, never fewer than 4 tiles per split.
    const int64_t base = (int64_t)batch * a->n_kv_heads * qp.row_groups;
    const int64_t want = std::max<int64_t>(1, cdiv(256, base));
    const int64_t by_len = std::max<int64_t>(1, n_tiles / 4);
    const int64_t ns = std::min(want, by_len);
    qp.tiles_per_split = (int32_t)cdiv(n_tiles, ns);
    qp.n_split = (int32_t)cdiv(n_tiles, qp.tiles_per_split);
  }
}

// Workspace of a query launch: tables, then (split-K, or always when
// `partials`) the partial O and (m, l) of every row.
void query_layout(const dbsa_attn_t* a, int32_t batch, size_t meta_ints, QueryPlan& qp,
                  bool partials = false) {
  qp.meta_bytes = meta_ints * sizeof(int32_t);
  qp.off_meta = 0;
  size_t cur = align_up(qp.meta_bytes);
  qp.partials = partials || qp.n_split > 1;
  if (qp.partials) {
    const size_t prow = (size_t)batch * a->n_kv_heads * qp.n_split * qp.rows;
    qp.off_po = cur;
    cur = align_up(cur + prow * a->head_dim * sizeof(float));
    qp.off_ml = cur;
    cur = align_up(cur + prow * 2 * sizeof(float));
  }
  qp.total = cur;
}

size_t seg_meta_ints(int32_t batch, int32_t stride, bool rot = false) {
  return (size_t)batch * stride * 3 + (size_t)batch * (rot ? 4 : 3);
}

void seg_init(SegPlan& sp, int32_t batch, int32_t stride, bool rot = false) {
  sp.stride = stride;
  sp.tables.assign(seg_meta_ints(batch, stride, rot), 0);
  sp.o_rot = rot ? (int32_t)((size_t)batch * stride * 3 + (size_t)batch * 3) : -1;
  sp.o_start = 0;
  sp.o_src = (size_t)batch * stride;
  sp.o_buf = 2 * (size_t)batch * stride;
  sp.o_nseg = 3 * (size_t)batch * stride;
  sp.o_pos0 = sp.o_nseg + batch;
  sp.o_dst = sp.o_pos0 + batch;
}

int launch_query_path(const dbsa_attn_t* a, int32_t batch, int32_t n_new, const void* q,
                      const void* k_new, const void* v_new, const void* k_pool,
                      const void* v_pool, void* k_buf, void* v_buf, int64_t cap, void* o,
                      const SegPlan& sp, const QueryPlan& qp, void* ws, hipStream_t s,
                      bool partials_only = false) {
  char* w = static_cast<char*>(ws);
  const bool bf16 = a->dtype == DBSA_BF16;
  // bf16: small tables ride in the kernel arguments (no copy, no extra
  // queue operation); otherwise they are staged into the workspace.
  const bool inl = bf16 && sp.tables.size() <= (size_t)kInlineInts;
  const int32_t* dt = reinterpret_cast<const int32_t*>(w + qp.off_meta);
  if (!inl) {
    const int rc = upload_ints(sp.tables.data(), sp.tables.size(), w + qp.off_meta, s);
    if (rc) return rc;
  }
  const RopeFreq freq = make_freq(a);
  hipError_t e;
  if (!bf16) {
    NewKVArgs na;
    na.k_new = k_new;
    na.v_new = v_new;
    na.k_dst = k_buf;
    na.v_dst = v_buf;
    na.dst_row = dt + sp.o_dst;
    na.pos0 = dt + sp.o_pos0;
    na.n_new = n_new;
    na.hkv = a->n_kv_heads;
    na.cap = cap;
    na.freq = freq;
    e = launch_new_kv(na, batch, a->head_dim, a->dtype, s);
    if (e != hipSuccess) return hip_fail(e, "launch new_kv");
  }

  QueryArgs qa;
  qa.q = q;
  qa.k_pool = k_pool;
  qa.v_pool = v_pool;
  qa.k_ctx = k_buf;
  qa.v_ctx = v_buf;
  qa.k_new = k_new;
  qa.v_new = v_new;
  qa.o = o;
  qa.part_o = qp.partials ? reinterpret_cast<float*>(w + qp.off_po) : nullptr;
  qa.part_ml = qp.partials ? reinterpret_cast<float*>(w + qp.off_ml) : nullptr;
  qa.meta = inl ? nullptr : dt;
  qa.seg.o_start = (int32_t)sp.o_start;
  qa.seg.o_src = (int32_t)sp.o_src;
  qa.seg.o_buf = (int32_t)sp.o_buf;
  qa.seg.o_nseg = (int32_t)sp.o_nseg;
  qa.seg.o_pos0 = (int32_t)sp.o_pos0;
  qa.seg.o_dst = (int32_t)sp.o_dst;
  qa.seg.o_rot = sp.o_rot;
  qa.seg.stride = sp.stride;
  qa.n_inline = inl ? (int32_t)sp.tables.size() : 0;
  if (inl) std::memcpy(qa.inl, sp.tables.data(), sp.tables.size() * sizeof(int32_t));
  qa.n_new = n_new;
  qa.hq = a->n_q_heads;
  qa.hkv = a->n_kv_heads;
  qa.batch = batch;
  qa.rows = qp.rows;
  qa.row_waves = qp.row_waves;
  qa.key_ways = qp.key_ways;
  qa.row_groups = qp.row_groups;
  qa.n_split = qp.n_split;
  qa.tiles_per_split = qp.tiles_per_split;
  qa.cap = cap;
  qa.q_scale = q_scale_of(a);
  qa.freq = freq;
  e = launch_query(qa, batch, a->head_dim, a->dtype, s);
  if (e != hipSuccess) return hip_fail(e, "launch query");
  if (qp.n_split > 1 && !partials_only) {
    CombineArgs ca;
    ca.part_o = qa.part_o;
    ca.part_ml = qa.part_ml;
    ca.o = o;
    ca.n_new = n_new;
    ca.hq = a->n_q_heads;
    ca.hkv = a->n_kv_heads;
    ca.rows = qp.rows;
    ca.n_split = qp.n_split;
    e = launch_combine(ca, batch, a->head_dim, a->dtype, s);
    if (e != hipSuccess) return hip_fail(e, "launch combine");
  }
  return DBSA_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return DBSA_OK;
  if (!ws) return fail(DBSA_EINVAL, "workspace is NULL (%zu bytes needed)", need);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(DBSA_EINVAL, "workspace must be %zu-byte aligned", kAlign);
  if (ws_bytes < need)
    return fail(DBSA_ENOSPC, "workspace too small: %zu bytes given, %zu needed", ws_bytes, need);
  return DBSA_OK;
}

int check_ptrs(std::initializer_list<const void*> ps, const char* names) {
  for (const void* p : ps)
    if (!p) return fail(DBSA_EINVAL, "NULL tensor pointer among (%s)", names);
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) % 16)
      return fail(DBSA_EINVAL, "tensor pointers must be 16-byte aligned (%s)", names);
  return DBSA_OK;
}

int check_meta(size_t bytes) {
  if (bytes > kMaxTableBytes)
    return fail(DBSA_EUNSUPPORTED, "per-call tables of %zu bytes exceed the %zu-byte limit",
                bytes, kMaxTableBytes);
  return DBSA_OK;
}

// Plans shared by the entry points and dbsa_workspace_bytes.
int plan_prefill(const dbsa_attn_t* a, const dbsa_blocks_t* b, Stage1Plan& p) {
  int rc = check_attn(a);
  if (!rc) rc = check_blocks(b, p.off);
  if (rc) return rc;
  p.n_tokens = p.off.back();
  p.row0 = 0;
  p.row1 = p.n_tokens;
  stage1_layout(a, p, true, b->sink, b->j);
  return check_meta(p.meta_bytes);
}

int plan_append(const dbsa_attn_t* a, const dbsa_blocks_t* b, int64_t new_len, Stage1Plan& p) {
  int rc = check_attn(a);
  if (!rc) rc = check_blocks(b, p.off);
  if (rc) return rc;
  if (new_len < 1) return fail(DBSA_EINVAL, "new_len must be >= 1");
  const int64_t n_old = p.off.back();
  if (n_old + new_len >= (int64_t(1) << 31) - 1024) return fail(DBSA_EINVAL, "pool too long");
  p.off.push_back((int32_t)(n_old + new_len));
  p.n_tokens = (int32_t)(n_old + new_len);
  p.row0 = (int32_t)n_old;
  p.row1 = p.n_tokens;
  stage1_layout(a, p, false, b->sink, b->j);
  return check_meta(p.meta_bytes);
}

int plan_gather(const dbsa_attn_t* a, const dbsa_blocks_t* b, const int32_t* ids, int32_t n_ids,
                int32_t batch, std::vector<int32_t>* tables, std::vector<int64_t>* lens,
                size_t* meta_bytes) {
  std::vector<int32_t> off;
  int rc = check_attn(a);
  if (!rc) rc = check_blocks(b, off);
  if (rc) return rc;
  if (batch < 1) return fail(DBSA_EINVAL, "batch must be >= 1");
  if (n_ids < 1) return fail(DBSA_EINVAL, "n_ids must be >= 1");
  *meta_bytes = (size_t)batch * (2 * n_ids + 1) * sizeof(int32_t);
  rc = check_meta(*meta_bytes);
  if (rc || !ids) return rc;
  rc = check_ids(ids, n_ids, batch, b->n_blocks);
  if (rc) return rc;
  if (tables) {
    tables->assign((size_t)batch * (2 * n_ids + 1), 0);
    int32_t* st = tables->data();
    int32_t* src = st + (size_t)batch * (n_ids + 1);
    lens->assign(batch, 0);
    for (int r = 0; r < batch; ++r) {
      int64_t pos = 0;
      for (int i = 0; i < n_ids; ++i) {
        const int blkid = ids[(int64_t)r * n_ids + i];
        st[(int64_t)r * (n_ids + 1) + i] = (int32_t)pos;
        src[(int64_t)r * n_ids + i] = off[blkid];
        pos += off[blkid + 1] - off[blkid];
      }
      st[(int64_t)r * (n_ids + 1) + n_ids] = (int32_t)pos;
      (*lens)[r] = pos;
    }
  }
  return DBSA_OK;
}

// ---------------------------------------------------------------------------
// Shared-block schedule of a Stage-2 batch (see k_shared.hip): tables,
// workspace layout and the tail / new-token pass.
// ---------------------------------------------------------------------------
struct SharedPlan {
  std::vector<int32_t> tab;   // off | bstart | istart | pairs | kslot | ublk | uslot
  SharedTables t{};
  int32_t rq = 0, n_pairs = 0;
  SegPlan sp;                 // tail / new-token pass
  QueryPlan qp;
  size_t off_tab = 0, off_k = 0, off_po = 0, off_pl = 0, off_queue = 0, off_tail = 0, total = 0;
};

// K-image tiles of block b: relative to the block (tile i = its tokens 64 i ..).
int64_t tiles_of_block(const std::vector<int32_t>& off, int b) {
  return cdiv(off[b + 1] - off[b], kKeyTile);
}

// Workspace layout (also the bound dbsa_workspace_bytes reports, with every
// block counted as selected when `ids` is null).
void shared_layout(const dbsa_attn_t* a, int32_t batch, int32_t n_ids, SharedPlan& p) {
  const size_t d = (size_t)a->head_dim;
  p.off_tab = 0;
  size_t cur = align_up(p.tab.size() * sizeof(int32_t));
  p.off_k = cur;
  cur = align_up(cur + (size_t)a->n_kv_heads * p.t.n_slots * kKeyTile * d * 2);
  const size_t prow = (size_t)batch * a->n_kv_heads * n_ids * p.rq;
  p.off_po = cur;
  cur = align_up(cur + prow * d * 2);
  p.off_pl = cur;
  cur = align_up(cur + prow * sizeof(float));
  p.off_queue = cur;
  cur = align_up(cur + kPrefillQueueWords * sizeof(uint32_t));
  p.off_tail = cur;
  p.total = cur + p.qp.total;
}

// Tables of the shared schedule.  ids == nullptr: sizes only, every block
// counted as selected (a bound over all ids of this shape).
int plan_shared(const dbsa_attn_t* a, const std::vector<int32_t>& off, const int32_t* ids,
                int32_t n_ids, int32_t batch, int32_t n_new, const int64_t* tail_len,
                SharedPlan& p) {
  const int nb = (int)off.size() - 1;
  const int G = a->n_q_heads / a->n_kv_heads;
  if (batch >= (1 << 15) || n_ids >= (1 << 16))
    return fail(DBSA_EUNSUPPORTED, "batch %d / n_ids %d: at most 32767 rows of 65535 ids", batch,
                n_ids);
  if ((int64_t)n_new * G > (1 << 24)) return fail(DBSA_EUNSUPPORTED, "too many query rows");
  p.rq = n_new * G;
  std::vector<int32_t> cnt(nb, 0);
  if (ids) {
    for (int64_t k = 0; k < (int64_t)batch * n_ids; ++k) cnt[ids[k]]++;
  } else {
    std::fill(cnt.begin(), cnt.end(), batch);  // (bound: every block, every row)
  }
  p.n_pairs = batch * n_ids;
  p.t.n_blocks = nb;
  std::vector<int32_t> bstart(nb + 1, 0), istart(nb + 1, 0), kslot(nb, -1), ublk, uslot(1, 0);
  int64_t items = 0, slots = 0;
  for (int b = 0; b < nb; ++b) {
    bstart[b + 1] = bstart[b] + (ids ? cnt[b] : 0);
    items += cdiv((int64_t)cnt[b] * p.rq, kPrefillRows);
    istart[b + 1] = (int32_t)std::min<int64_t>(items, INT32_MAX);
    if (cnt[b] > 0) {
      kslot[b] = (int32_t)slots;
      ublk.push_back(b);
      slots += tiles_of_block(off, b);
      uslot.push_back((int32_t)std::min<int64_t>(slots, INT32_MAX));
    }
  }
  if (items * a->n_kv_heads >= INT32_MAX || slots >= INT32_MAX)
    return fail(DBSA_EUNSUPPORTED, "batch too large for one call");
  p.t.n_items = (int32_t)items;
  p.t.n_slots = (int32_t)slots;
  p.t.n_used = (int32_t)ublk.size();
  // Table block.
  p.t.o_off = 0;
  p.t.o_bstart = nb + 1;
  p.t.o_istart = 2 * (nb + 1);
  p.t.o_pairs = 3 * (nb + 1);
  p.t.o_kslot = p.t.o_pairs + 2 * p.n_pairs;
  p.t.o_ublk = p.t.o_kslot + nb;
  p.t.o_uslot = p.t.o_ublk + p.t.n_used;
  p.tab.assign((size_t)p.t.o_uslot + p.t.n_used + 1, 0);
  int32_t* tb = p.tab.data();
  std::copy(off.begin(), off.end(), tb + p.t.o_off);
  std::copy(bstart.begin(), bstart.end(), tb + p.t.o_bstart);
  std::copy(istart.begin(), istart.end(), tb + p.t.o_istart);
  std::copy(kslot.begin(), kslot.end(), tb + p.t.o_kslot);
  std::copy(ublk.begin(), ublk.end(), tb + p.t.o_ublk);
  std::copy(uslot.begin(), uslot.end(), tb + p.t.o_uslot);
  // Tail / new-token pass: per row, the tail buffer (virtual 0 .. tail_len)
  // and the new tokens after it, turned by the row's gathered length T'.
  int64_t max_tail = 0;
  for (int q = 0; q < batch; ++q) max_tail = std::max<int64_t>(max_tail, tail_len ? tail_len[q] : 0);
  seg_init(p.sp, batch, 3, true);
  if (ids) {
    std::vector<int32_t> fill(bstart.begin(), bstart.end() - 1);
    for (int q = 0; q < batch; ++q) {
      int64_t tp = 0;
      for (int i = 0; i < n_ids; ++i) {
        const int b = ids[(int64_t)q * n_ids + i];
        tp += off[b + 1] - off[b];
      }
      const int64_t pos0 = tp + tail_len[q];
      if (pos0 + n_new >= (int64_t(1) << 31) - 1024) return fail(DBSA_EINVAL, "context too long");
      int64_t start = 0;
      for (int i = 0; i < n_ids; ++i) {
        const int b = ids[(int64_t)q * n_ids + i];
        const int64_t shift = pos0 - start + off[b];  // Q turn of token 0 against pool-rotated keys
        if (shift + n_new >= (int64_t(1) << 31) - 1024)
          return fail(DBSA_EUNSUPPORTED, "pool position + context length exceeds 2^31");
        int32_t* pr = tb + p.t.o_pairs + 2 * (size_t)fill[b]++;
        pr[0] = (q << 16) | i;
        pr[1] = (int32_t)shift;
        start += off[b + 1] - off[b];
      }
      int32_t* t = p.sp.tables.data();
      const size_t r3 = (size_t)q * 3;
      t[p.sp.o_start + r3 + 0] = 0;
      t[p.sp.o_src + r3 + 0] = 0;
      t[p.sp.o_buf + r3 + 0] = 1;
      t[p.sp.o_start + r3 + 1] = (int32_t)tail_len[q];
      t[p.sp.o_src + r3 + 1] = 0;
      t[p.sp.o_buf + r3 + 1] = 2;
      t[p.sp.o_start + r3 + 2] = (int32_t)(tail_len[q] + n_new);
      t[p.sp.o_nseg + q] = 2;
      t[p.sp.o_pos0 + q] = (int32_t)tail_len[q];
      t[p.sp.o_dst + q] = (int32_t)tail_len[q];
      t[p.sp.o_rot + q] = (int32_t)tp;
    }
  }
  query_split(a, batch, n_new, max_tail + n_new, p.qp);
  query_layout(a, batch, p.sp.tables.size(), p.qp, true);
  shared_layout(a, batch, n_ids, p);
  return check_meta(std::max(p.tab.size(), p.sp.tables.size()) * sizeof(int32_t));
}

int launch_shared_path(const dbsa_attn_t* a, int32_t batch, int32_t n_ids, int32_t n_new,
                       int32_t n_tokens, const void* k_pool, const void* v_pool, const void* q,
                       const void* k_new, const void* v_new, void* k_tail, void* v_tail,
                       int64_t tail_capacity, void* o, const SharedPlan& p, void* ws,
                       hipStream_t s) {
  char* w = static_cast<char*>(ws);
  int rc = upload_ints(p.tab.data(), p.tab.size(), w + p.off_tab, s);
  if (rc) return rc;
  const RopeFreq freq = make_freq(a);
  const int32_t* tab = reinterpret_cast<const int32_t*>(w + p.off_tab);
  hipError_t e;
  if (p.t.n_slots > 0) {
    SharedPackArgs pk;
    pk.k = k_pool;
    pk.k_tiles = w + p.off_k;
    pk.tab = tab;
    pk.t = p.t;
    pk.n_tokens = n_tokens;
    pk.hkv = a->n_kv_heads;
    pk.freq = freq;
    pk.queue = reinterpret_cast<uint32_t*>(w + p.off_queue);
    e = launch_shared_pack(pk, a->head_dim, s);
    if (e != hipSuccess) return hip_fail(e, "launch shared pack");
    SharedArgs sa;
    sa.q = q;
    sa.k_tiles = w + p.off_k;
    sa.v = v_pool;
    sa.part_o = reinterpret_cast<uint16_t*>(w + p.off_po);
    sa.part_lam = reinterpret_cast<float*>(w + p.off_pl);
    sa.tab = tab;
    sa.t = p.t;
    sa.n_tokens = n_tokens;
    sa.n_ids = n_ids;
    sa.n_new = n_new;
    sa.hq = a->n_q_heads;
    sa.hkv = a->n_kv_heads;
    sa.rq = p.rq;
    sa.q_scale = q_scale_of(a);
    sa.freq = freq;
    sa.queue = pk.queue;
    rc = compute_units(&sa.n_workers);
    if (rc) return rc;
    e = launch_shared(sa, a->head_dim, s);
    if (e != hipSuccess) return hip_fail(e, "launch shared");
  }
  rc = launch_query_path(a, batch, n_new, q, k_new, v_new, nullptr, nullptr, k_tail, v_tail,
                         tail_capacity, o, p.sp, p.qp, w + p.off_tail, s, true);
  if (rc) return rc;
  MergeArgs ma;
  ma.part_o = reinterpret_cast<const uint16_t*>(w + p.off_po);
  ma.part_lam = reinterpret_cast<const float*>(w + p.off_pl);
  ma.tail_o = reinterpret_cast<const float*>(w + p.off_tail + p.qp.off_po);
  ma.tail_ml = reinterpret_cast<const float*>(w + p.off_tail + p.qp.off_ml);
  ma.o = o;
  ma.n_ids = n_ids;
  ma.n_split = p.qp.n_split;
  ma.rq = p.rq;
  ma.n_new = n_new;
  ma.hq = a->n_q_heads;
  ma.hkv = a->n_kv_heads;
  e = launch_merge(ma, batch, a->head_dim, s);
  if (e != hipSuccess) return hip_fail(e, "launch merge");
  return DBSA_OK;
}

}  // namespace
}  // namespace dbsa

using namespace dbsa;

extern "C" {

const char* dbsa_last_error(void) { return g_err; }

const char* dbsa_version(void) { return "dbsa-gfx950 0.1.0"; }

size_t dbsa_workspace_bytes(int op, const dbsa_attn_t* attn, const dbsa_blocks_t* blocks,
                            int64_t rows, int32_t batch, int32_t n_ids, int64_t max_ctx) {
  g_err[0] = 0;
  switch (op) {
    case DBSA_OP_PREFILL: {
      Stage1Plan p;
      return plan_prefill(attn, blocks, p) ? 0 : p.total;
    }
    case DBSA_OP_APPEND: {
      Stage1Plan p;
      return plan_append(attn, blocks, rows, p) ? 0 : p.total;
    }
    case DBSA_OP_GATHER: {
      size_t mb = 0;
      if (plan_gather(attn, blocks, nullptr, n_ids, batch, nullptr, nullptr, &mb)) return 0;
      return align_up(mb);
    }
    case DBSA_OP_GATHER_SPANS: {
      if (check_attn(attn)) return 0;
      if (batch < 1 || n_ids < 1) {
        fail(DBSA_EINVAL, "need batch >= 1 and n_spans >= 1");
        return 0;
      }
      const size_t mb = (size_t)batch * (2 * (size_t)n_ids + 1) * sizeof(int32_t);
      if (check_meta(mb)) return 0;
      return align_up(mb);
    }
    case DBSA_OP_QUERY_BATCHED: {
      std::vector<int32_t> off;
      if (check_attn(attn) || check_blocks(blocks, off)) return 0;
      if (batch < 1 || rows < 1 || n_ids < 1 || max_ctx < rows || max_ctx >= (int64_t(1) << 31)) {
        fail(DBSA_EINVAL, "need batch, n_new, n_ids >= 1 and n_new <= max_ctx < 2^31");
        return 0;
      }
      if (attn->dtype != DBSA_BF16)
        return dbsa_workspace_bytes(DBSA_OP_QUERY_GATHERED, attn, blocks, rows, batch, n_ids,
                                    max_ctx);
      SharedPlan p;
      std::vector<int64_t> tl(batch, max_ctx - rows);
      if (plan_shared(attn, off, nullptr, n_ids, batch, (int32_t)rows, tl.data(), p)) return 0;
      return p.total;
    }
    case DBSA_OP_QUERY:
    case DBSA_OP_QUERY_GATHERED:
    case DBSA_OP_QUERY_SPANS: {
      if (check_attn(attn)) return 0;
      if (batch < 1 || rows < 1 || max_ctx < rows || max_ctx >= (int64_t(1) << 31)) {
        fail(DBSA_EINVAL, "need batch >= 1, n_new >= 1 and n_new <= max_ctx < 2^31");
        return 0;
      }
      if (op != DBSA_OP_QUERY && n_ids < 1) {
        fail(DBSA_EINVAL, "n_ids (n_spans) must be >= 1");
        return 0;
      }
      const int32_t stride = op == DBSA_OP_QUERY ? 3 : n_ids + 3;
      QueryPlan qp;
      query_split(attn, batch, (int32_t)rows, max_ctx, qp);
      query_layout(attn, batch, seg_meta_ints(batch, stride), qp);
      if (check_meta(qp.meta_bytes)) return 0;
      return qp.total;
    }
    default:
      fail(DBSA_EINVAL, "unknown op %d", op);
      return 0;
  }
}

int dbsa_prefill(const dbsa_attn_t* attn, const dbsa_blocks_t* blocks, const void* q,
                 const void* k, const void* v, void* o, void* ws, size_t ws_bytes,
                 void* stream) {
  g_err[0] = 0;
  Stage1Plan p;
  int rc = plan_prefill(attn, blocks, p);
  if (!rc) rc = check_ptrs({q, k, v, o}, "q, k, v, o");
  if (!rc) rc = check_ws(ws, ws_bytes, p.total);
  if (rc) return rc;
  return launch_stage1(attn, blocks, p, q, 0, k, v, o, ws, static_cast<hipStream_t>(stream));
}

int dbsa_prefill_layers(const dbsa_attn_t* attn, const dbsa_blocks_t* blocks, int32_t n_layers,
                        const void* q, int64_t q_layer_stride, const void* k, const void* v,
                        int64_t kv_layer_stride, void* o, int64_t o_layer_stride, void* ws,
                        size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  Stage1Plan p;
  int rc = plan_prefill(attn, blocks, p);
  if (!rc) rc = check_ptrs({q, k, v, o}, "q, k, v, o");
  if (!rc) rc = check_ws(ws, ws_bytes, p.total);
  if (rc) return rc;
  if (n_layers < 1) return fail(DBSA_EINVAL, "n_layers must be >= 1");
  const int64_t eb = elem_bytes(attn);
  const int64_t q_extent = (int64_t)p.n_tokens * attn->n_q_heads * attn->head_dim;
  const int64_t kv_extent = (int64_t)p.n_tokens * attn->n_kv_heads * attn->head_dim;
  if (n_layers > 1) {
    if (o_layer_stride < q_extent)
      return fail(DBSA_EINVAL, "o_layer_stride %lld is below one layer of o (%lld elements)",
                  (long long)o_layer_stride, (long long)q_extent);
    if (q_layer_stride != 0 && q_layer_stride < q_extent)
      return fail(DBSA_EINVAL, "q_layer_stride must be 0 or >= %lld elements",
                  (long long)q_extent);
    if (kv_layer_stride != 0 && kv_layer_stride < kv_extent)
      return fail(DBSA_EINVAL, "kv_layer_stride must be 0 or >= %lld elements",
                  (long long)kv_extent);
    if ((q_layer_stride * eb) % 16 || (kv_layer_stride * eb) % 16 || (o_layer_stride * eb) % 16)
      return fail(DBSA_EINVAL, "layer strides must be multiples of 16 bytes");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t l = 0; l < n_layers; ++l) {
    const char* ql = static_cast<const char*>(q) + l * q_layer_stride * eb;
    const char* kl = static_cast<const char*>(k) + l * kv_layer_stride * eb;
    const char* vl = static_cast<const char*>(v) + l * kv_layer_stride * eb;
    char* ol = static_cast<char*>(o) + l * o_layer_stride * eb;
    rc = launch_stage1(attn, blocks, p, ql, 0, kl, vl, ol, ws, s, l == 0);
    if (rc) return rc;
  }
  return DBSA_OK;
}

int dbsa_append_block(const dbsa_attn_t* attn, const dbsa_blocks_t* existing, int32_t new_len,
                      const void* q_new, const void* k_new, const void* v_new, void* k_cache,
                      void* v_cache, int64_t cache_capacity_tokens, void* o_new, void* ws,
                      size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  Stage1Plan p;
  int rc = plan_append(attn, existing, new_len, p);
  if (!rc) rc = check_ptrs({q_new, k_new, v_new, k_cache, v_cache, o_new},
                           "q_new, k_new, v_new, k_cache, v_cache, o_new");
  if (!rc && p.n_tokens > cache_capacity_tokens)
    rc = fail(DBSA_ENOSPC, "cache holds %lld tokens, %d needed", (long long)cache_capacity_tokens,
              p.n_tokens);
  if (!rc) rc = check_ws(ws, ws_bytes, p.total);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The new block's K/V join the unrotated cache [Notes, Method > Stage 1, items 3-4].
  const size_t row_bytes = (size_t)attn->n_kv_heads * attn->head_dim * elem_bytes(attn);
  char* kc = static_cast<char*>(k_cache) + (size_t)p.row0 * row_bytes;
  char* vc = static_cast<char*>(v_cache) + (size_t)p.row0 * row_bytes;
  hipError_t e = hipMemcpyAsync(kc, k_new, (size_t)new_len * row_bytes, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(vc, v_new, (size_t)new_len * row_bytes, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(append K/V)");
  return launch_stage1(attn, existing, p, q_new, p.row0, k_cache, v_cache, o_new, ws, s);
}

}  // extern "C"

namespace {

// Pool token spans of each batch row (source token, length), in context
// order: empty spans dropped, back-to-back spans merged.
typedef std::vector<std::vector<std::pair<int32_t, int32_t>>> RowSpans;

void add_span(std::vector<std::pair<int32_t, int32_t>>& row, int32_t src, int32_t len) {
  if (len <= 0) return;
  if (!row.empty() && row.back().first + row.back().second == src) {
    row.back().second += len;
    return;
  }
  row.emplace_back(src, len);
}

// Blocks given by id (anchor first): one span per block.
RowSpans spans_of_ids(const std::vector<int32_t>& off, const int32_t* ids, int32_t n_ids,
                      int32_t batch) {
  RowSpans rs(batch);
  for (int b = 0; b < batch; ++b)
    for (int i = 0; i < n_ids; ++i) {
      const int blkid = ids[(int64_t)b * n_ids + i];
      add_span(rs[b], off[blkid], off[blkid + 1] - off[blkid]);
    }
  return rs;
}

int check_spans(const int32_t* span_src, const int32_t* span_len, int32_t n_spans, int32_t batch,
                int64_t pool_tokens, RowSpans& rs) {
  if (!span_src || !span_len) return fail(DBSA_EINVAL, "span_src or span_len is NULL");
  if (batch < 1) return fail(DBSA_EINVAL, "batch must be >= 1");
  if (n_spans < 1) return fail(DBSA_EINVAL, "n_spans must be >= 1");
  if (pool_tokens < 1 || pool_tokens >= (int64_t(1) << 31))
    return fail(DBSA_EINVAL, "pool_tokens must be in [1, 2^31)");
  rs.assign(batch, {});
  for (int b = 0; b < batch; ++b) {
    int64_t total = 0;
    for (int i = 0; i < n_spans; ++i) {
      const int64_t k = (int64_t)b * n_spans + i;
      const int64_t src = span_src[k], len = span_len[k];
      if (len < 0 || src < 0 || src + len > pool_tokens)
        return fail(DBSA_EINVAL, "span [%d][%d] = (%lld, %lld) outside the pool of %lld tokens", b,
                    i, (long long)src, (long long)len, (long long)pool_tokens);
      total += len;
      add_span(rs[b], (int32_t)src, (int32_t)len);
    }
    if (total < 1) return fail(DBSA_EINVAL, "batch row %d selects no tokens", b);
    if (total >= (int64_t(1) << 31) - 1024) return fail(DBSA_EINVAL, "context too long");
  }
  return DBSA_OK;
}

size_t max_spans(const RowSpans& rs) {
  size_t n = 0;
  for (const auto& r : rs) n = std::max(n, r.size());
  return n;
}

// Gather + re-RoPE of pool spans (see RowSpans): row b's spans are written in
// order at positions 0..T'_b-1.  Tables: start [batch][n + 1] | src [batch][n]
// with n = the most spans of any row (shorter rows padded with empty spans).
int gather_spans(const dbsa_attn_t* attn, const RowSpans& rs, int32_t batch, const void* k_pool,
                 const void* v_pool, void* k_out, void* v_out, int64_t out_capacity_tokens,
                 int64_t* ctx_len_out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_ptrs({k_pool, v_pool, k_out, v_out}, "k_pool, v_pool, k_out, v_out");
  if (!rc && !ctx_len_out) rc = fail(DBSA_EINVAL, "ctx_len_out is NULL");
  if (rc) return rc;
  const int32_t n = (int32_t)max_spans(rs);
  const size_t mb = (size_t)batch * (2 * n + 1) * sizeof(int32_t);
  rc = check_meta(mb);
  if (rc) return rc;
  std::vector<int32_t> tables((size_t)batch * (2 * n + 1), 0);
  int32_t* st = tables.data();
  int32_t* src = st + (size_t)batch * (n + 1);
  int64_t max_len = 0;
  std::vector<int64_t> lens(batch, 0);
  for (int r = 0; r < batch; ++r) {
    int64_t pos = 0;
    for (int i = 0; i < n; ++i) {
      st[(int64_t)r * (n + 1) + i] = (int32_t)pos;
      if (i < (int)rs[r].size()) {
        src[(int64_t)r * n + i] = rs[r][i].first;
        pos += rs[r][i].second;
      }
    }
    st[(int64_t)r * (n + 1) + n] = (int32_t)pos;
    lens[r] = pos;
    max_len = std::max(max_len, pos);
  }
  if (max_len > out_capacity_tokens)
    return fail(DBSA_ENOSPC, "gathered context of %lld tokens exceeds out_capacity_tokens %lld",
                (long long)max_len, (long long)out_capacity_tokens);
  rc = check_ws(ws, ws_bytes, align_up(mb));
  if (rc) return rc;
  for (int r = 0; r < batch; ++r) ctx_len_out[r] = lens[r];
  hipStream_t s = static_cast<hipStream_t>(stream);
  GatherArgs ga;
  const bool inl = tables.size() <= (size_t)kInlineInts;
  if (inl) {
    std::memcpy(ga.inl, tables.data(), tables.size() * sizeof(int32_t));
  } else {
    rc = upload_ints(tables.data(), tables.size(), ws, s);
    if (rc) return rc;
  }
  ga.n_inline = inl ? (int32_t)tables.size() : 0;
  ga.tab = static_cast<const int32_t*>(ws);
  ga.batch = batch;
  ga.k_pool = k_pool;
  ga.v_pool = v_pool;
  ga.k_out = k_out;
  ga.v_out = v_out;
  ga.n_ids = n;
  ga.hkv = attn->n_kv_heads;
  ga.cap = out_capacity_tokens;
  ga.max_len = (int32_t)max_len;
  ga.freq = make_freq(attn);
  hipError_t e = launch_gather(ga, batch, attn->head_dim, attn->dtype, s);
  if (e != hipSuccess) return hip_fail(e, "launch gather");
  return DBSA_OK;
}

}  // namespace

extern "C" {

int dbsa_gather_rope(const dbsa_attn_t* attn, const dbsa_blocks_t* blocks, const int32_t* ids,
                     int32_t n_ids, int32_t batch, const void* k_pool, const void* v_pool,
                     void* k_out, void* v_out, int64_t out_capacity_tokens, int64_t* ctx_len_out,
                     void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  std::vector<int32_t> off;
  int rc = check_attn(attn);
  if (!rc) rc = check_blocks(blocks, off);
  if (!rc) rc = check_ids(ids, n_ids, batch, blocks->n_blocks);
  if (rc) return rc;
  return gather_spans(attn, spans_of_ids(off, ids, n_ids, batch), batch, k_pool, v_pool, k_out,
                      v_out, out_capacity_tokens, ctx_len_out, ws, ws_bytes, stream);
}

int dbsa_gather_rope_spans(const dbsa_attn_t* attn, const int32_t* span_src,
                           const int32_t* span_len, int32_t n_spans, int32_t batch,
                           int64_t pool_tokens, const void* k_pool, const void* v_pool,
                           void* k_out, void* v_out, int64_t out_capacity_tokens,
                           int64_t* ctx_len_out, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  RowSpans rs;
  int rc = check_attn(attn);
  if (!rc) rc = check_spans(span_src, span_len, n_spans, batch, pool_tokens, rs);
  if (rc) return rc;
  return gather_spans(attn, rs, batch, k_pool, v_pool, k_out, v_out, out_capacity_tokens,
                      ctx_len_out, ws, ws_bytes, stream);
}

int dbsa_query_attn(const dbsa_attn_t* attn, int32_t batch, int32_t n_new, const void* q,
                    const void* k_new, const void* v_new, void* k_ctx, void* v_ctx,
                    const int64_t* ctx_len, int64_t ctx_capacity, void* o, void* ws,
                    size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  int rc = check_attn(attn);
  if (rc) return rc;
  if (batch < 1) return fail(DBSA_EINVAL, "batch must be >= 1");
  if (n_new < 0) return fail(DBSA_EINVAL, "n_new must be >= 0");
  if (n_new == 0) return DBSA_OK;  // nothing to attend
  if (!ctx_len) return fail(DBSA_EINVAL, "ctx_len is NULL");
  rc = check_ptrs({q, k_new, v_new, k_ctx, v_ctx, o}, "q, k_new, v_new, k_ctx, v_ctx, o");
  if (rc) return rc;
  int64_t max_ctx = 0;
  for (int b = 0; b < batch; ++b) {
    if (ctx_len[b] < 0) return fail(DBSA_EINVAL, "ctx_len[%d] < 0", b);
    if (ctx_len[b] + n_new > ctx_capacity)
      return fail(DBSA_ENOSPC, "ctx_len[%d] + n_new = %lld exceeds ctx_capacity %lld", b,
                  (long long)(ctx_len[b] + n_new), (long long)ctx_capacity);
    max_ctx = std::max(max_ctx, ctx_len[b] + n_new);
  }
  if (max_ctx >= (int64_t(1) << 31) - 1024) return fail(DBSA_EINVAL, "context too long");
  QueryPlan qp;
  query_split(attn, batch, n_new, max_ctx, qp);
  SegPlan sp;
  seg_init(sp, batch, 3);
  query_layout(attn, batch, sp.tables.size(), qp);
  rc = check_meta(qp.meta_bytes);
  if (!rc) rc = check_ws(ws, ws_bytes, qp.total);
  if (rc) return rc;
  // bf16: context buffer rows [0, ctx_len), then the new tokens read from
  // k_new / v_new.  float32: the new tokens are appended first (new_kv) and
  // the whole range is read from the context buffer.
  const bool bf16 = attn->dtype == DBSA_BF16;
  for (int b = 0; b < batch; ++b) {
    int32_t* t = sp.tables.data() + 0;
    const size_t r3 = (size_t)b * 3;
    const int32_t cl = (int32_t)ctx_len[b];
    t[sp.o_start + r3 + 0] = 0;
    t[sp.o_src + r3 + 0] = 0;
    t[sp.o_buf + r3 + 0] = 1;
    if (bf16) {
      t[sp.o_start + r3 + 1] = cl;
      t[sp.o_src + r3 + 1] = 0;
      t[sp.o_buf + r3 + 1] = 2;
      t[sp.o_start + r3 + 2] = cl + n_new;
      t[sp.o_nseg + b] = 2;
    } else {
      t[sp.o_start + r3 + 1] = cl + n_new;
      t[sp.o_nseg + b] = 1;
    }
    t[sp.o_pos0 + b] = cl;
    t[sp.o_dst + b] = cl;
  }
  return launch_query_path(attn, batch, n_new, q, k_new, v_new, nullptr, nullptr, k_ctx, v_ctx,
                           ctx_capacity, o, sp, qp, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

int scratch_of_current_device(void** out);

// Query tokens over pool spans gathered and re-rotated inside the attention's
// loads, then the row's tail buffer, then (bf16) the new tokens.  With
// static_scratch, `ws` is ignored: the library's scratch array (ws_bytes
// long) serves as the workspace.
int query_spans(const dbsa_attn_t* attn, const RowSpans& rs, int32_t batch,
                const void* k_pool, const void* v_pool, int32_t n_new, const void* q,
                const void* k_new, const void* v_new, void* k_tail, void* v_tail,
                const int64_t* tail_len, int64_t tail_capacity, void* o, void* ws,
                size_t ws_bytes, void* stream, bool static_scratch = false) {
  if (n_new == 0) return DBSA_OK;
  if (!tail_len) return fail(DBSA_EINVAL, "tail_len is NULL");
  int rc = check_ptrs({k_pool, v_pool, q, k_new, v_new, k_tail, v_tail, o},
                      "k_pool, v_pool, q, k_new, v_new, k_tail, v_tail, o");
  if (rc) return rc;
  const int32_t n_sp = (int32_t)max_spans(rs);
  if (n_sp + 2 > kMaxSegments)
    return fail(DBSA_EUNSUPPORTED,
                "%d pool spans (after merging back-to-back ones) exceed the %d supported per row",
                n_sp, kMaxSegments - 2);
  // Segments: the pool spans (rotated on load), then the row's tail buffer,
  // then (bf16) the new tokens read from k_new / v_new; float32 appends the
  // new tokens to the tail buffer first and reads them there.
  const bool bf16 = attn->dtype == DBSA_BF16;
  const int32_t stride = n_sp + 3;
  SegPlan sp;
  seg_init(sp, batch, stride);
  int64_t max_ctx = 0;
  for (int b = 0; b < batch; ++b) {
    if (tail_len[b] < 0) return fail(DBSA_EINVAL, "tail_len[%d] < 0", b);
    if (tail_len[b] + n_new > tail_capacity)
      return fail(DBSA_ENOSPC, "tail_len[%d] + n_new = %lld exceeds tail_capacity %lld", b,
                  (long long)(tail_len[b] + n_new), (long long)tail_capacity);
    int32_t* t = sp.tables.data();
    const size_t row = (size_t)b * stride;
    const int ns = (int)rs[b].size();
    int64_t pos = 0;
    for (int i = 0; i < ns; ++i) {
      t[sp.o_start + row + i] = (int32_t)pos;
      t[sp.o_src + row + i] = rs[b][i].first;
      t[sp.o_buf + row + i] = 0;
      pos += rs[b][i].second;
    }
    const int64_t total = pos + tail_len[b] + n_new;
    if (total >= (int64_t(1) << 31) - 1024) return fail(DBSA_EINVAL, "context too long");
    t[sp.o_start + row + ns] = (int32_t)pos;  // tail segment
    t[sp.o_src + row + ns] = 0;
    t[sp.o_buf + row + ns] = 1;
    if (bf16) {
      t[sp.o_start + row + ns + 1] = (int32_t)(pos + tail_len[b]);  // new tokens
      t[sp.o_src + row + ns + 1] = 0;
      t[sp.o_buf + row + ns + 1] = 2;
      t[sp.o_start + row + ns + 2] = (int32_t)total;
      t[sp.o_nseg + b] = ns + 2;
    } else {
      t[sp.o_start + row + ns + 1] = (int32_t)total;
      t[sp.o_nseg + b] = ns + 1;
    }
    t[sp.o_pos0 + b] = (int32_t)(pos + tail_len[b]);
    t[sp.o_dst + b] = (int32_t)tail_len[b];
    max_ctx = std::max(max_ctx, total);
  }
  QueryPlan qp;
  query_split(attn, batch, n_new, max_ctx, qp);
  query_layout(attn, batch, sp.tables.size(), qp);
  rc = check_meta(qp.meta_bytes);
  if (!rc && static_scratch) {
    // The library's own scratch array: its size is checked before the first
    // HIP call, then its device address is looked up.
    if (qp.total > ws_bytes)
      rc = fail(DBSA_ENOSPC,
                "this call needs %zu bytes of scratch; the no-allocation entry point has a fixed "
                "%zu-byte scratch array (fewer query tokens or a smaller batch per call fit)",
                qp.total, ws_bytes);
    if (!rc) rc = scratch_of_current_device(&ws);
  }
  if (!rc) rc = check_ws(ws, ws_bytes, qp.total);
  if (rc) return rc;
  return launch_query_path(attn, batch, n_new, q, k_new, v_new, k_pool, v_pool, k_tail, v_tail,
                           tail_capacity, o, sp, qp, ws, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

int dbsa_query_attn_gathered(const dbsa_attn_t* attn, const dbsa_blocks_t* blocks,
                             const int32_t* ids, int32_t n_ids, int32_t batch,
                             const void* k_pool, const void* v_pool, int32_t n_new,
                             const void* q, const void* k_new, const void* v_new, void* k_tail,
                             void* v_tail, const int64_t* tail_len, int64_t tail_capacity,
                             void* o, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  std::vector<int32_t> off;
  int rc = check_attn(attn);
  if (!rc) rc = check_blocks(blocks, off);
  if (rc) return rc;
  if (batch < 1) return fail(DBSA_EINVAL, "batch must be >= 1");
  if (n_new < 0) return fail(DBSA_EINVAL, "n_new must be >= 0");
  rc = check_ids(ids, n_ids, batch, blocks->n_blocks);
  if (rc) return rc;
  if (n_new == 0) return DBSA_OK;
  return query_spans(attn, spans_of_ids(off, ids, n_ids, batch), batch, k_pool, v_pool, n_new, q,
                     k_new, v_new, k_tail, v_tail, tail_len, tail_capacity, o, ws, ws_bytes,
                     stream);
}

int dbsa_query_attn_batched(const dbsa_attn_t* attn, const dbsa_blocks_t* blocks,
                            const int32_t* ids, int32_t n_ids, int32_t batch, const void* k_pool,
                            const void* v_pool, int32_t n_new, const void* q, const void* k_new,
                            const void* v_new, void* k_tail, void* v_tail,
                            const int64_t* tail_len, int64_t tail_capacity, void* o, void* ws,
                            size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  std::vector<int32_t> off;
  int rc = check_attn(attn);
  if (!rc) rc = check_blocks(blocks, off);
  if (rc) return rc;
  if (batch < 1) return fail(DBSA_EINVAL, "batch must be >= 1");
  if (n_new < 0) return fail(DBSA_EINVAL, "n_new must be >= 0");
  rc = check_ids(ids, n_ids, batch, blocks->n_blocks);
  if (rc) return rc;
  if (n_new == 0) return DBSA_OK;
  if (attn->dtype != DBSA_BF16)  // the float32 path has no shared schedule: same result per row
    return dbsa_query_attn_gathered(attn, blocks, ids, n_ids, batch, k_pool, v_pool, n_new, q,
                                    k_new, v_new, k_tail, v_tail, tail_len, tail_capacity, o, ws,
                                    ws_bytes, stream);
  if (!tail_len) return fail(DBSA_EINVAL, "tail_len is NULL");
  rc = check_ptrs({k_pool, v_pool, q, k_new, v_new, k_tail, v_tail, o},
                  "k_pool, v_pool, q, k_new, v_new, k_tail, v_tail, o");
  if (rc) return rc;
  for (int b = 0; b < batch; ++b) {
    if (tail_len[b] < 0) return fail(DBSA_EINVAL, "tail_len[%d] < 0", b);
    if (tail_len[b] + n_new > tail_capacity)
      return fail(DBSA_ENOSPC, "tail_len[%d] + n_new = %lld exceeds tail_capacity %lld", b,
                  (long long)(tail_len[b] + n_new), (long long)tail_capacity);
  }
  SharedPlan p;
  rc = plan_shared(attn, off, ids, n_ids, batch, n_new, tail_len, p);
  if (!rc) rc = check_ws(ws, ws_bytes, p.total);
  if (rc) return rc;
  return launch_shared_path(attn, batch, n_ids, n_new, off.back(), k_pool, v_pool, q, k_new, v_new,
                            k_tail, v_tail, tail_capacity, o, p, ws,
                            static_cast<hipStream_t>(stream));
}

int dbsa_query_attn_spans(const dbsa_attn_t* attn, const int32_t* span_src,
                          const int32_t* span_len, int32_t n_spans, int32_t batch,
                          int64_t pool_tokens, const void* k_pool, const void* v_pool,
                          int32_t n_new, const void* q, const void* k_new, const void* v_new,
                          void* k_tail, void* v_tail, const int64_t* tail_len,
                          int64_t tail_capacity, void* o, void* ws, size_t ws_bytes,
                          void* stream) {
  g_err[0] = 0;
  RowSpans rs;
  int rc = check_attn(attn);
  if (!rc) rc = check_spans(span_src, span_len, n_spans, batch, pool_tokens, rs);
  if (rc) return rc;
  if (n_new < 0) return fail(DBSA_EINVAL, "n_new must be >= 0");
  if (n_new == 0) return DBSA_OK;
  return query_spans(attn, rs, batch, k_pool, v_pool, n_new, q, k_new, v_new, k_tail, v_tail,
                     tail_len, tail_capacity, o, ws, ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The no-allocation variant of dbsa_query_attn_gathered, for callers that
// cannot allocate (HIP graph capture, tight serving loops, harnesses that
// forbid allocation).  Its scratch (split-K partials and the per-call tables
// that do not fit the kernel arguments) is this file-scope device array: one
// copy per GPU, loaded with the library's code object and held until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// handed to kernels.  Calls on one GPU share the array: calls that may overlap
// on one GPU (two streams) race.  Nothing in it has to start at zero: every
// call writes each scratch byte it later reads.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = size_t(DBSA_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DBSA_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % kAlign)
      return fail(DBSA_EHIP, "scratch array has no usable device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DBSA_OK;
}

}  // namespace

extern "C" {

int dbsa_query_attn_gathered_noalloc(const dbsa_attn_t* attn, const dbsa_blocks_t* blocks,
                                     const int32_t* ids, int32_t n_ids, int32_t batch,
                                     const void* k_pool, const void* v_pool, int32_t n_new,
                                     const void* q, const void* k_new, const void* v_new,
                                     void* k_tail, void* v_tail, const int64_t* tail_len,
                                     int64_t tail_capacity, void* o, void* stream) {
  g_err[0] = 0;
  std::vector<int32_t> off;
  int rc = check_attn(attn);
  if (!rc) rc = check_blocks(blocks, off);
  if (rc) return rc;
  if (batch < 1) return fail(DBSA_EINVAL, "batch must be >= 1");
  if (n_new < 0) return fail(DBSA_EINVAL, "n_new must be >= 0");
  rc = check_ids(ids, n_ids, batch, blocks->n_blocks);
  if (rc) return rc;
  if (n_new == 0) return DBSA_OK;
  return query_spans(attn, spans_of_ids(off, ids, n_ids, batch), batch, k_pool, v_pool, n_new, q,
                     k_new, v_new, k_tail, v_tail, tail_len, tail_capacity, o, nullptr,
                     kScratchBytes, stream, true);
}

}  // extern "C"
