// Internal declarations shared by the host library and the gfx950 kernels.
//
// Method: "Efficient Many-Shot In-Context Learning with Dynamic Block-Sparse
// Attention" (paper-notes page, ACL 2025), cited as [Notes, section].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dbsa {

// ---------------------------------------------------------------------------
// Tiling constants of the bf16 MFMA kernels.
// ---------------------------------------------------------------------------
constexpr int kKeyTile = 64;      // keys per K/V tile (one LDS stage)
constexpr int kRowsPerWave = 32;  // query rows per wavefront (MFMA N dimension)
constexpr int kPrefillWaves = 8;  // waves per prefill workgroup (2 per SIMD)
constexpr int kPrefillRows = kRowsPerWave * kPrefillWaves;  // 256 query rows per workgroup
constexpr int kPrefillStages = 4;  // LDS stages per K ring and per V ring
constexpr int kPrefillPackHeads = 4;  // most query heads of one KV head per prefill workgroup
constexpr int kPrefillQueueWords = 8;  // prefill work counters, one per XCD
constexpr int kMaxSegments = 1024;  // context segments per batch row in Stage 2
constexpr int kQueryLoaders = 4;   // Stage-2 wavefronts that load and rotate the tiles
constexpr int kQueryLead = 3;      // tiles each of their threads keeps in flight
constexpr int kMaxHalf = 64;       // head_dim / 2 upper bound (head_dim <= 128)

// RoPE frequencies in revolutions per position: w_i / (2 pi), w_i = theta^(-2i/d),
// computed on the host in double precision.
struct RopeFreq {
  double rev[kMaxHalf];
};

// ---------------------------------------------------------------------------
// Stage 1: K rotation into MFMA-ready tile images.
// ---------------------------------------------------------------------------
// Key tiles are the 64-token tiles of the pool.  Only tiles in [0, sink_tiles)
// and [win_tile0, win_tile1) are materialised; slot(kt) maps them densely.
struct PackArgs {
  const void* k;        // [n_tokens][hkv][d] unrotated
  void* k_tiles;        // [hkv][n_slots][64][d] rotated, LDS byte image
  int32_t n_tokens;     // keys beyond are zero-filled
  int32_t hkv;
  int32_t sink_tiles;   // tiles [0, sink_tiles) materialised
  int32_t win_tile0;    // tiles [win_tile0, win_tile1) materialised
  int32_t win_tile1;
  int32_t n_slots;      // sink_tiles + (win_tile1 - win_tile0)
  RopeFreq freq;
  uint32_t* queue;      // non-null: the prefill's 8 work counters, zeroed here
};

// Small per-call int32 tables travel in the kernel arguments (kInlineInts
// ints at most, read through the kernarg segment pointer so no private copy
// is made); larger ones are written into the workspace by k_upload launches,
// each carrying kInlineInts ints in its own arguments.  Either way the copy
// is ordered on the caller's stream and needs no host staging memory.
constexpr int kInlineInts = 512;

// One k_upload launch carries up to kUploadInts ints (the argument block
// stays under 4 KiB).  Its duration is mostly the latency of reading the
// argument block, so fewer, larger launches are faster.
constexpr int kUploadInts = 960;
struct UploadArgs {
  int32_t* dst;
  int32_t n;
  int32_t v[kUploadInts];
};

struct PrefillArgs {
  const void* q;            // [n_tokens][hq][d] unrotated (rows of this call)
  const void* k_tiles;      // from PackArgs
  const void* v;            // [n_keys][hkv][d] values (natural layout, read directly)
  void* o;                  // [rows][hq][d]
  const int32_t* offsets;   // device int32[n_blocks + 1], block start tokens (n_inline == 0)
  int32_t n_blocks;
  int32_t sink;
  int32_t j;
  int32_t row0, row1;       // absolute query rows [row0, row1) of this call
  int32_t q_row0;           // absolute row of q[0] / o[0]
  int32_t hq, hkv;
  int32_t n_qtiles;         // ceil((row1 - row0) / (kPrefillRows >> pack_log2))
  int32_t pack_log2;        // 2^pack_log2 query heads of one KV head share a workgroup (and
                            // every K/V tile it loads): kPrefillRows >> pack_log2 tokens each
  int32_t n_keys;           // keys available (rows of v)
  int32_t sink_tiles, win_tile0, n_slots;  // key-tile slot map (see PackArgs)
  float q_scale;            // softmax scale * log2(e), folded into Q
  RopeFreq freq;
  // Split keys (n_split > 1, short walks such as an append): the key tiles of
  // each query tile are cut into n_split consecutive parts, one workgroup
  // each, which leave unnormalised O and (m, l) per row in part_o / part_ml,
  // laid out [hkv][n_split][rows * G][d] (row (t - row0) * G + head in group),
  // for k_combine.
  int32_t n_split;
  float* part_o;
  float* part_ml;
  // Whole walks (n_split == 1): a persistent grid of n_workers workgroups
  // takes the items from 8 counters (kPrefillQueueWords), zeroed by the pack
  // kernel of the same call.
  uint32_t* queue;
  int32_t n_workers;
  int32_t n_inline;         // > 0: the offsets are `inl` below
  int32_t inl[kInlineInts];
};

// ---------------------------------------------------------------------------
// Stage 2
// ---------------------------------------------------------------------------
// The context of batch row b is a list of segments of virtual positions.
// Segment s covers positions [start[s], start[s+1]); its tokens are read from
// `src` token index onward in buffer `buf`:
//   0  the unrotated pool (rotated on load at the virtual position),
//   1  the row's own rotated context buffer,
//   2  the call's new tokens (rotated on load; written back, rotated, to the
//      context buffer at dst_row + token).
// The tables are int32 arrays at these offsets of one table block, which
// travels in the kernel arguments when it fits (kInlineInts) and otherwise in
// the workspace.
struct SegTable {
  int32_t o_start;   // [batch][stride]  (start[nseg] = context length)
  int32_t o_src;     // [batch][stride]
  int32_t o_buf;     // [batch][stride]
  int32_t o_nseg;    // [batch]
  int32_t o_pos0;    // [batch] position of new token 0 (= keys before it)
  int32_t o_dst;     // [batch] context-buffer row of new token 0
  int32_t o_rot;     // [batch] rotation offset added to every position of the row, or -1
                     // for none (positions are then the virtual positions themselves)
  int32_t stride;
};

struct GatherArgs {
  const void* k_pool;
  const void* v_pool;
  void* k_out;            // [batch][cap][hkv][d]
  void* v_out;
  const int32_t* tab;     // device table (n_inline == 0): start | src, see below
  int32_t n_ids, hkv, batch;
  int64_t cap;
  int32_t max_len;        // max T'_b
  RopeFreq freq;
  int32_t n_inline;       // > 0: the table is `inl` below
  int32_t inl[kInlineInts];
  // table: start [batch][n_ids + 1] (output start token of each id, then T'_b),
  //        src [batch][n_ids] (pool start token of each id)
};

struct NewKVArgs {
  const void* k_new;      // [batch][n_new][hkv][d]
  const void* v_new;
  void* k_dst;            // [batch][cap][hkv][d]
  void* v_dst;
  const int32_t* dst_row; // [batch] index in the buffer of new token 0
  const int32_t* pos0;    // [batch] position of new token 0
  int32_t n_new, hkv;
  int64_t cap;
  RopeFreq freq;
};

struct QueryArgs {
  const void* q;          // [batch][n_new][hq][d]
  const void* k_pool;     // may be null when no segment uses buffer 0
  const void* v_pool;
  void* k_ctx;            // [batch][cap][hkv][d] (buffer 1; new rows are written here)
  void* v_ctx;
  const void* k_new;      // [batch][n_new][hkv][d] (buffer 2)
  const void* v_new;
  void* o;                // [batch][n_new][hq][d] (when part_o is null)
  float* part_o;          // [batch][hkv][n_split][rows][d] partials, when not null (always
                          // when n_split > 1; o is then written by a merge kernel)
  float* part_ml;         // [batch][hkv][n_split][rows][2]
  const int32_t* meta;    // table block in device memory (when n_inline == 0)
  SegTable seg;
  int32_t n_inline;       // > 0: the table block is `inl` below
  int32_t n_new, hq, hkv, batch;
  int32_t rows;           // n_new * (hq / hkv) packed rows per kv head
  int32_t row_waves;      // 32-row attention wavefronts per workgroup: 1 .. 4
  int32_t key_ways;       // 2: two wavefronts per 32 rows, one per key half (row_waves <= 2)
  int32_t row_groups;     // row groups of 32 * row_waves rows
  int32_t n_split;        // key splits per (batch, kv head, row group)
  int32_t tiles_per_split;
  int64_t cap;
  float q_scale;          // softmax scale * log2(e)
  RopeFreq freq;
  int32_t inl[kInlineInts];
};

// ---------------------------------------------------------------------------
// Stage 2 for a batch with block loads shared across the queries that chose
// each block.  K tiles are rotated once per call at their pool positions; a
// workgroup takes 256 rows (query, token, head in group) of the queries that
// selected one block and turns each query's Q by its placement shift (RoPE
// scores depend only on position differences).  Per (query, block) it leaves
// a partial: O / l in bf16 and lambda = m + log2(l) (log2 units, softmax scale
// folded in).  Tables (int32, one block `tab`):
//   off     [n_blocks + 1]  block start tokens
//   bstart  [n_blocks + 1]  pairs of block b: pairs[bstart[b] .. bstart[b+1])
//   istart  [n_blocks + 1]  work items of block b: istart[b] .. istart[b+1]
//   pairs   [n_pairs][2]    (batch row << 16 | slot of b in the row's ids,
//                            Q rotation position of the row's token 0)
//   kslot   [n_blocks]      first K-image slot of block b's tiles (-1: unused)
//   ublk    [n_used]        blocks selected by some row, ascending
//   uslot   [n_used + 1]    first K-image slot of each of them
// ---------------------------------------------------------------------------
struct SharedTables {
  int32_t o_off, o_bstart, o_istart, o_pairs, o_kslot, o_ublk, o_uslot;
  int32_t n_blocks, n_used, n_slots, n_items;
};

struct SharedPackArgs {
  const void* k;            // [n_tokens][hkv][d] unrotated pool
  void* k_tiles;            // [hkv][n_slots][64][d] rotated at pool positions, LDS image
  const int32_t* tab;
  SharedTables t;
  int32_t n_tokens, hkv;
  RopeFreq freq;
  uint32_t* queue;          // k_shared_bf16's kPrefillQueueWords work counters, zeroed here
};

struct SharedArgs {
  const void* q;            // [batch][n_new][hq][d] unrotated
  const void* k_tiles;      // from SharedPackArgs
  const void* v;            // [n_tokens][hkv][d] pool values
  uint16_t* part_o;         // [batch][hkv][n_ids][rq][d] bf16: O / l
  float* part_lam;          // [batch][hkv][n_ids][rq]: m + log2(l)
  const int32_t* tab;
  SharedTables t;
  int32_t n_tokens, n_ids, n_new, hq, hkv;
  int32_t rq;               // rows per (batch row, kv head) = n_new * (hq / hkv)
  float q_scale;            // softmax scale * log2(e)
  RopeFreq freq;
  uint32_t* queue;          // work counters (see queue_claim)
  int32_t n_workers;        // persistent workgroups (compute units)
};

struct MergeArgs {
  const uint16_t* part_o;   // block partials (SharedArgs)
  const float* part_lam;
  const float* tail_o;      // the tail / new-token pass: [batch][hkv][n_split][rq][d] O, unnormalised
  const float* tail_ml;     // [batch][hkv][n_split][rq][2] (m, l)
  void* o;                  // [batch][n_new][hq][d]
  int32_t n_ids, n_split, rq, n_new, hq, hkv;
};

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  void* o;
  int32_t n_new, hq, hkv, rows, n_split;
};

// Launchers (each returns the launch status; all enqueue on `stream`).
hipError_t launch_upload(const UploadArgs& a, hipStream_t stream);
hipError_t launch_pack(const PackArgs& a, int head_dim, int dtype, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int dtype, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, int batch, int head_dim, int dtype,
                         hipStream_t stream);
hipError_t launch_new_kv(const NewKVArgs& a, int batch, int head_dim, int dtype,
                         hipStream_t stream);
hipError_t launch_query(const QueryArgs& a, int batch, int head_dim, int dtype,
                        hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, int batch, int head_dim, int dtype,
                          hipStream_t stream);
hipError_t launch_shared_pack(const SharedPackArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_shared(const SharedArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int batch, int head_dim, hipStream_t stream);

}  // namespace dbsa
