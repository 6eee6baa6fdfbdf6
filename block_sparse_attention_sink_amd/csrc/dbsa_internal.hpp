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
};

struct PrefillArgs {
  const void* q;            // [n_tokens][hq][d] unrotated (rows of this call)
  const void* k_tiles;      // from PackArgs
  const void* v;            // [n_keys][hkv][d] values (natural layout, read directly)
  void* o;                  // [rows][hq][d]
  const int32_t* offsets;   // device int32[n_blocks + 1], block start tokens
  int32_t n_blocks;
  int32_t sink;
  int32_t j;
  int32_t row0, row1;       // absolute query rows [row0, row1) of this call
  int32_t q_row0;           // absolute row of q[0] / o[0]
  int32_t hq, hkv;
  int32_t n_qtiles;         // ceil((row1 - row0) / kPrefillRows)
  int32_t n_keys;           // keys available (rows of v)
  int32_t sink_tiles, win_tile0, n_slots;  // key-tile slot map (see PackArgs)
  float q_scale;            // softmax scale * log2(e), folded into Q
  RopeFreq freq;
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
constexpr int kInlineInts = 512;
struct SegTable {
  int32_t o_start;   // [batch][stride]  (start[nseg] = context length)
  int32_t o_src;     // [batch][stride]
  int32_t o_buf;     // [batch][stride]
  int32_t o_nseg;    // [batch]
  int32_t o_pos0;    // [batch] position of new token 0 (= keys before it)
  int32_t o_dst;     // [batch] context-buffer row of new token 0
  int32_t stride;
};

struct GatherArgs {
  const void* k_pool;
  const void* v_pool;
  void* k_out;            // [batch][cap][hkv][d]
  void* v_out;
  const int32_t* start;   // [batch][n_ids + 1] output start token of each id
  const int32_t* src;     // [batch][n_ids] pool start token of each id
  int32_t n_ids, hkv;
  int64_t cap;
  int32_t max_len;        // max T'_b
  RopeFreq freq;
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
  void* o;                // [batch][n_new][hq][d] (when n_split == 1)
  float* part_o;          // [batch][hkv][n_split][rows][d] (when n_split > 1)
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

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  void* o;
  int32_t n_new, hq, hkv, rows, n_split;
};

// Launchers (each returns the launch status; all enqueue on `stream`).
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

}  // namespace dbsa
