// Host planner: BSR structure -> work tiles, split-KV partitions, merge table.
// Pure host code; never calls the HIP runtime.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "bsa.h"

namespace bsa {

// Record widths of the int32 tables (see bsa_plan_export in bsa.h).
constexpr int kTileInts = 8;
constexpr int kMergeInts = 8;

// Trace build (BSA_TRACE, a separate library for tests): each kernel records
// per planner tile what its loops actually did, kTraceInts int32 per tile after
// the split partials: {times processed, first column entry walked, last entry
// walked + 1, valid keys counted, partial offset written, kv head, first row,
// rows, key tokens outside [0, N) met (and masked), 7 x unused}.
constexpr int kTraceInts = 16;

// Tile record fields.
enum TileField { T_ROWBLOCK = 0, T_KVHEAD, T_ROW0, T_NROWS, T_COLB, T_COLE, T_PART, T_KEYS };
// Merge record fields.
enum MergeField { MG_ROWBLOCK = 0, MG_KVHEAD, MG_ROW0, MG_NROWS, MG_PART0, MG_NSPLIT, MG_STRIDE };

// Auto split-KV rule constants (kv_splits == 0).
#ifndef BSA_AUTO_TILES_PER_CU
#define BSA_AUTO_TILES_PER_CU 4
#endif
constexpr int kAutoTilesPerCu = BSA_AUTO_TILES_PER_CU;  // aim for this many tiles per CU
constexpr int kAutoMinSplitKeys = 256;   // never cut a row tile into pieces below this many keys
constexpr int kMaxSplits = 64;           // hard cap on partitions per row tile
#ifndef BSA_TILE_MAX_ROWS
#define BSA_TILE_MAX_ROWS 256
#endif
constexpr int kTileMaxRows = BSA_TILE_MAX_ROWS;  // largest row tile of the generic kernel (128 or 256)
// Generic kernel: 256-row tiles unless that gives fewer than this many tiles
// per CU (then 128-row tiles, so that two workgroups share a CU).
#ifndef BSA_TILE_SMALL_GRID_PER_CU
#define BSA_TILE_SMALL_GRID_PER_CU 8
#endif
constexpr int kTileSmallGridPerCu = BSA_TILE_SMALL_GRID_PER_CU;
// Decode kernel: a workgroup of 8 waves takes a group of
// decode_heads_per_wg(num_kv_heads) kv heads, the largest power of two up to
// 8 that divides num_kv_heads (one head per wave when it is 8).  With
// kv_splits == 0 the tiles are a balanced partition over the workgroups the
// device holds at once (8 waves at 2 waves per SIMD: one per CU), each taking
// at least kBalancedMinKeys keys.
constexpr int kDecodeWaves = 8;
constexpr int kDecodeWgPerCu = 1;
constexpr int kBalancedMinKeys = 256;
inline int32_t decode_heads_per_wg(int32_t num_kv_heads) {
  const int32_t low = num_kv_heads & -num_kv_heads;
  return low < kDecodeWaves ? low : kDecodeWaves;
}

struct Plan {
  // validated request
  bsa_plan_desc_t d{};
  int64_t MB = 0, NB = 0;
  int32_t group = 1;
  float sm_scale = 0.f;
  // selected kernel
  int32_t kernel = BSA_KERNEL_TILE;
  int32_t tile_rows = 0;
  int32_t key_tile = 0;
  int32_t num_cus = 0;
  // tables
  std::vector<int32_t> tiles;    // kTileInts per tile, launch order
  std::vector<int32_t> merges;   // kMergeInts per merge
  std::vector<int32_t> cols;     // column blocks per row block, ascending, causally trimmed
  std::vector<int32_t> lens;     // valid length of each cols entry, empty when every block is full
  std::vector<int32_t> wg_ptr;   // workgroup w runs tiles wg_ptr[w] .. wg_ptr[w+1]-1, in order
  // Element-mask bit planes (element masks or variable blocks; empty otherwise):
  // plane r (r < R) holds, for column-list entry e and key c < C of its block,
  // the visibility of query row I*R + r (I = the entry's row block) at bit
  // e*C + c: word (e*C + c) / 32, bit (e*C + c) % 32.  mask_plane_words words
  // per plane, padded so that a key tile read past a list's end stays inside.
  std::vector<uint32_t> mbits;
  int64_t mask_plane_words = 0;
  int32_t max_splits = 1;
  int32_t heads_per_wg = 1;      // kv heads per tile group (decode kernel: one workgroup)
  int64_t partial_floats = 0;
  int64_t valid_pairs = 0;
  // workspace layout (bytes)
  int64_t off_tiles = 0, off_merges = 0, off_cols = 0, off_lens = 0, off_wg = 0, off_zero = 0, off_mbits = 0;
  int64_t table_bytes = 0, partial_bytes = 0, workspace_bytes = 0;
  std::vector<uint8_t> table_blob;  // exact image of the table region
  uint64_t id = 0;                  // process-unique plan id
};

// Validates `desc` and builds every table.  `num_cus` must be > 0 here (the
// C ABI layer resolves 0 from the device).  On failure returns a status and
// sets `err`.
bsa_status_t build_plan(const bsa_plan_desc_t& desc, int32_t num_cus, Plan& plan, std::string& err);

}  // namespace bsa
