// Internal declarations of the gfx950 submanifold sparse convolution library.
// Not part of the public ABI (that is include/spconv.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace spconv {

// Rows per tile.  One 64-lane wavefront covers one tile in the map build
// (one ballot per tile and offset), and the forward's workgroup owns whole
// tiles, so per-tile list ranges are all the forward needs from the map.
constexpr int kTileRows = 64;
// Tiles per chunk of the count / compaction grid (4 waves x 16 tiles).
constexpr int kChunkTiles = 64;
constexpr int kChunkRows = kTileRows * kChunkTiles;

// Hash table: open addressing over 16-byte slots {key, row}, probed in
// aligned windows of 4 slots (64 bytes) by a group of 4 lanes.
constexpr int kWindowSlots = 4;
constexpr uint64_t kEmptyKey = ~0ull;

// Device error flags (bit set in summary[0]).
constexpr unsigned long long kFlagDuplicate = 1ull;
constexpr unsigned long long kFlagRange = 2ull;
constexpr unsigned long long kFlagTableFull = 4ull;

struct Slot {
  unsigned long long key;
  int32_t row;
  int32_t pad;
};

// Layout of the small device summary the host reads once per build:
//   [0] error flags, [1] total entries E, [2 + k] entries of offset k.
constexpr int kSummaryHead = 2;

struct BuildPlan {
  int64_t n = 0;
  int32_t K = 0, KV = 0, centre = 0, half = 0, mask_words = 0;
  int64_t tiles = 0;        // ceil(n / kTileRows)
  int64_t chunks = 0;       // ceil(tiles / kChunkTiles)
  int64_t table_slots = 0;  // power of two >= 2n, >= 64
};

// Workspace of one build (carved from a single allocation).
struct BuildScratch {
  Slot* table = nullptr;            // table_slots
  uint32_t* masks = nullptr;        // mask_words x n, word-major
  int32_t* nbr = nullptr;           // KV x n, offset-major; only entries whose mask bit is set are valid
  int64_t* chunk_sum = nullptr;     // KV x chunks, then its exclusive scan in place
  long long* summary = nullptr;     // kSummaryHead + KV
};

size_t build_scratch_bytes(const BuildPlan& p);
void carve_build_scratch(const BuildPlan& p, void* base, BuildScratch* s);

// Map-build launches (all asynchronous on `stream`).
hipError_t launch_build_front(const BuildPlan& p, const int32_t* coords, const BuildScratch& s,
                              hipStream_t stream);
hipError_t launch_build_compact(const BuildPlan& p, const BuildScratch& s, int64_t total,
                                int32_t* in_idx, int32_t* out_idx, int32_t* tile_off,
                                hipStream_t stream);

// Forward launch.  dtype: 0 f32, 1 f16, 2 bf16.
struct ForwardArgs {
  const void* feats;
  const void* weights;
  void* out;
  const int32_t* in_idx;
  const int32_t* out_idx;
  const int32_t* tile_off;  // KV * tiles + 1
  int64_t n;
  int64_t tiles;
  int32_t KV;
  int32_t cin;
  int32_t cout;
  int32_t dtype;
};
hipError_t launch_forward(const ForwardArgs& a, hipStream_t stream);

}  // namespace spconv
