// Internal declarations of the gfx950 submanifold sparse convolution library.
// Not part of the public ABI (that is include/spconv.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

namespace spconv {

// Rows per tile.  One 64-lane wavefront covers one tile in the map build
// (one ballot per tile and offset), and the forward's workgroup owns whole
// tiles, so per-tile list ranges are all the forward needs from the map.
constexpr int kTileRows = 64;
// Tiles per group of the count / compaction grid (one count workgroup of 16
// waves, one tile each, per group).  A chunk is `group_tiles` consecutive
// groups, chosen so that an offset has at most kMaxChunks chunks: each
// compaction workgroup sums the counts of the chunks before it.
constexpr int kGroupTiles = 16;
constexpr int kMaxChunks = 128;

// Per tile, the input rows of its first kTileSlots non-centre entries in the
// order the small-channel forward stages them: by offset, then by output row
// (slot s of tile t at tile_rows[t * kTileSlots + s]).  With it the forward
// loads a tile's gather indices together with the tile's masks instead of
// after them.
constexpr int kTileSlots = 128;

// The map's row order (the order the forward computes rows in): for K > 1
// and at least kOrderMinRows rows, the rows of each window of kOrderWindow
// consecutive input rows sorted stably by a kOrderKeyBits-bit key of their
// neighbour set; otherwise the input order.  A window is a multiple of
// kTileRows, so a tile never straddles two.  Below kOrderMinRows the forward
// is bound by per-tile latency rather than by the weights and rows it
// fetches, and the order does not repay its build time.
constexpr int kOrderWindow = 4096;
constexpr int kOrderKeyBits = 16;
constexpr int64_t kOrderMinRows = 262144;

// Coordinate table: open addressing over 16-byte slots (64-bit key, int32 row,
// flags), probed in aligned windows of 8 slots (128 bytes, one L2 line).  A
// key first claims its preferred slot (x & 3 in a hash-chosen half of its home
// window); an EMPTY preferred slot therefore means the key is absent.  The
// table has at least 4 slots per voxel.
constexpr int kWindowSlots = 8;
constexpr int kTableSlotsPerVoxel = 4;
constexpr uint64_t kEmptyKey = ~0ull;

// Device error flags (bit set in summary[0]).
constexpr unsigned long long kFlagDuplicate = 1ull;
constexpr unsigned long long kFlagRange = 2ull;
constexpr unsigned long long kFlagTableFull = 4ull;

// Layout of the small device summary the host reads once per build:
//   [0] error flags, [1] unused, [2 + k] entries of offset k.
constexpr int kSummaryHead = 2;

// Exclusive prefix sum over the lanes of a wavefront of values in [0, 2^BITS),
// bit plane by bit plane: a ballot of bit b, counted below the lane (mbcnt),
// weighs 2^b.  No cross-lane data movement, so no LDS round trips.
template <int BITS>
__device__ __forceinline__ int wave_prefix_small(int v) {
  int excl = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    const unsigned long long m = __ballot((v >> b) & 1);
    const int below = static_cast<int>(__builtin_amdgcn_mbcnt_hi(
        static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
    excl += below << b;
  }
  return excl;
}

struct BuildPlan {
  int64_t n = 0;
  int32_t K = 0, KV = 0, centre = 0;
  int64_t tiles = 0;        // ceil(n / kTileRows)
  int64_t group_tiles = 0;  // tiles per chunk (a multiple of kGroupTiles)
  int64_t chunks = 0;       // ceil(tiles / group_tiles) <= kMaxChunks
  int64_t table_slots = 0;  // power of two >= kTableSlotsPerVoxel n, >= 64
  bool ordered = false;     // rows reordered by neighbour set (see kOrderWindow)
};
BuildPlan make_plan(int64_t n, int32_t K);

// Workspace of one build (carved from a single allocation).
// Neighbour flags of a row: offsets after the centre as bits of
// pos_words(K) 32-bit words (written by the row's own probe lane), offsets
// before the centre as bytes in a 16-byte aligned record of neg_bytes(K)
// (written by the lanes of the neighbours, as mirror entries).
__host__ __device__ constexpr int pos_words(int K) { return ((K * K * K - 1) / 2 + 31) / 32; }
__host__ __device__ constexpr int neg_bytes(int K) { return ((K * K * K - 1) / 2 + 15) / 16 * 16; }

struct BuildScratch {
  ulonglong2* table = nullptr;   // table_slots 16-byte slots: .x key, .y row
  uint4* occ = nullptr;          // occupancy map: table_slots / 4 buckets of 16 bytes
  uint32_t* pos_bits = nullptr;  // n x pos_words(K)
  uint8_t* neg_flags = nullptr;  // n x neg_bytes(K)
  int32_t* nbr = nullptr;        // KV x n, offset-major; valid where the flag is set
  int64_t* chunk_sum = nullptr;  // KV x groups entry counts (per kGroupTiles tiles)
  int32_t* tile_base = nullptr;  // KV x tiles: slot of offset k's first entry in tile t
  long long* summary = nullptr;  // kSummaryHead + KV
  int32_t* group_base = nullptr;  // KV x groups: first list position of each group (ordered maps)
};

size_t build_scratch_bytes(const BuildPlan& p);
void carve_build_scratch(const BuildPlan& p, void* base, BuildScratch* s);

// Device buffers owned by a map (one allocation).
struct MapBuffers {
  int32_t* in_idx = nullptr;                // capacity KV * n
  int32_t* out_idx = nullptr;               // capacity KV * n
  int32_t* tile_off = nullptr;              // KV * tiles + 1
  unsigned long long* tile_mask = nullptr;  // KV * tiles
  int32_t* tile_rows = nullptr;             // tiles * kTileSlots (slots past a tile's entries unset)
  int32_t* perm = nullptr;                  // n: row at each position of the forward's order (NULL: identity)
};
size_t map_buffer_bytes(const BuildPlan& p);
void carve_map_buffers(const BuildPlan& p, void* base, MapBuffers* m);

// The whole map build (all asynchronous on `stream`).  When it completes,
// host_summary (pinned host memory, kSummaryHead + KV values) holds the flags
// and the per-offset counts, and for a map in the input order (!p.ordered)
// the scratch's coordinate table and occupancy map are clear again.
// table_clear: they are clear already (the last build on this scratch was
// such a map with the same table size), so the clearing launch is skipped.
hipError_t launch_build(const BuildPlan& p, const int32_t* coords, const BuildScratch& s,
                        const MapBuffers& m, long long* host_summary, bool table_clear, hipStream_t stream);

// Forward launch.  dtype: 0 f32, 1 f16, 2 bf16.
struct ForwardArgs {
  const void* feats;
  const void* weights;
  void* out;
  const int32_t* in_idx;
  const int32_t* out_idx;
  const int32_t* tile_off;                  // KV * tiles + 1
  const unsigned long long* tile_mask;      // KV * tiles
  const int32_t* tile_rows;                 // tiles * kTileSlots
  const int32_t* perm;                      // n, or NULL (identity): output row of each position
  int64_t n;
  int64_t tiles;
  int32_t KV;
  int32_t cin;
  int32_t cout;
  int32_t dtype;
  int32_t centre;   // offset whose list is the identity (read by position), -1: none (strided maps)
  int64_t n_in;     // rows of feats (n for a submanifold map)
  // The weights already in MFMA operand order with the zero row after them
  // (what launch_prep_weights writes, tiled_workspace_bytes(a) bytes), or
  // NULL: the wide and tiled paths then write that copy into their workspace.
  const void* prepared = nullptr;
};
hipError_t launch_forward(const ForwardArgs& a, hipStream_t stream);

// Mid / large channel path (forward_tiled.hip): needs a workspace of
// tiled_workspace_bytes(a) bytes for the weights in MFMA operand order
// (none when a.prepared holds them).
bool tiled_supported(const ForwardArgs& a);
size_t tiled_workspace_bytes(const ForwardArgs& a);
hipError_t launch_forward_tiled(const ForwardArgs& a, void* workspace, hipStream_t stream);
// Writes the weights in MFMA operand order and a 512-byte zero row into the
// workspace (tiled_workspace_bytes(a) bytes).
hipError_t launch_prep_weights(const ForwardArgs& a, void* workspace, hipStream_t stream);
const uint4* workspace_zero_row(const ForwardArgs& a, const void* workspace);
// Wide path (forward_wide.hip): gathered rows staged in LDS, shared by the
// waves of a workgroup.  Its workspace (wide_workspace_bytes(a) bytes) starts
// with the prepared weights and zero row (launch_prep_weights; absent when
// a.prepared holds them), followed by fp32 partial outputs when a small
// layer splits its offsets.
bool wide_supported(const ForwardArgs& a);
size_t wide_workspace_bytes(const ForwardArgs& a);
hipError_t launch_forward_wide(const ForwardArgs& a, void* workspace, hipStream_t stream);
// Backward (backward.hip).  The data gradient runs the forward over the
// same map with W'_k = W_{K^3-1-k}^T, which launch_mirror_transpose writes
// ([K^3][C_out][C_in], mirror_workspace_bytes); the weight gradient needs
// wgrad_workspace_bytes of fp32 partial sums.
hipError_t launch_mirror_transpose(const void* w, void* wt, int KV, int cin, int cout, int dtype,
                                   hipStream_t stream);
size_t mirror_workspace_bytes(int KV, int cin, int cout, int dtype);
struct WgradArgs {
  const void* feats;     // [n][cin]
  const void* grad_out;  // [n][cout]
  float* grad_w;         // [KV][cin][cout], fp32
  const int32_t* in_idx;
  const int32_t* out_idx;
  const int32_t* tile_off;  // KV * tiles + 1: list k starts at tile_off[k * tiles]
  int64_t n;     // output rows (grad_out)
  int64_t n_in;  // input rows (feats)
  int64_t tiles;
  int32_t KV;
  int32_t cin;
  int32_t cout;
  int32_t dtype;
};
size_t wgrad_workspace_bytes(const WgradArgs& a);
hipError_t launch_wgrad(const WgradArgs& a, void* workspace, hipStream_t stream);
// True when the small-channel kernel (every W_d resident in LDS) serves `a`.
bool small_supported(const ForwardArgs& a);

// ---- Strided maps and their transposes (map_strided.hip, map_build.hip) ----
// Output coordinates of a strided map: candidates, sort and unique.  m =
// n_in x ca^3 candidate keys (ca = ceil(K / stride) choices per axis),
// sorted in blocks of 4096.
struct OutCoordPlan {
  int64_t n_in = 0;
  int K = 0, lo = 0, stride = 0, ca = 0;
  int64_t m = 0;
  int64_t blocks = 0;
};
OutCoordPlan out_coord_plan(int64_t n_in, int K, int stride);
size_t out_coord_scratch_bytes(const OutCoordPlan& p);
// Candidates, sort and per-block run counts; the number of outputs goes to
// *n_out (a device word).
hipError_t launch_out_coords_count(const OutCoordPlan& p, const int32_t* coords, void* scratch, long long* n_out,
                                   hipStream_t stream);
// The outputs' coordinates (int32 [n_out][4]) from the same scratch.
hipError_t launch_out_coords_write(const OutCoordPlan& p, void* scratch, int32_t* out_coords, hipStream_t stream);

// Coordinate table of n rows (table_slots_for(n) slots, a quarter as many
// occupancy buckets); clears summary[0 .. summary_len) and raises the
// duplicate and range flags in summary[0].
int64_t table_slots_for(int64_t n);
hipError_t launch_table_build(const int32_t* coords, int64_t n, ulonglong2* table, int64_t table_slots, uint4* occ,
                              long long* summary, int summary_len, hipStream_t stream);
// A map without an identity offset over nq output rows (query coordinates
// qcoords): every offset probed in the other side's table (mode 0: the input
// at stride x q + d; mode 1: the strided output q' with stride x q' + d = p),
// then tile masks and lists as for a submanifold map (centre -1).
struct GeneralMapArgs {
  const int32_t* qcoords = nullptr;
  int64_t nq = 0;
  const ulonglong2* table = nullptr;
  int64_t table_slots = 0;
  int K = 0, lo = 0, stride = 1, mode = 0;
  uint32_t* flags = nullptr;   // nq x 4 words
  int32_t* nbr = nullptr;      // K^3 x nq
  int64_t* chunk_sum = nullptr;
  int32_t* tile_base = nullptr;
  long long* summary = nullptr;       // per-offset totals at kSummaryHead + k (zero on entry)
  long long* host_summary = nullptr;  // the summary is copied here when the lists are done
  MapBuffers map;
};
size_t general_scratch_bytes(int64_t nq, int K);
void carve_general_scratch(int64_t nq, int K, void* base, GeneralMapArgs* g);
hipError_t launch_general_map(const GeneralMapArgs& g, hipStream_t stream);

// ---- Weight-stationary forward with adaptive grouping (grouped.hip) ----
// At most K^3 = 343 offsets (K = 7).
constexpr int kMaxGroupEntries = 343;
// The groups of one (epsilon, S) choice over a map's per-offset counts:
// entries (offsets) in execution order, group by group; every member of a
// group is padded to the group's largest map.
struct GroupPlan {
  std::vector<int> entries;        // offset of each entry
  std::vector<int> entry_group;    // group of each entry
  std::vector<int> group_first;    // first entry of each group, then the entry count
  std::vector<int64_t> group_pad;  // rows of each member of a group (its largest map)
  int groups = 0;
  int64_t padded_rows = 0;         // rows of the padded batches (sum over entries of pad)
  int64_t list_rows = 0;           // entries of the map (sum over entries of their list sizes)
  int64_t tiles = 0;               // 64-row gather tiles over all entries
};
GroupPlan make_group_plan(const int64_t* counts, int KV, int centre, double epsilon, double S);
bool grouped_supported(const ForwardArgs& a);
size_t grouped_workspace_bytes(const ForwardArgs& a, const GroupPlan& p);
hipError_t launch_forward_grouped(const ForwardArgs& a, const GroupPlan& p, void* workspace, hipStream_t stream);

}  // namespace spconv
