// Kernel-map construction for submanifold sparse convolution on gfx950.
//
// The map ("rulebook") of a K^3 submanifold convolution holds, for every
// offset d, the entries (P, Q) with P = Q + d among the active voxels
// ("Sparse inputs and sparse convolution", section "The map is the
// computation"; sign as in "Sparse convolution for point clouds", section
// "The map and the update rule").  Outputs are the inputs (section "The fix:
// compute only where an input exists"), so one coordinate table serves both
// sides (the SparseConvNet blog, section 2, builds one table per side).
//
// Coordinate table: open addressing over 64-bit keys (b, z, y, x packed in
// 16-bit fields), probed in aligned windows of 4 keys (32 bytes) with linear
// probing over windows; the row of a key sits in a parallel array at the same
// slot and is read only on a hit.  The home window of a key hashes
// (b, z, y, x >> 2): the four keys of an aligned run of x share a home window,
// so the x-neighbours a voxel looks up for one (dz, dy) fall into one or two
// windows, which a lane keeps in registers between lookups.
//
// Pipeline (one stream, six launches, then one read-back of a small summary):
//   k_init     clear the table, the neighbour bitmasks and the summary
//   k_insert   one lane per voxel: scan the window, claim the first free slot
//              with a 64-bit CAS; an equal key raises the duplicate flag
//   k_probe    one lane per (voxel, (dz, dy) row of the positive half): look up
//              Q + d for the offsets d > 0 (lexicographic in (dz, dy, dx)) of
//              that row.  A hit also records the mirror entry (Q, P, -d),
//              since (P, Q, d) <-> (Q, P, -d) ("Sparse inputs and sparse
//              convolution", section "A symmetry you can check on the slide"),
//              so (K^3 - 1) / 2 of the K^3 offsets are probed.  Bits go to
//              per-row neighbour masks, indices to an offset-major scratch
//              table.
//   k_count    one workgroup per 1024-row chunk: per-tile row masks of every
//              offset (ballots of the mask bits) and per-chunk counts
//   k_scan     one workgroup: exclusive scan of the (offset, chunk) counts in
//              offset-major order into list offsets and per-offset totals
//   k_compact  per (offset, chunk): each entry's place from the scan and the
//              tile mask; lists come out grouped by offset ("sorted by weight
//              offset", section "Nine entries become two") and ordered by
//              output row within an offset.
// The lists are sized for the bound of K^3 entries per voxel, so nothing on
// the device waits for the host; the host reads the summary once at the end.
#include "internal.h"

namespace spconv {
namespace {

__device__ __forceinline__ unsigned long long pack_key(int b, int z, int y, int x) {
  return (static_cast<unsigned long long>(static_cast<uint32_t>(b)) << 48) |
         (static_cast<unsigned long long>(static_cast<uint32_t>(z)) << 32) |
         (static_cast<unsigned long long>(static_cast<uint32_t>(y)) << 16) |
         static_cast<unsigned long long>(static_cast<uint32_t>(x));
}

// 64-bit finalizer of MurmurHash3 (fmix64): a bijective avalanche mix.
__device__ __forceinline__ unsigned long long mix64(unsigned long long h) {
  h ^= h >> 33;
  h *= 0xff51afd7ed558ccdull;
  h ^= h >> 33;
  h *= 0xc4ceb9fe1a85ec53ull;
  h ^= h >> 33;
  return h;
}

// Home window of a key: hash of the key without the two low bits of x.
__device__ __forceinline__ unsigned long long home_window(unsigned long long key,
                                                          unsigned long long window_mask) {
  return mix64(key >> 2) & window_mask;
}

__device__ __forceinline__ bool coord_in_range(int v) { return v >= 0 && v < 65536; }

__device__ __forceinline__ void raise_flag(long long* summary, unsigned long long bit) {
  atomicOr(reinterpret_cast<unsigned long long*>(summary), bit);
}

__global__ __launch_bounds__(256) void k_init(ulonglong2* keys2, int64_t key_pairs,
                                              uint32_t* masks, int64_t mask_elems,
                                              long long* summary, int summary_len) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const ulonglong2 empty = make_ulonglong2(kEmptyKey, kEmptyKey);
  for (int64_t i = t0; i < key_pairs; i += stride) keys2[i] = empty;
  for (int64_t i = t0; i < mask_elems; i += stride) masks[i] = 0u;
  for (int64_t i = t0; i < summary_len; i += stride) summary[i] = 0;
}

// One lane per voxel.
__global__ __launch_bounds__(256) void k_insert(const int4* __restrict__ coords, int64_t n,
                                                unsigned long long* keys, int32_t* rows,
                                                unsigned long long window_mask,
                                                long long* summary) {
  const int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v >= n) return;
  const int4 c = coords[v];
  if (c.x < 0 || c.x >= 32768 || !coord_in_range(c.y) || !coord_in_range(c.z) ||
      !coord_in_range(c.w)) {
    raise_flag(summary, kFlagRange);
    return;
  }
  const unsigned long long key = pack_key(c.x, c.y, c.z, c.w);
  unsigned long long w = home_window(key, window_mask);
  // Every window is left for the next one as soon as it is seen full, so the
  // search visits each window at most once; the bound is reached only by a
  // table without a free slot, which reports a full table.
  const unsigned long long max_steps = window_mask + 1;
  // Keys of one aligned x-run share a home window; each first tries its own
  // slot x & 3 so that neighbours inserted together do not contend.  Any free
  // slot of the first non-full window is valid for linear probing, since a
  // lookup scans whole windows and stops at the first one with a free slot.
  //
  // The window is read with plain (cacheable) loads.  A stale view can only
  // show EMPTY where a key already sits, never a wrong key; a failed CAS
  // returns the slot's true key, which replaces the stale one.  Candidates are
  // tried in a fixed order (the preferred slot, then increasing slot index),
  // so two inserters of one key always meet on the slot the first one
  // claimed and the second sees its key: duplicates are always detected.
  const int pref = c.w & (kWindowSlots - 1);
  for (unsigned long long step = 0; step < max_steps; ++step) {
    unsigned long long* win = keys + w * kWindowSlots;
    const ulonglong2 v01 = reinterpret_cast<const ulonglong2*>(win)[0];
    const ulonglong2 v23 = reinterpret_cast<const ulonglong2*>(win)[1];
    unsigned long long view[kWindowSlots] = {v01.x, v01.y, v23.x, v23.y};
    bool moved = false;
    for (int attempt = 0; attempt <= kWindowSlots; ++attempt) {
      bool dup = false;
      int target = -1;
#pragma unroll
      for (int j = kWindowSlots - 1; j >= 0; --j) {
        dup |= (view[j] == key);
        if (view[j] == kEmptyKey) target = j;
      }
      if (dup) {
        raise_flag(summary, kFlagDuplicate);
        return;
      }
      if (view[pref] == kEmptyKey) target = pref;
      if (target < 0) {  // window full: next window
        moved = true;
        break;
      }
      const unsigned long long old = atomicCAS(&win[target], kEmptyKey, key);
      if (old == kEmptyKey) {
        rows[w * kWindowSlots + target] = static_cast<int32_t>(v);
        return;
      }
      view[target] = old;  // learn the true key and try again
    }
    if (moved) w = (w + 1) & window_mask;
  }
  raise_flag(summary, kFlagTableFull);
}

// Row of `key`, or -1.  The window at index `cw` (keys in ck[]) is the one
// loaded last; it is reused when a search reaches it again.
__device__ __forceinline__ int64_t find_row(unsigned long long key,
                                            const unsigned long long* __restrict__ keys,
                                            const int32_t* __restrict__ rows,
                                            unsigned long long window_mask,
                                            unsigned long long& cw, ulonglong2 (&ck)[2],
                                            bool& overflow) {
  unsigned long long w = home_window(key, window_mask);
  for (unsigned long long step = 0; step <= window_mask; ++step) {
    if (w != cw) {
      const ulonglong2* p = reinterpret_cast<const ulonglong2*>(keys + w * kWindowSlots);
      ck[0] = p[0];
      ck[1] = p[1];
      cw = w;
    }
    const unsigned long long k0 = ck[0].x, k1 = ck[0].y, k2 = ck[1].x, k3 = ck[1].y;
    int hit = -1;
    if (k3 == key) hit = 3;
    if (k2 == key) hit = 2;
    if (k1 == key) hit = 1;
    if (k0 == key) hit = 0;
    if (hit >= 0) return rows[w * kWindowSlots + hit];
    if (k0 == kEmptyKey || k1 == kEmptyKey || k2 == kEmptyKey || k3 == kEmptyKey) return -1;
    w = (w + 1) & window_mask;
  }
  overflow = true;
  return -1;
}

// Grid: x covers voxels, y = index j of a (dz, dy) row of the positive half,
// in lexicographic order: j = 0 is (0, 0) (probing dx > 0 only), then (0, 1..r),
// then (1..r, -r..r).
__global__ __launch_bounds__(256) void k_probe(const int4* __restrict__ coords, int64_t n, int K,
                                               int KV, const unsigned long long* __restrict__ keys,
                                               const int32_t* __restrict__ rows,
                                               unsigned long long window_mask,
                                               int32_t* __restrict__ nbr, uint32_t* masks,
                                               long long* summary) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= n) return;
  const int r = (K - 1) / 2;
  const int j = blockIdx.y;
  int dz, dy;
  if (j == 0) {
    dz = 0;
    dy = 0;
  } else if (j <= r) {
    dz = 0;
    dy = j;
  } else {
    dz = 1 + (j - r - 1) / K;
    dy = (j - r - 1) % K - r;
  }
  const int dx_lo = (j == 0) ? 1 : -r;
  const int4 c = coords[q];
  const int z = c.y + dz, y = c.z + dy;
  if (!coord_in_range(z) || !coord_in_range(y)) return;  // never wraps
  unsigned long long cw = ~0ull;
  ulonglong2 ck[2];
  bool overflow = false;
  // The offsets of one (dz, dy) row are K consecutive indices, so they span at
  // most two 32-bit mask words.
  const int krow = (dz + r) * K * K + (dy + r) * K + r;  // k of (dz, dy, 0)
  const int w0 = (krow - r) >> 5;
  uint32_t own0 = 0u, own1 = 0u;
  for (int dx = dx_lo; dx <= r; ++dx) {
    const int x = c.w + dx;
    if (!coord_in_range(x)) continue;
    const int64_t p = find_row(pack_key(c.x, z, y, x), keys, rows, window_mask, cw, ck, overflow);
    if (p < 0 || p >= n) continue;  // miss (a claimed slot always holds a row in range)
    const int kpos = krow + dx;
    const int kneg = KV - 1 - kpos;
    nbr[static_cast<int64_t>(kpos) * n + q] = static_cast<int32_t>(p);
    nbr[static_cast<int64_t>(kneg) * n + p] = static_cast<int32_t>(q);
    if ((kpos >> 5) == w0) {
      own0 |= 1u << (kpos & 31);
    } else {
      own1 |= 1u << (kpos & 31);
    }
    atomicOr(&masks[static_cast<int64_t>(kneg >> 5) * n + p], 1u << (kneg & 31));
  }
  // Other lanes' mirror bits land in this voxel's words too, hence atomics.
  if (own0) atomicOr(&masks[static_cast<int64_t>(w0) * n + q], own0);
  if (own1) atomicOr(&masks[static_cast<int64_t>(w0 + 1) * n + q], own1);
  if (overflow) raise_flag(summary, kFlagTableFull);
}

// Exclusive scan, in place and in offset-major order, of the KV x chunks
// counts by one 1024-thread workgroup; totals go to the summary, E to
// *tile_off_end.
__device__ void scan_chunk_sums(int64_t* a, int KV, int64_t chunks, long long* summary,
                                int32_t* tile_off_end, int64_t* part) {
  constexpr int kT = 1024;
  const int t = threadIdx.x;
  const int64_t m = static_cast<int64_t>(KV) * chunks;
  const int64_t per = (m + kT - 1) / kT;
  const int64_t b = t * per;
  const int64_t e = (b + per < m) ? b + per : m;
  int64_t s = 0;
  for (int64_t i = b; i < e; ++i) s += a[i];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < kT; off <<= 1) {
    const int64_t add = (t >= off) ? part[t - off] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  const int64_t total = part[kT - 1];
  int64_t base = part[t] - s;
  for (int64_t i = b; i < e; ++i) {
    const int64_t val = a[i];
    a[i] = base;
    base += val;
  }
  __syncthreads();
  if (t == 0) {
    summary[1] = total;
    *tile_off_end = static_cast<int32_t>(total);
  }
  for (int k = t; k < KV; k += kT) {
    const int64_t lo = a[static_cast<int64_t>(k) * chunks];
    const int64_t hi = (k + 1 < KV) ? a[static_cast<int64_t>(k + 1) * chunks] : total;
    summary[kSummaryHead + k] = hi - lo;
  }
}

// One workgroup of 1024 threads (16 waves) per chunk of kChunkTiles = 16
// tiles, one tile per wave.  Per tile and offset k, a ballot of mask bit k is
// the tile's row mask; lane k mod 64 keeps it (slot k / 64), stores it to
// tile_mask[k][t] and counts it.  Per-chunk counts go to chunk_sum[k][chunk].
template <int K>
__global__ __launch_bounds__(1024) void k_count(const uint32_t* __restrict__ masks, int64_t n,
                                                int64_t tiles, int64_t chunks,
                                                unsigned long long* __restrict__ tile_mask,
                                                int64_t* chunk_sum) {
  constexpr int KV = K * K * K;
  constexpr int centre = (KV - 1) / 2;
  constexpr int NS = (KV + 63) / 64;          // offsets per lane
  constexpr int KW = (KV + 31) / 32;          // mask words per row
  const int64_t chunk = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = chunk * kChunkTiles + wave;
  const int64_t q = t * kTileRows + lane;
  const bool valid = (t < tiles) && (q < n);
  unsigned long long mine[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) mine[s] = 0ull;
  if (t < tiles) {
#pragma unroll
    for (int w = 0; w < KW; ++w) {
      const uint32_t mw = valid ? masks[static_cast<int64_t>(w) * n + q] : 0u;
#pragma unroll
      for (int bit = 0; bit < 32; ++bit) {
        const int k = 32 * w + bit;
        if (k < KV) {
          const unsigned long long bal = __ballot(k == centre ? valid : ((mw >> bit) & 1u) != 0u);
          if (lane == (k & 63)) mine[k >> 6] = bal;
        }
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int k = s * 64 + lane;
      if (k < KV) tile_mask[static_cast<int64_t>(k) * tiles + t] = mine[s];
    }
  }
  __shared__ int part[kChunkTiles][NS * 64];
#pragma unroll
  for (int s = 0; s < NS; ++s) part[wave][s * 64 + lane] = __popcll(mine[s]);
  __syncthreads();
  for (int k = threadIdx.x; k < KV; k += 1024) {
    int sum = 0;
#pragma unroll
    for (int w = 0; w < kChunkTiles; ++w) sum += part[w][k];
    chunk_sum[static_cast<int64_t>(k) * chunks + chunk] = sum;
  }
}

// One workgroup of 1024 threads scans the chunk counts (a kernel boundary
// orders it after k_count, which is far cheaper than a device-wide fence on a
// GPU whose L2 caches are per XCD).
__global__ __launch_bounds__(1024) void k_scan(int64_t* chunk_sum, int KV, int64_t chunks,
                                               long long* summary, int32_t* tile_off_end) {
  __shared__ int64_t scan_part[1024];
  scan_chunk_sums(chunk_sum, KV, chunks, summary, tile_off_end, scan_part);
}

// Grid: x = chunk, y = offset k; 256 threads, wave w places the entries of
// tiles chunk * 16 + 4 w + [0, 4) from their tile masks.  tile_off[k * tiles
// + t] = first entry of tile t in list k (tile_off[KV * tiles] = E is written
// by the scan).
__global__ __launch_bounds__(256) void k_compact(const unsigned long long* __restrict__ tile_mask,
                                                 const int32_t* __restrict__ nbr, int64_t n,
                                                 int64_t tiles, int centre, int64_t chunks,
                                                 const int64_t* __restrict__ chunk_base,
                                                 int32_t* __restrict__ in_idx,
                                                 int32_t* __restrict__ out_idx,
                                                 int32_t* __restrict__ tile_off) {
  constexpr int kTilesPerWave = kChunkTiles / 4;
  const int k = blockIdx.y;
  const int64_t chunk = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool is_centre = (k == centre);
  // lane i < kTilesPerWave holds the mask of the wave's tile i
  const int64_t tl = chunk * kChunkTiles + wave * kTilesPerWave + lane;
  const unsigned long long my_mask =
      (lane < kTilesPerWave && tl < tiles) ? tile_mask[static_cast<int64_t>(k) * tiles + tl] : 0ull;
  int wsum = __popcll(my_mask);
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) wsum += __shfl_xor(wsum, d);  // the wave's total
  __shared__ int part[4];
  if (lane == 0) part[wave] = wsum;
  __syncthreads();
  int64_t base = chunk_base[static_cast<int64_t>(k) * chunks + chunk];
  for (int w = 0; w < wave; ++w) base += part[w];
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int32_t* nk = nbr + static_cast<int64_t>(k) * n;
#pragma unroll
  for (int i = 0; i < kTilesPerWave; ++i) {
    const int64_t t = chunk * kChunkTiles + wave * kTilesPerWave + i;
    if (t < tiles) {
      const unsigned long long m = __shfl(my_mask, i);
      if (lane == 0) tile_off[static_cast<int64_t>(k) * tiles + t] = static_cast<int32_t>(base);
      if ((m >> lane) & 1ull) {
        const int64_t q = t * kTileRows + lane;
        const int64_t pos = base + __popcll(m & below);
        in_idx[pos] = is_centre ? static_cast<int32_t>(q) : nk[q];
        out_idx[pos] = static_cast<int32_t>(q);
      }
      base += __popcll(m);
    }
  }
}

int grid_for(int64_t work, int per_block, int cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return static_cast<int>(g);
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

size_t build_scratch_bytes(const BuildPlan& p) {
  size_t b = 0;
  b += align_up(static_cast<size_t>(p.table_slots) * sizeof(unsigned long long), 256);
  b += align_up(static_cast<size_t>(p.table_slots) * sizeof(int32_t), 256);
  b += align_up(static_cast<size_t>(p.mask_words) * p.n * sizeof(uint32_t), 256);
  b += align_up(static_cast<size_t>(p.KV) * p.n * sizeof(int32_t), 256);
  b += align_up(static_cast<size_t>(p.KV) * p.chunks * sizeof(int64_t), 256);
  b += align_up(static_cast<size_t>(kSummaryHead + p.KV) * sizeof(long long), 256);
  return b;
}

void carve_build_scratch(const BuildPlan& p, void* base, BuildScratch* s) {
  char* c = static_cast<char*>(base);
  s->keys = reinterpret_cast<unsigned long long*>(c);
  c += align_up(static_cast<size_t>(p.table_slots) * sizeof(unsigned long long), 256);
  s->rows = reinterpret_cast<int32_t*>(c);
  c += align_up(static_cast<size_t>(p.table_slots) * sizeof(int32_t), 256);
  s->masks = reinterpret_cast<uint32_t*>(c);
  c += align_up(static_cast<size_t>(p.mask_words) * p.n * sizeof(uint32_t), 256);
  s->nbr = reinterpret_cast<int32_t*>(c);
  c += align_up(static_cast<size_t>(p.KV) * p.n * sizeof(int32_t), 256);
  s->chunk_sum = reinterpret_cast<int64_t*>(c);
  c += align_up(static_cast<size_t>(p.KV) * p.chunks * sizeof(int64_t), 256);
  s->summary = reinterpret_cast<long long*>(c);
}

size_t map_buffer_bytes(const BuildPlan& p) {
  const size_t cap = static_cast<size_t>(p.KV) * p.n;
  const size_t tiles = static_cast<size_t>(p.KV) * p.tiles;
  return 2 * align_up(cap * sizeof(int32_t), 256) + align_up((tiles + 1) * sizeof(int32_t), 256) +
         align_up(tiles * sizeof(unsigned long long), 256);
}

void carve_map_buffers(const BuildPlan& p, void* base, MapBuffers* m) {
  const size_t cap = static_cast<size_t>(p.KV) * p.n;
  const size_t tiles = static_cast<size_t>(p.KV) * p.tiles;
  char* c = static_cast<char*>(base);
  m->in_idx = reinterpret_cast<int32_t*>(c);
  c += align_up(cap * sizeof(int32_t), 256);
  m->out_idx = reinterpret_cast<int32_t*>(c);
  c += align_up(cap * sizeof(int32_t), 256);
  m->tile_off = reinterpret_cast<int32_t*>(c);
  c += align_up((tiles + 1) * sizeof(int32_t), 256);
  m->tile_mask = reinterpret_cast<unsigned long long*>(c);
}

hipError_t launch_build(const BuildPlan& p, const int32_t* coords, const BuildScratch& s,
                        const MapBuffers& m, hipStream_t stream) {
  const int64_t mask_elems = static_cast<int64_t>(p.mask_words) * p.n;
  const int64_t key_pairs = p.table_slots / 2;
  const int64_t init_work = key_pairs > mask_elems ? key_pairs : mask_elems;
  hipLaunchKernelGGL(k_init, dim3(grid_for(init_work, 256, 4096)), dim3(256), 0, stream,
                     reinterpret_cast<ulonglong2*>(s.keys), key_pairs, s.masks, mask_elems,
                     s.summary, kSummaryHead + p.KV);
  const unsigned long long window_mask =
      static_cast<unsigned long long>(p.table_slots / kWindowSlots) - 1ull;
  const int4* c4 = reinterpret_cast<const int4*>(coords);
  const unsigned gx = static_cast<unsigned>((p.n + 255) / 256);
  hipLaunchKernelGGL(k_insert, dim3(gx), dim3(256), 0, stream, c4, p.n, s.keys, s.rows,
                     window_mask, s.summary);
  if (p.K > 1) {
    const int r = (p.K - 1) / 2;
    const unsigned rows = static_cast<unsigned>(1 + r + r * p.K);  // (dz, dy) rows with d > 0
    hipLaunchKernelGGL(k_probe, dim3(gx, rows), dim3(256), 0, stream, c4, p.n, p.K, p.KV, s.keys,
                       s.rows, window_mask, s.nbr, s.masks, s.summary);
  }
  const dim3 gc(static_cast<unsigned>(p.chunks));
  switch (p.K) {
    case 1:
      hipLaunchKernelGGL(k_count<1>, gc, dim3(1024), 0, stream, s.masks, p.n, p.tiles, p.chunks,
                         m.tile_mask, s.chunk_sum);
      break;
    case 3:
      hipLaunchKernelGGL(k_count<3>, gc, dim3(1024), 0, stream, s.masks, p.n, p.tiles, p.chunks,
                         m.tile_mask, s.chunk_sum);
      break;
    case 5:
      hipLaunchKernelGGL(k_count<5>, gc, dim3(1024), 0, stream, s.masks, p.n, p.tiles, p.chunks,
                         m.tile_mask, s.chunk_sum);
      break;
    case 7:
      hipLaunchKernelGGL(k_count<7>, gc, dim3(1024), 0, stream, s.masks, p.n, p.tiles, p.chunks,
                         m.tile_mask, s.chunk_sum);
      break;
    default:
      return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, stream, s.chunk_sum, p.KV, p.chunks,
                     s.summary, m.tile_off + static_cast<int64_t>(p.KV) * p.tiles);
  hipLaunchKernelGGL(k_compact, dim3(static_cast<unsigned>(p.chunks), static_cast<unsigned>(p.KV)),
                     dim3(256), 0, stream, m.tile_mask, s.nbr, p.n, p.tiles, p.centre, p.chunks,
                     s.chunk_sum, m.in_idx, m.out_idx, m.tile_off);
  return hipGetLastError();
}

}  // namespace spconv
