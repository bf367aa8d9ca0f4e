// Kernel-map construction for submanifold sparse convolution on gfx950.
//
// The map ("rulebook") of a K^3 submanifold convolution holds, for every
// offset d, the entries (P, Q) with P = Q + d among the active voxels
// ("Sparse inputs and sparse convolution", section "The map is the
// computation"; sign as in "Sparse convolution for point clouds", section
// "The map and the update rule").  Outputs are the inputs (section "The fix:
// compute only where an input exists"), so one coordinate table serves both
// sides (SparseConvNet blog, section 2, builds one table per side).
//
// Pipeline (one stream, five launches before the single host read-back):
//   k_init     clear the hash table, the neighbour bitmasks and the summary
//   k_insert   pack (b, z, y, x) into a 64-bit key; 4-lane groups probe
//              aligned 4-slot windows and claim a slot with a 64-bit CAS;
//              an equal key raises the duplicate flag
//   k_probe    4-lane groups look up Q + d for the (K^3 - 1) / 2 offsets with
//              k(d) > centre only; a hit also records the mirror entry
//              (Q, P, -d), since (P, Q, d) <-> (Q, P, -d) ("Sparse inputs and
//              sparse convolution", section "A symmetry you can check on the
//              slide"); bits go to per-row neighbour masks, indices to an
//              offset-major scratch table
//   k_count    per (offset, 4096-row chunk): popcount of mask bits by ballot
//   k_scan     one workgroup: exclusive scan over (offset, chunk) counts in
//              offset-major order, giving list offsets and per-offset counts
// and after the read-back (the host sizes the lists exactly):
//   k_compact  per (offset, chunk): ballot ranks place each entry; lists come
//              out grouped by offset ("sorted by weight offset", section
//              "Nine entries become two") and ordered by output row within an
//              offset; per-tile list starts are recorded for the forward.
#include "internal.h"

namespace spconv {
namespace {

constexpr int kGroup = 4;  // lanes per hash query

__device__ __forceinline__ unsigned long long pack_key(int b, int z, int y, int x) {
  return (static_cast<unsigned long long>(static_cast<uint32_t>(b)) << 48) |
         (static_cast<unsigned long long>(static_cast<uint32_t>(z)) << 32) |
         (static_cast<unsigned long long>(static_cast<uint32_t>(y)) << 16) |
         static_cast<unsigned long long>(static_cast<uint32_t>(x));
}

// 64-bit finalizer of MurmurHash3 (fmix64): a bijective avalanche mix, so
// neighbouring coordinates land in unrelated windows.
__device__ __forceinline__ unsigned long long mix64(unsigned long long h) {
  h ^= h >> 33;
  h *= 0xff51afd7ed558ccdull;
  h ^= h >> 33;
  h *= 0xc4ceb9fe1a85ec53ull;
  h ^= h >> 33;
  return h;
}

__device__ __forceinline__ bool coord_in_range(int v) { return v >= 0 && v < 65536; }

__device__ __forceinline__ void raise_flag(long long* summary, unsigned long long bit) {
  atomicOr(reinterpret_cast<unsigned long long*>(summary), bit);
}

__global__ __launch_bounds__(256) void k_init(uint4* table, int64_t slots, uint32_t* masks,
                                              int64_t mask_elems, long long* summary,
                                              int summary_len) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const uint4 empty = make_uint4(0xffffffffu, 0xffffffffu, 0xffffffffu, 0u);  // key ~0, row -1
  for (int64_t i = t0; i < slots; i += stride) table[i] = empty;
  for (int64_t i = t0; i < mask_elems; i += stride) masks[i] = 0u;
  for (int64_t i = t0; i < summary_len; i += stride) summary[i] = 0;
}

// One 4-lane group per voxel.  Group-uniform control flow throughout: every
// decision is taken from the group's 4 ballot bits or a value broadcast from
// one of its lanes.
__global__ __launch_bounds__(256) void k_insert(const int4* __restrict__ coords, int64_t n,
                                                Slot* table, unsigned long long window_mask,
                                                long long* summary) {
  const int64_t v = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kGroup;
  if (v >= n) return;
  const int lane = threadIdx.x & 63;
  const int sub = lane & (kGroup - 1);
  const int gbase = lane & ~(kGroup - 1);
  const int4 c = coords[v];
  if (c.x < 0 || c.x >= 32768 || !coord_in_range(c.y) || !coord_in_range(c.z) ||
      !coord_in_range(c.w)) {
    if (sub == 0) raise_flag(summary, kFlagRange);
    return;
  }
  const unsigned long long key = pack_key(c.x, c.y, c.z, c.w);
  unsigned long long w = mix64(key) & window_mask;
  // Each window is visited at most kWindowSlots + 1 times (every failed CAS
  // means one more slot of it was claimed), so this bound is never reached on
  // a table with a free slot; reaching it reports a full table.
  const unsigned long long max_steps = (window_mask + 1) * (kWindowSlots + 1);
  for (unsigned long long step = 0; step < max_steps; ++step) {
    Slot* win = table + w * kWindowSlots;
    // Device-scope atomic load: other CUs may have claimed slots since the
    // kernel started, and a stale cached view must not be trusted.
    const unsigned long long cur =
        __hip_atomic_load(&win[sub].key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long hit = (__ballot(cur == key) >> gbase) & 0xfull;
    if (hit) {
      if (sub == 0) raise_flag(summary, kFlagDuplicate);
      return;
    }
    const unsigned long long free_bits = (__ballot(cur == kEmptyKey) >> gbase) & 0xfull;
    if (!free_bits) {
      w = (w + 1) & window_mask;
      continue;
    }
    const int leader = __ffsll(static_cast<long long>(free_bits)) - 1;
    unsigned long long old = 0;
    if (sub == leader) {
      old = atomicCAS(&win[sub].key, kEmptyKey, key);
      if (old == kEmptyKey) win[sub].row = static_cast<int32_t>(v);
    }
    old = __shfl(old, gbase + leader);
    if (old == kEmptyKey) return;  // claimed
    if (old == key) {              // the same key won the slot first
      if (sub == 0) raise_flag(summary, kFlagDuplicate);
      return;
    }
    // another key took the slot: look at the same window again
  }
  if (sub == 0) raise_flag(summary, kFlagTableFull);
}

// Grid: x covers voxels (4 lanes each), y = index j of the positive offset
// k = centre + 1 + j.  Consecutive groups take consecutive voxels for the same
// offset, so coordinate reads and the positive-side scratch writes coalesce.
__global__ __launch_bounds__(256) void k_probe(const int4* __restrict__ coords, int64_t n, int K,
                                               int KV, int centre, const Slot* __restrict__ table,
                                               unsigned long long window_mask,
                                               int32_t* __restrict__ nbr, uint32_t* masks,
                                               long long* summary) {
  const int64_t q = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kGroup;
  if (q >= n) return;
  const int lane = threadIdx.x & 63;
  const int sub = lane & (kGroup - 1);
  const int gbase = lane & ~(kGroup - 1);
  const int kpos = centre + 1 + static_cast<int>(blockIdx.y);
  const int kneg = KV - 1 - kpos;
  const int r = (K - 1) / 2;
  const int dz = kpos / (K * K) - r;
  const int dy = (kpos / K) % K - r;
  const int dx = kpos % K - r;
  const int4 c = coords[q];
  const int z = c.y + dz, y = c.z + dy, x = c.w + dx;
  if (!coord_in_range(z) || !coord_in_range(y) || !coord_in_range(x)) return;  // never wraps
  const unsigned long long key = pack_key(c.x, z, y, x);
  unsigned long long w = mix64(key) & window_mask;
  for (unsigned long long step = 0; step <= window_mask; ++step) {
    const Slot s = table[w * kWindowSlots + sub];
    const unsigned long long hit = (__ballot(s.key == key) >> gbase) & 0xfull;
    if (hit) {
      if (sub == __ffsll(static_cast<long long>(hit)) - 1) {
        const int64_t p = s.row;
        if (p < 0 || p >= n) {  // a claimed slot always holds its row; never index out of bounds
          raise_flag(summary, kFlagTableFull);
          return;
        }
        nbr[static_cast<int64_t>(kpos) * n + q] = static_cast<int32_t>(p);
        nbr[static_cast<int64_t>(kneg) * n + p] = static_cast<int32_t>(q);
        atomicOr(&masks[static_cast<int64_t>(kpos >> 5) * n + q], 1u << (kpos & 31));
        atomicOr(&masks[static_cast<int64_t>(kneg >> 5) * n + p], 1u << (kneg & 31));
      }
      return;
    }
    if ((__ballot(s.key == kEmptyKey) >> gbase) & 0xfull) return;  // miss
    w = (w + 1) & window_mask;
  }
  if (sub == 0) raise_flag(summary, kFlagTableFull);
}

__device__ __forceinline__ bool has_entry(const uint32_t* __restrict__ mword, uint32_t bit,
                                          bool is_centre, int64_t q, int64_t n) {
  if (q >= n) return false;
  return is_centre || (mword[q] & bit) != 0u;
}

// Grid: x = chunk of kChunkTiles tiles, y = offset k.  Wave w counts tiles
// chunk * 64 + 16 w + [0, 16).
__global__ __launch_bounds__(256) void k_count(const uint32_t* __restrict__ masks, int64_t n,
                                               int64_t tiles, int centre, int64_t chunks,
                                               int64_t* __restrict__ chunk_sum) {
  const int k = blockIdx.y;
  const int64_t chunk = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t* mword = masks + static_cast<int64_t>(k >> 5) * n;
  const uint32_t bit = 1u << (k & 31);
  const bool is_centre = (k == centre);
  int cnt = 0;
  for (int i = 0; i < 16; ++i) {
    const int64_t t = chunk * kChunkTiles + wave * 16 + i;
    if (t >= tiles) break;
    cnt += __popcll(__ballot(has_entry(mword, bit, is_centre, t * kTileRows + lane, n)));
  }
  __shared__ int part[4];
  if (lane == 0) part[wave] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    chunk_sum[static_cast<int64_t>(k) * chunks + chunk] = part[0] + part[1] + part[2] + part[3];
  }
}

// One workgroup of 1024 threads: exclusive scan of the KV x chunks counts in
// offset-major order (so the base of (k, chunk) is the list offset of k plus
// the entries of k in earlier chunks); totals go to the summary.
__global__ __launch_bounds__(1024) void k_scan(int64_t* __restrict__ a, int64_t m, int KV,
                                               int64_t chunks, long long* summary) {
  __shared__ int64_t part[1024];
  const int t = threadIdx.x;
  const int64_t per = (m + 1023) / 1024;
  const int64_t b = t * per;
  const int64_t e = (b + per < m) ? b + per : m;
  int64_t s = 0;
  for (int64_t i = b; i < e; ++i) s += a[i];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int64_t add = (t >= off) ? part[t - off] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  const int64_t total = part[1023];
  int64_t base = part[t] - s;
  for (int64_t i = b; i < e; ++i) {
    const int64_t val = a[i];
    a[i] = base;
    base += val;
  }
  __syncthreads();
  if (t == 0) summary[1] = total;
  for (int k = t; k < KV; k += 1024) {
    const int64_t lo = a[static_cast<int64_t>(k) * chunks];
    const int64_t hi = (k + 1 < KV) ? a[static_cast<int64_t>(k + 1) * chunks] : total;
    summary[kSummaryHead + k] = hi - lo;
  }
}

// Grid: x = chunk, y = offset k.  Same tile walk as k_count; ballot ranks
// give each entry its place.  tile_off[k * tiles + t] = first entry of tile t
// in list k; tile_off[KV * tiles] = E.
__global__ __launch_bounds__(256) void k_compact(const uint32_t* __restrict__ masks,
                                                 const int32_t* __restrict__ nbr, int64_t n,
                                                 int64_t tiles, int KV, int centre, int64_t chunks,
                                                 const int64_t* __restrict__ chunk_base,
                                                 int64_t total, int32_t* __restrict__ in_idx,
                                                 int32_t* __restrict__ out_idx,
                                                 int32_t* __restrict__ tile_off) {
  const int k = blockIdx.y;
  const int64_t chunk = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t* mword = masks + static_cast<int64_t>(k >> 5) * n;
  const uint32_t bit = 1u << (k & 31);
  const bool is_centre = (k == centre);
  unsigned long long bal[16];
  int wcnt = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t t = chunk * kChunkTiles + wave * 16 + i;
    bal[i] = (t < tiles) ? __ballot(has_entry(mword, bit, is_centre, t * kTileRows + lane, n)) : 0ull;
    wcnt += __popcll(bal[i]);
  }
  __shared__ int part[4];
  if (lane == 0) part[wave] = wcnt;
  __syncthreads();
  int64_t base = chunk_base[static_cast<int64_t>(k) * chunks + chunk];
  for (int w = 0; w < wave; ++w) base += part[w];
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int32_t* nk = nbr + static_cast<int64_t>(k) * n;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t t = chunk * kChunkTiles + wave * 16 + i;
    if (t < tiles) {
      if (lane == 0) tile_off[static_cast<int64_t>(k) * tiles + t] = static_cast<int32_t>(base);
      const int64_t q = t * kTileRows + lane;
      if ((bal[i] >> lane) & 1ull) {
        const int64_t pos = base + __popcll(bal[i] & below);
        in_idx[pos] = is_centre ? static_cast<int32_t>(q) : nk[q];
        out_idx[pos] = static_cast<int32_t>(q);
      }
      base += __popcll(bal[i]);
    }
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    tile_off[static_cast<int64_t>(KV) * tiles] = static_cast<int32_t>(total);
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
  b += align_up(static_cast<size_t>(p.table_slots) * sizeof(Slot), 256);
  b += align_up(static_cast<size_t>(p.mask_words) * p.n * sizeof(uint32_t), 256);
  b += align_up(static_cast<size_t>(p.KV) * p.n * sizeof(int32_t), 256);
  b += align_up(static_cast<size_t>(p.KV) * p.chunks * sizeof(int64_t), 256);
  b += align_up(static_cast<size_t>(kSummaryHead + p.KV) * sizeof(long long), 256);
  return b;
}

void carve_build_scratch(const BuildPlan& p, void* base, BuildScratch* s) {
  char* c = static_cast<char*>(base);
  s->table = reinterpret_cast<Slot*>(c);
  c += align_up(static_cast<size_t>(p.table_slots) * sizeof(Slot), 256);
  s->masks = reinterpret_cast<uint32_t*>(c);
  c += align_up(static_cast<size_t>(p.mask_words) * p.n * sizeof(uint32_t), 256);
  s->nbr = reinterpret_cast<int32_t*>(c);
  c += align_up(static_cast<size_t>(p.KV) * p.n * sizeof(int32_t), 256);
  s->chunk_sum = reinterpret_cast<int64_t*>(c);
  c += align_up(static_cast<size_t>(p.KV) * p.chunks * sizeof(int64_t), 256);
  s->summary = reinterpret_cast<long long*>(c);
}

hipError_t launch_build_front(const BuildPlan& p, const int32_t* coords, const BuildScratch& s,
                              hipStream_t stream) {
  const int64_t mask_elems = static_cast<int64_t>(p.mask_words) * p.n;
  int64_t init_work = p.table_slots > mask_elems ? p.table_slots : mask_elems;
  hipLaunchKernelGGL(k_init, dim3(grid_for(init_work, 256, 4096)), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(s.table), p.table_slots, s.masks, mask_elems,
                     s.summary, kSummaryHead + p.KV);
  const unsigned long long window_mask =
      static_cast<unsigned long long>(p.table_slots / kWindowSlots) - 1ull;
  const int4* c4 = reinterpret_cast<const int4*>(coords);
  const int64_t lanes = p.n * kGroup;
  const unsigned gx = static_cast<unsigned>((lanes + 255) / 256);
  hipLaunchKernelGGL(k_insert, dim3(gx), dim3(256), 0, stream, c4, p.n, s.table, window_mask,
                     s.summary);
  if (p.half > 0) {
    hipLaunchKernelGGL(k_probe, dim3(gx, static_cast<unsigned>(p.half)), dim3(256), 0, stream, c4,
                       p.n, p.K, p.KV, p.centre, s.table, window_mask, s.nbr, s.masks, s.summary);
  }
  hipLaunchKernelGGL(k_count, dim3(static_cast<unsigned>(p.chunks), static_cast<unsigned>(p.KV)),
                     dim3(256), 0, stream, s.masks, p.n, p.tiles, p.centre, p.chunks, s.chunk_sum);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, stream, s.chunk_sum,
                     static_cast<int64_t>(p.KV) * p.chunks, p.KV, p.chunks, s.summary);
  return hipGetLastError();
}

hipError_t launch_build_compact(const BuildPlan& p, const BuildScratch& s, int64_t total,
                                int32_t* in_idx, int32_t* out_idx, int32_t* tile_off,
                                hipStream_t stream) {
  hipLaunchKernelGGL(k_compact, dim3(static_cast<unsigned>(p.chunks), static_cast<unsigned>(p.KV)),
                     dim3(256), 0, stream, s.masks, s.nbr, p.n, p.tiles, p.KV, p.centre, p.chunks,
                     s.chunk_sum, total, in_idx, out_idx, tile_off);
  return hipGetLastError();
}

}  // namespace spconv
