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
// Coordinate table: open addressing over 16-byte slots (64-bit key with b, z,
// y, x in 16-bit fields; the row; a "displaced" bit), probed in aligned
// windows of 8 slots (128 bytes) with linear probing over windows.  The home
// window of a key hashes (b, z, y, x >> 2), so the four keys of an aligned run
// of x share a window (in a hash-chosen half), and each key first claims its
// own slot x & 3 there.  A
// key that loses its preferred slot marks that slot displaced before going
// elsewhere.  A lookup therefore settles on the preferred slot alone
// (the key, EMPTY, or another key in an unmarked slot: absent) except in the
// few marked slots, where the window is scanned.
//
// Pipeline (one stream, six launches, seven for an ordered map, one fewer
// when the table is already clear; the last one also writes the small
// summary into the host's pinned memory):
//   k_init     clear the table and the occupancy map, unless the previous
//              build on the same scratch (same table size) left them clear
//   k_claim    one lane per voxel: a plain store of its row claims its
//              preferred slot (last writer wins); it also clears the
//              voxel's negative-half flags, and the summary
//   k_insert   one lane per voxel: the winner writes its key; a loser is a
//              duplicate of the winner or takes the first unreserved free slot
//              by CAS (the only atomics of the insert)
//   k_probe    one lane per voxel: look up Q + d for the (K^3 - 1) / 2
//              offsets d after the centre (lexicographic in (dz, dy, dx)),
//              their loads in flight together.  A hit also records the mirror
//              entry (Q, P, -d), since (P, Q, d) <-> (Q, P, -d) ("Sparse
//              inputs and sparse convolution", section "A symmetry you can
//              check on the slide"), so half of the offsets are probed.  Each
//              (row, offset) cell has one writer, so flags and neighbour rows
//              are plain stores.
//   k_order    (ordered maps) per window of kOrderWindow rows, the rows sorted
//              by a 16-bit key of their neighbour flags: the map's row order
//              (perm); then the window's tiles counted as k_count counts them
//   k_count    (maps in the input order) per 64-row tile and offset, a
//              ballot of the flags is the tile's row mask; per-group counts
//              and per-offset totals
//   k_scan     (ordered maps) per offset: each group's first list position
//   k_compact  per (offset, chunk): the list start from the totals and the
//              counts of earlier chunks, then each entry's place from the tile
//              masks; lists come out grouped by offset ("sorted by weight
//              offset", section "Nine entries become two") and in the row
//              order within an offset; then its grid clears the table and
//              the occupancy map for the next build on the scratch.  An
//              ordered map uses k_compact_window: per (offset, window), the
//              probe's neighbour column of the window's rows staged in LDS
//              with coalesced loads, then read through the permutation (its
//              table is cleared by k_init in the next build).
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

// Home window of a key: hash of the key without the two low bits of x, so an
// aligned run of 4 x values shares it.  The run takes the half of the window
// chosen by a high hash bit (independent of the window index), and each key
// its slot x & 3 in that half.
__device__ __forceinline__ unsigned long long key_hash(unsigned long long key) { return mix64(key >> 2); }
__device__ __forceinline__ unsigned long long home_window(unsigned long long key,
                                                          unsigned long long window_mask) {
  return key_hash(key) & window_mask;
}
__device__ __forceinline__ unsigned long long preferred_slot(unsigned long long key,
                                                             unsigned long long window_mask) {
  const unsigned long long h = key_hash(key);
  return (h & window_mask) * kWindowSlots + ((h >> 60) & 4ull) + (key & 3ull);
}

// Occupancy map: buckets of 16 bytes, one per run of 16 x values of a
// (b, z, y) line, at a hash of (b, z, y, x >> 4); byte x & 15 is set when
// that voxel is present.  A probe reads a whole bucket per line of
// neighbours (K = 3: 5 lines cover the 13 offsets), so most absent
// neighbours are settled without touching the table.  Buckets of different
// runs may coincide: a set byte is a candidate, confirmed in the table; a
// clear byte is a certain miss.
__device__ __forceinline__ unsigned long long occ_bucket(int b, int z, int y, int xr,
                                                         unsigned long long bucket_mask) {
  return mix64(pack_key(b, z, y, xr) + 0x9e3779b97f4a7c15ull) & bucket_mask;
}

__device__ __forceinline__ unsigned long long lane_u64(unsigned long long v, int src) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), src));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), src));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

__device__ __forceinline__ bool coord_in_range(int v) { return v >= 0 && v < 65536; }

__device__ __forceinline__ bool voxel_in_range(int4 c) {
  return c.x >= 0 && c.x < 32768 && coord_in_range(c.y) && coord_in_range(c.z) && coord_in_range(c.w);
}

// Slot fields: .x is the key; the low 32 bits of .y the row, the high 32 bits
// flags (bit 0: a key was displaced from this slot).  Row and flags are
// separate words so that neither write can clobber the other.
constexpr uint32_t kSlotDisplaced = 1u;
__device__ __forceinline__ uint32_t* slot_row(ulonglong2* s) {
  return reinterpret_cast<uint32_t*>(&s->y);
}
__device__ __forceinline__ uint32_t* slot_flags(ulonglong2* s) {
  return reinterpret_cast<uint32_t*>(&s->y) + 1;
}

__device__ __forceinline__ void raise_flag(long long* summary, unsigned long long bit) {
  atomicOr(reinterpret_cast<unsigned long long*>(summary), bit);
}

// Unit i of the table's clear state (16 bytes each): table slot i as
// (EMPTY, row -1, no flags) for i < slots, then occupancy bucket i - slots as
// zeros.
__device__ __forceinline__ void clear_table_unit(uint4* table, int64_t slots, uint4* occ, int64_t buckets,
                                                 int64_t i) {
  if (i < slots) {
    table[i] = make_uint4(0xffffffffu, 0xffffffffu, 0xffffffffu, 0u);  // key ~0, row -1, no flags
  } else if (i - slots < buckets) {
    occ[i - slots] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// Clears the table slots and the occupancy map (kInitUnits 16-byte units per
// thread, a workgroup's stores contiguous).  A build whose scratch's last
// build left a table of the same size clear (k_compact, the last kernel of a
// map in the input order, clears it) skips this launch.
constexpr int kInitUnits = 4;
__global__ __launch_bounds__(256) void k_init(uint4* table, int64_t slots, uint4* occ, int64_t buckets) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * blockDim.x * kInitUnits + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kInitUnits; ++u) clear_table_unit(table, slots, occ, buckets, base + u * blockDim.x);
}

// Insert, phase 1 (one lane per voxel): claim the preferred slot of the home
// window with a plain store of the row; the last writer wins.  The voxel's
// byte of the occupancy map is set too (every writer stores 1).  Each lane
// also clears its voxel's negative-half flag record (nbu 16-byte units; the
// probe, a later kernel, sets them), and the first workgroup the summary.
__global__ __launch_bounds__(256) void k_claim(const int4* __restrict__ coords, int64_t n, ulonglong2* table,
                                               uint8_t* occ, unsigned long long window_mask,
                                               unsigned long long bucket_mask, uint4* neg, int nbu,
                                               long long* summary, int summary_len) {
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < summary_len; i += blockDim.x) summary[i] = 0;
  }
  const int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v >= n) return;
  const int4 c = coords[v];
  if (voxel_in_range(c)) {  // out of range: reported by phase 2
    const unsigned long long key = pack_key(c.x, c.y, c.z, c.w);
    *slot_row(&table[preferred_slot(key, window_mask)]) = static_cast<uint32_t>(v);
    occ[occ_bucket(c.x, c.y, c.z, c.w >> 4, bucket_mask) * 16 + (c.w & 15)] = 1;
  }
  // after the load (a store before it would hold up its wait)
  for (int u = 0; u < nbu; ++u) neg[v * nbu + u] = make_uint4(0u, 0u, 0u, 0u);
}

__device__ __forceinline__ bool same_voxel(int4 a, int4 b) {
  return a.x == b.x && a.y == b.y && a.z == b.z && a.w == b.w;
}

// Insert, phase 2 (one lane per voxel; phase 1 is complete, a kernel
// boundary).  The winner of a preferred slot writes its key there with a
// plain store.  A loser whose winner has the same coordinates is a duplicate;
// otherwise it marks the slot displaced and takes, by CAS, the first slot
// that no phase-1 winner reserved and no other loser took, in an order fixed
// by the key (increasing or decreasing slot index, by a hash bit, window
// after window).  Two losers with one key thus always meet on the slot the
// first one took, so duplicates are always detected.  Views are read with plain loads; a stale view can only show a
// slot free that has since been taken (slots are never released), and a
// failed CAS returns the slot's true key.  Every window is left as soon as it
// is seen full, so the search visits each window at most once.
__global__ __launch_bounds__(256) void k_insert(const int4* __restrict__ coords, int64_t n,
                                                ulonglong2* table, unsigned long long window_mask,
                                                long long* summary) {
  const int64_t v = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v >= n) return;
  const int4 c = coords[v];
  if (!voxel_in_range(c)) {
    raise_flag(summary, kFlagRange);
    return;
  }
  const unsigned long long key = pack_key(c.x, c.y, c.z, c.w);
  unsigned long long w = home_window(key, window_mask);
  ulonglong2* pslot = &table[preferred_slot(key, window_mask)];
  const uint32_t claim = *slot_row(pslot);
  if (claim == static_cast<uint32_t>(v)) {
    pslot->x = key;
    return;
  }
  // claim is another voxel's row (phase 1 wrote one for every voxel in range).
  // The winner's coordinates (the duplicate check) and the home window are
  // loaded together; the displaced mark is stored after the search, so that
  // no store sits between these loads and the CAS.
  const int4 cw = coords[claim < static_cast<uint64_t>(n) ? claim : 0];
  ulonglong2 e0[kWindowSlots];
#pragma unroll
  for (int j = 0; j < kWindowSlots; ++j) e0[j] = table[w * kWindowSlots + j];
  if (claim < static_cast<uint64_t>(n) && same_voxel(cw, c)) {
    raise_flag(summary, kFlagDuplicate);
    return;
  }
  const bool descending = ((key_hash(key) >> 40) & 1ull) != 0ull;
  const unsigned long long max_steps = window_mask + 1;
  for (unsigned long long step = 0; step < max_steps; ++step) {
    ulonglong2* win = table + w * kWindowSlots;
    unsigned long long view[kWindowSlots];
    bool reserved[kWindowSlots];
    // A slot reserved by a phase-1 winner holds (or is about to hold) that
    // winner's key, which differs from ours: equal keys prefer the same slot,
    // and our own slot's winner was compared above.
#pragma unroll
    for (int j = 0; j < kWindowSlots; ++j) {
      const ulonglong2 e = (step == 0) ? e0[j] : win[j];
      view[j] = e.x;
      reserved[j] = (static_cast<uint32_t>(e.y) != 0xffffffffu);
    }
    bool moved = false;
    for (int attempt = 0; attempt <= kWindowSlots; ++attempt) {
      // the first free slot in ascending or, for half the keys (a hash bit),
      // descending order, so that losers sharing a window race for one slot
      // less often; equal keys take the same order
      bool dup = false;
      int first = -1, last = -1;
#pragma unroll
      for (int j = kWindowSlots - 1; j >= 0; --j) {
        dup |= (view[j] == key);
        if (view[j] == kEmptyKey && !reserved[j]) first = j;
      }
#pragma unroll
      for (int j = 0; j < kWindowSlots; ++j) {
        if (view[j] == kEmptyKey && !reserved[j]) last = j;
      }
      const int target = descending ? last : first;
      if (dup) {
        *slot_flags(pslot) = kSlotDisplaced;
        raise_flag(summary, kFlagDuplicate);
        return;
      }
      if (target < 0) {  // window full: next window
        moved = true;
        break;
      }
      const unsigned long long old =
          atomicCAS(reinterpret_cast<unsigned long long*>(&win[target]), kEmptyKey, key);
      if (old == kEmptyKey) {
        *slot_row(&win[target]) = static_cast<uint32_t>(v);
        *slot_flags(pslot) = kSlotDisplaced;  // every writer stores the same value
        return;
      }
      view[target] = old;  // learn the true key and try again
    }
    if (moved) w = (w + 1) & window_mask;
  }
  *slot_flags(pslot) = kSlotDisplaced;
  raise_flag(summary, kFlagTableFull);
}

// Row of `key` by scanning windows from its home window, or -1.
__device__ __forceinline__ int64_t find_row_scan(unsigned long long key, const ulonglong2* __restrict__ table,
                                 unsigned long long window_mask, bool& overflow) {
  unsigned long long w = home_window(key, window_mask);
  for (unsigned long long step = 0; step <= window_mask; ++step) {
    const ulonglong2* win = table + w * kWindowSlots;
    int64_t found = -1;
    bool empty = false;
#pragma unroll
    for (int j = 0; j < kWindowSlots; ++j) {
      const ulonglong2 e = win[j];
      if (e.x == key) found = static_cast<int64_t>(static_cast<uint32_t>(e.y));
      empty |= (e.x == kEmptyKey);
    }
    if (found >= 0) return found;
    if (empty) return -1;
    w = (w + 1) & window_mask;
  }
  overflow = true;
  return -1;
}

// Offset of index j in the positive half (k = centre + 1 + j) as (dz, dy, dx).
template <int K>
__device__ __forceinline__ void positive_offset(int j, int& dz, int& dy, int& dx) {
  constexpr int R = (K - 1) / 2, centre = (K * K * K - 1) / 2;
  const int k = centre + 1 + j;
  dz = k / (K * K) - R;
  dy = (k / K) % K - R;
  dx = k % K - R;
}

// Lines of the positive half: line 0 is (dz, dy) = (0, 0) with dx in [1, R];
// lines 1..R are (0, dy) and the rest (dz > 0, dy) with dx in [-R, R], in
// the same lexicographic order as the offsets, so a line's offsets are a
// contiguous range of positive indices starting at its first.
template <int K>
struct PosLine {
  static constexpr int R = (K - 1) / 2, W = 2 * R + 1;
  static constexpr int kLines = 1 + R + R * W;
  static constexpr int dz(int l) { return l <= R ? 0 : 1 + (l - R - 1) / W; }
  static constexpr int dy(int l) { return l <= R ? l : -R + (l - R - 1) % W; }
  static constexpr int dx_lo(int l) { return l == 0 ? 1 : -R; }
  static constexpr int count(int l) { return l == 0 ? R : W; }
  static constexpr int first(int l) { return l == 0 ? 0 : R + (l - 1) * W; }
};

// Records the entry (P = p, Q = q, offset k) and its mirror (Q, P, -d).
template <int K>
__device__ __forceinline__ void emit_pair(int j, int64_t q, int32_t p, int64_t n, int32_t* __restrict__ nbr,
                                          uint8_t* __restrict__ neg_flags) {
  constexpr int KV = K * K * K, centre = (KV - 1) / 2, NB = neg_bytes(K);
  const int k = centre + 1 + j;
  const int kneg = centre - 1 - j;  // = KV - 1 - k
  nbr[static_cast<int64_t>(k) * n + q] = p;
  nbr[static_cast<int64_t>(kneg) * n + p] = static_cast<int32_t>(q);
  neg_flags[static_cast<int64_t>(p) * NB + kneg] = 1;
}

// Rows fit 27 bits (n K^3 < 2^31 with K >= 3), lookup indices of a step the
// other 5.
constexpr int kHitRowBits = 27;

// One lane per voxel Q: the (K^3 - 1) / 2 offsets after the centre, a few
// lines of neighbours at a time, each in rounds of loads:
//   1. the occupancy bucket(s) of every line (two when its x range crosses a
//      run boundary): a clear byte settles a lookup as a miss;
//   2. the preferred slot of each candidate: the key is a hit; EMPTY, or
//      another key in a slot not marked displaced, a miss;
//   3. the whole home window of each candidate on a displaced slot (a second
//      pass scans further windows when it is full).
// Within a round every load is issued before any is used, and all stores
// come after the last round: vector-memory counters retire in order, so a
// store issued between loads would make the later loads' waits wait for its
// write acknowledgement too.  A hit on P = Q + d stores the bit of (Q, d) in
// Q's positive-half flag word, the neighbour row at [k][Q], and the mirror
// entry (P, Q, -d).
template <int K>
__global__ __launch_bounds__(256) void k_probe(const int4* __restrict__ coords, int64_t n,
                                               const ulonglong2* __restrict__ table,
                                               const uint4* __restrict__ occ, unsigned long long window_mask,
                                               unsigned long long bucket_mask, int32_t* __restrict__ nbr,
                                               uint32_t* __restrict__ pos_bits,
                                               uint8_t* __restrict__ neg_flags, long long* summary) {
  using L = PosLine<K>;
  constexpr int PW = pos_words(K);
  constexpr int kLinesPerStep = 32 / L::W;         // lines whose buckets are in flight together
  constexpr int kMaxLook = kLinesPerStep * L::W;   // lookups of a step (<= 32)
  constexpr int kCand = 4, kPend = 2;              // loads per lane per round of steps 2 and 3
  static_assert(kMaxLook <= 32, "a step's lookups fit a 32-bit mask");
  static_assert(kMaxLook <= (1 << (32 - kHitRowBits)), "a lookup index fits the hit's high bits");
  // A step's hits (lookup index in the step, high bits; the neighbour's row,
  // low bits), in LDS: the lane's e-th at hits[e * 256 + lane in the
  // workgroup].  Kept out of registers, where an array indexed by the lookup
  // costs a compare and a select per element at every write, and out of
  // global memory until the step's last load (a store before a load would
  // hold up that load's wait).
  __shared__ uint32_t hits[kMaxLook * 256];
  auto record = [&](int js, int64_t p, int& nh) {
    hits[nh * 256 + threadIdx.x] = (static_cast<uint32_t>(js) << kHitRowBits) | static_cast<uint32_t>(p);
    ++nh;
  };
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= n) return;
  const int4 c = coords[q];
  const bool ok = voxel_in_range(c);  // a voxel out of range (a reported error) gets no entries
  bool overflow = false;
  uint32_t bits[PW > 0 ? PW : 1];
#pragma unroll
  for (int w = 0; w < PW; ++w) bits[w] = 0u;
  auto key_of = [&](int j) {
    int dz, dy, dx;
    positive_offset<K>(j, dz, dy, dx);
    return pack_key(c.x, c.y + dz, c.z + dy, c.w + dx);
  };
#pragma unroll
  for (int l0 = 0; l0 < L::kLines; l0 += kLinesPerStep) {
    const int j0 = L::first(l0);
    // 1. occupancy buckets of the step's lines
    uint4 v0[kLinesPerStep], v1[kLinesPerStep];
    int xr0[kLinesPerStep];
#pragma unroll
    for (int i = 0; i < kLinesPerStep; ++i) {
      const int l = l0 + i;
      if (l < L::kLines) {
        const int zz = c.y + L::dz(l), yy = c.z + L::dy(l);
        const bool line_ok = ok && coord_in_range(zz) && coord_in_range(yy);
        const int xlo = max(c.w + L::dx_lo(l), 0), xhi = min(c.w + L::dx_lo(l) + L::count(l) - 1, 65535);
        xr0[i] = xlo >> 4;
        const int xr1 = xhi >> 4;
        const unsigned long long b0 = line_ok ? occ_bucket(c.x, zz, yy, xlo >> 4, bucket_mask) : 0ull;
        v0[i] = occ[b0];  // unconditional (bucket 0 exists), so the loads batch
        v1[i] = make_uint4(0u, 0u, 0u, 0u);
        if (line_ok && xr1 != xr0[i]) v1[i] = occ[occ_bucket(c.x, zz, yy, xr1, bucket_mask)];
      }
    }
    uint32_t cand = 0u;  // bit i: lookup j0 + i has its occupancy byte set
#pragma unroll
    for (int i = 0; i < kLinesPerStep; ++i) {
      const int l = l0 + i;
      if (l < L::kLines) {
        const int zz = c.y + L::dz(l), yy = c.z + L::dy(l);
        const bool line_ok = ok && coord_in_range(zz) && coord_in_range(yy);
#pragma unroll
        for (int e = 0; e < L::W; ++e) {
          if (e < L::count(l)) {
            const int x = c.w + L::dx_lo(l) + e;
            const uint4 v = ((x >> 4) == xr0[i]) ? v0[i] : v1[i];
            const int by = x & 15;
            const uint32_t word = (by < 4) ? v.x : (by < 8) ? v.y : (by < 12) ? v.z : v.w;
            const bool set = line_ok && coord_in_range(x) && ((word >> (8 * (by & 3))) & 0xffu) != 0u;
            cand |= set ? (1u << (L::first(l) - j0 + e)) : 0u;
          }
        }
      }
    }
    int nh = 0;  // hits of the step so far, in hits[] (LDS)
    uint32_t pend = 0u;
    // 2. preferred slots of the candidates
    while (cand != 0u) {
      int js[kCand];
      unsigned long long ks[kCand];
      ulonglong2 sv[kCand];
#pragma unroll
      for (int u = 0; u < kCand; ++u) {
        js[u] = -1;
        ks[u] = 0ull;
        if (cand != 0u) {
          js[u] = __ffs(cand) - 1;
          cand &= cand - 1u;
          ks[u] = key_of(j0 + js[u]);
          sv[u] = table[preferred_slot(ks[u], window_mask)];
        }
      }
#pragma unroll
      for (int u = 0; u < kCand; ++u) {
        if (js[u] >= 0) {
          if (sv[u].x == ks[u]) {
            const int64_t p = static_cast<int64_t>(static_cast<uint32_t>(sv[u].y));
            if (p < n) record(js[u], p, nh);
          } else if (sv[u].x != kEmptyKey &&
                     (static_cast<uint32_t>(sv[u].y >> 32) & kSlotDisplaced) != 0u) {
            pend |= 1u << js[u];
          }
        }
      }
    }
    // 3. candidates on displaced slots: whole home windows, every one loaded
    // before any is scanned
    while (pend != 0u) {
      int js[kPend];
      unsigned long long ks[kPend];
      ulonglong2 wv[kPend][kWindowSlots];
#pragma unroll
      for (int u = 0; u < kPend; ++u) {
        js[u] = -1;
        ks[u] = 0ull;
        if (pend != 0u) {
          js[u] = __ffs(pend) - 1;
          pend &= pend - 1u;
          ks[u] = key_of(j0 + js[u]);
          const ulonglong2* win = table + home_window(ks[u], window_mask) * kWindowSlots;
#pragma unroll
          for (int s2 = 0; s2 < kWindowSlots; ++s2) wv[u][s2] = win[s2];
        }
      }
#pragma unroll
      for (int u = 0; u < kPend; ++u) {
        if (js[u] >= 0) {
          int64_t p = -1;
          bool empty = false;
#pragma unroll
          for (int s2 = 0; s2 < kWindowSlots; ++s2) {
            if (wv[u][s2].x == ks[u]) p = static_cast<int64_t>(static_cast<uint32_t>(wv[u][s2].y));
            empty |= (wv[u][s2].x == kEmptyKey);
          }
          if (p < 0 && !empty) p = find_row_scan(ks[u], table, window_mask, overflow);  // full window
          if (p >= 0 && p < n) record(js[u], p, nh);
        }
      }
    }
    for (int e = 0; e < nh; ++e) {
      const uint32_t hv = hits[e * 256 + threadIdx.x];
      const int j = j0 + static_cast<int>(hv >> kHitRowBits);
      bits[j >> 5] |= 1u << (j & 31);
      emit_pair<K>(j, q, static_cast<int32_t>(hv & ((1u << kHitRowBits) - 1u)), n, nbr, neg_flags);
    }
  }
#pragma unroll
  for (int w = 0; w < PW; ++w) pos_bits[q * PW + w] = bits[w];
  if (overflow) raise_flag(summary, kFlagTableFull);
}

// Offsets whose neighbour flags form a row's order key, most significant
// first: the offsets next to the centre (every coordinate within one step)
// in index order, then the others in index order, kOrderKeyBits of them.
template <int K>
struct KeyOffsets {
  int k[kOrderKeyBits];
  int count;
  constexpr KeyOffsets() : k{}, count(0) {
    constexpr int R = (K - 1) / 2, KV = K * K * K, C = (KV - 1) / 2;
    for (int pass = 0; pass < 2; ++pass) {
      for (int kk = 0; kk < KV && count < kOrderKeyBits; ++kk) {
        if (kk == C) continue;
        const int dz = kk / (K * K) - R, dy = (kk / K) % K - R, dx = kk % K - R;
        const bool inner = dz >= -1 && dz <= 1 && dy >= -1 && dy <= 1 && dx >= -1 && dx <= 1;
        if ((pass == 0) == inner) k[count++] = kk;
      }
    }
  }
};

// Order key of row q: bit kOrderKeyBits - 1 - i set when the row has a
// neighbour at the i-th key offset (the probe's flags).
template <int K>
__device__ __forceinline__ uint32_t order_key(const uint32_t* __restrict__ pos_bits,
                                              const uint8_t* __restrict__ neg_flags, int64_t q) {
  constexpr int KV = K * K * K, centre = (KV - 1) / 2;
  constexpr int PW = pos_words(K), NB = neg_bytes(K), NV = NB / 16;
  constexpr KeyOffsets<K> ko{};
  uint32_t pw[PW];
  uint4 nv[NV];
#pragma unroll
  for (int w = 0; w < PW; ++w) pw[w] = pos_bits[q * PW + w];
#pragma unroll
  for (int v = 0; v < NV; ++v) nv[v] = *reinterpret_cast<const uint4*>(neg_flags + q * NB + 16 * v);
  uint32_t key = 0u;
#pragma unroll
  for (int i = 0; i < ko.count; ++i) {
    const int k = ko.k[i];
    bool f;
    if (k < centre) {
      const uint4 v = nv[k / 16];
      const uint32_t word = ((k % 16) / 4 == 0) ? v.x : ((k % 16) / 4 == 1) ? v.y : ((k % 16) / 4 == 2) ? v.z : v.w;
      f = ((word >> (8 * (k % 4))) & 0xffu) != 0u;
    } else {
      const int j = k - centre - 1;
      f = ((pw[j >> 5] >> (j & 31)) & 1u) != 0u;
    }
    key |= static_cast<uint32_t>(f) << (kOrderKeyBits - 1 - i);
  }
  return key;
}

// The count of tile t (positions t * kTileRows + lane of the row order) by
// one wave, each lane holding the row at its position (`valid` false past
// n): per offset k, a ballot of the rows' flags is the tile's row mask; lane
// k mod 64 stores it to tile_mask[k][t], with tile_base[k][t], the number of
// the tile's non-centre entries at offsets before k, and adds its population
// to cnt[k / 64].
template <int K>
__device__ __forceinline__ void count_tile(const uint32_t* __restrict__ pos_bits,
                                           const uint8_t* __restrict__ neg_flags, int64_t row, bool valid,
                                           int64_t t, int64_t tiles, unsigned long long* __restrict__ tile_mask,
                                           int32_t* __restrict__ tile_base, int (&cnt)[(K * K * K + 63) / 64]) {
  constexpr int KV = K * K * K;
  constexpr int centre = (KV - 1) / 2;
  constexpr int NS = (KV + 63) / 64;  // offsets per lane
  constexpr int PW = pos_words(K), NB = neg_bytes(K), NV = NB / 16;
  const int lane = threadIdx.x & 63;
  uint32_t pw[PW > 0 ? PW : 1];
  uint4 nv[NV > 0 ? NV : 1];
#pragma unroll
  for (int w = 0; w < PW; ++w) pw[w] = pos_bits[row * PW + w];
#pragma unroll
  for (int v = 0; v < NV; ++v) nv[v] = *reinterpret_cast<const uint4*>(neg_flags + row * NB + 16 * v);
  unsigned long long mine[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) mine[s] = 0ull;
  const unsigned long long vmask = __ballot(valid);  // lanes holding a row
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int jj = 0; jj < 64; ++jj) {
      const int k = s * 64 + jj;
      if (k < KV) {
        bool f;
        if (k == centre) {
          f = true;
        } else if (k < centre) {
          const uint4 v = nv[k / 16];
          const uint32_t word = ((k % 16) / 4 == 0) ? v.x : ((k % 16) / 4 == 1) ? v.y : ((k % 16) / 4 == 2) ? v.z : v.w;
          f = ((word >> (8 * (k % 4))) & 0xffu) != 0u;
        } else {
          const int j = k - centre - 1;
          f = ((pw[j >> 5] >> (j & 31)) & 1u) != 0u;
        }
        const unsigned long long bal = __ballot(f) & vmask;
        if (lane == jj) mine[s] = bal;
      }
    }
  }
  int before = 0;  // non-centre entries of the tile at offsets of earlier slots
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int k = s * 64 + lane;
    const int c = (k < KV && k != centre) ? static_cast<int>(__popcll(mine[s])) : 0;
    const int excl = wave_prefix_small<7>(c);
    if (k < KV) {
      tile_mask[static_cast<int64_t>(k) * tiles + t] = mine[s];
      tile_base[static_cast<int64_t>(k) * tiles + t] = before + excl;
    }
    before += __builtin_amdgcn_readlane(excl + c, 63);
    cnt[s] += __popcll(mine[s]);
  }
}

// The map's row order ("TorchSparse: regular computation from irregular
// sparsity", section "TorchSparse++: overlap memory with computation": rows
// reordered by their neighbour bitmask, so that rows computed together need
// the same weights).  One workgroup of 1024 threads per window of
// kOrderWindow consecutive rows sorts the window's rows stably by key and
// writes perm[w0 + i] = the row at sorted position i (each row's key is
// order_key of its flags); windows keep rows near
// their neighbours in space, and tiles never straddle two.  An LSD radix sort
// over 8-bit digits in LDS: element e of the window sits with wave
// e / (E x 64), round (e / 64) mod E, lane e mod 64, and within a pass a
// wave ranks its own elements round by round (lanes with equal digits found
// by eight ballots, counts kept in the wave's row of the histogram), so that
// the only workgroup barriers are those around the per-digit scan and the
// scatter.  Rows past n sort last (key ~0 and the largest positions).
// The sorted window is then counted in place of a separate pass: wave w
// holds the window's tiles w E .. w E + E - 1 (position e of tile t in lane
// e mod 64), counts each with count_tile, and the waves of each group of
// kGroupTiles tiles add their counts through LDS into chunk_sum[k][group]
// (one chunk per group) and the window's into the per-offset totals.
constexpr int kOrderThreads = 1024;
constexpr int kOrderPerThread = kOrderWindow / kOrderThreads;
constexpr int kOrderWaves = kOrderThreads / 64;
constexpr int kOrderPasses = (kOrderKeyBits + 7) / 8;
constexpr int kOrderGroups = kOrderWindow / (kTileRows * kGroupTiles);
static_assert(kTileRows == 64 && kGroupTiles % kOrderPerThread == 0, "a wave's rounds are whole tiles of one group");
template <int K>
__global__ __launch_bounds__(kOrderThreads) void k_order(const uint32_t* __restrict__ pos_bits,
                                                          const uint8_t* __restrict__ neg_flags, int64_t n,
                                                          int32_t* __restrict__ perm, int64_t tiles, int64_t groups,
                                                          unsigned long long* __restrict__ tile_mask,
                                                          int32_t* __restrict__ tile_base,
                                                          int64_t* __restrict__ chunk_sum, long long* summary) {
  constexpr int E = kOrderPerThread;
  __shared__ unsigned long long buf[kOrderWindow];
  __shared__ uint32_t hist[kOrderWaves * 256];
  __shared__ uint32_t wtot[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t w0 = static_cast<int64_t>(blockIdx.x) * kOrderWindow;
  const int64_t wn = (n - w0 < kOrderWindow) ? n - w0 : kOrderWindow;
  const unsigned long long below = (1ull << lane) - 1ull;
  uint32_t key[E], idx[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int e = (wave * E + j) * 64 + lane;
    idx[j] = static_cast<uint32_t>(e);
    const uint32_t kv = order_key<K>(pos_bits, neg_flags, w0 + (e < wn ? e : wn - 1));  // unconditional loads batch
    key[j] = (e < wn) ? kv : ~0u;
  }
#pragma unroll 1
  for (int pass = 0; pass < kOrderPasses; ++pass) {
    const int shift = 8 * pass;
    uint32_t* row = hist + wave * 256;
    for (int d = lane; d < 256; d += 64) row[d] = 0u;
    // Lanes with the digit of each round (independent of one another, so
    // computed for all rounds first), then the rounds' counts in order: each
    // lane reads its digit's count so far and every lane of the digit writes
    // the same new count (LDS operations of a wave run in order, so a round
    // sees the rounds before it).
    uint32_t rank[E], cnt[E], dig[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const uint32_t d = (key[j] >> shift) & 255u;
      unsigned long long peers = ~0ull;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const unsigned long long bb = __ballot((d >> b) & 1u);
        peers &= ((d >> b) & 1u) ? bb : ~bb;
      }
      dig[j] = d;
      rank[j] = static_cast<uint32_t>(__popcll(peers & below));
      cnt[j] = static_cast<uint32_t>(__popcll(peers));
    }
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const uint32_t base = row[dig[j]];
      rank[j] += base;
      row[dig[j]] = base + cnt[j];
    }
    __syncthreads();
    // Per digit (thread d < 256): the counts of earlier waves become each
    // wave's base, and an exclusive scan over digits gives the digit starts.
    uint32_t tot = 0u, incl = 0u;
    if (threadIdx.x < 256) {
      const int d = threadIdx.x;
#pragma unroll
      for (int w = 0; w < kOrderWaves; ++w) {
        const uint32_t c = hist[w * 256 + d];
        hist[w * 256 + d] = tot;
        tot += c;
      }
      incl = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_up(incl, o);
        if (lane >= o) incl += u;
      }
      if (lane == 63) wtot[wave] = incl;
    }
    __syncthreads();
    if (threadIdx.x < 256) {
      const int d = threadIdx.x;
      uint32_t start = incl - tot;
      for (int w = 0; w < wave; ++w) start += wtot[w];
#pragma unroll
      for (int w = 0; w < kOrderWaves; ++w) hist[w * 256 + d] += start;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < E; ++j) {
      buf[hist[wave * 256 + dig[j]] + rank[j]] = (static_cast<unsigned long long>(key[j]) << 32) | idx[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const unsigned long long u = buf[(wave * E + j) * 64 + lane];
      key[j] = static_cast<uint32_t>(u >> 32);
      idx[j] = static_cast<uint32_t>(u);
    }
    __syncthreads();  // every read of buf and of the histogram done before the next pass
  }
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int e = (wave * E + j) * 64 + lane;
    if (e < wn) perm[w0 + e] = static_cast<int32_t>(w0 + idx[j]);
  }
  constexpr int KV = K * K * K, NS = (KV + 63) / 64;
  int cnt[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) cnt[s] = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * (kOrderWindow / kTileRows) + wave * E + j;
    if (t < tiles) {  // uniform over the wave
      const int e = (wave * E + j) * 64 + lane;
      const bool valid = e < wn;
      count_tile<K>(pos_bits, neg_flags, w0 + (valid ? idx[j] : 0u), valid, t, tiles, tile_mask, tile_base, cnt);
    }
  }
  // Per-wave counts through LDS (buf is free: the last pass ended on a barrier).
  static_assert(kOrderWaves * NS * 64 * sizeof(int) <= sizeof(buf), "counts fit the sort buffer");
  int* part = reinterpret_cast<int*>(buf);
#pragma unroll
  for (int s = 0; s < NS; ++s) part[wave * NS * 64 + s * 64 + lane] = cnt[s];
  __syncthreads();
  constexpr int WG = kOrderWaves / kOrderGroups;  // waves per group
  for (int k = threadIdx.x; k < KV; k += kOrderThreads) {
    long long total = 0;
#pragma unroll
    for (int g = 0; g < kOrderGroups; ++g) {
      int sum = 0;
#pragma unroll
      for (int w = 0; w < WG; ++w) sum += part[(g * WG + w) * NS * 64 + k];
      const int64_t gi = static_cast<int64_t>(blockIdx.x) * kOrderGroups + g;
      if (gi < groups) chunk_sum[static_cast<int64_t>(k) * groups + gi] = sum;
      total += sum;
    }
    if (total != 0) {
      atomicAdd(reinterpret_cast<unsigned long long*>(&summary[kSummaryHead + k]),
                static_cast<unsigned long long>(total));
    }
  }
}

// Maps in the input order (ordered maps are counted by k_order): one
// workgroup of 1024 threads (16 waves) per chunk of group_tiles tiles, one
// tile per wave at a time (launched with chunks of one group, so each wave
// counts one tile with count_tile).  Per-chunk counts go to
// chunk_sum[k][chunk] and are added to the per-offset totals in the summary.
template <int K>
__global__ __launch_bounds__(1024) void k_count(const uint32_t* __restrict__ pos_bits,
                                                const uint8_t* __restrict__ neg_flags,
                                                const int32_t* __restrict__ perm, int64_t n,
                                                int64_t tiles, int64_t group_tiles, int64_t chunks,
                                                unsigned long long* __restrict__ tile_mask,
                                                int32_t* __restrict__ tile_base,
                                                int64_t* __restrict__ chunk_sum, long long* summary) {
  constexpr int KV = K * K * K;
  constexpr int NS = (KV + 63) / 64;  // offsets per lane
  const int64_t chunk = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int cnt[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) cnt[s] = 0;
  for (int64_t g = 0; g < group_tiles; g += kGroupTiles) {
    const int64_t t = chunk * group_tiles + g + wave;
    if (t >= tiles) break;  // tiles of later groups are past the end too
    const int64_t q = t * kTileRows + lane;  // position in the row order
    const bool valid = q < n;
    const int64_t qp = valid ? q : n - 1;
    const int64_t qs = perm != nullptr ? static_cast<int64_t>(perm[qp]) : qp;  // its row
    count_tile<K>(pos_bits, neg_flags, qs, valid, t, tiles, tile_mask, tile_base, cnt);
  }
  __shared__ int part[kGroupTiles][NS * 64];
#pragma unroll
  for (int s = 0; s < NS; ++s) part[wave][s * 64 + lane] = cnt[s];
  __syncthreads();
  for (int k = threadIdx.x; k < KV; k += 1024) {
    int sum = 0;
#pragma unroll
    for (int w = 0; w < kGroupTiles; ++w) sum += part[w][k];
    chunk_sum[static_cast<int64_t>(k) * chunks + chunk] = sum;
    if (sum != 0) {
      atomicAdd(reinterpret_cast<unsigned long long*>(&summary[kSummaryHead + k]),
                static_cast<unsigned long long>(sum));
    }
  }
}

// Grid: x = chunk, y = offset k; 256 threads, wave w places the entries of
// the quarter w of the chunk's tiles, in tile order.  The workgroup's first
// list position is the sum of the totals of offsets before k and of the
// counts of chunks of offset k before this one (k_count has completed: a
// kernel boundary).  tile_off[k * tiles + t] = first entry of tile t in list
// k; the last workgroup also writes tile_off[KV * tiles] = E.  A non-centre
// entry also goes to its tile's slot table (tile_rows), at slot
// tile_base[k][t] + its rank in the tile's mask, when that is below
// kTileSlots.
__global__ __launch_bounds__(256) void k_compact(const unsigned long long* __restrict__ tile_mask,
                                                 const int32_t* __restrict__ tile_base,
                                                 const int32_t* __restrict__ nbr, int64_t n,
                                                 int64_t tiles, int centre, int KV, int64_t group_tiles,
                                                 int64_t chunks, const int64_t* __restrict__ chunk_sum,
                                                 const long long* __restrict__ summary,
                                                 int32_t* __restrict__ in_idx,
                                                 int32_t* __restrict__ out_idx,
                                                 int32_t* __restrict__ tile_off,
                                                 int32_t* __restrict__ tile_rows,
                                                 long long* __restrict__ host_summary, uint4* table,
                                                 int64_t slots, uint4* occ, int64_t buckets) {
  const int k = blockIdx.y;
  const int64_t chunk = blockIdx.x;
  // The summary is final (its writers ran in earlier kernels): the first
  // workgroup hands it to the host's pinned slot, which saves a copy launch.
  if (chunk == 0 && k == 0) {
    for (int i = threadIdx.x; i < kSummaryHead + KV; i += blockDim.x) host_summary[i] = summary[i];
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool is_centre = (k == centre);
  const int64_t per = group_tiles / 4;  // tiles of this wave
  const int64_t t0 = chunk * group_tiles + wave * per;
  __shared__ long long s_base;
  __shared__ long long s_wave[4];
  if (wave == 0) {
    long long s = 0;
    for (int i = lane; i < k; i += 64) s += summary[kSummaryHead + i];
    // the counts were taken per group of kGroupTiles tiles
    const int64_t groups = (tiles + kGroupTiles - 1) / kGroupTiles;
    const int64_t before = chunk * (group_tiles / kGroupTiles);
    for (int64_t cc = lane; cc < before; cc += 64) s += chunk_sum[static_cast<int64_t>(k) * groups + cc];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) s += __shfl_xor(s, d);
    if (lane == 0) s_base = s;
  }
  // The wave's tiles in rounds of 64, one tile mask per lane: the round's
  // entry count, then (after the workgroup base is known) each tile's first
  // position by a wave prefix sum.
  const int64_t rounds = (per + 63) / 64;
  long long wsum = 0;
  for (int64_t rd = 0; rd < rounds; ++rd) {
    const int64_t t = t0 + rd * 64 + lane;
    if (rd * 64 + lane < per && t < tiles) wsum += __popcll(tile_mask[static_cast<int64_t>(k) * tiles + t]);
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) wsum += __shfl_xor(wsum, d);
  if (lane == 0) s_wave[wave] = wsum;
  __syncthreads();
  long long base = s_base;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int32_t* nk = nbr + static_cast<int64_t>(k) * n;
  constexpr int kBatch = 8;  // tiles whose neighbour rows are loaded together
  for (int64_t rd = 0; rd < rounds; ++rd) {
    const int64_t tr = t0 + rd * 64;
    const bool have = rd * 64 + lane < per && tr + lane < tiles;
    const unsigned long long mt = have ? tile_mask[static_cast<int64_t>(k) * tiles + tr + lane] : 0ull;
    const int sb = have && !is_centre ? tile_base[static_cast<int64_t>(k) * tiles + tr + lane] : 0;
    const int ct = __popcll(mt);
    const int incl = wave_prefix_small<7>(ct) + ct;
    if (have) tile_off[static_cast<int64_t>(k) * tiles + tr + lane] = static_cast<int32_t>(base + incl - ct);
    const int nt = static_cast<int>(per - rd * 64 < 64 ? per - rd * 64 : 64);
    for (int b0 = 0; b0 < nt; b0 += kBatch) {
      int32_t src[kBatch];
      if (is_centre) {
#pragma unroll
        for (int i = 0; i < kBatch; ++i) src[i] = static_cast<int32_t>((tr + b0 + i) * kTileRows + lane);
      } else {
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {  // all loads before any store (clamped rows)
          const int64_t q = (tr + b0 + i) * kTileRows + lane;
          src[i] = nk[q < n ? q : n - 1];
        }
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (b0 + i < nt) {
          const unsigned long long m = lane_u64(mt, b0 + i);
          const long long tb = base + __builtin_amdgcn_readlane(incl - ct, b0 + i);
          const int sbi = __builtin_amdgcn_readlane(sb, b0 + i);
          if ((m >> lane) & 1ull) {
            const int rank = __popcll(m & below);
            const int64_t pos = tb + rank;
            in_idx[pos] = src[i];
            out_idx[pos] = static_cast<int32_t>((tr + b0 + i) * kTileRows + lane);
            if (!is_centre && sbi + rank < kTileSlots) {
              tile_rows[(tr + b0 + i) * kTileSlots + sbi + rank] = src[i];
            }
          }
        }
      }
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  if (k == KV - 1 && chunk == chunks - 1 && wave == 3 && lane == 0) {
    tile_off[static_cast<int64_t>(KV) * tiles] = static_cast<int32_t>(base);
  }
  // The coordinate table and occupancy map (slots > 0) are no longer read
  // (the probe, their last reader, has completed): leave them clear for the
  // next build on this scratch, spread over the whole grid.
  const int64_t wg = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * gridDim.y * blockDim.x;
  for (int64_t i = wg * blockDim.x + threadIdx.x; i < slots + buckets; i += stride)
    clear_table_unit(table, slots, occ, buckets, i);
}

// Ordered maps, one workgroup per offset k (1024 threads): list positions.
// The first entry of offset k is the sum of the totals of the offsets before
// it (the summary, final since k_count), and each group of kGroupTiles tiles
// starts after the groups before it: group_base[k][g] = that sum plus an
// exclusive scan of the per-group counts.
__global__ __launch_bounds__(1024) void k_scan(const int64_t* __restrict__ chunk_sum, int64_t groups,
                                               const long long* __restrict__ summary,
                                               int32_t* __restrict__ group_base) {
  const int k = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __shared__ long long s_wave[16];
  __shared__ long long s_base;
  if (wave == 0) {
    long long b = 0;
    for (int i = lane; i < k; i += 64) b += summary[kSummaryHead + i];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) b += __shfl_xor(b, d);
    if (lane == 0) s_base = b;
  }
  __syncthreads();
  long long running = s_base;
  for (int64_t c0 = 0; c0 < groups; c0 += 1024) {
    const int64_t g = c0 + tid;
    const long long v = g < groups ? chunk_sum[static_cast<int64_t>(k) * groups + g] : 0;
    long long incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const long long u = __shfl_up(incl, d);
      if (lane >= d) incl += u;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    long long before = running, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const long long t = s_wave[w];
      if (w < wave) before += t;
      total += t;
    }
    if (g < groups) group_base[static_cast<int64_t>(k) * groups + g] = static_cast<int32_t>(before + incl - v);
    running += total;
    __syncthreads();  // s_wave is rewritten by the next round
  }
}

// Ordered maps.  Grid: x = window of kOrderWindow positions (kWindowGroups
// groups of kGroupTiles tiles), y = offset k; one wave per group.  The
// positions of a window hold a permutation of the window's rows, so the
// probe's neighbour column of those rows at offset k (nbr[k][w0 .. w0 +
// window)) is first copied into LDS with coalesced loads and then read
// through perm.  A group's first list position comes from k_scan (a
// launch of its own: summing the counts of the groups before it here, one
// dependent load round per 64 groups, took 14 us longer at K = 5 on 8 LiDAR
// frames).
// Wave w places the entries of group w of the window: each
// tile's first list position (group_base plus the earlier tiles' counts, a
// wave prefix sum) goes to tile_off[k][t], and each entry, at its rank in the
// tile's mask, gets the row at its position (out_idx) and that row's
// neighbour (in_idx; the row itself at the centre).  A non-centre entry also
// goes to its tile's slot table (tile_rows), at slot tile_base[k][t] + rank,
// when that is below kTileSlots.  The workgroup of the last offset and window
// also writes tile_off[KV * tiles] = E, and the first one hands the summary
// to the host's pinned slot.
// The neighbour column is read once and out_idx is not read by the forward:
// both go non-temporal, so that the map build leaves more of the caches to
// the forward that follows it (8 frames: the in-step forward 249 -> 242 us
// at K = 3, 279 -> 265 us at K = 5).  Maps in the input order are small
// enough to stay cached and keep plain accesses (k_compact).
constexpr int kWindowGroups = kOrderWindow / (kTileRows * kGroupTiles);
static_assert(kWindowGroups * kTileRows * kGroupTiles == kOrderWindow, "whole groups per window");
__global__ __launch_bounds__(64 * kWindowGroups) void k_compact_window(
    const unsigned long long* __restrict__ tile_mask, const int32_t* __restrict__ tile_base,
    const int32_t* __restrict__ nbr, const int32_t* __restrict__ perm, int64_t n, int64_t tiles, int centre,
    int KV, const int32_t* __restrict__ group_base, const long long* __restrict__ summary,
    int32_t* __restrict__ in_idx, int32_t* __restrict__ out_idx,
    int32_t* __restrict__ tile_off, int32_t* __restrict__ tile_rows, long long* __restrict__ host_summary) {
  __shared__ int32_t col[kOrderWindow];
  const int k = blockIdx.y;
  const int64_t win = blockIdx.x;
  const int64_t w0 = win * kOrderWindow;
  const int64_t wn = (n - w0 < kOrderWindow) ? n - w0 : kOrderWindow;
  if (win == 0 && k == 0) {
    for (int i = threadIdx.x; i < kSummaryHead + KV; i += blockDim.x) host_summary[i] = summary[i];
  }
  const bool is_centre = (k == centre);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t groups = (tiles + kGroupTiles - 1) / kGroupTiles;
  const int64_t g = win * kWindowGroups + wave;
  const bool active = g < groups;
  // Issued together: the column of the window's rows, the wave's tile
  // masks and (once the masks are in) the rows at the present positions.
  constexpr int kPerThread = kOrderWindow / (64 * kWindowGroups);
  int32_t cv[kPerThread];
  if (!is_centre) {
    const int32_t* nk = nbr + static_cast<int64_t>(k) * n + w0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int e = i * 64 * kWindowGroups + static_cast<int>(threadIdx.x);
      cv[i] = __builtin_nontemporal_load(&nk[e < wn ? e : wn - 1]);
    }
  }
  const int64_t t0 = g * kGroupTiles;
  const int64_t tl = t0 + lane;
  const bool have = active && lane < kGroupTiles && tl < tiles;
  const unsigned long long mt = have ? tile_mask[static_cast<int64_t>(k) * tiles + tl] : 0ull;
  const int sb = (have && !is_centre) ? tile_base[static_cast<int64_t>(k) * tiles + tl] : 0;
  const int nt = active ? static_cast<int>(tiles - t0 < kGroupTiles ? tiles - t0 : kGroupTiles) : 0;
  int32_t row[kGroupTiles];
#pragma unroll
  for (int i = 0; i < kGroupTiles; ++i) {
    const unsigned long long m = (i < nt) ? lane_u64(mt, i) : 0ull;
    const int64_t q = (t0 + i) * kTileRows + lane;
    row[i] = ((m >> lane) & 1ull) ? perm[q] : static_cast<int32_t>(w0);
  }
  // This group's first list position (k_scan).
  const int base = active ? group_base[static_cast<int64_t>(k) * groups + g] : 0;
  if (!is_centre) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int e = i * 64 * kWindowGroups + static_cast<int>(threadIdx.x);
      if (e < wn) col[e] = cv[i];
    }
  }
  __syncthreads();
  if (!active) return;  // no barrier follows
  const int ct = __popcll(mt);
  const int excl = wave_prefix_small<7>(ct);
  if (have) tile_off[static_cast<int64_t>(k) * tiles + tl] = base + excl;
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int i = 0; i < kGroupTiles; ++i) {
    const unsigned long long m = (i < nt) ? lane_u64(mt, i) : 0ull;
    if ((m >> lane) & 1ull) {
      const int32_t src = is_centre ? row[i] : col[row[i] - w0];
      const int rank = __popcll(m & below);
      const int64_t pos = base + __builtin_amdgcn_readlane(excl, i) + rank;
      in_idx[pos] = src;
      __builtin_nontemporal_store(row[i], &out_idx[pos]);
      const int sbi = __builtin_amdgcn_readlane(sb, i);
      if (!is_centre && sbi + rank < kTileSlots) tile_rows[(t0 + i) * kTileSlots + sbi + rank] = src;
    }
  }
  if (k == KV - 1 && g == groups - 1 && lane == nt - 1) tile_off[static_cast<int64_t>(KV) * tiles] = base + excl + ct;
}

// ---- Strided maps and their transposes ------------------------------------
// One lane per row of the map's output side (query q, coordinates qc[q]); for
// every offset k of the K^3 kernel (components lo .. lo + K - 1) the row of
// the other side that pairs with it, looked up in that side's table:
//   mode 0 (strided map; "Sparse inputs and sparse convolution", section "The
//          map is the computation": look up s q + d): the input at s q + d;
//   mode 1 (its transpose): the strided output q' with s q' + d = p, p the
//          query's coordinates, when (p - d) / s is integral and >= 0.
// nbr[k][q] = that row or -1, and bit k of the query's flag words is set on a
// hit.  All offsets are probed (no mirror symmetry halves them here).  A
// batch of kAllBatch lookups issues its preferred-slot loads together.
constexpr int kAllBatch = 8;
constexpr int kAllFlagWords = 4;  // K <= 5: K^3 <= 125 offsets
template <int K>
__global__ __launch_bounds__(256) void k_probe_all(const int4* __restrict__ qc, int64_t nq,
                                                   const ulonglong2* __restrict__ table,
                                                   unsigned long long window_mask, int lo, int s, int mode,
                                                   int32_t* __restrict__ nbr, uint32_t* __restrict__ flags,
                                                   long long* summary) {
  constexpr int KV = K * K * K;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= nq) return;
  const int4 c = qc[q];
  // Per axis, the coordinate each kernel component probes (-1: none): the
  // offsets combine one component per axis, so the divisions run K times per
  // axis instead of once per offset.
  int tq[3][K];
  {
    const int p[3] = {c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 3; ++i) {
#pragma unroll
      for (int dd = 0; dd < K; ++dd) {
        const int d = dd + lo;
        int t;
        if (mode == 0) {
          t = s * p[i] + d;
          t = (t >= 0 && t < 65536) ? t : -1;
        } else {
          const int v = p[i] - d;
          t = (v >= 0 && v % s == 0) ? v / s : -1;
        }
        tq[i][dd] = t;
      }
    }
  }
  uint32_t fw[kAllFlagWords] = {0u, 0u, 0u, 0u};
  bool overflow = false;
#pragma unroll
  for (int k0 = 0; k0 < KV; k0 += kAllBatch) {
    unsigned long long key[kAllBatch];
    bool ok[kAllBatch];
    ulonglong2 e[kAllBatch];
#pragma unroll
    for (int j = 0; j < kAllBatch; ++j) {
      const int k = k0 + j;
      if (k < KV) {
        const int tz = tq[0][k / (K * K)], ty = tq[1][(k / K) % K], tx = tq[2][k % K];
        ok[j] = tz >= 0 && ty >= 0 && tx >= 0;
        key[j] = ok[j] ? pack_key(c.x, tz, ty, tx) : kEmptyKey;
      } else {
        ok[j] = false;
        key[j] = kEmptyKey;
      }
    }
#pragma unroll
    for (int j = 0; j < kAllBatch; ++j) {
      e[j] = make_ulonglong2(kEmptyKey, 0ull);
      if (ok[j]) e[j] = table[preferred_slot(key[j], window_mask)];
    }
#pragma unroll
    for (int j = 0; j < kAllBatch; ++j) {
      const int k = k0 + j;
      if (k < KV) {
        int64_t row = -1;
        if (ok[j]) {
          if (e[j].x == key[j]) {
            row = static_cast<int64_t>(static_cast<uint32_t>(e[j].y));
          } else if (e[j].x != kEmptyKey && ((e[j].y >> 32) & kSlotDisplaced) != 0ull) {
            row = find_row_scan(key[j], table, window_mask, overflow);
          }
        }
        nbr[static_cast<int64_t>(k) * nq + q] = static_cast<int32_t>(row);
        if (row >= 0) fw[k >> 5] |= 1u << (k & 31);
      }
    }
  }
#pragma unroll
  for (int w = 0; w < kAllFlagWords; ++w) flags[q * kAllFlagWords + w] = fw[w];
  if (overflow) raise_flag(summary, kFlagTableFull);
}

// Tile masks of a map without an identity offset: as k_count (one tile of 64
// output rows per wave, one group of kGroupTiles tiles per workgroup), from
// the probe's flag words; every offset's entries count in the slot bases.
template <int NS>
__global__ __launch_bounds__(1024) void k_count_all(const uint32_t* __restrict__ flags, int KV, int64_t n,
                                                    int64_t tiles, int64_t group_tiles, int64_t chunks,
                                                    unsigned long long* __restrict__ tile_mask,
                                                    int32_t* __restrict__ tile_base,
                                                    int64_t* __restrict__ chunk_sum, long long* summary) {
  const int64_t chunk = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int cnt[NS];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) cnt[sl] = 0;
  for (int64_t g = 0; g < group_tiles; g += kGroupTiles) {
    const int64_t t = chunk * group_tiles + g + wave;
    if (t >= tiles) break;
    const int64_t q = t * kTileRows + lane;
    const bool valid = q < n;
    uint32_t fw[kAllFlagWords];
#pragma unroll
    for (int w = 0; w < kAllFlagWords; ++w) fw[w] = valid ? flags[q * kAllFlagWords + w] : 0u;
    unsigned long long mine[NS];
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      mine[sl] = 0ull;
#pragma unroll
      for (int jj = 0; jj < 64; ++jj) {
        const int k = sl * 64 + jj;
        if (k < KV) {
          const unsigned long long bal = __ballot(((fw[k >> 5] >> (k & 31)) & 1u) != 0u);
          if (lane == jj) mine[sl] = bal;
        }
      }
    }
    int before = 0;
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      const int k = sl * 64 + lane;
      const int cc = k < KV ? static_cast<int>(__popcll(mine[sl])) : 0;
      const int excl = wave_prefix_small<7>(cc);
      if (k < KV) {
        tile_mask[static_cast<int64_t>(k) * tiles + t] = mine[sl];
        tile_base[static_cast<int64_t>(k) * tiles + t] = before + excl;
      }
      before += __builtin_amdgcn_readlane(excl + cc, 63);
      cnt[sl] += cc;
    }
  }
  __shared__ int part[kGroupTiles][NS * 64];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) part[wave][sl * 64 + lane] = cnt[sl];
  __syncthreads();
  for (int k = threadIdx.x; k < KV; k += 1024) {
    int sum = 0;
#pragma unroll
    for (int w = 0; w < kGroupTiles; ++w) sum += part[w][k];
    chunk_sum[static_cast<int64_t>(k) * chunks + chunk] = sum;
    if (sum != 0) {
      atomicAdd(reinterpret_cast<unsigned long long*>(&summary[kSummaryHead + k]),
                static_cast<unsigned long long>(sum));
    }
  }
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Occupancy buckets: a power of two, one per 4 table slots (at least one
// per voxel), so that about a quarter to a half are in use.
int64_t occ_buckets(const BuildPlan& p) { return p.table_slots / 4; }

template <int K>
void launch_probe_count(const BuildPlan& p, const int4* c4, const BuildScratch& s, const MapBuffers& m,
                        unsigned long long window_mask, hipStream_t stream) {
  const unsigned gx = static_cast<unsigned>((p.n + 255) / 256);
  if (K > 1) {
    hipLaunchKernelGGL((k_probe<K>), dim3(gx), dim3(256), 0, stream, c4, p.n, s.table, s.occ, window_mask,
                       static_cast<unsigned long long>(occ_buckets(p) - 1), s.nbr, s.pos_bits, s.neg_flags,
                       s.summary);
  }
  const int64_t groups = (p.tiles + kGroupTiles - 1) / kGroupTiles;
  if constexpr (K > 1) {
    if (p.ordered) {
      const unsigned windows = static_cast<unsigned>((p.n + kOrderWindow - 1) / kOrderWindow);
      hipLaunchKernelGGL((k_order<K>), dim3(windows), dim3(kOrderThreads), 0, stream, s.pos_bits, s.neg_flags, p.n,
                         m.perm, p.tiles, groups, m.tile_mask, s.tile_base, s.chunk_sum, s.summary);
      return;
    }
  }
  hipLaunchKernelGGL((k_count<K>), dim3(static_cast<unsigned>(groups)), dim3(1024), 0, stream,
                     s.pos_bits, s.neg_flags, nullptr, p.n, p.tiles, static_cast<int64_t>(kGroupTiles), groups,
                     m.tile_mask, s.tile_base, s.chunk_sum, s.summary);
}

}  // namespace

BuildPlan make_plan(int64_t n, int32_t K) {
  BuildPlan p;
  p.n = n;
  p.K = K;
  p.KV = K * K * K;
  p.centre = (p.KV - 1) / 2;
  p.tiles = (n + kTileRows - 1) / kTileRows;
  const int64_t groups = (p.tiles + kGroupTiles - 1) / kGroupTiles;
  const int64_t groups_per_chunk = (groups + kMaxChunks - 1) / kMaxChunks;
  p.group_tiles = groups_per_chunk * kGroupTiles;
  p.chunks = (p.tiles + p.group_tiles - 1) / p.group_tiles;
  int64_t slots = 64;
  while (slots < kTableSlotsPerVoxel * n) slots <<= 1;
  p.table_slots = slots;
  p.ordered = K > 1 && n >= kOrderMinRows;
  return p;
}

size_t build_scratch_bytes(const BuildPlan& p) {
  size_t b = 0;
  b += align_up(static_cast<size_t>(p.table_slots) * sizeof(ulonglong2), 256);
  b += align_up(static_cast<size_t>(occ_buckets(p)) * sizeof(uint4), 256);
  b += align_up(static_cast<size_t>(pos_words(p.K)) * p.n * sizeof(uint32_t), 256);
  b += align_up(static_cast<size_t>(neg_bytes(p.K)) * p.n, 256);
  b += align_up(static_cast<size_t>(p.KV) * p.n * sizeof(int32_t), 256);
  b += align_up(static_cast<size_t>(p.KV) * ((p.tiles + kGroupTiles - 1) / kGroupTiles) * sizeof(int64_t), 256);
  b += align_up(static_cast<size_t>(p.KV) * p.tiles * sizeof(int32_t), 256);
  b += align_up(static_cast<size_t>(kSummaryHead + p.KV) * sizeof(long long), 256);
  if (p.ordered) {
    b += align_up(static_cast<size_t>(p.KV) * ((p.tiles + kGroupTiles - 1) / kGroupTiles) * sizeof(int32_t), 256);
  }
  return b;
}

void carve_build_scratch(const BuildPlan& p, void* base, BuildScratch* s) {
  char* c = static_cast<char*>(base);
  s->table = reinterpret_cast<ulonglong2*>(c);
  c += align_up(static_cast<size_t>(p.table_slots) * sizeof(ulonglong2), 256);
  s->occ = reinterpret_cast<uint4*>(c);
  c += align_up(static_cast<size_t>(occ_buckets(p)) * sizeof(uint4), 256);
  s->pos_bits = reinterpret_cast<uint32_t*>(c);
  c += align_up(static_cast<size_t>(pos_words(p.K)) * p.n * sizeof(uint32_t), 256);
  s->neg_flags = reinterpret_cast<uint8_t*>(c);
  c += align_up(static_cast<size_t>(neg_bytes(p.K)) * p.n, 256);
  s->nbr = reinterpret_cast<int32_t*>(c);
  c += align_up(static_cast<size_t>(p.KV) * p.n * sizeof(int32_t), 256);
  s->chunk_sum = reinterpret_cast<int64_t*>(c);
  c += align_up(static_cast<size_t>(p.KV) * ((p.tiles + kGroupTiles - 1) / kGroupTiles) * sizeof(int64_t), 256);
  s->tile_base = reinterpret_cast<int32_t*>(c);
  c += align_up(static_cast<size_t>(p.KV) * p.tiles * sizeof(int32_t), 256);
  s->summary = reinterpret_cast<long long*>(c);
  c += align_up(static_cast<size_t>(kSummaryHead + p.KV) * sizeof(long long), 256);
  s->group_base = p.ordered ? reinterpret_cast<int32_t*>(c) : nullptr;
}

size_t map_buffer_bytes(const BuildPlan& p) {
  const size_t cap = static_cast<size_t>(p.KV) * p.n;
  const size_t tiles = static_cast<size_t>(p.KV) * p.tiles;
  return 2 * align_up(cap * sizeof(int32_t), 256) + align_up((tiles + 1) * sizeof(int32_t), 256) +
         align_up(tiles * sizeof(unsigned long long), 256) +
         align_up(static_cast<size_t>(p.tiles) * kTileSlots * sizeof(int32_t), 256) +
         (p.ordered ? align_up(static_cast<size_t>(p.n) * sizeof(int32_t), 256) : 0);
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
  c += align_up(tiles * sizeof(unsigned long long), 256);
  m->tile_rows = reinterpret_cast<int32_t*>(c);
  c += align_up(static_cast<size_t>(p.tiles) * kTileSlots * sizeof(int32_t), 256);
  m->perm = p.ordered ? reinterpret_cast<int32_t*>(c) : nullptr;
}

hipError_t launch_build(const BuildPlan& p, const int32_t* coords, const BuildScratch& s,
                        const MapBuffers& m, long long* host_summary, bool table_clear, hipStream_t stream) {
  if (!table_clear) {
    const int64_t units = p.table_slots + occ_buckets(p);
    const int64_t init_blocks = (units + 256 * kInitUnits - 1) / (256 * kInitUnits);
    hipLaunchKernelGGL(k_init, dim3(static_cast<unsigned>(init_blocks)), dim3(256), 0, stream,
                       reinterpret_cast<uint4*>(s.table), p.table_slots, s.occ, occ_buckets(p));
  }
  const unsigned long long window_mask =
      static_cast<unsigned long long>(p.table_slots / kWindowSlots) - 1ull;
  const int4* c4 = reinterpret_cast<const int4*>(coords);
  const unsigned gx = static_cast<unsigned>((p.n + 255) / 256);
  hipLaunchKernelGGL(k_claim, dim3(gx), dim3(256), 0, stream, c4, p.n, s.table,
                     reinterpret_cast<uint8_t*>(s.occ), window_mask,
                     static_cast<unsigned long long>(occ_buckets(p) - 1), reinterpret_cast<uint4*>(s.neg_flags),
                     neg_bytes(p.K) / 16, s.summary, kSummaryHead + p.KV);
  hipLaunchKernelGGL(k_insert, dim3(gx), dim3(256), 0, stream, c4, p.n, s.table, window_mask, s.summary);
  switch (p.K) {
    case 1: launch_probe_count<1>(p, c4, s, m, window_mask, stream); break;
    case 3: launch_probe_count<3>(p, c4, s, m, window_mask, stream); break;
    case 5: launch_probe_count<5>(p, c4, s, m, window_mask, stream); break;
    case 7: launch_probe_count<7>(p, c4, s, m, window_mask, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (p.ordered) {
    const int64_t groups = (p.tiles + kGroupTiles - 1) / kGroupTiles;
    hipLaunchKernelGGL(k_scan, dim3(static_cast<unsigned>(p.KV)), dim3(1024), 0, stream, s.chunk_sum, groups,
                       s.summary, s.group_base);
    const unsigned windows = static_cast<unsigned>((p.n + kOrderWindow - 1) / kOrderWindow);
    hipLaunchKernelGGL(k_compact_window, dim3(windows, static_cast<unsigned>(p.KV)), dim3(64 * kWindowGroups), 0,
                       stream, m.tile_mask, s.tile_base, s.nbr, m.perm, p.n, p.tiles, p.centre, p.KV, s.group_base,
                       s.summary, m.in_idx, m.out_idx, m.tile_off, m.tile_rows, host_summary);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_compact, dim3(static_cast<unsigned>(p.chunks), static_cast<unsigned>(p.KV)),
                     dim3(256), 0, stream, m.tile_mask, s.tile_base, s.nbr, p.n, p.tiles, p.centre, p.KV,
                     p.group_tiles, p.chunks, s.chunk_sum, s.summary, m.in_idx, m.out_idx,
                     m.tile_off, m.tile_rows, host_summary, reinterpret_cast<uint4*>(s.table), p.table_slots,
                     s.occ, occ_buckets(p));
  return hipGetLastError();
}

hipError_t launch_table_build(const int32_t* coords, int64_t n, ulonglong2* table, int64_t table_slots, uint4* occ,
                              long long* summary, int summary_len, hipStream_t stream) {
  const int64_t buckets = table_slots / 4;
  const int64_t units = table_slots + buckets;
  const int64_t init_blocks = (units + 256 * kInitUnits - 1) / (256 * kInitUnits);
  hipLaunchKernelGGL(k_init, dim3(static_cast<unsigned>(init_blocks)), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(table), table_slots, occ, buckets);
  const unsigned long long window_mask = static_cast<unsigned long long>(table_slots / kWindowSlots) - 1ull;
  const int4* c4 = reinterpret_cast<const int4*>(coords);
  const unsigned gx = static_cast<unsigned>((n + 255) / 256);
  hipLaunchKernelGGL(k_claim, dim3(gx), dim3(256), 0, stream, c4, n, table, reinterpret_cast<uint8_t*>(occ),
                     window_mask, static_cast<unsigned long long>(buckets - 1), static_cast<uint4*>(nullptr), 0, summary,
                     summary_len);
  hipLaunchKernelGGL(k_insert, dim3(gx), dim3(256), 0, stream, c4, n, table, window_mask, summary);
  return hipGetLastError();
}

int64_t table_slots_for(int64_t n) {
  int64_t slots = 64;
  while (slots < kTableSlotsPerVoxel * n) slots <<= 1;
  return slots;
}

hipError_t launch_general_map(const GeneralMapArgs& g, hipStream_t stream) {
  if (g.nq <= 0) return hipSuccess;
  const unsigned long long window_mask = static_cast<unsigned long long>(g.table_slots / kWindowSlots) - 1ull;
  {
    const dim3 grid(static_cast<unsigned>((g.nq + 255) / 256));
    const int4* qc = reinterpret_cast<const int4*>(g.qcoords);
    switch (g.K) {
      case 1:
        hipLaunchKernelGGL(k_probe_all<1>, grid, dim3(256), 0, stream, qc, g.nq, g.table, window_mask, g.lo, g.stride,
                           g.mode, g.nbr, g.flags, g.summary);
        break;
      case 2:
        hipLaunchKernelGGL(k_probe_all<2>, grid, dim3(256), 0, stream, qc, g.nq, g.table, window_mask, g.lo, g.stride,
                           g.mode, g.nbr, g.flags, g.summary);
        break;
      case 3:
        hipLaunchKernelGGL(k_probe_all<3>, grid, dim3(256), 0, stream, qc, g.nq, g.table, window_mask, g.lo, g.stride,
                           g.mode, g.nbr, g.flags, g.summary);
        break;
      case 4:
        hipLaunchKernelGGL(k_probe_all<4>, grid, dim3(256), 0, stream, qc, g.nq, g.table, window_mask, g.lo, g.stride,
                           g.mode, g.nbr, g.flags, g.summary);
        break;
      case 5:
        hipLaunchKernelGGL(k_probe_all<5>, grid, dim3(256), 0, stream, qc, g.nq, g.table, window_mask, g.lo, g.stride,
                           g.mode, g.nbr, g.flags, g.summary);
        break;
      default:
        return hipErrorInvalidValue;
    }
  }
  const int64_t tiles = (g.nq + kTileRows - 1) / kTileRows;
  const int64_t groups = (tiles + kGroupTiles - 1) / kGroupTiles;
  const int KV = g.K * g.K * g.K;
  if (KV <= 64) {
    hipLaunchKernelGGL(k_count_all<1>, dim3(static_cast<unsigned>(groups)), dim3(1024), 0, stream, g.flags, KV,
                       g.nq, tiles, static_cast<int64_t>(kGroupTiles), groups, g.map.tile_mask, g.tile_base,
                       g.chunk_sum, g.summary);
  } else {
    hipLaunchKernelGGL(k_count_all<2>, dim3(static_cast<unsigned>(groups)), dim3(1024), 0, stream, g.flags, KV,
                       g.nq, tiles, static_cast<int64_t>(kGroupTiles), groups, g.map.tile_mask, g.tile_base,
                       g.chunk_sum, g.summary);
  }
  // k_compact with chunks of whole groups, at most kMaxChunks of them
  const int64_t groups_per_chunk = (groups + kMaxChunks - 1) / kMaxChunks;
  const int64_t group_tiles = groups_per_chunk * kGroupTiles;
  const int64_t chunks = (tiles + group_tiles - 1) / group_tiles;
  hipLaunchKernelGGL(k_compact, dim3(static_cast<unsigned>(chunks), static_cast<unsigned>(KV)), dim3(256), 0, stream,
                     g.map.tile_mask, g.tile_base, g.nbr, g.nq, tiles, -1, KV, group_tiles, chunks, g.chunk_sum,
                     g.summary, g.map.in_idx, g.map.out_idx, g.map.tile_off, g.map.tile_rows, g.host_summary,
                     static_cast<uint4*>(nullptr), int64_t(0), static_cast<uint4*>(nullptr), int64_t(0));
  return hipGetLastError();
}

size_t general_scratch_bytes(int64_t nq, int K) {
  const int64_t KV = static_cast<int64_t>(K) * K * K;
  const int64_t tiles = (nq + kTileRows - 1) / kTileRows;
  const int64_t groups = (tiles + kGroupTiles - 1) / kGroupTiles;
  return align_up(static_cast<size_t>(nq) * kAllFlagWords * sizeof(uint32_t), 256) +
         align_up(static_cast<size_t>(KV) * nq * sizeof(int32_t), 256) +
         align_up(static_cast<size_t>(KV) * groups * sizeof(int64_t), 256) +
         align_up(static_cast<size_t>(KV) * tiles * sizeof(int32_t), 256);
}

void carve_general_scratch(int64_t nq, int K, void* base, GeneralMapArgs* g) {
  const int64_t KV = static_cast<int64_t>(K) * K * K;
  const int64_t tiles = (nq + kTileRows - 1) / kTileRows;
  const int64_t groups = (tiles + kGroupTiles - 1) / kGroupTiles;
  char* c = static_cast<char*>(base);
  g->flags = reinterpret_cast<uint32_t*>(c);
  c += align_up(static_cast<size_t>(nq) * kAllFlagWords * sizeof(uint32_t), 256);
  g->nbr = reinterpret_cast<int32_t*>(c);
  c += align_up(static_cast<size_t>(KV) * nq * sizeof(int32_t), 256);
  g->chunk_sum = reinterpret_cast<int64_t*>(c);
  c += align_up(static_cast<size_t>(KV) * groups * sizeof(int64_t), 256);
  g->tile_base = reinterpret_cast<int32_t*>(c);
}

}  // namespace spconv
