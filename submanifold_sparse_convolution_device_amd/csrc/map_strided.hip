// Output coordinates of a strided sparse convolution on gfx950.
//
// A strided map ("Sparse inputs and sparse convolution", section "The map is
// the computation": for each output q and offset d, look up s q + d) has the
// outputs of the regular output definition (SparseConvNet blog, section 2:
// an output is computed where the kernel covers at least one active input):
// the grid points q >= 0 with an input at s q + d for some offset d of the
// K^3 kernel (components lo .. lo + K - 1, lo = -floor((K - 1) / 2)).  They
// are produced in lexicographic (b, z, y, x) order, the order a unique-based
// voxelizer emits:
//   key format        (k_bounds_partial, k_key_format) the range of each
//                     output field, from the inputs' ranges: a key packs
//                     (b, z, y, x) minus their lower bounds in just the bits
//                     the ranges need, b highest, so that its order is still
//                     the lexicographic order; an unused slot holds the
//                     smallest value above every key (1 << width);
//   k_out_candidates  one lane per input p: per axis the kernel components d
//                     with p - d divisible by s and (p - d) / s in
//                     [0, 2^16); every combination's key;
//   radix sort        stable LSD over the bytes the keys use (passes past
//                     them exit at once; the format decides on the device,
//                     so the host waits for nothing): per pass a
//                     digit histogram per block of 4096 keys (k_rs_count), an
//                     exclusive scan over (digit, block) (per tile of 4096
//                     counts, then the tiles' totals, then each tile's prefix
//                     added) and a stable scatter (k_rs_scatter: ranks within a block by
//                     ballots, in element order);
//   unique            a key that differs from its predecessor (and is not ~0)
//                     starts a run: per-block counts, their exclusive scan
//                     (the total is the number of outputs) and the unpacked
//                     coordinates at their ranks.
#include "internal.h"

#include <algorithm>
#include <climits>

namespace spconv {
namespace {

constexpr int kSortThreads = 1024;
constexpr int kSortPer = 4;
constexpr int kSortBlock = kSortThreads * kSortPer;
constexpr int kSortWaves = kSortThreads / 64;
constexpr unsigned long long kNoKey = ~0ull;

// How the output keys of one build are packed (written by k_key_format).
struct KeyFormat {
  int32_t lo[4];     // lower bound of b, z, y, x
  int32_t shift[4];  // bit position of b, z, y, x in the key
  int32_t npass;     // 8-bit radix passes the keys need (the invalid marker included)
  int32_t unused;
  unsigned long long invalid;  // 1 << (total width): above every key
};

__device__ __forceinline__ unsigned long long pack_out(const KeyFormat& f, int b, int z, int y, int x) {
  return (static_cast<unsigned long long>(static_cast<uint32_t>(b - f.lo[0])) << f.shift[0]) |
         (static_cast<unsigned long long>(static_cast<uint32_t>(z - f.lo[1])) << f.shift[1]) |
         (static_cast<unsigned long long>(static_cast<uint32_t>(y - f.lo[2])) << f.shift[2]) |
         (static_cast<unsigned long long>(static_cast<uint32_t>(x - f.lo[3])) << f.shift[3]);
}

__device__ __forceinline__ int4 unpack_out(const KeyFormat& f, unsigned long long k) {
  auto field = [&](int i, int next) {
    const unsigned long long bits = k >> f.shift[i];
    const int w = next - f.shift[i];
    return static_cast<int>(bits & ((w >= 64) ? ~0ull : ((1ull << w) - 1ull))) + f.lo[i];
  };
  // field widths: x up to y's shift, y up to z's, z up to b's, b up to the total
  const int total = 63 - __clzll(static_cast<long long>(f.invalid));
  return make_int4(field(0, total), field(1, f.shift[0]), field(2, f.shift[1]), field(3, f.shift[2]));
}

__device__ __forceinline__ bool in_range(int4 c) {
  return c.x >= 0 && c.x < 32768 && c.y >= 0 && c.y < 65536 && c.z >= 0 && c.z < 65536 && c.w >= 0 && c.w < 65536;
}

// Per workgroup of 256 inputs (a grid-stride share of them): the minimum and
// maximum of b, z, y, x over the inputs in range, to part[8 blk .. 8 blk + 8)
// (minima, then maxima; an empty share gives min > max).
constexpr int kBoundsBlocks = 512;
__global__ __launch_bounds__(256) void k_bounds_partial(const int4* __restrict__ coords, int64_t n,
                                                        int32_t* __restrict__ part) {
  __shared__ int32_t red[8][4];
  int mn[4] = {INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX}, mx[4] = {INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN};
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
    const int4 c = coords[i];
    if (!in_range(c)) continue;
    const int v[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      mn[f] = min(mn[f], v[f]);
      mx[f] = max(mx[f], v[f]);
    }
  }
#pragma unroll
  for (int f = 0; f < 4; ++f) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      mn[f] = min(mn[f], __shfl_xor(mn[f], o));
      mx[f] = max(mx[f], __shfl_xor(mx[f], o));
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      red[f][wave] = mn[f];
      red[4 + f][wave] = mx[f];
    }
  }
  __syncthreads();
  if (threadIdx.x < 8) {
    const int f = threadIdx.x;
    int r = red[f][0];
    for (int w = 1; w < 4; ++w) r = (f < 4) ? min(r, red[f][w]) : max(r, red[f][w]);
    part[static_cast<int64_t>(blockIdx.x) * 8 + f] = r;
  }
}

__device__ __forceinline__ int floor_div(int a, int s) { return (a >= 0) ? a / s : -((-a + s - 1) / s); }
__device__ __forceinline__ int bit_width(uint32_t v) { return v == 0u ? 0 : 32 - __clz(static_cast<int>(v)); }

// One wave: the inputs' bounds from the partials, then the outputs' bounds
// (an output q of an input p has q = (p - d) / s for a component d in
// lo .. lo + K - 1, and 0 <= q < 2^16) and the key format.
__global__ __launch_bounds__(64) void k_key_format(const int32_t* __restrict__ part, int nparts, int K, int lo,
                                                   int s, KeyFormat* __restrict__ fmt) {
  const int lane = threadIdx.x;
  int mn[4] = {INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX}, mx[4] = {INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN};
  for (int i = lane; i < nparts; i += 64) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      mn[f] = min(mn[f], part[8 * i + f]);
      mx[f] = max(mx[f], part[8 * i + 4 + f]);
    }
  }
#pragma unroll
  for (int f = 0; f < 4; ++f) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      mn[f] = min(mn[f], __shfl_xor(mn[f], o));
      mx[f] = max(mx[f], __shfl_xor(mx[f], o));
    }
  }
  if (lane != 0) return;
  KeyFormat k;
  int width[4] = {0, 0, 0, 0};
  if (mn[0] > mx[0]) {  // no input in range: no candidate key is used
#pragma unroll
    for (int f = 0; f < 4; ++f) k.lo[f] = 0;
  } else {
    k.lo[0] = mn[0];
    width[0] = bit_width(static_cast<uint32_t>(mx[0] - mn[0]));
#pragma unroll
    for (int f = 1; f < 4; ++f) {
      const int qlo = max(0, floor_div(mn[f] - (lo + K - 1), s));
      const int qhi = min(65535, max(qlo, floor_div(mx[f] - lo, s)));
      k.lo[f] = qlo;
      width[f] = bit_width(static_cast<uint32_t>(qhi - qlo));
    }
  }
  k.shift[3] = 0;
  k.shift[2] = width[3];
  k.shift[1] = width[3] + width[2];
  k.shift[0] = width[3] + width[2] + width[1];
  const int total = k.shift[0] + width[0];  // at most 15 + 3 x 16 = 63
  k.invalid = 1ull << total;
  k.npass = (total + 1 + 7) / 8;
  k.unused = 0;
  *fmt = k;
}

constexpr int kMaxAxisChoices = 8;

// The grid coordinates q = (p - d) / s of one axis, for the kernel components
// d in lo .. lo + K - 1 that divide evenly and land in [0, 2^16).
__device__ __forceinline__ int axis_choices(int p, int K, int lo, int s, int (&q)[kMaxAxisChoices]) {
  int n = 0;
  for (int d = lo; d < lo + K; ++d) {
    const int v = p - d;
    if (v >= 0 && v % s == 0 && v / s < 65536 && n < kMaxAxisChoices) q[n++] = v / s;
  }
  return n;
}

// One lane per input row; `ca` choices per axis at most, ca^3 key slots per
// input.
__global__ __launch_bounds__(256) void k_out_candidates(const int4* __restrict__ coords, int64_t n, int K, int lo,
                                                        int s, int ca, const KeyFormat* __restrict__ fmtp,
                                                        unsigned long long* __restrict__ keys) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const KeyFormat fmt = *fmtp;
  const int4 c = coords[i];
  const int64_t base = i * static_cast<int64_t>(ca) * ca * ca;
  const bool ok_in = in_range(c);  // out-of-range inputs are reported by the table build
  int qz[kMaxAxisChoices], qy[kMaxAxisChoices], qx[kMaxAxisChoices];
  const int nz = ok_in ? axis_choices(c.y, K, lo, s, qz) : 0;
  const int ny = ok_in ? axis_choices(c.z, K, lo, s, qy) : 0;
  const int nx = ok_in ? axis_choices(c.w, K, lo, s, qx) : 0;
  for (int a = 0; a < ca; ++a)
    for (int b = 0; b < ca; ++b)
      for (int e = 0; e < ca; ++e) {
        const bool ok = a < nz && b < ny && e < nx;
        keys[base + (a * ca + b) * ca + e] = ok ? pack_out(fmt, c.x, qz[a], qy[b], qx[e]) : fmt.invalid;
      }
}

// Element e of a block sits in round (e / 64) mod kSortPer of wave
// e / (kSortPer x 64), lane e mod 64, so a wave's rounds walk its elements in
// order and ranks by (wave, round, lane) are ranks in element order.
__device__ __forceinline__ int64_t sort_index(int64_t block, int wave, int j, int lane) {
  return block * kSortBlock + (static_cast<int64_t>(wave) * kSortPer + j) * 64 + lane;
}

// Digit histogram of one block: hist[d * blocks + block].
__global__ __launch_bounds__(kSortThreads) void k_rs_count(const unsigned long long* __restrict__ keys, int64_t m,
                                                           int shift, int64_t blocks, uint32_t* __restrict__ hist,
                                                           const KeyFormat* __restrict__ fmt) {
  if (shift >= 8 * fmt->npass) return;  // a pass past the keys' bytes (uniform)
  __shared__ uint32_t h[256];
  for (int i = threadIdx.x; i < 256; i += kSortThreads) h[i] = 0u;
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < kSortPer; ++j) {
    const int64_t g = sort_index(blockIdx.x, wave, j, lane);
    if (g < m) atomicAdd(&h[(keys[g] >> shift) & 255u], 1u);
  }
  __syncthreads();
  for (int d = threadIdx.x; d < 256; d += kSortThreads) hist[static_cast<int64_t>(d) * blocks + blockIdx.x] = h[d];
}

// In-place exclusive scan of `count` values by one workgroup: each thread
// sums a contiguous run, the runs' sums are scanned across the workgroup,
// and each thread rewrites its run.  The total goes to *total when non-null.
__global__ __launch_bounds__(1024) void k_scan_excl(uint32_t* __restrict__ v, int64_t count,
                                                    long long* __restrict__ total, const KeyFormat* __restrict__ fmt,
                                                    int shift) {
  if (fmt != nullptr && shift >= 8 * fmt->npass) return;  // a skipped sort pass (uniform)
  __shared__ unsigned long long wsum[16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t per = (count + 1023) / 1024;
  const int64_t lo = tid * per;
  const int64_t hi = (lo + per < count) ? lo + per : count;
  unsigned long long sum = 0;
  for (int64_t i = lo; i < hi; ++i) sum += v[i];
  unsigned long long incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  unsigned long long base = incl - sum;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  for (int64_t i = lo; i < hi; ++i) {
    const uint32_t x = v[i];
    v[i] = static_cast<uint32_t>(base);
    base += x;
  }
  if (tid == 1023 && total != nullptr) {
    unsigned long long all = 0;
    for (int w = 0; w < 16; ++w) all += wsum[w];
    *total = static_cast<long long>(all);
  }
}

// Multi-workgroup exclusive scan, pass 1: workgroup t scans its tile of
// kScanTile values in place (thread i holds values 4 i .. 4 i + 3 of the tile)
// and writes the tile's total to part[t].  Pass 2 scans part (k_scan_excl,
// one workgroup, few values); pass 3 (k_scan_add) adds each tile's prefix.
constexpr int kScanTile = 4096;
__global__ __launch_bounds__(1024) void k_scan_tile(uint32_t* __restrict__ v, int64_t count,
                                                    uint32_t* __restrict__ part, const KeyFormat* __restrict__ fmt,
                                                    int shift) {
  if (fmt != nullptr && shift >= 8 * fmt->npass) return;
  __shared__ uint32_t wsum[16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanTile + 4 * tid;
  uint32_t x[4];
  uint32_t sum = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = (base + j < count) ? v[base + j] : 0u;
    sum += x[j];
  }
  uint32_t incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t run = incl - sum;
  for (int w = 0; w < wave; ++w) run += wsum[w];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (base + j < count) v[base + j] = run;
    run += x[j];
  }
  if (tid == 1023) part[blockIdx.x] = run;  // the last thread's running value is the tile's total
}

__global__ __launch_bounds__(256) void k_scan_add(uint32_t* __restrict__ v, int64_t count,
                                                  const uint32_t* __restrict__ part, const KeyFormat* __restrict__ fmt,
                                                  int shift) {
  if (fmt != nullptr && shift >= 8 * fmt->npass) return;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count) v[i] += part[i / kScanTile];
}

// Stable scatter of one block for the byte at `shift`: key at element e goes
// to offs[d * blocks + block] (the scanned histogram) + its rank among the
// block's keys of digit d that precede it.
__global__ __launch_bounds__(kSortThreads) void k_rs_scatter(const unsigned long long* __restrict__ in,
                                                             unsigned long long* __restrict__ out, int64_t m,
                                                             int shift, int64_t blocks,
                                                             const uint32_t* __restrict__ offs,
                                                             const KeyFormat* __restrict__ fmt) {
  if (shift >= 8 * fmt->npass) return;  // a pass past the keys' bytes (uniform)
  __shared__ uint32_t hist[kSortWaves * 256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  uint32_t* row = hist + wave * 256;
  for (int d = lane; d < 256; d += 64) row[d] = 0u;
  unsigned long long key[kSortPer];
  uint32_t dig[kSortPer], rank[kSortPer];
  bool valid[kSortPer];
#pragma unroll
  for (int j = 0; j < kSortPer; ++j) {
    const int64_t g = sort_index(blockIdx.x, wave, j, lane);
    valid[j] = g < m;
    key[j] = valid[j] ? in[g] : kNoKey;
    const uint32_t d = static_cast<uint32_t>((key[j] >> shift) & 255u);
    dig[j] = d;
    unsigned long long peers = __ballot(valid[j]);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const unsigned long long bb = __ballot((d >> b) & 1u);
      peers &= ((d >> b) & 1u) ? bb : ~bb;
    }
    rank[j] = static_cast<uint32_t>(__popcll(peers & below));
    const uint32_t cnt = static_cast<uint32_t>(__popcll(peers));
    // lanes of one digit read the count so far and write the same new count
    // (a wave's LDS operations run in order, so round j sees the rounds before)
    const uint32_t before = row[d];
    rank[j] += before;
    if (valid[j]) row[d] = before + cnt;
  }
  __syncthreads();
  // per digit: each wave's start within the block
  if (threadIdx.x < 256) {
    const int d = threadIdx.x;
    uint32_t run = 0u;
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) {
      const uint32_t c = hist[w * 256 + d];
      hist[w * 256 + d] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kSortPer; ++j) {
    if (valid[j]) {
      const uint32_t d = dig[j];
      const int64_t pos = static_cast<int64_t>(offs[static_cast<int64_t>(d) * blocks + blockIdx.x]) + hist[wave * 256 + d] + rank[j];
      out[pos] = key[j];
    }
  }
}

__device__ __forceinline__ bool run_start(const unsigned long long* __restrict__ keys, int64_t g, int64_t m,
                                          unsigned long long invalid) {
  if (g >= m) return false;
  const unsigned long long k = keys[g];
  return k != invalid && (g == 0 || keys[g - 1] != k);
}

// The sorted keys: an odd number of passes leaves them in the second buffer.
__device__ __forceinline__ const unsigned long long* sorted_keys(const unsigned long long* a,
                                                                 const unsigned long long* b, const KeyFormat& f) {
  return (f.npass & 1) ? b : a;
}

// Runs starting in each block.
__global__ __launch_bounds__(kSortThreads) void k_uniq_count(const unsigned long long* __restrict__ ka,
                                                             const unsigned long long* __restrict__ kb, int64_t m,
                                                             const KeyFormat* __restrict__ fmtp,
                                                             uint32_t* __restrict__ cnt) {
  const KeyFormat fmt = *fmtp;
  const unsigned long long* keys = sorted_keys(ka, kb, fmt);
  __shared__ uint32_t total;
  if (threadIdx.x == 0) total = 0u;
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t c = 0u;
#pragma unroll
  for (int j = 0; j < kSortPer; ++j) c += run_start(keys, sort_index(blockIdx.x, wave, j, lane), m, fmt.invalid) ? 1u : 0u;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if (lane == 0) atomicAdd(&total, c);
  __syncthreads();
  if (threadIdx.x == 0) cnt[blockIdx.x] = total;
}

// The coordinates of each run's key at offs[block] + its rank in the block.
__global__ __launch_bounds__(kSortThreads) void k_uniq_write(const unsigned long long* __restrict__ ka,
                                                             const unsigned long long* __restrict__ kb, int64_t m,
                                                             const KeyFormat* __restrict__ fmtp,
                                                             const uint32_t* __restrict__ offs,
                                                             int4* __restrict__ out) {
  const KeyFormat fmt = *fmtp;
  const unsigned long long* keys = sorted_keys(ka, kb, fmt);
  __shared__ uint32_t wtot[kSortWaves];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  bool st[kSortPer];
  uint32_t rank[kSortPer];
  uint32_t run = 0u;
#pragma unroll
  for (int j = 0; j < kSortPer; ++j) {
    st[j] = run_start(keys, sort_index(blockIdx.x, wave, j, lane), m, fmt.invalid);
    const unsigned long long b = __ballot(st[j]);
    rank[j] = run + static_cast<uint32_t>(__popcll(b & below));
    run += static_cast<uint32_t>(__popcll(b));
  }
  if (lane == 0) wtot[wave] = run;
  __syncthreads();
  uint32_t base = offs[blockIdx.x];
  for (int w = 0; w < wave; ++w) base += wtot[w];
#pragma unroll
  for (int j = 0; j < kSortPer; ++j) {
    if (st[j]) {
      out[base + rank[j]] = unpack_out(fmt, keys[sort_index(blockIdx.x, wave, j, lane)]);
    }
  }
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

struct OutScratch {
  unsigned long long* a;
  unsigned long long* b;
  uint32_t* hist;
  uint32_t* cnt;
  uint32_t* part;       // tile totals of the multi-workgroup scan
  int32_t* bounds;      // kBoundsBlocks x 8 partial bounds
  KeyFormat* fmt;
};

int64_t scan_tiles(int64_t count) { return (count + kScanTile - 1) / kScanTile; }

// Exclusive scan of v[0 .. count) in place; the total to *total when non-null.
// With fmt, the scan of the sort pass at `shift` (skipped past the keys' bytes).
void launch_scan(uint32_t* v, int64_t count, uint32_t* part, long long* total, const KeyFormat* fmt, int shift,
                 hipStream_t stream) {
  const int64_t tiles = scan_tiles(count);
  hipLaunchKernelGGL(k_scan_tile, dim3(static_cast<unsigned>(tiles)), dim3(1024), 0, stream, v, count, part, fmt,
                     shift);
  hipLaunchKernelGGL(k_scan_excl, dim3(1), dim3(1024), 0, stream, part, tiles, total, fmt, shift);
  hipLaunchKernelGGL(k_scan_add, dim3(static_cast<unsigned>((count + 255) / 256)), dim3(256), 0, stream, v, count,
                     static_cast<const uint32_t*>(part), fmt, shift);
}

OutScratch carve_out_scratch(const OutCoordPlan& p, void* base) {
  OutScratch s;
  char* c = static_cast<char*>(base);
  s.a = reinterpret_cast<unsigned long long*>(c);
  c += align256(static_cast<size_t>(p.m) * sizeof(unsigned long long));
  s.b = reinterpret_cast<unsigned long long*>(c);
  c += align256(static_cast<size_t>(p.m) * sizeof(unsigned long long));
  s.hist = reinterpret_cast<uint32_t*>(c);
  c += align256(static_cast<size_t>(256) * p.blocks * sizeof(uint32_t));
  s.cnt = reinterpret_cast<uint32_t*>(c);
  c += align256(static_cast<size_t>(p.blocks) * sizeof(uint32_t));
  s.part = reinterpret_cast<uint32_t*>(c);
  c += align256(static_cast<size_t>(scan_tiles(256 * p.blocks)) * sizeof(uint32_t));
  s.bounds = reinterpret_cast<int32_t*>(c);
  c += align256(static_cast<size_t>(kBoundsBlocks) * 8 * sizeof(int32_t));
  s.fmt = reinterpret_cast<KeyFormat*>(c);
  return s;
}

}  // namespace

OutCoordPlan out_coord_plan(int64_t n_in, int K, int stride) {
  OutCoordPlan p;
  p.n_in = n_in;
  p.K = K;
  p.lo = -((K - 1) / 2);
  p.stride = stride;
  p.ca = (K + stride - 1) / stride;
  p.m = n_in * p.ca * p.ca * p.ca;
  p.blocks = (p.m + kSortBlock - 1) / kSortBlock;
  return p;
}

size_t out_coord_scratch_bytes(const OutCoordPlan& p) {
  return 2 * align256(static_cast<size_t>(p.m) * sizeof(unsigned long long)) +
         align256(static_cast<size_t>(256) * p.blocks * sizeof(uint32_t)) +
         align256(static_cast<size_t>(p.blocks) * sizeof(uint32_t)) +
         align256(static_cast<size_t>(scan_tiles(256 * p.blocks)) * sizeof(uint32_t)) +
         align256(static_cast<size_t>(kBoundsBlocks) * 8 * sizeof(int32_t)) + align256(sizeof(KeyFormat));
}

hipError_t launch_out_coords_count(const OutCoordPlan& p, const int32_t* coords, void* scratch, long long* n_out,
                                   hipStream_t stream) {
  const OutScratch s = carve_out_scratch(p, scratch);
  const int4* c4 = reinterpret_cast<const int4*>(coords);
  const int nb = static_cast<int>(std::min<int64_t>(kBoundsBlocks, (p.n_in + 255) / 256));
  hipLaunchKernelGGL(k_bounds_partial, dim3(static_cast<unsigned>(nb)), dim3(256), 0, stream, c4, p.n_in, s.bounds);
  hipLaunchKernelGGL(k_key_format, dim3(1), dim3(64), 0, stream, static_cast<const int32_t*>(s.bounds), nb, p.K,
                     p.lo, p.stride, s.fmt);
  hipLaunchKernelGGL(k_out_candidates, dim3(static_cast<unsigned>((p.n_in + 255) / 256)), dim3(256), 0, stream, c4,
                     p.n_in, p.K, p.lo, p.stride, p.ca, static_cast<const KeyFormat*>(s.fmt), s.a);
  unsigned long long* src = s.a;
  unsigned long long* dst = s.b;
  const unsigned grid = static_cast<unsigned>(p.blocks);
  for (int pass = 0; pass < 8; ++pass) {
    // passes past the keys' bytes return at once (their launches cost a few
    // microseconds; the key format is on the device)
    const int shift = 8 * pass;
    hipLaunchKernelGGL(k_rs_count, dim3(grid), dim3(kSortThreads), 0, stream, src, p.m, shift, p.blocks, s.hist,
                       static_cast<const KeyFormat*>(s.fmt));
    launch_scan(s.hist, static_cast<int64_t>(256) * p.blocks, s.part, nullptr, s.fmt, shift, stream);
    hipLaunchKernelGGL(k_rs_scatter, dim3(grid), dim3(kSortThreads), 0, stream, src, dst, p.m, shift, p.blocks,
                       s.hist, static_cast<const KeyFormat*>(s.fmt));
    unsigned long long* t = src;
    src = dst;
    dst = t;
  }
  // the sorted keys are in s.a after an even number of executed passes, in s.b after an odd one
  hipLaunchKernelGGL(k_uniq_count, dim3(grid), dim3(kSortThreads), 0, stream, static_cast<const unsigned long long*>(s.a),
                     static_cast<const unsigned long long*>(s.b), p.m, static_cast<const KeyFormat*>(s.fmt), s.cnt);
  launch_scan(s.cnt, p.blocks, s.part, n_out, nullptr, 0, stream);
  return hipGetLastError();
}

hipError_t launch_out_coords_write(const OutCoordPlan& p, void* scratch, int32_t* out_coords, hipStream_t stream) {
  const OutScratch s = carve_out_scratch(p, scratch);
  hipLaunchKernelGGL(k_uniq_write, dim3(static_cast<unsigned>(p.blocks)), dim3(kSortThreads), 0, stream,
                     static_cast<const unsigned long long*>(s.a), static_cast<const unsigned long long*>(s.b), p.m,
                     static_cast<const KeyFormat*>(s.fmt), static_cast<const uint32_t*>(s.cnt),
                     reinterpret_cast<int4*>(out_coords));
  return hipGetLastError();
}

}  // namespace spconv
