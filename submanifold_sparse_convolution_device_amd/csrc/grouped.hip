// Weight-stationary forward with adaptive grouping on gfx950: the comparison
// dataflow of "TorchSparse: regular computation from irregular sparsity",
// sections "The spectrum: separate, dense, grouped" and "How the groups are
// chosen".
//
// Instead of one fused output-stationary kernel, the forward runs in phases
// over groups of offsets:
//   gather   (k_gs_gather, one launch) the input rows of every offset into a
//            padded batch: entry e (one offset) holds its list's rows, then
//            zero rows up to the largest map of its group (its `pad`);
//   GEMM     (k_gs_gemm, one launch per group: the batched matrix product)
//            Y = A_e x W_k for every entry of the group on MFMA, in fp32,
//            the padded rows included (the grouping's redundant work; their
//            products are not stored).  A workgroup stages a column slice of
//            W_k in LDS once and streams 256 batch rows through it;
//   reduce   (k_gs_reduce, one launch) every output row sums the Y rows of
//            its entries in offset order and is written once, rounded to the
//            dtype: the pages' scatter, deterministic here (no atomics).
// Y is laid out like the map's lists: the product of list entry i is Y row i.
// The groups (make_group_plan) follow the pages: the offsets with entries,
// the identity offset apart, in decreasing map size (ties by index), cut into
// runs while the padded rows stay at most epsilon of a run's padded batch; a
// run whose largest map is at least S runs as separate products (each offset
// padded to its own size only).  (The page describes the paper's scan in
// kernel order but sorts by size in its figure and tuner; only the size order
// makes epsilon = 0 pair the mirror offsets, its symmetric grouping.)  The
// host makes the plan from the map's counts; a one-wave kernel writes the
// device's entry table.
#include "internal.h"

#include <algorithm>

namespace spconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ floatx4 mfma(uint4 a, uint4 b, floatx4 c) {
  if constexpr (__is_same(T, _Float16)) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
__device__ __forceinline__ uint16_t round_bits(float v) {
  if constexpr (__is_same(T, _Float16)) return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
  else return bf16_bits_rne(v);
}

constexpr int kGsRows = 64;          // rows of a gather tile
constexpr int kGsWgRows = 256;       // batch rows one GEMM workgroup streams through its weights
constexpr int kGsQB = 2;             // 16-row blocks a wave computes at once
constexpr int kGsWeightLds = 32768;  // bytes of a workgroup's weight slice
constexpr int kReduceRows = 16;      // output rows of a reduction workgroup
constexpr int kReduceBatch = 8;      // product rows a reduction thread loads before adding them

// One entry of the grouped computation: one offset, its list and its padded
// rows in the batch buffer.
struct GsEntry {
  int32_t k;
  int32_t len;   // entries of offset k
  int32_t pad;   // rows in the batch (the largest map of the group)
  int32_t blk0;  // first 64-row gather tile of this entry among all entries' tiles
  int64_t off;   // list start of offset k (its first Y row)
  int64_t base;  // first row of the entry in A
};

// The plan as the host made it: the offset and padded size of each entry,
// in execution order.
struct GsPlanArgs {
  int32_t n;
  int16_t k[kMaxGroupEntries];
  int32_t pad[kMaxGroupEntries];
};

constexpr int kSetupPer = (kMaxGroupEntries + 63) / 64;

// One wave: lane l fills entries l * kSetupPer ..; the A rows and gather
// tiles before each entry come from a wave prefix sum of the lanes' totals.
__global__ __launch_bounds__(64) void k_gs_setup(GsPlanArgs p, const int32_t* __restrict__ tile_off, int64_t tiles,
                                                 GsEntry* __restrict__ ent) {
  const int lane = threadIdx.x;
  const int e0 = lane * kSetupPer;
  int64_t rows = 0;
  int32_t blks = 0;
  int32_t lo[kSetupPer], hi[kSetupPer];
#pragma unroll
  for (int i = 0; i < kSetupPer; ++i) {
    const int e = e0 + i;
    lo[i] = hi[i] = 0;
    if (e < p.n) {
      const int64_t k = p.k[e];
      lo[i] = tile_off[k * tiles];
      hi[i] = tile_off[(k + 1) * tiles];
      rows += p.pad[e];
      blks += (p.pad[e] + kGsRows - 1) / kGsRows;
    }
  }
  int64_t r_incl = rows;
  int32_t b_incl = blks;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t r = __shfl_up(r_incl, d);
    const int32_t b = __shfl_up(b_incl, d);
    if (lane >= d) {
      r_incl += r;
      b_incl += b;
    }
  }
  int64_t base = r_incl - rows;
  int32_t blk = b_incl - blks;
#pragma unroll
  for (int i = 0; i < kSetupPer; ++i) {
    const int e = e0 + i;
    if (e < p.n) {
      GsEntry g;
      g.k = p.k[e];
      g.len = hi[i] - lo[i];
      g.pad = p.pad[e];
      g.blk0 = blk;
      g.off = lo[i];
      g.base = base;
      ent[e] = g;
      base += g.pad;
      blk += (g.pad + kGsRows - 1) / kGsRows;
    }
  }
}

// The entry whose gather tiles hold tile `blk` (entries are in tile order).
__device__ __forceinline__ int find_entry(const GsEntry* __restrict__ ent, int n, int32_t blk) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (ent[mid].blk0 <= blk) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Gather: workgroup = one 64-row tile of one entry; each thread copies
// 16-byte pieces of the tile's rows (the input row of the list entry, or
// zeros past the list).
template <typename T>
__global__ __launch_bounds__(256) void k_gs_gather(const T* __restrict__ feats, const int32_t* __restrict__ in_idx,
                                                   const GsEntry* __restrict__ ent, int n_ent, int cin,
                                                   T* __restrict__ A) {
  const GsEntry e = ent[find_entry(ent, n_ent, static_cast<int32_t>(blockIdx.x))];
  const int32_t r0 = (static_cast<int32_t>(blockIdx.x) - e.blk0) * kGsRows;
  const int per_row = cin * static_cast<int>(sizeof(T)) / 16;
  for (int p = threadIdx.x; p < kGsRows * per_row; p += 256) {
    const int rr = p / per_row, c = p % per_row;
    const int32_t r = r0 + rr;
    if (r >= e.pad) continue;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < e.len) {
      const int64_t src = in_idx[e.off + r];
      v = reinterpret_cast<const uint4*>(feats + src * cin)[c];
    }
    reinterpret_cast<uint4*>(A + (e.base + r) * cin)[c] = v;
  }
}

// GEMM of one group: workgroup (row chunk x, column slice y, entry z of the
// group).  The slice's NCB 16-column blocks of W_k, in MFMA operand order
// (k_prep_weights: lane (g, r) of block cb and chunk ch holds
// W[32 ch + 8 g + i][16 cb + r], i < 8), are staged in LDS; then each wave
// takes kGsQB 16-row blocks at a time (8 channels of chunk ch of batch row
// 16 q + r per lane: the B operand) and accumulates D = W^T A^T: lane (g, r)
// ends with output columns 16 cb + 4 g + j of batch row 16 q + r.  PC chunks
// of B are loaded before their MFMAs.
template <typename T, int NCB, int PC>
__global__ __launch_bounds__(256) void k_gs_gemm(const uint16_t* __restrict__ A, const uint4* __restrict__ wop,
                                                 const GsEntry* __restrict__ ent, int e_first, int nch, int ncbg,
                                                 float* __restrict__ Y) {
  extern __shared__ uint4 s_w[];  // [NCB][nch][64]
  const GsEntry e = ent[e_first + blockIdx.z];
  const int cb0 = blockIdx.y * NCB;
  const int cin = nch * 32, cout = ncbg * 16;
  for (int i = threadIdx.x; i < NCB * nch * 64; i += 256) {
    const int lane = i & 63, ch = (i >> 6) % nch, cb = (i >> 6) / nch;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (cb0 + cb < ncbg) v = wop[((static_cast<int64_t>(e.k) * ncbg + cb0 + cb) * nch + ch) * 64 + lane];
    s_w[i] = v;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int32_t r_end = min(e.pad, static_cast<int32_t>(blockIdx.x + 1) * kGsWgRows);
  for (int32_t rb = static_cast<int32_t>(blockIdx.x) * kGsWgRows + wave * 16 * kGsQB; rb < r_end;
       rb += 4 * 16 * kGsQB) {
    floatx4 acc[kGsQB][NCB];
#pragma unroll
    for (int q = 0; q < kGsQB; ++q)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[q][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int ch0 = 0; ch0 < nch; ch0 += PC) {
      uint4 b[kGsQB][PC];
#pragma unroll
      for (int q = 0; q < kGsQB; ++q) {
        const int32_t row = rb + 16 * q + r;
        const uint16_t* src = A + (e.base + (row < e.pad ? row : 0)) * cin + 32 * ch0 + 8 * g;
#pragma unroll
        for (int c = 0; c < PC; ++c) {
          b[q][c] = make_uint4(0u, 0u, 0u, 0u);
          if (row < e.pad) b[q][c] = *reinterpret_cast<const uint4*>(src + 32 * c);
        }
      }
#pragma unroll
      for (int c = 0; c < PC; ++c) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const uint4 a = s_w[(cb * nch + ch0 + c) * 64 + lane];
#pragma unroll
          for (int q = 0; q < kGsQB; ++q) acc[q][cb] = mfma<T>(a, b[q][c], acc[q][cb]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kGsQB; ++q) {
      const int32_t row = rb + 16 * q + r;
      if (row < e.len) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          if (cb0 + cb < ncbg) {
            *reinterpret_cast<floatx4*>(Y + (e.off + row) * cout + 16 * (cb0 + cb) + 4 * g) = acc[q][cb];
          }
        }
      }
    }
  }
}

// Reduce: workgroup = kReduceRows rows of one 64-row output tile (so that
// small maps still fill the chip).  The tile's masks and first list
// positions per offset are staged in LDS; then each thread sums 4 columns of
// one row over the offsets present, in offset order, from Y (the entry's list
// position: the tile's first position plus its rank in the mask), and writes
// the row once, rounded to the dtype.  A thread issues the loads of
// kReduceBatch offsets before adding them (latency, not bandwidth, bounds
// the small layers).
template <typename T>
__global__ __launch_bounds__(256) void k_gs_reduce(const float* __restrict__ Y,
                                                   const unsigned long long* __restrict__ tile_mask,
                                                   const int32_t* __restrict__ tile_off,
                                                   const int32_t* __restrict__ perm, int64_t n, int64_t tiles,
                                                   int KV, int cout, T* __restrict__ out) {
  __shared__ unsigned long long s_mask[kMaxGroupEntries];
  __shared__ int32_t s_pos[kMaxGroupEntries];
  const int64_t t = blockIdx.x / (kGsRows / kReduceRows);
  const int r0 = static_cast<int>(blockIdx.x % (kGsRows / kReduceRows)) * kReduceRows;
  for (int k = threadIdx.x; k < KV; k += blockDim.x) {
    s_mask[k] = tile_mask[static_cast<int64_t>(k) * tiles + t];
    s_pos[k] = tile_off[static_cast<int64_t>(k) * tiles + t];
  }
  __syncthreads();
  const int tpr = cout / 4;  // threads per row, 4 columns each (cout <= 1024: tpr <= 256)
  const int rows_per_pass = static_cast<int>(blockDim.x) / tpr;
  if (static_cast<int>(threadIdx.x) >= rows_per_pass * tpr) return;
  const int c4 = threadIdx.x % tpr;
  for (int rr = r0 + static_cast<int>(threadIdx.x) / tpr; rr < r0 + kReduceRows; rr += rows_per_pass) {
    const int64_t q = t * kGsRows + rr;
    if (q >= n) break;
    const unsigned long long below = (rr == 0) ? 0ull : (~0ull >> (64 - rr));
    // The sums run in offset order; an absent offset adds +0, which changes
    // no sum (acc starts at +0, so it is never -0).
    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < KV; k0 += kReduceBatch) {
      floatx4 v[kReduceBatch];
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j) {
        const int k = k0 + j;
        v[j] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (k < KV) {
          const unsigned long long m = s_mask[k];
          if ((m >> rr) & 1ull) {
            const int64_t yr = static_cast<int64_t>(s_pos[k]) + __popcll(m & below);
            v[j] = *reinterpret_cast<const floatx4*>(Y + yr * cout + 4 * c4);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j) acc += v[j];
    }
    const int64_t orow = perm != nullptr ? static_cast<int64_t>(perm[q]) : q;
    u16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = round_bits<T>(acc[i]);
    *reinterpret_cast<u16x4*>(out + orow * cout + 4 * c4) = o;
  }
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

struct GsLayout {
  size_t wop_b, a_b, y_b, ent_b;
};

GsLayout gs_layout(const ForwardArgs& a, const GroupPlan& p) {
  GsLayout l;
  l.wop_b = align256(tiled_workspace_bytes(a));
  l.a_b = align256(static_cast<size_t>(p.padded_rows) * a.cin * 2);
  l.y_b = align256(static_cast<size_t>(p.list_rows) * a.cout * sizeof(float));
  l.ent_b = align256(sizeof(GsEntry) * kMaxGroupEntries);
  return l;
}

// Weight slice of a GEMM workgroup: NCB 16-column blocks, NCB x nch KiB of
// operands, within kGsWeightLds and no wider than the output.
int gemm_ncb(int nch, int ncbg) {
  int ncb = 8;
  while (ncb > 1 && ncb * nch * 1024 > kGsWeightLds) ncb /= 2;
  while (ncb > 1 && ncb / 2 >= ncbg) ncb /= 2;
  return ncb;
}

int gemm_pc(int nch) {
  if (nch % 4 == 0) return 4;
  if (nch % 2 == 0) return 2;
  return 1;
}

template <typename T, int NCB, int PC>
void launch_gemm_group(const uint16_t* A, const uint4* wop, const GsEntry* ent, int e_first, int count, int64_t pad,
                       int nch, int ncbg, float* Y, hipStream_t stream) {
  const unsigned gx = static_cast<unsigned>((pad + kGsWgRows - 1) / kGsWgRows);
  const unsigned gy = static_cast<unsigned>((ncbg + NCB - 1) / NCB);
  const size_t lds = static_cast<size_t>(NCB) * nch * 64 * sizeof(uint4);
  hipLaunchKernelGGL((k_gs_gemm<T, NCB, PC>), dim3(gx, gy, static_cast<unsigned>(count)), dim3(256), lds, stream, A,
                     wop, ent, e_first, nch, ncbg, Y);
}

template <typename T, int NCB>
void launch_gemm_pc(int pc, const uint16_t* A, const uint4* wop, const GsEntry* ent, int e_first, int count,
                    int64_t pad, int nch, int ncbg, float* Y, hipStream_t stream) {
  if (pc == 4) launch_gemm_group<T, NCB, 4>(A, wop, ent, e_first, count, pad, nch, ncbg, Y, stream);
  else if (pc == 2) launch_gemm_group<T, NCB, 2>(A, wop, ent, e_first, count, pad, nch, ncbg, Y, stream);
  else launch_gemm_group<T, NCB, 1>(A, wop, ent, e_first, count, pad, nch, ncbg, Y, stream);
}

template <typename T>
hipError_t launch_typed(const ForwardArgs& a, const GroupPlan& p, void* ws, hipStream_t stream) {
  const GsLayout l = gs_layout(a, p);
  char* c = static_cast<char*>(ws);
  const uint4* wop = reinterpret_cast<const uint4*>(c);
  T* A = reinterpret_cast<T*>(c + l.wop_b);
  float* Y = reinterpret_cast<float*>(c + l.wop_b + l.a_b);
  GsEntry* ent = reinterpret_cast<GsEntry*>(c + l.wop_b + l.a_b + l.y_b);
  const int n_ent = static_cast<int>(p.entries.size());
  GsPlanArgs pa;
  pa.n = n_ent;
  for (int i = 0; i < kMaxGroupEntries; ++i) {
    pa.k[i] = static_cast<int16_t>(i < n_ent ? p.entries[i] : 0);
    pa.pad[i] = i < n_ent ? static_cast<int32_t>(p.group_pad[p.entry_group[i]]) : 0;
  }
  hipError_t e = launch_prep_weights(a, ws, stream);
  if (e != hipSuccess) return e;
  if (n_ent > 0) {
    hipLaunchKernelGGL(k_gs_setup, dim3(1), dim3(64), 0, stream, pa, a.tile_off, a.tiles, ent);
    hipLaunchKernelGGL(k_gs_gather<T>, dim3(static_cast<unsigned>(p.tiles)), dim3(256), 0, stream,
                       static_cast<const T*>(a.feats), a.in_idx, static_cast<const GsEntry*>(ent), n_ent, a.cin, A);
    const int nch = a.cin / 32, ncbg = a.cout / 16;
    const int ncb = gemm_ncb(nch, ncbg), pc = gemm_pc(nch);
    const uint16_t* A16 = reinterpret_cast<const uint16_t*>(A);
    for (int gi = 0; gi < p.groups; ++gi) {
      const int e_first = p.group_first[gi], count = p.group_first[gi + 1] - e_first;
      const int64_t pad = p.group_pad[gi];
      switch (ncb) {
        case 8: launch_gemm_pc<T, 8>(pc, A16, wop, ent, e_first, count, pad, nch, ncbg, Y, stream); break;
        case 4: launch_gemm_pc<T, 4>(pc, A16, wop, ent, e_first, count, pad, nch, ncbg, Y, stream); break;
        case 2: launch_gemm_pc<T, 2>(pc, A16, wop, ent, e_first, count, pad, nch, ncbg, Y, stream); break;
        default: launch_gemm_pc<T, 1>(pc, A16, wop, ent, e_first, count, pad, nch, ncbg, Y, stream); break;
      }
    }
  }
  // kReduceRows rows of tpr threads each, at most 256 threads
  const unsigned reduce_threads = static_cast<unsigned>(std::min(256, kReduceRows * (a.cout / 4)));
  hipLaunchKernelGGL(k_gs_reduce<T>, dim3(static_cast<unsigned>(a.tiles * (kGsRows / kReduceRows))),
                     dim3(reduce_threads), 0, stream,
                     static_cast<const float*>(Y), a.tile_mask, a.tile_off, a.perm, a.n, a.tiles, a.KV, a.cout,
                     static_cast<T*>(a.out));
  return hipGetLastError();
}

}  // namespace

GroupPlan make_group_plan(const int64_t* counts, int KV, int centre, double epsilon, double S) {
  std::vector<int> order;
  for (int k = 0; k < KV; ++k)
    if (counts[k] > 0 && k != centre) order.push_back(k);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return counts[x] > counts[y]; });
  std::vector<std::vector<int>> runs;
  std::vector<int> cur;
  int64_t cur_max = 0, cur_sum = 0;
  for (int k : order) {
    const int64_t mx = std::max(cur_max, counts[k]);
    const int64_t tot = cur_sum + counts[k];
    const int64_t m = static_cast<int64_t>(cur.size()) + 1;
    // redundant computation ratio of the run with k added: its padded rows
    // over the padded batch's rows
    const double ratio = static_cast<double>(m * mx - tot) / static_cast<double>(m * mx);
    if (!cur.empty() && ratio > epsilon) {
      runs.push_back(cur);
      cur.assign(1, k);
      cur_max = counts[k];
      cur_sum = counts[k];
    } else {
      cur.push_back(k);
      cur_max = mx;
      cur_sum = tot;
    }
  }
  if (!cur.empty()) runs.push_back(cur);
  std::vector<std::vector<int>> groups;
  if (centre >= 0 && centre < KV && counts[centre] > 0) groups.push_back({centre});
  for (const auto& g : runs) {
    int64_t mx = 0;
    for (int k : g) mx = std::max(mx, counts[k]);
    if (static_cast<double>(mx) >= S) {
      for (int k : g) groups.push_back({k});
    } else {
      groups.push_back(g);
    }
  }
  GroupPlan p;
  for (size_t gi = 0; gi < groups.size(); ++gi) {
    int64_t mx = 0;
    for (int k : groups[gi]) mx = std::max(mx, counts[k]);
    p.group_first.push_back(static_cast<int>(p.entries.size()));
    p.group_pad.push_back(mx);
    for (int k : groups[gi]) {
      p.entries.push_back(k);
      p.entry_group.push_back(static_cast<int>(gi));
      p.padded_rows += mx;
      p.list_rows += counts[k];
      p.tiles += (mx + kGsRows - 1) / kGsRows;
    }
  }
  p.group_first.push_back(static_cast<int>(p.entries.size()));
  p.groups = static_cast<int>(groups.size());
  return p;
}

bool grouped_supported(const ForwardArgs& a) {
  return (a.dtype == 1 || a.dtype == 2) && a.cin % 32 == 0 && a.cout % 16 == 0 && a.KV <= kMaxGroupEntries;
}

size_t grouped_workspace_bytes(const ForwardArgs& a, const GroupPlan& p) {
  const GsLayout l = gs_layout(a, p);
  return l.wop_b + l.a_b + l.y_b + l.ent_b;
}

hipError_t launch_forward_grouped(const ForwardArgs& a, const GroupPlan& p, void* workspace, hipStream_t stream) {
  if (!grouped_supported(a)) return hipErrorNotSupported;
  if (a.dtype == 1) return launch_typed<_Float16>(a, p, workspace, stream);
  return launch_typed<__bf16>(a, p, workspace, stream);
}

}  // namespace spconv
