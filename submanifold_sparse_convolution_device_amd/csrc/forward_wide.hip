// Forward of a submanifold sparse convolution for wide channel counts
// (C_in 64, 128 or 256; C_out a multiple of 64, of 32 at C_in = 256) on
// gfx950.
//
// Same computation as the other forward kernels: for every output row Q,
// f_out(Q) = sum over map entries (P, Q, W_d) of f_in(P) x W_d ("Sparse
// convolution for point clouds", section "The map and the update rule"),
// accumulated on chip per output row and written once.
//
// Work unit: a task of TB 16-row blocks (one or two 64-row tiles) and a
// group of NW x NCB x 16 output columns.  Wave w of the workgroup owns NCB
// 16-column blocks of all TB blocks, so its accumulators are TB x NCB MFMA
// tiles.  Large layers use one column group (every column of a task in one
// workgroup, so a gathered row is shared by all of them); small ones split
// the columns and shorten the tasks so that the grid still fills the chip.
// The task walks the offsets that occur in its rows.  Per offset d:
//   * the gathered input rows of the task's blocks (B operands, zero for
//     rows without a neighbour at d) are copied from global memory straight
//     into LDS (buffer loads to LDS: lane l of a load writes 16 bytes at
//     l x 16; a row without a neighbour reads past the buffer's end, where
//     the load's bounds check returns zeros), whole rows per copy, shared by
//     all waves of the workgroup;
//   * each wave keeps its slice of W_d (A operands, from a copy of the weights
//     in operand order) in registers and applies it to every block present;
// and the work is software-pipelined: while offset i runs on MFMA, the
// weights and gathered rows of offset i + 1 and the row indices of offset
// i + 2 are loaded, their load instructions spread between the MFMA groups
// so that they issue in the matrix core's shadow.  A step begins by waiting
// for all of them (and, by a barrier, for the other waves' row copies).
// The epilogue rounds the accumulators, regroups pairs of column blocks
// between lanes so that each lane holds 8 consecutive columns of its row,
// and streams them out with non-temporal 16-byte stores (split offsets
// write fp32 partials instead, summed by k_reduce_splits).
#include "internal.h"

#include <type_traits>
#include <utility>

namespace spconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Four fp32 values rounded to nearest even in the output type, packed.
template <typename T>
__device__ __forceinline__ u16x4 pack4(floatx4 v) {
  u16x4 o;
  if constexpr (__is_same(T, _Float16)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[i]));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = bf16_bits_rne(v[i]);
  }
  return o;
}

template <typename T>
__device__ __forceinline__ void store4(T* dst, floatx4 v) {
  *reinterpret_cast<u16x4*>(dst) = pack4<T>(v);
}

template <typename T>
__device__ __forceinline__ floatx4 mfma(uint4 a, uint4 b, floatx4 c) {
  if constexpr (__is_same(T, _Float16)) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

__device__ __forceinline__ int lane_i32(int v, int src) { return __builtin_amdgcn_readlane(v, src); }
__device__ __forceinline__ unsigned long long lane_u64(unsigned long long v, int src) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), src));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), src));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup barrier that orders only what the kernel orders by hand.
// __syncthreads() also makes global memory visible, which drains every load
// in flight (the prefetches included).  Here the copies into LDS that a step
// needs are waited for by count (wait_vm) before the barrier, and the LDS
// reads of the stage complete inside their own asm block, so a bare barrier
// (a compiler barrier on both sides) is enough.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The B operands of one staged block read block by block (read_chunks) are
// written as asm because the compiler, unable to tell the two stage buffers
// apart, would otherwise wait for every copy into LDS still in flight before
// each read, the next offset's included; the asm also keeps it from waiting
// for the reads themselves before their registers are needed.
template <int... I, typename F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N - 1, in order.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// The NCH chunks of one staged block: one 16-byte LDS read per chunk at
// addr[ch] + OFF, left in flight.
template <int NCH, int OFF>
__device__ __forceinline__ void read_chunks(const uint32_t (&addr)[NCH], u32x4 (&v)[NCH]) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset range");
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v[ch]) : "v"(addr[ch]), "i"(OFF) : "memory");
}

// Waits until at most N LDS (or scalar-memory) operations are in flight and
// only then releases v: the registers pass through the asm, so nothing that
// reads them can be scheduled before the wait.
template <int N, int TB>
__device__ __forceinline__ void wait_lgkm(u32x4 (&v)[TB]) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  if constexpr (TB == 2) {
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(v[0]), "+v"(v[1]) : "i"(N) : "memory");
  } else if constexpr (TB == 8) {
    asm volatile("s_waitcnt lgkmcnt(%8)"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
                 : "i"(N)
                 : "memory");
  } else {
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]) : "i"(N) : "memory");
  }
}

// s_waitcnt with only a vector-memory count (the other counters unconstrained).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int CIN, int TB, int NCB, int NW>
struct WideShape {
  static constexpr int NCH = CIN / 32;            // 32-wide ci chunks
  static constexpr int TPT = TB / 4;              // 64-row tiles per task
  static constexpr int BPW = TB / NW;             // blocks staged by each wave
  static constexpr int COLS = NW * NCB * 16;      // output columns of a workgroup
  // A staged row is SEG 16-byte segments; one copy instruction moves RPI
  // whole rows (64 lanes x 16 bytes), so a block takes IPB of them.  Whole
  // rows per instruction matter: the gather's cost follows the number of
  // distinct rows an instruction touches, not its bytes.
  static constexpr int SEG = CIN / 8;
  static constexpr int RPI = 64 / SEG;
  static constexpr int IPB = 16 / RPI;
  // Rows sharing one 256-byte LDS bank period.
  static constexpr int RP = SEG * 16 >= 256 ? 1 : 256 / (SEG * 16);
  static constexpr int LOADS_A = NCB * NCH;       // weight loads per wave and offset
  static constexpr int LOADS_B = BPW * IPB;       // LDS copies per wave and offset
  static constexpr int LOADS_I = BPW;             // index loads per wave and offset
  static constexpr int BLOCK_BYTES = 16 * SEG * 16;  // one staged 16-row block
  static constexpr int STAGE_BYTES = TB * BLOCK_BYTES;
  static size_t lds_bytes() { return static_cast<size_t>(2) * STAGE_BYTES; }
  static_assert(TB == 4 || TB == 8, "tasks of one or two tiles");
  static_assert(BPW >= 1 && BPW * NW == TB, "blocks split evenly over the waves");
};

// Segment swizzle of staged row i: its 16-byte segment c sits at position
// c ^ seg_swizzle(i), so that the 16 rows a B-operand read touches at one
// segment fall on distinct LDS banks.
template <int SEG, int RP>
__device__ __forceinline__ int seg_swizzle(int i) {
  return (i / RP) & ((SEG < 16 ? SEG : 16) - 1);
}

// Buffer resource word 3 for raw 32-bit-element loads (gfx9 data format 32,
// no swizzle): the bounds check then compares each byte offset with the
// record count, the buffer's size in bytes.
constexpr int kBufferWord3 = 0x00020000;
// Largest feature buffer the row copies address (see wide_supported).
constexpr int64_t kWideMaxFeatureBytes = (int64_t{1} << 32) - 4096;

// Per-offset state the pipeline carries: the offset, and for each of the
// (up to) two tiles its row mask and first list position (wave-uniform).
struct OffsetRef {
  int k;
  unsigned long long m0, m1;
  int lo0, lo1;
  uint32_t pm;  // bit b: 16-row block b has at least one entry
};

template <typename T, int CIN, int TB, int NCB, int NW>
__global__ __launch_bounds__(64 * NW) void k_forward_wide(
    const uint16_t* __restrict__ feats_raw, const uint4* __restrict__ wop, T* __restrict__ out,
    const int32_t* __restrict__ in_idx, const int32_t* __restrict__ tile_off,
    const unsigned long long* __restrict__ tile_mask, const int32_t* __restrict__ perm, int64_t n, int64_t n_in,
    int64_t tiles, int64_t tasks, int groups, int splits, float* __restrict__ part, int KV, int cout, int centre_k) {
  using Sh = WideShape<CIN, TB, NCB, NW>;
  constexpr int NCH = Sh::NCH, BPW = Sh::BPW, TPT = Sh::TPT;
  constexpr int SEG = Sh::SEG, RPI = Sh::RPI, IPB = Sh::IPB, RP = Sh::RP, BLOCK_BYTES = Sh::BLOCK_BYTES;
  extern __shared__ uint4 bstage[];  // [2][TB] staged blocks of 16 rows
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  // Consecutive work units on one XCD (workgroups are dealt to the 8 XCDs in
  // turn), so that units sharing rows share an L2: a task's column groups
  // are adjacent, and so are neighbouring tasks.  The grid is a multiple of
  // 8 workgroups, which makes the remapping a permutation of [0, grid).
  const int64_t per_xcd = gridDim.x / 8;
  const int64_t bid = blockIdx.x;
  const int64_t unit = (bid % 8) * per_xcd + bid / 8;
  if (unit >= tasks * groups * splits) return;  // uniform over the workgroup
  // unit = (task x groups + column group) x splits + offset share
  const int share = static_cast<int>(unit % splits);
  const int64_t tg = unit / splits;
  const int64_t task = tg / groups;
  const int cg = static_cast<int>(tg - task * groups);
  const int64_t t0 = TPT * task, t1 = t0 + 1;
  const int64_t q0 = t0 * kTileRows;
  const int col0 = cg * Sh::COLS + wave * NCB * 16;  // this wave's first output column
  // The output row of each of the lane's TB rows (position q0 + 16 b + r;
  // -1 past the last row), loaded now so that the epilogue's stores wait
  // for nothing.
  int32_t out_row[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    const int64_t qpos = q0 + 16 * b + r;
    out_row[b] = qpos < n ? (perm != nullptr ? perm[qpos] : static_cast<int32_t>(qpos)) : -1;
  }

  // Task metadata: lane k (and k - 64) holds offset k's masks and list starts.
  unsigned long long mA0 = 0ull, mA1 = 0ull, mB0 = 0ull, mB1 = 0ull;
  int lA0 = 0, lA1 = 0, lB0 = 0, lB1 = 0;
  if (lane < KV) {
    mA0 = tile_mask[static_cast<int64_t>(lane) * tiles + t0];
    lA0 = tile_off[static_cast<int64_t>(lane) * tiles + t0];
    if (TPT == 2 && t1 < tiles) {
      mA1 = tile_mask[static_cast<int64_t>(lane) * tiles + t1];
      lA1 = tile_off[static_cast<int64_t>(lane) * tiles + t1];
    }
  }
  if (lane + 64 < KV) {
    mB0 = tile_mask[static_cast<int64_t>(lane + 64) * tiles + t0];
    lB0 = tile_off[static_cast<int64_t>(lane + 64) * tiles + t0];
    if (TPT == 2 && t1 < tiles) {
      mB1 = tile_mask[static_cast<int64_t>(lane + 64) * tiles + t1];
      lB1 = tile_off[static_cast<int64_t>(lane + 64) * tiles + t1];
    }
  }
  unsigned long long todo0 = __ballot((mA0 | mA1) != 0ull), todo1 = __ballot((mB0 | mB1) != 0ull);
  // With splits > 1 the task's offsets are dealt round-robin over the
  // splits workgroups of the unit, each summing its share into its own fp32
  // partial output: the share's offsets are picked out of the task's once,
  // here.  (splits is a power of two.)
  if (splits > 1) {
    const int share_u = __builtin_amdgcn_readfirstlane(share);
    const int smask = __builtin_amdgcn_readfirstlane(splits - 1);
    unsigned long long keep0 = 0ull, keep1 = 0ull;
    int seen = 0;
    for (unsigned long long t = todo0; t != 0ull; t &= t - 1ull)
      if ((seen++ & smask) == share_u) keep0 |= t & (~t + 1ull);
    for (unsigned long long t = todo1; t != 0ull; t &= t - 1ull)
      if ((seen++ & smask) == share_u) keep1 |= t & (~t + 1ull);
    todo0 = keep0;
    todo1 = keep1;
  }
  auto pick = [&](unsigned long long& todo, int base) -> int {
    if (todo == 0ull) return -1;
    const int kk = base + __ffsll(static_cast<long long>(todo)) - 1;
    todo &= todo - 1ull;
    return kk;
  };
  // The next offset's state; pm, the blocks present, is computed here once
  // for the tests around that offset's MFMA groups and row copies.
  auto next_ref = [&]() -> OffsetRef {
    OffsetRef o{-1, 0ull, 0ull, 0, 0, 0u};
    int k = pick(todo0, 0);
    if (k < 0) k = pick(todo1, 64);
    if (k >= 0) {
      const int s = k & 63;
      o.k = k;
      o.m0 = lane_u64(k < 64 ? mA0 : mB0, s);
      o.m1 = lane_u64(k < 64 ? mA1 : mB1, s);
      o.lo0 = lane_i32(k < 64 ? lA0 : lB0, s);
      o.lo1 = lane_i32(k < 64 ? lA1 : lB1, s);
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        const unsigned long long m = (b < 4) ? o.m0 : o.m1;
        if (((m >> (16 * (b & 3))) & 0xffffull) != 0ull) o.pm |= 1u << b;
      }
    }
    return o;
  };

  // The loads that prepare an offset, one at a time so that they can be
  // spread through the MFMAs of the offset before (see run).
  //   Index load j (< BPW): the input row of lane (g, r)'s row 16 b + r of the
  //     wave's staged block b = wave + NW j at offset o; -1 where there is no
  //     entry (the load itself is unconditional: in_idx[0] stands in).
  auto load_idx_one = [&](const OffsetRef& o, int32_t (&idx)[BPW], int j) {
    const int b = wave + NW * j;
    const unsigned long long m = (b < 4) ? o.m0 : o.m1;
    const int bit = 16 * (b & 3) + r;
    const bool has = o.k >= 0 && ((m >> bit) & 1ull);
    const int rank = __popcll(m & ((1ull << bit) - 1ull));
    const int lo = (b < 4) ? o.lo0 : o.lo1;
    // The centre offset reads the task's own rows (the row at each position:
    // perm, or the position itself), not its list.
    const int64_t qpos = q0 + 16 * b + r;
    const bool centre = o.k == centre_k;  // wave-uniform; centre_k = -1: no identity offset
    int32_t v;
    if (centre && perm == nullptr) v = static_cast<int32_t>(qpos);
    else v = centre ? perm[has ? qpos : 0] : in_idx[has ? lo + rank : 0];
    // An OR with the "no entry" mask rather than a select on the loaded
    // value: a select would let the compiler move the load under a branch
    // and wait for it there.
    idx[j] = v | (has ? 0 : -1);
  };
  //   Row copies of the wave's staged block jj (< BPW), IPB of them under
  //     one test of the block's bit (a block with no entry at the offset is
  //     skipped, its MFMAs too): copy q moves rows [RPI q, RPI q + RPI) of
  //     the block, whole rows, from global memory straight into B stage
  //     `buf`; lane l copies segment (l % SEG) ^ swizzle of row RPI q + l /
  //     SEG, whose input row is srow[jj IPB + q] (-1: no entry; its byte
  //     offset wraps to just below 2^32, past the end of the features, whose
  //     size the host keeps below that, so the load returns zeros).  srow
  //     comes from copy_rows, which moves the index of row i from lane i of
  //     idx (a cross-lane read, done before the MFMAs start, where its wait
  //     costs nothing).
  auto copy_rows = [&](const int32_t (&idx)[BPW], int32_t (&srow)[Sh::LOADS_B]) {
#pragma unroll
    for (int j = 0; j < Sh::LOADS_B; ++j) srow[j] = __shfl(idx[j / IPB], RPI * (j % IPB) + lane / SEG);
    // Settle the cross-lane reads here: their results pass through an asm,
    // so the wait for them lands before the stage reads start instead of
    // between them (where it would also wait for those).
#pragma unroll
    for (int j = 0; j < Sh::LOADS_B; ++j) asm volatile("" : "+v"(srow[j]));
  };
  const __amdgpu_buffer_rsrc_t frsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(feats_raw), 0, static_cast<int>(static_cast<uint32_t>(n_in * CIN * 2)), kBufferWord3);
  auto stage_block = [&](const OffsetRef& o, int buf, const int32_t (&srow)[Sh::LOADS_B], int jj) {
    const int b = wave + NW * jj;
    if (((o.pm >> b) & 1u) == 0u) return;  // wave-uniform
#pragma unroll
    for (int q = 0; q < IPB; ++q) {
      const int i = RPI * q + lane / SEG;
      const int c = (lane % SEG) ^ seg_swizzle<SEG, RP>(i);
      const uint32_t voff = static_cast<uint32_t>(srow[jj * IPB + q]) * (CIN * 2u) + static_cast<uint32_t>(c) * 16u;
      uint4* dst = bstage + ((buf * TB + b) * BLOCK_BYTES + q * RPI * SEG * 16) / 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(frsrc, (lds_void*)dst, 16, static_cast<int>(voff), 0, 0, 0);
    }
  };
  //   Weight load j (< NCB x NCH): this wave's slice of W_k in operand order.
  const int ncbg = cout / 16;
  const int cb0 = col0 / 16;
  auto load_a_one = [&](const OffsetRef& o, uint4 (&a)[NCB][NCH], int j) {
    const int k = o.k < 0 ? 0 : o.k;
    const int cb = j / NCH, ch = j % NCH;
    a[cb][ch] = wop[((static_cast<int64_t>(k) * ncbg + cb0 + cb) * NCH + ch) * 64 + lane];
  };
  constexpr int A = Sh::LOADS_A, I = Sh::LOADS_I;
  constexpr int kLoads = BPW + A + I;  // items: copy groups, weights, indices

  floatx4 acc[TB][NCB];
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[b][cb] = floatx4{0.f, 0.f, 0.f, 0.f};

  typedef __attribute__((address_space(3))) uint4 lds_uint4;
  const uint32_t stage_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_uint4*)bstage));
  // Per-lane LDS addresses of the NCH chunks of block 0 of stage 0: lane
  // (g, r) reads row r, segment 4 ch + g (swizzled); other blocks and the
  // other stage are immediate offsets.
  uint32_t caddr[NCH];
  {
    const int swz = seg_swizzle<SEG, RP>(r);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
      caddr[ch] = stage_addr + static_cast<uint32_t>(r * SEG * 16 + ((4 * ch + g) ^ swz) * 16);
  }
  // MFMAs of offset o from stage BUF and weights a, block by block (one
  // test of the block's bit per block).  The loads of the next offset
  // (load(item), items 0 .. kLoads - 1: the row-copy groups, weights, then
  // the indices of the offset after) are issued a few at a time after each
  // block's MFMAs, where they issue while the matrix core is busy instead
  // of stalling the wave before the offset starts.
  auto run = [&](const OffsetRef& o, auto buf_tag, const uint4 (&a)[NCB][NCH], auto&& load) {
    constexpr int BUF = decltype(buf_tag)::value;
    const uint32_t pm = o.pm;
    // Block-major: block b + 1's chunks are read while block b runs on MFMA.
    u32x4 bv[2][NCH];
    read_chunks<NCH, BUF * TB * BLOCK_BYTES>(caddr, bv[0]);
    static_for<TB>([&](auto b_tag) {
      constexpr int b = decltype(b_tag)::value;
      if constexpr (b + 1 < TB) {
        read_chunks<NCH, (BUF * TB + b + 1) * BLOCK_BYTES>(caddr, bv[(b + 1) & 1]);
        wait_lgkm<NCH, NCH>(bv[b & 1]);
      } else {
        wait_lgkm<0, NCH>(bv[b & 1]);
      }
      if (pm & (1u << b)) {
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            acc[b][cb] = mfma<T>(a[cb][ch], __builtin_bit_cast(uint4, bv[b & 1][ch]), acc[b][cb]);
      }
#pragma unroll
      for (int it = b * kLoads / TB; it < (b + 1) * kLoads / TB; ++it) load(it);
    });
  };

  // Prologue: indices of offsets 0 and 1, weights and rows of offset 0 (the
  // first offset always exists: every row of the task has its centre entry).
  OffsetRef o0 = next_ref();
  OffsetRef o1 = next_ref();
  OffsetRef o2 = next_ref();
  int32_t ix0[BPW], ix1[BPW];
  uint4 ax[NCB][NCH], ay[NCB][NCH];
#pragma unroll
  for (int j = 0; j < BPW; ++j) load_idx_one(o0, ix0, j);
#pragma unroll
  for (int j = 0; j < BPW; ++j) load_idx_one(o1, ix1, j);
#pragma unroll
  for (int j = 0; j < A; ++j) load_a_one(o0, ax, j);
  int32_t srow[Sh::LOADS_B];
  copy_rows(ix0, srow);
#pragma unroll
  for (int jj = 0; jj < BPW; ++jj) stage_block(o0, 0, srow, jj);

  // Steady state, two offsets per trip so that the register sets alternate
  // without copies.  One step: wait for every load of the step before (this
  // offset's rows, weights and the next offset's indices) and for the other
  // waves' row copies (barrier; it also ends every wave's reads of the stage
  // the step refills), then run this offset while loading the next.
  while (true) {
    // ---- offset o0: weights ax, stage 0; loads rows of o1 (from ix1) into
    // stage 1, its weights into ay, the indices of o2 into ix0
    wait_vm<0>();
    lds_barrier();
    copy_rows(ix1, srow);
    run(o0, std::integral_constant<int, 0>{}, ax, [&](int it) {
      if (it < BPW) stage_block(o1, 1, srow, it);
      else if (it < BPW + A) load_a_one(o1, ay, it - BPW);
      else load_idx_one(o2, ix0, it - BPW - A);
    });
    if (o1.k < 0) break;
    OffsetRef o3 = next_ref();
    // ---- offset o1: weights ay, stage 1; loads for o2 and the indices of o3
    wait_vm<0>();
    lds_barrier();
    copy_rows(ix0, srow);
    run(o1, std::integral_constant<int, 1>{}, ay, [&](int it) {
      if (it < BPW) stage_block(o2, 0, srow, it);
      else if (it < BPW + A) load_a_one(o2, ax, it - BPW);
      else load_idx_one(o3, ix1, it - BPW - A);
    });
    if (o2.k < 0) break;
    o0 = o2;
    o1 = o3;
    o2 = next_ref();
  }
  wait_vm<0>();  // no copy into LDS may be left in flight at exit

  // Epilogue.  D element (row 4 g + i, column r) of block (b, cb) is output
  // column col0 + 16 cb + 4 g + i of row out_row[b].
  if (splits == 1) {
    // Rounded to the output type, then each pair of column blocks (2 p,
    // 2 p + 1) is regrouped between the lanes of rows g and g ^ 1 (lanes l
    // and l ^ 16: one v_permlane16_swap per dword) so that every lane holds
    // 8 consecutive columns: an even g columns 32 p + 4 g .. + 7 (its own
    // four of block 2 p, then its partner's), an odd g columns
    // 32 p + 16 + 4 (g - 1) .. + 7 (its partner's four of block 2 p + 1,
    // then its own).  A store then writes 16 bytes per lane, 64 contiguous
    // bytes per row, instead of 8-byte fragments (8 frames, K = 3, C = 128:
    // 272 -> 258 us).
    static_assert(NCB % 2 == 0, "column blocks in pairs");
    const int colp = col0 + 4 * (g & ~1) + 16 * (g & 1);
#pragma unroll
    for (int b = 0; b < TB; ++b) {
#pragma unroll
      for (int p = 0; p < NCB / 2; ++p) {
        const uint2 x = __builtin_bit_cast(uint2, pack4<T>(acc[b][2 * p]));
        const uint2 y = __builtin_bit_cast(uint2, pack4<T>(acc[b][2 * p + 1]));
        const auto s0 = __builtin_amdgcn_permlane16_swap(x.x, y.x, false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(x.y, y.y, false, false);
        // Non-temporal: the output is not read again here, and streaming it
        // past the caches leaves them to the gathered rows and the weights
        // (8 frames, K = 3, C = 128: 256 -> 230 us).
        if (out_row[b] >= 0)
          __builtin_nontemporal_store(
              u32x4{s0[0], s1[0], s0[1], s1[1]},
              reinterpret_cast<u32x4*>(out + static_cast<int64_t>(out_row[b]) * cout + colp + 32 * p));
      }
    }
  } else {
    // A share of split offsets writes its fp32 partial sums (k_reduce_splits
    // adds the shares and rounds).
    float* pout = part + static_cast<int64_t>(share) * n * cout;
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      if (out_row[b] >= 0) {
        const int64_t q = out_row[b];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          *reinterpret_cast<floatx4*>(pout + q * cout + col0 + 16 * cb + 4 * g) = acc[b][cb];
      }
    }
  }
}

// Sum of the splits fp32 partial outputs, rounded to the output type (each
// thread four consecutive values).
template <typename T>
__global__ __launch_bounds__(256) void k_reduce_splits(const float* __restrict__ part, T* __restrict__ out,
                                                       int64_t count4, int64_t stride, int splits) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= count4) return;
  floatx4 s = reinterpret_cast<const floatx4*>(part)[i];
  for (int p = 1; p < splits; ++p) s += reinterpret_cast<const floatx4*>(part + p * stride)[i];
  store4<T>(out + 4 * i, s);
}

template <typename T, int CIN, int TB, int NCB, int NW>
hipError_t launch_wide_shape(const ForwardArgs& a, int splits, const uint4* wop, float* part, hipStream_t stream) {
  using Sh = WideShape<CIN, TB, NCB, NW>;
  const int64_t tasks = (a.tiles + Sh::TPT - 1) / Sh::TPT;
  const int groups = a.cout / Sh::COLS;
  static bool raised = false;
  if (!raised) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_forward_wide<T, CIN, TB, NCB, NW>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(Sh::lds_bytes()));
    if (e != hipSuccess) return e;
    raised = true;
  }
  const int64_t grid = (tasks * groups * splits + 7) / 8 * 8;
  hipLaunchKernelGGL((k_forward_wide<T, CIN, TB, NCB, NW>), dim3(static_cast<unsigned>(grid)), dim3(64 * NW),
                     Sh::lds_bytes(), stream, static_cast<const uint16_t*>(a.feats), wop, static_cast<T*>(a.out),
                     a.in_idx, a.tile_off, a.tile_mask, a.perm, a.n, a.n_in, a.tiles, tasks, groups, splits, part,
                     a.KV, a.cout, a.centre);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int64_t count4 = a.n * a.cout / 4;
  hipLaunchKernelGGL(k_reduce_splits<T>, dim3(static_cast<unsigned>((count4 + 255) / 256)), dim3(256), 0, stream,
                     part, static_cast<T*>(a.out), count4, a.n * a.cout, splits);
  return hipGetLastError();
}

// The compiled shapes: (C_in, task blocks, column blocks per wave, waves).
// Tasks are one tile (TB = 4): measured against two-tile tasks, which halve
// the weight traffic per row, the smaller register and LDS footprint (two
// waves per SIMD) wins on every workload here.  Column blocks per wave are 4
// (64 columns) at C_in = 128 and 2 at 64 and 256.  At 64, two waves per
// workgroup sharing the staged rows hide more latency than one (LiDAR frame
// step 84.0 -> 79.4 us, 8 frames at K = 5 770 -> 738 us); one block per wave
// lost 50 us on the latter, two lost 6 us at 128.  At 256 a wave's
// double-buffered weight slice would not fit otherwise.
struct WideChoice {
  int tb, ncb, nw, splits;
};

int wide_ncb(int cin) { return cin == 128 ? 4 : 2; }
constexpr int kMaxSplits = 8;

bool wide_compiled(int cin, int tb, int nw) {
  if (nw != 1 && nw != 2 && nw != 4) return false;
  return tb == 4 && (cin == 64 || cin == 128 || cin == 256);
}

int wide_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, v = 0;
    cus = (hipGetDevice(&dev) == hipSuccess &&
           hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
              ? v
              : 256;
  }
  return cus;
}

// Largest workgroups (every column of a task in one, up to 4 waves), unless
// the grid would leave CUs idle: then the offsets of a task split over up to
// kMaxSplits workgroups (fp32 partials, one reduction; no input row is read
// twice), and only then narrower workgroups (more column groups, each
// gathering the task's rows again).
bool choose_wide(const ForwardArgs& a, WideChoice* out) {
  const int ncb = wide_ncb(a.cin);
  const int per_wave = 16 * ncb;
  if (a.cout % per_wave != 0) return false;
  const int waves_total = a.cout / per_wave;
  int nw = 4;
  while (nw > 1 && waves_total % nw != 0) nw /= 2;
  const int64_t want = 2 * static_cast<int64_t>(wide_cus());
  auto units = [&](int tb, int w) { return (a.tiles + tb / 4 - 1) / (tb / 4) * (a.cout / (per_wave * w)); };
  const int tb = 4;
  if (!wide_compiled(a.cin, tb, nw)) return false;
  // Splits cost a pass over fp32 partials: only for grids under one
  // workgroup per CU.
  int splits = 1;
  if (units(tb, nw) < want / 2) {
    while (splits < kMaxSplits && units(tb, nw) * splits < want && 2 * splits <= a.KV) splits *= 2;
  }
  while (nw > 1 && units(tb, nw) * splits < want && wide_compiled(a.cin, tb, nw / 2)) nw /= 2;
  *out = WideChoice{tb, ncb, nw, splits};
  return true;
}

template <typename T, int CIN, int NCB>
hipError_t launch_wide_cin(const ForwardArgs& a, const WideChoice& c, const uint4* wop, float* part,
                           hipStream_t stream) {
  if (c.tb != 4) return hipErrorNotSupported;
  if (c.nw == 4) return launch_wide_shape<T, CIN, 4, NCB, 4>(a, c.splits, wop, part, stream);
  if (c.nw == 2) return launch_wide_shape<T, CIN, 4, NCB, 2>(a, c.splits, wop, part, stream);
  return launch_wide_shape<T, CIN, 4, NCB, 1>(a, c.splits, wop, part, stream);
}

template <typename T>
hipError_t launch_wide_typed(const ForwardArgs& a, const WideChoice& c, const uint4* wop, float* part,
                             hipStream_t stream) {
  if (a.cin == 64) return launch_wide_cin<T, 64, 2>(a, c, wop, part, stream);
  if (a.cin == 128) return launch_wide_cin<T, 128, 4>(a, c, wop, part, stream);
  return launch_wide_cin<T, 256, 2>(a, c, wop, part, stream);
}

}  // namespace

bool wide_supported(const ForwardArgs& a) {
  if (a.dtype != 1 && a.dtype != 2) return false;
  if (a.KV > 128) return false;
  if (a.cin != 64 && a.cin != 128 && a.cin != 256) return false;
  // Row copies address the features with 32-bit byte offsets, and a missing
  // row's offset (just below 2^32) must stay past their end.
  if (a.n_in * a.cin * 2 > kWideMaxFeatureBytes) return false;
  WideChoice c;
  return choose_wide(a, &c);
}

size_t wide_workspace_bytes(const ForwardArgs& a) {
  WideChoice c;
  const size_t base = a.prepared != nullptr ? 0 : tiled_workspace_bytes(a);
  if (!choose_wide(a, &c) || c.splits == 1) return base;
  return base + static_cast<size_t>(c.splits) * a.n * a.cout * sizeof(float);
}

hipError_t launch_forward_wide(const ForwardArgs& a, void* workspace, hipStream_t stream) {
  WideChoice c;
  if (!choose_wide(a, &c)) return hipErrorNotSupported;
  const uint4* wop = static_cast<const uint4*>(a.prepared != nullptr ? a.prepared : workspace);
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         (a.prepared != nullptr ? 0 : tiled_workspace_bytes(a)));
  if (a.dtype == 1) return launch_wide_typed<_Float16>(a, c, wop, part, stream);
  return launch_wide_typed<__bf16>(a, c, wop, part, stream);
}

}  // namespace spconv
