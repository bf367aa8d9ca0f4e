// Forward of a submanifold sparse convolution for wide channel counts
// (C_in 64 with C_out 64, 128 or 256; C_in 128 with C_out 128 or 256) on
// gfx950.
//
// Same computation as the other forward kernels: for every output row Q,
// f_out(Q) = sum over map entries (P, Q, W_d) of f_in(P) x W_d ("Sparse
// convolution for point clouds", section "The map and the update rule"),
// accumulated on chip per output row and written once.
//
// Work unit: a task of 128 output rows (two 64-row tiles, eight 16-row blocks)
// and all C_out columns.  The workgroup has C_out / 64 waves; wave w owns
// columns [64 w, 64 w + 64) of all 128 rows, so its accumulators are
// 8 blocks x 4 column blocks of MFMA tiles.  The task walks the offsets that
// occur in its rows.  Per offset d:
//   * the gathered input rows of the eight blocks (B operands, zero for rows
//     without a neighbour at d) are copied from global memory straight into
//     LDS in MFMA operand order (global_load_lds: lane l of a load writes
//     16 bytes at l x 16), shared by all waves of the task, so each entry's
//     input row leaves memory once;
//   * each wave keeps its slice of W_d (A operands, from a copy of the weights
//     in operand order) in registers and applies it to every block present;
// and the work is software-pipelined: while offset i runs on MFMA, the
// weights and gathered rows of offset i + 1 and the row indices of offset
// i + 2 are loaded, their load instructions spread between the MFMA groups
// so that they issue in the matrix core's shadow.  A step begins by waiting
// for all of them (and, by a barrier, for the other waves' row copies).
#include "internal.h"

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

template <typename T>
__device__ __forceinline__ void store4(T* dst, floatx4 v) {
  u16x4 o;
  if constexpr (__is_same(T, _Float16)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[i]));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = bf16_bits_rne(v[i]);
  }
  *reinterpret_cast<u16x4*>(dst) = o;
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

// The B operands of the eight blocks of one 32-wide ci chunk: eight 16-byte
// LDS reads at `addr` + j * STRIDE bytes, left in flight.  Written as asm
// because the compiler, unable to tell the two stage buffers apart, would
// otherwise wait for every copy into LDS still in flight before each read,
// the next offset's included; the asm also keeps it from waiting for the
// reads themselves before their registers are needed.
template <int STRIDE>
__device__ __forceinline__ void read_stage8(uint32_t addr, u32x4 (&v)[8]) {
  static_assert(7 * STRIDE < 65536, "ds_read offset range");
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:%9\n\t"
      "ds_read_b128 %2, %8 offset:%10\n\t"
      "ds_read_b128 %3, %8 offset:%11\n\t"
      "ds_read_b128 %4, %8 offset:%12\n\t"
      "ds_read_b128 %5, %8 offset:%13\n\t"
      "ds_read_b128 %6, %8 offset:%14\n\t"
      "ds_read_b128 %7, %8 offset:%15"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(addr), "i"(STRIDE), "i"(2 * STRIDE), "i"(3 * STRIDE), "i"(4 * STRIDE), "i"(5 * STRIDE),
        "i"(6 * STRIDE), "i"(7 * STRIDE)
      : "memory");
}

// Waits until at most N LDS (or scalar-memory) operations are in flight and
// only then releases v: the registers pass through the asm, so nothing that
// reads them can be scheduled before the wait.
template <int N>
__device__ __forceinline__ void wait_lgkm(u32x4 (&v)[8]) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
               : "i"(N)
               : "memory");
}

// s_waitcnt with only a vector-memory count (the other counters unconstrained).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

constexpr int kTaskBlocks = 8;  // 16-row blocks per task (two tiles)
constexpr int kTaskRows = 16 * kTaskBlocks;

template <int CIN, int NW>
struct WideShape {
  static constexpr int NCH = CIN / 32;            // 32-wide ci chunks
  static constexpr int NCB = 4;                   // 16-wide column blocks per wave
  static constexpr int BPW = kTaskBlocks / NW;    // blocks staged by each wave
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
  static constexpr int BLOCK_BYTES = 16 * SEG * 16;     // one staged 16-row block
  static constexpr int STAGE = kTaskBlocks * BLOCK_BYTES / 16;  // uint4 per B stage
  static size_t lds_bytes() { return static_cast<size_t>(2) * STAGE * sizeof(uint4); }
};

// Segment swizzle of staged row i: its 16-byte segment c sits at position
// c ^ seg_swizzle(i), so that the 16 rows a B-operand read touches at one
// segment fall on distinct LDS banks.
template <int SEG, int RP>
__device__ __forceinline__ int seg_swizzle(int i) {
  return (i / RP) & ((SEG < 16 ? SEG : 16) - 1);
}

// Per-offset state the pipeline carries: the offset, and for each of the two
// tiles its row mask and first list position (wave-uniform).
struct OffsetRef {
  int k;
  unsigned long long m0, m1;
  int lo0, lo1;
};

template <typename T, int CIN, int NW>
__global__ __launch_bounds__(64 * NW) void k_forward_wide(
    const uint16_t* __restrict__ feats_raw, const uint4* __restrict__ wop, T* __restrict__ out,
    const int32_t* __restrict__ in_idx, const int32_t* __restrict__ tile_off,
    const unsigned long long* __restrict__ tile_mask, const uint4* __restrict__ zero_row, int64_t n,
    int64_t tiles, int64_t tasks, int KV, int cout) {
  using Sh = WideShape<CIN, NW>;
  constexpr int NCH = Sh::NCH, NCB = Sh::NCB, BPW = Sh::BPW, STAGE = Sh::STAGE;
  constexpr int SEG = Sh::SEG, RPI = Sh::RPI, IPB = Sh::IPB, RP = Sh::RP, BLOCK_BYTES = Sh::BLOCK_BYTES;
  static_assert(STAGE * 2 * 16 == 2 * kTaskBlocks * BLOCK_BYTES, "stage size");
  extern __shared__ uint4 bstage[];  // [2][kTaskBlocks][NCH][64]
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  // Consecutive tasks on one XCD (workgroups are dealt to the 8 XCDs in turn),
  // so that tasks sharing neighbour rows share an L2.  The grid is a multiple
  // of 8 workgroups, which makes the remapping a permutation of [0, grid).
  const int64_t per_xcd = gridDim.x / 8;
  const int64_t bid = blockIdx.x;
  const int64_t task = (bid % 8) * per_xcd + bid / 8;
  if (task >= tasks) return;  // uniform over the workgroup
  const int64_t t0 = 2 * task, t1 = t0 + 1;
  const int64_t q0 = t0 * kTileRows;

  // Task metadata: lane k (and k - 64) holds offset k's masks and list starts.
  unsigned long long mA0 = 0ull, mA1 = 0ull, mB0 = 0ull, mB1 = 0ull;
  int lA0 = 0, lA1 = 0, lB0 = 0, lB1 = 0;
  if (lane < KV) {
    mA0 = tile_mask[static_cast<int64_t>(lane) * tiles + t0];
    lA0 = tile_off[static_cast<int64_t>(lane) * tiles + t0];
    if (t1 < tiles) {
      mA1 = tile_mask[static_cast<int64_t>(lane) * tiles + t1];
      lA1 = tile_off[static_cast<int64_t>(lane) * tiles + t1];
    }
  }
  if (lane + 64 < KV) {
    mB0 = tile_mask[static_cast<int64_t>(lane + 64) * tiles + t0];
    lB0 = tile_off[static_cast<int64_t>(lane + 64) * tiles + t0];
    if (t1 < tiles) {
      mB1 = tile_mask[static_cast<int64_t>(lane + 64) * tiles + t1];
      lB1 = tile_off[static_cast<int64_t>(lane + 64) * tiles + t1];
    }
  }
  unsigned long long todo0 = __ballot((mA0 | mA1) != 0ull), todo1 = __ballot((mB0 | mB1) != 0ull);
  auto next_ref = [&]() -> OffsetRef {
    OffsetRef o{-1, 0ull, 0ull, 0, 0};
    int k = -1;
    if (todo0) {
      k = __ffsll(static_cast<long long>(todo0)) - 1;
      todo0 &= todo0 - 1ull;
    } else if (todo1) {
      k = 64 + __ffsll(static_cast<long long>(todo1)) - 1;
      todo1 &= todo1 - 1ull;
    }
    if (k >= 0) {
      const int s = k & 63;
      o.k = k;
      o.m0 = lane_u64(k < 64 ? mA0 : mB0, s);
      o.m1 = lane_u64(k < 64 ? mA1 : mB1, s);
      o.lo0 = lane_i32(k < 64 ? lA0 : lB0, s);
      o.lo1 = lane_i32(k < 64 ? lA1 : lB1, s);
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
    const int32_t v = in_idx[has ? lo + rank : 0];  // the centre's list holds the row itself
    // An OR with the "no entry" mask rather than a select on the loaded
    // value: a select would let the compiler move the load under a branch
    // and wait for it there.
    idx[j] = v | (has ? 0 : -1);
  };
  //   Row copy j (< BPW x IPB): rows [RPI q, RPI q + RPI) of staged block
  //     jj (q = j % IPB, jj = j / IPB), whole rows, from global memory
  //     straight into B stage `buf`: lane l copies segment (l % SEG) ^ swizzle
  //     of row RPI q + l / SEG, whose input row is srow[j] (-1: a zero row).
  //     A block with no entry at the offset is skipped (its MFMAs are too).
  //     srow comes from copy_rows, which moves the index of row i from lane
  //     i of idx (a cross-lane read, done before the MFMAs start, where its
  //     wait costs nothing).
  auto copy_rows = [&](const int32_t (&idx)[BPW], int32_t (&srow)[Sh::LOADS_B]) {
#pragma unroll
    for (int j = 0; j < Sh::LOADS_B; ++j) srow[j] = __shfl(idx[j / IPB], RPI * (j % IPB) + lane / SEG);
    // Settle the cross-lane reads here: their results pass through an asm,
    // so the wait for them lands before the stage reads start instead of
    // between them (where it would also wait for those).
#pragma unroll
    for (int j = 0; j < Sh::LOADS_B; ++j) asm volatile("" : "+v"(srow[j]));
  };
  auto stage_b_one = [&](const OffsetRef& o, int buf, const int32_t (&srow)[Sh::LOADS_B], int j) {
    const int jj = j / IPB, q = j % IPB;
    const int b = wave + NW * jj;
    const unsigned long long m = (b < 4) ? o.m0 : o.m1;
    if (((m >> (16 * (b & 3))) & 0xffffull) == 0ull) return;  // wave-uniform
    const int i = RPI * q + lane / SEG;
    const int c = (lane % SEG) ^ seg_swizzle<SEG, RP>(i);
    const int32_t src_row = srow[j];
    const void* src = (src_row >= 0)
                          ? static_cast<const void*>(feats_raw + static_cast<int64_t>(src_row) * CIN + c * 8)
                          : static_cast<const void*>(zero_row + c);
    uint4* dst = bstage + ((buf * kTaskBlocks + b) * BLOCK_BYTES + q * RPI * SEG * 16) / 16;
    __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
  };
  //   Weight load j (< NCB x NCH): this wave's slice of W_k in operand order.
  const int ncbg = cout / 16;
  auto load_a_one = [&](const OffsetRef& o, uint4 (&a)[NCB][NCH], int j) {
    const int k = o.k < 0 ? 0 : o.k;
    const int cb = j / NCH, ch = j % NCH;
    a[cb][ch] = wop[((static_cast<int64_t>(k) * ncbg + NCB * wave + cb) * NCH + ch) * 64 + lane];
  };
  constexpr int A = Sh::LOADS_A, B = Sh::LOADS_B, I = Sh::LOADS_I;
  constexpr int kLoads = A + B + I;

  floatx4 acc[kTaskBlocks][NCB];
#pragma unroll
  for (int b = 0; b < kTaskBlocks; ++b)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[b][cb] = floatx4{0.f, 0.f, 0.f, 0.f};

  typedef __attribute__((address_space(3))) uint4 lds_uint4;
  const uint32_t stage_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_uint4*)bstage));
  // MFMAs of offset o from stage `buf` and weights a.  The loads of the next
  // offset (load(item), items 0 .. kLoads - 1: rows, weights, then the
  // indices of the offset after) are issued a few at a time between the
  // MFMA groups of the blocks, where they issue while the matrix core is
  // busy instead of stalling the wave before the offset starts.
  auto run = [&](const OffsetRef& o, int buf, const uint4 (&a)[NCB][NCH], auto&& load) {
    uint32_t pm = 0u;  // blocks with at least one entry
#pragma unroll
    for (int b = 0; b < kTaskBlocks; ++b) {
      const unsigned long long m = (b < 4) ? o.m0 : o.m1;
      if (((m >> (16 * (b & 3))) & 0xffffull) != 0ull) pm |= 1u << b;
    }
    pm = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(pm)));
    constexpr int kSlots = NCH * kTaskBlocks;
    // Chunk ch + 1's reads are in flight while chunk ch runs on MFMA; the
    // wait before a chunk's MFMAs leaves only the newer chunk's eight reads.
    // Lane (g, r) reads row r, segment 4 ch + g (swizzled) of each block.
    u32x4 bv[2][kTaskBlocks];
    const uint32_t base = stage_addr + static_cast<uint32_t>(buf * kTaskBlocks * BLOCK_BYTES + r * SEG * 16);
    const int swz = seg_swizzle<SEG, RP>(r);
    auto chunk_addr = [&](int ch) { return base + static_cast<uint32_t>(((4 * ch + g) ^ swz) * 16); };
    read_stage8<BLOCK_BYTES>(chunk_addr(0), bv[0]);
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      if (ch + 1 < NCH) {
        read_stage8<BLOCK_BYTES>(chunk_addr(ch + 1), bv[(ch + 1) & 1]);
        wait_lgkm<kTaskBlocks>(bv[ch & 1]);
      } else {
        wait_lgkm<0>(bv[ch & 1]);
      }
#pragma unroll
      for (int b = 0; b < kTaskBlocks; ++b) {
        if (pm & (1u << b)) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            acc[b][cb] = mfma<T>(a[cb][ch], __builtin_bit_cast(uint4, bv[ch & 1][b]), acc[b][cb]);
        }
        const int slot = ch * kTaskBlocks + b;
#pragma unroll
        for (int it = slot * kLoads / kSlots; it < (slot + 1) * kLoads / kSlots; ++it) load(it);
      }
    }
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
  for (int j = 0; j < B; ++j) stage_b_one(o0, 0, srow, j);

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
    run(o0, 0, ax, [&](int it) {
      if (it < B) stage_b_one(o1, 1, srow, it);
      else if (it < B + A) load_a_one(o1, ay, it - B);
      else load_idx_one(o2, ix0, it - B - A);
    });
    if (o1.k < 0) break;
    OffsetRef o3 = next_ref();
    // ---- offset o1: weights ay, stage 1; loads for o2 and the indices of o3
    wait_vm<0>();
    lds_barrier();
    copy_rows(ix0, srow);
    run(o1, 1, ay, [&](int it) {
      if (it < B) stage_b_one(o2, 0, srow, it);
      else if (it < B + A) load_a_one(o2, ax, it - B);
      else load_idx_one(o3, ix1, it - B - A);
    });
    if (o2.k < 0) break;
    o0 = o2;
    o1 = o3;
    o2 = next_ref();
  }
  wait_vm<0>();  // no copy into LDS may be left in flight at exit

  // Epilogue: D element (row 4 g + i, column r) of block (b, cb) is output
  // column 64 wave + 16 cb + 4 g + i of row q0 + 16 b + r.
#pragma unroll
  for (int b = 0; b < kTaskBlocks; ++b) {
    const int64_t q = q0 + 16 * b + r;
    if (q < n) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) store4<T>(out + q * cout + 64 * wave + 16 * cb + 4 * g, acc[b][cb]);
    }
  }
}

template <typename T, int CIN, int NW>
hipError_t launch_wide_shape(const ForwardArgs& a, const uint4* wop, const uint4* zero_row, hipStream_t stream) {
  using Sh = WideShape<CIN, NW>;
  const int64_t tasks = (a.tiles + 1) / 2;
  static bool raised = false;
  if (!raised) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_forward_wide<T, CIN, NW>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(Sh::lds_bytes()));
    if (e != hipSuccess) return e;
    raised = true;
  }
  const int64_t grid = (tasks + 7) / 8 * 8;
  hipLaunchKernelGGL((k_forward_wide<T, CIN, NW>), dim3(static_cast<unsigned>(grid)), dim3(64 * NW),
                     Sh::lds_bytes(), stream, static_cast<const uint16_t*>(a.feats), wop, static_cast<T*>(a.out),
                     a.in_idx, a.tile_off, a.tile_mask, zero_row, a.n, a.tiles, tasks, a.KV, a.cout);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_wide_typed(const ForwardArgs& a, const uint4* wop, const uint4* zero_row, hipStream_t stream) {
  const int nw = a.cout / 64;
  if (a.cin == 64) {
    if (nw == 1) return launch_wide_shape<T, 64, 1>(a, wop, zero_row, stream);
    if (nw == 2) return launch_wide_shape<T, 64, 2>(a, wop, zero_row, stream);
    return launch_wide_shape<T, 64, 4>(a, wop, zero_row, stream);
  }
  if (nw == 2) return launch_wide_shape<T, 128, 2>(a, wop, zero_row, stream);
  return launch_wide_shape<T, 128, 4>(a, wop, zero_row, stream);
}

}  // namespace

// Shapes whose per-offset load counts fit the 6-bit vector-memory counter
// and whose double-buffered weights fit the registers.
bool wide_supported(const ForwardArgs& a) {
  if (a.dtype != 1 && a.dtype != 2) return false;
  if (a.KV > 128) return false;
  if (a.cin == 64) return a.cout == 64 || a.cout == 128 || a.cout == 256;
  if (a.cin == 128) return a.cout == 128 || a.cout == 256;
  return false;
}

hipError_t launch_forward_wide(const ForwardArgs& a, const uint4* wop, const uint4* zero_row,
                               hipStream_t stream) {
  if (a.dtype == 1) return launch_wide_typed<_Float16>(a, wop, zero_row, stream);
  return launch_wide_typed<__bf16>(a, wop, zero_row, stream);
}

}  // namespace spconv
