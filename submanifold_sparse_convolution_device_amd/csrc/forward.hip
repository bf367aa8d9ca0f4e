// Fused forward of a submanifold sparse convolution on gfx950.
//
// Computes, for every output row Q,
//     f_out(Q) = sum over map entries (P, Q, W_d) of f_in(P) x W_d
// ("Sparse convolution for point clouds", section "The map and the update
// rule"; the whole layer as one loop over the map: "Sparse inputs and sparse
// convolution", section "The map is the computation").
//
// Dataflow.  The pages' GPU baseline runs gather -> matmul -> scatter as three
// launches per offset ("Sparse inputs and sparse convolution", section
// "Gather, matmul, scatter"), re-reading a shared feature row once per offset
// and leaving the phases unoverlapped ("TorchSparse: regular computation from
// irregular sparsity", sections "Why this wastes most of the GPU" and
// "TorchSparse++: overlap memory with computation").  Here one launch is
// output-stationary: a workgroup owns a tile of 64 output rows and a block of
// CB output channels, walks the offsets that occur in the tile, and keeps the
// partial sums in MFMA accumulators; each output row is written once, with no
// atomics.
//   * Centre offset: the identity map, so the tile's own rows are read
//     directly (a plain dense GEMM, no index list).
//   * Other offsets: the tile's entries are a contiguous range of each
//     offset's list (lists are grouped by offset and ordered by output row),
//     located through tile_off; they are staged once per tile into an LDS
//     row -> input-row table, and each wave gathers its 16 rows' inputs by
//     index straight into MFMA operand registers (16 bytes per lane).
//   * W_d is staged into LDS transposed ([co][ci]) so that a lane's MFMA
//     operand is one 16-byte LDS read.
// MFMA formulation: D[co][q] += W^T[co][ci] * F^T[ci][q], with
// v_mfma_f32_16x16x32_{f16,bf16} (fp32 accumulate) for half types and
// v_mfma_f32_16x16x4_f32 for fp32.  For the A (16 x K) and B (K x 16)
// operands, lane l supplies row / column (l mod 16) and a k-slice selected by
// l / 16; the same slice is used for both operands, so the sum over ci is
// exact regardless of how the hardware orders k within a slice.  D element
// (row 4 (l / 16) + i, column l mod 16) sits in accumulator i of lane l.
#include "internal.h"

#include <cstdlib>

namespace spconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int kOffsetsPerStage = 32;  // offsets whose index tables share one LDS stage
constexpr int kThreads = 256;

// Round to nearest even, fp32 -> bf16 bits (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int kVec = 4;     // elements per 16-byte load
  static constexpr int kChunk = 16;  // ci per step: 4 lane groups x 4
  static constexpr int kPad = 4;     // LDS row padding (elements)
  __device__ static void store4(float* dst, floatx4 v) { *reinterpret_cast<floatx4*>(dst) = v; }
};
template <>
struct Elem<_Float16> {
  static constexpr int kVec = 8;
  static constexpr int kChunk = 32;  // one 16x16x32 MFMA: 4 lane groups x 8
  static constexpr int kPad = 8;
  __device__ static u16x4 pack4(floatx4 v) {
    u16x4 o;
    for (int i = 0; i < 4; ++i) {
      const _Float16 h = static_cast<_Float16>(v[i]);  // v_cvt_f16_f32: round to nearest even
      o[i] = __builtin_bit_cast(uint16_t, h);
    }
    return o;
  }
  __device__ static void store4(_Float16* dst, floatx4 v) { *reinterpret_cast<u16x4*>(dst) = pack4(v); }
};
template <>
struct Elem<__bf16> {
  static constexpr int kVec = 8;
  static constexpr int kChunk = 32;
  static constexpr int kPad = 8;
  __device__ static u16x4 pack4(floatx4 v) {
    u16x4 o;
    for (int i = 0; i < 4; ++i) o[i] = bf16_bits_rne(v[i]);
    return o;
  }
  __device__ static void store4(__bf16* dst, floatx4 v) { *reinterpret_cast<u16x4*>(dst) = pack4(v); }
};

// One ci-chunk of MFMA work for NCB co-blocks.  b_src is the lane's gathered
// feature slice (read only when b_ok: the row exists and the slice is inside
// c_in), wt_row the lane's transposed-weight slice in LDS for co-block 0
// (read only when a_ok), advanced by 16 rows per co-block.  Every lane of the
// wave takes part in every MFMA; lanes without data supply zeros.
template <typename T, int NCB>
struct Step;

template <int NCB>
struct Step<_Float16, NCB> {
  __device__ static void run(floatx4 (&acc)[NCB], const _Float16* b_src, bool b_ok,
                             const _Float16* wt_row, bool a_ok, int wt_block_stride) {
    half8 b = {};
    if (b_ok) b = *reinterpret_cast<const half8*>(b_src);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      half8 a = {};
      if (a_ok) a = *reinterpret_cast<const half8*>(wt_row + cb * wt_block_stride);
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[cb], 0, 0, 0);
    }
  }
};

template <int NCB>
struct Step<__bf16, NCB> {
  __device__ static void run(floatx4 (&acc)[NCB], const __bf16* b_src, bool b_ok,
                             const __bf16* wt_row, bool a_ok, int wt_block_stride) {
    bf16x8 b = {};
    if (b_ok) b = *reinterpret_cast<const bf16x8*>(b_src);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      bf16x8 a = {};
      if (a_ok) a = *reinterpret_cast<const bf16x8*>(wt_row + cb * wt_block_stride);
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[cb], 0, 0, 0);
    }
  }
};

template <int NCB>
struct Step<float, NCB> {
  __device__ static void run(floatx4 (&acc)[NCB], const float* b_src, bool b_ok,
                             const float* wt_row, bool a_ok, int wt_block_stride) {
    floatx4 b = {};
    if (b_ok) b = *reinterpret_cast<const floatx4*>(b_src);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      floatx4 a = {};
      if (a_ok) a = *reinterpret_cast<const floatx4*>(wt_row + cb * wt_block_stride);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc[cb], 0, 0, 0);
      }
    }
  }
};

template <typename T, int CB>
__global__ __launch_bounds__(kThreads) void k_forward(
    const T* __restrict__ feats, const T* __restrict__ weights, T* __restrict__ out,
    const int32_t* __restrict__ in_idx, const unsigned long long* __restrict__ tile_mask,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ perm, int64_t n, int64_t tiles, int KV,
    int cin, int cout, int centre) {
  constexpr int NCB = CB / 16;
  constexpr int VEC = Elem<T>::kVec;
  constexpr int CHUNK = Elem<T>::kChunk;
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* nbr_lds = reinterpret_cast<int32_t*>(smem);            // [kOffsetsPerStage][64]
  int32_t* lo_lds = nbr_lds + kOffsetsPerStage * kTileRows;       // [kOffsetsPerStage]
  int32_t* hi_lds = lo_lds + kOffsetsPerStage;                    // [kOffsetsPerStage]
  T* wt = reinterpret_cast<T*>(hi_lds + kOffsetsPerStage);        // [CB][ldw], 16-byte aligned
  const int ldw = cin + Elem<T>::kPad;

  const int64_t tile = blockIdx.x;
  const int co0 = blockIdx.y * CB;
  const int64_t q0 = tile * kTileRows;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  // centre: the offset whose list is the identity (read by position), or -1
  // for maps without one (strided and transposed maps).
  const int row_in_tile = wave * 16 + r;
  const int64_t q = q0 + row_in_tile;  // position in the map's row order
  const int32_t qrow = q < n ? (perm != nullptr ? perm[q] : static_cast<int32_t>(q)) : -1;  // its row

  floatx4 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < KV; kb += kOffsetsPerStage) {
    const int kn = (KV - kb < kOffsetsPerStage) ? KV - kb : kOffsetsPerStage;
    __syncthreads();  // previous stage's LDS readers are done
    for (int i = tid; i < kn; i += kThreads) {
      const int64_t base = static_cast<int64_t>(kb + i) * tiles + tile;
      lo_lds[i] = tile_off[base];
      hi_lds[i] = tile_off[base + 1];
    }
    for (int i = tid; i < kn * kTileRows; i += kThreads) nbr_lds[i] = -1;
    __syncthreads();
    // position -> input-row table of this tile for the stage's offsets: the
    // tile's entries at offset k follow its row mask, one per set bit
    for (int i = 0; i < kn; ++i) {
      if (kb + i == centre) continue;
      const int lo = lo_lds[i];
      if (lo == hi_lds[i]) continue;
      const unsigned long long m = tile_mask[static_cast<int64_t>(kb + i) * tiles + tile];
      for (int row = tid; row < kTileRows; row += kThreads) {
        if ((m >> row) & 1ull) {
          const unsigned long long lower = row == 0 ? 0ull : (m & (~0ull >> (64 - row)));
          nbr_lds[i * kTileRows + row] = in_idx[lo + __popcll(lower)];
        }
      }
    }
    for (int i = 0; i < kn; ++i) {
      const int k = kb + i;
      if (lo_lds[i] == hi_lds[i]) continue;  // no entry of offset k in this tile
      __syncthreads();  // table writes visible; previous offset's weight readers done
      // Stage W_k[:, co0 : co0 + CB] transposed into wt[co][ci].
      const T* wk = weights + static_cast<int64_t>(k) * cin * cout;
      constexpr int VPR = CB / VEC;  // 16-byte vectors per ci row of the block
      for (int v = tid; v < cin * VPR; v += kThreads) {
        const int ci = v / VPR;
        const int cv = (v - ci * VPR) * VEC;
        const int co = co0 + cv;
        T vals[VEC];
        if (co < cout) {
          const uint4 raw = *reinterpret_cast<const uint4*>(wk + static_cast<int64_t>(ci) * cout + co);
          __builtin_memcpy(vals, &raw, sizeof(raw));
        } else {
#pragma unroll
          for (int j = 0; j < VEC; ++j) vals[j] = static_cast<T>(0.0f);
        }
#pragma unroll
        for (int j = 0; j < VEC; ++j) wt[(cv + j) * ldw + ci] = vals[j];
      }
      __syncthreads();
      const int32_t src = (k == centre) ? qrow : nbr_lds[i * kTileRows + row_in_tile];
      if (__ballot(src >= 0) == 0ull) continue;  // none of this wave's 16 rows uses offset k
      const T* frow = feats + static_cast<int64_t>(src < 0 ? 0 : src) * cin;
      const T* wrow = wt + r * ldw;
      // The offset's products are summed on their own and added to the
      // row's total once: fp32 rounding then runs along chains of C_in / 4
      // MFMA steps and of one addition per offset, not along all of them
      // (at C_in = 512 that keeps fp32 within 1e-5 of the output's RMS).
      floatx4 part[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) part[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
      for (int c = 0; c < cin; c += CHUNK) {
        const int cc = c + g * (CHUNK / 4);
        const bool inside = cc < cin;
        const int ccs = inside ? cc : 0;
        Step<T, NCB>::run(part, frow + ccs, inside && src >= 0, wrow + ccs, inside, 16 * ldw);
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] += part[cb];
    }
  }

  // Epilogue: fp32 -> dtype, each output row written once.
  if (q < n) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int co = co0 + cb * 16 + 4 * g;
      if (co < cout) Elem<T>::store4(out + static_cast<int64_t>(qrow) * cout + co, acc[cb]);
    }
  }
}

// ---------------------------------------------------------------------------
// Small-channel kernel: every W_d fits in LDS at once.
//
// A workgroup stages all K^3 weight matrices into LDS once, already in MFMA
// operand order (per offset, co-block and ci-chunk, 64 lanes x 16 bytes), so
// a lane's A operand is one 16-byte read.  Each wave then owns one 64-row
// output tile at a time, independently of the other waves:
//   1. lanes k < K^3 read the tile's row mask and list start for offset k
//      (written by the map build); the tile's own rows are loaded straight
//      into B-operand registers and the centre offset runs on them as a dense
//      GEMM;
//   2. the tile's non-centre entries are numbered in offset order (a wave
//      prefix sum of the mask popcounts).  Entry s of offset k sits at list
//      position tile_off[k] + s - base_k, so a lane finds the input row of a
//      stage slot with one index load, then loads that whole row; the
//      stage's rows go to the wave's LDS stage in one burst;
//   3. per offset present in the tile, per 16-row block that uses it, one
//      MFMA per (co-block, ci-chunk) with B read from the stage (zero for
//      rows without that neighbour);
//   4. the accumulators are rounded to the output dtype and each output row is
//      written once.
// A tile with more entries than the stage holds is processed in slot ranges
// of kStageEntries; an entry belongs to exactly one range, and the rows of
// the next range are in flight while the current one runs on MFMA.
// ---------------------------------------------------------------------------
constexpr int kSmallWaves = 12;    // most waves per workgroup
constexpr int kSpares = 2;         // spare waves that take halves of heavy tiles
constexpr int kSplitMin = 64;      // fewest entries of a tile whose upper half a spare takes
static_assert(kSplitMin > 0, "a shared tile's owner must fill its stage");
constexpr int kStageRounds = 2;    // 64-slot rounds per stage
constexpr int kStageEntries = 64 * kStageRounds;  // plus one zero row per wave
static_assert(kStageEntries == kTileSlots, "a whole-tile stage is the tile's slot table");
constexpr size_t kSmallLdsCap = 160 * 1024;  // one workgroup per CU

template <typename T, int CIN, int COUT>
struct SmallShape {
  static constexpr int CHUNK = Elem<T>::kChunk;
  static constexpr int VEC = Elem<T>::kVec;
  static constexpr int NCH = CIN / CHUNK;
  static constexpr int NCB = COUT / 16;
  static constexpr int ROWV = CIN * static_cast<int>(sizeof(T)) / 16;  // 16-byte vectors per row
  static_assert(CIN % CHUNK == 0 && COUT % 16 == 0, "shape");
  static size_t wbytes(int KV) { return static_cast<size_t>(KV) * NCB * NCH * 64 * 16; }
  static size_t stage_bytes() { return static_cast<size_t>(ROWV) * (kStageEntries + 1) * 16; }
  // Weights, one stage per wave, then three ints per wave for splitting
  // tiles (tile, weight, stage-ready flag).
  static size_t lds_bytes(int KV, int waves) {
    return wbytes(KV) + static_cast<size_t>(waves) * stage_bytes() + 16 * ((kSmallWaves * 12 + 15) / 16);
  }
};

template <typename T, int NCB>
__device__ __forceinline__ void mfma_block(floatx4 (&acc)[NCB], const uint4 (&a)[NCB], uint4 b) {
  if constexpr (sizeof(T) == 4) {
    const floatx4 bv = __builtin_bit_cast(floatx4, b);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const floatx4 av = __builtin_bit_cast(floatx4, a[cb]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bv[j], acc[cb], 0, 0, 0);
    }
  } else if constexpr (__is_same(T, _Float16)) {
    const half8 bv = __builtin_bit_cast(half8, b);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a[cb]), bv, acc[cb], 0, 0, 0);
    }
  } else {
    const bf16x8 bv = __builtin_bit_cast(bf16x8, b);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[cb]), bv, acc[cb], 0, 0, 0);
    }
  }
}

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lane_i32(int v, int src) { return __builtin_amdgcn_readlane(v, src); }
__device__ __forceinline__ unsigned long long lane_u64(unsigned long long v, int src) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), src));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), src));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// Position of lane l's 16-byte operand inside a 64-lane operand block in LDS.
// The XOR spreads the eight 16-byte writes that eight consecutive threads make
// together while staging (slots 8m + j, m = 0..7) over all banks; reads by
// lanes 8m..8m+7 stay one contiguous 128-byte row.
__device__ __forceinline__ int operand_slot(int l) { return l ^ ((l >> 3) & 7); }

// Stages every W_d into operand order: element i of lane (g, r) of block
// (k, cb, ch) is W[k][ch * CHUNK + g * VEC + i][cb * 16 + r].  Each thread
// reads VEC x VEC blocks (VEC rows of ci, VEC columns of co, 16 bytes per
// row), transposes them in registers, and writes VEC 16-byte operand vectors.
// The first block of a thread is split into a load (weight_block_load) and a
// store (weight_block_store) so that the caller can overlap its latency.
template <typename T, int CIN, int COUT>
struct WeightBlock {
  static constexpr int VEC = Elem<T>::kVec;
  uint4 rows[VEC];
  int b;
};

template <typename T, int CIN, int COUT>
__device__ __forceinline__ void weight_block_load(WeightBlock<T, CIN, COUT>& wb, const T* __restrict__ weights,
                                                  int b, int nblk) {
  constexpr int VEC = Elem<T>::kVec, RB = CIN / VEC, CBK = COUT / VEC;
  wb.b = b;
  if (b >= nblk) return;
  const int k = b / (RB * CBK);
  const int rem = b - k * RB * CBK;
  const int ci0 = (rem / CBK) * VEC, co0 = (rem % CBK) * VEC;
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    wb.rows[i] = *reinterpret_cast<const uint4*>(weights + (static_cast<int64_t>(k) * CIN + ci0 + i) * COUT + co0);
  }
}

template <typename T, int CIN, int COUT>
__device__ __forceinline__ void weight_block_store(const WeightBlock<T, CIN, COUT>& wb, uint4* wl, int nblk) {
  using Sh = SmallShape<T, CIN, COUT>;
  constexpr int CHUNK = Sh::CHUNK, VEC = Sh::VEC, NCH = Sh::NCH, NCB = Sh::NCB;
  constexpr int RB = CIN / VEC, CBK = COUT / VEC;
  if (wb.b >= nblk) return;
  const int k = wb.b / (RB * CBK);
  const int rem = wb.b - k * RB * CBK;
  const int ci0 = (rem / CBK) * VEC, co0 = (rem % CBK) * VEC;
  T blk[VEC][VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) __builtin_memcpy(blk[i], &wb.rows[i], sizeof(uint4));
  const int ch = ci0 / CHUNK, g = (ci0 % CHUNK) / VEC;
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    T col[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) col[i] = blk[i][j];
    const int co = co0 + j;
    const size_t slot = ((static_cast<size_t>(k) * NCB + (co >> 4)) * NCH + ch) * 64 + operand_slot(g * 16 + (co & 15));
    uint4 v;
    __builtin_memcpy(&v, col, sizeof(v));
    wl[slot] = v;
  }
}

// Per-wave state of one tile: offset k's row mask, list start and first
// stage slot live in lane k.
struct TileMeta {
  unsigned long long mk;
  int lok;
  int basek;
  int total;
};

// The rows [row_lo, row_hi) of a tile's metadata (whole = [0, 64)): the
// masks keep those rows' bits and list starts move past the rows before.
__device__ __forceinline__ TileMeta window_meta(unsigned long long mk, int lok, int row_lo, int row_hi, int KV,
                                                int centre, int lane) {
  TileMeta tm;
  const unsigned long long below = row_lo == 0 ? 0ull : (~0ull >> (64 - row_lo));
  const unsigned long long upto = row_hi == 64 ? ~0ull : (~0ull >> (64 - row_hi));
  tm.mk = mk & upto & ~below;
  tm.lok = lok + static_cast<int>(__popcll(mk & below));
  const int cnt = (lane < KV && lane != centre) ? __popcll(tm.mk) : 0;
  tm.basek = wave_prefix_small<7>(cnt);
  tm.total = lane_i32(tm.basek + cnt, 63);
  return tm;
}

// Lane k < KV loads offset k's row mask and list start of tile t.
__device__ __forceinline__ void load_meta(const unsigned long long* __restrict__ tile_mask,
                                          const int32_t* __restrict__ tile_off, int64_t t, int64_t tiles, int KV,
                                          int lane, unsigned long long& mk, int& lok) {
  mk = 0ull;
  lok = 0;
  if (lane < KV) {
    mk = tile_mask[static_cast<int64_t>(lane) * tiles + t];
    lok = tile_off[static_cast<int64_t>(lane) * tiles + t];
  }
}

template <typename T, int CIN>
__device__ __forceinline__ TileMeta tile_meta(const unsigned long long* __restrict__ tile_mask,
                                              const int32_t* __restrict__ tile_off, int64_t t,
                                              int64_t tiles, int KV, int centre, int lane) {
  unsigned long long mk;
  int lok;
  load_meta(tile_mask, tile_off, t, tiles, KV, lane, mk, lok);
  return window_meta(mk, lok, 0, kTileRows, KV, centre, lane);
}

// Stage layout of a wave: chunk-major, stage[v * kStageStride + slot] is the
// 16-byte chunk v of the row in stage slot `slot`; slot kStageEntries is a
// zero row.  Consecutive slots are consecutive 16-byte words, so lanes reading
// one chunk of consecutive slots hit distinct banks.
constexpr int kStageStride = kStageEntries + 1;

// List positions of stage slots s0 + lane + 64 rd.  Entries are numbered in
// offset order: offset k's entries of this tile are slots [base_k, base_k +
// cnt_k) and list positions [tile_off_k, tile_off_k + cnt_k), both in output
// row order.  Slots past the tile's entries get position 0 (a valid entry; its
// row lands in a stage slot nothing reads).
__device__ __forceinline__ void stage_positions(const TileMeta& tm, int cntk, int s0, int lane,
                                                int (&pos)[kStageRounds]) {
#pragma unroll
  for (int rd = 0; rd < kStageRounds; ++rd) pos[rd] = 0;
  unsigned long long todo = __ballot(cntk > 0 && tm.basek < s0 + kStageEntries && tm.basek + cntk > s0);
  while (todo) {
    const int k = __ffsll(static_cast<long long>(todo)) - 1;
    todo &= todo - 1ull;
    const int base = lane_i32(tm.basek, k), c = lane_i32(cntk, k), lo = lane_i32(tm.lok, k);
#pragma unroll
    for (int rd = 0; rd < kStageRounds; ++rd) {
      const int e = s0 + lane + 64 * rd - base;
      if (e >= 0 && e < c) pos[rd] = lo + e;
    }
  }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Rows of one stage in flight (native vectors, so they stay in registers
// across the MFMA loop that overlaps their loads).
template <int ROWV>
struct StageRows {
  u32x4 v[kStageRounds][ROWV];
};

// Input rows of the slots whose list positions are idx_pos (all loads issued
// before any is used).
template <typename T, int CIN>
__device__ __forceinline__ void load_stage_rows(const T* __restrict__ feats, const int32_t* __restrict__ in_idx,
                                                const int (&pos)[kStageRounds],
                                                StageRows<CIN * static_cast<int>(sizeof(T)) / 16>& rows) {
  constexpr int ROWV = CIN * static_cast<int>(sizeof(T)) / 16;
  int32_t src[kStageRounds];
#pragma unroll
  for (int rd = 0; rd < kStageRounds; ++rd) src[rd] = in_idx[pos[rd]];
#pragma unroll
  for (int rd = 0; rd < kStageRounds; ++rd) {
    const u32x4* rowp = reinterpret_cast<const u32x4*>(feats + static_cast<int64_t>(src[rd]) * CIN);
#pragma unroll
    for (int v = 0; v < ROWV; ++v) rows.v[rd][v] = rowp[v];
  }
}

// Input rows of stage slots lane + 64 rd, read from the tile's slot table
// (srow, loaded with the tile's masks); slots at or past `total` load row 0,
// a valid row that nothing reads.
template <typename T, int CIN>
__device__ __forceinline__ void load_slot_rows(const T* __restrict__ feats, const int32_t (&srow)[kStageRounds],
                                               int total, int lane,
                                               StageRows<CIN * static_cast<int>(sizeof(T)) / 16>& rows) {
  constexpr int ROWV = CIN * static_cast<int>(sizeof(T)) / 16;
#pragma unroll
  for (int rd = 0; rd < kStageRounds; ++rd) {
    const int32_t src = lane + 64 * rd < total ? srow[rd] : 0;
    const u32x4* rowp = reinterpret_cast<const u32x4*>(feats + static_cast<int64_t>(src) * CIN);
#pragma unroll
    for (int v = 0; v < ROWV; ++v) rows.v[rd][v] = rowp[v];
  }
}

template <int ROWV>
__device__ __forceinline__ void commit_stage(uint4* stage, const StageRows<ROWV>& rows, int lane) {
#pragma unroll
  for (int rd = 0; rd < kStageRounds; ++rd)
#pragma unroll
    for (int v = 0; v < ROWV; ++v) *reinterpret_cast<u32x4*>(stage + v * kStageStride + lane + 64 * rd) = rows.v[rd][v];
}

// One unit of MFMA work: the rows of a pair of 16-row blocks (32 rows) that
// have a neighbour at offset k, with at least one of them in the current
// stage range.  All fields are wave-uniform.  lo is the stage slot of the
// pair's first entry at k relative to the range start; sub has bit i set when
// row i of the pair has that neighbour.  k < 0 marks the end of a walk.  One
// read of W_k serves both blocks: a pair of blocks has 40% fewer items than
// its blocks one by one on the indoor scene.
struct Item {
  int k;
  int lo;
  uint32_t sub;
};

// A operands (W_k for every co-block) and the B operands of one item's two
// blocks.  A lane whose row has no entry in range reads the stage's zero row.
// An item with k < 0 reads offset 0 and the zero row (a harmless read that
// keeps the LDS wait counts the same on every path).
template <int NCH, int NCB>
struct ItemOps {
  uint4 a[NCH][NCB];
  uint4 b[2][NCH];
};

template <typename T, int CIN, int COUT>
__device__ __forceinline__ void load_item(ItemOps<CIN / Elem<T>::kChunk, COUT / 16>& op, const uint4* wl,
                                          const uint4* stage_g, const Item& it, int lim, int r,
                                          uint32_t below_r, int aslot) {
  constexpr int NCH = CIN / Elem<T>::kChunk, NCB = COUT / 16;
  const int k = it.k < 0 ? 0 : it.k;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) op.a[ch][cb] = wl[((static_cast<size_t>(k) * NCB + cb) * NCH + ch) * 64 + aslot];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // row r of block h: its slot follows the pair's entries at k in the rows before it
    const uint32_t before = h == 0 ? below_r : (0xffffu | (below_r << 16));
    const int ls0 = it.lo + __popc(it.sub & before);
    const bool has = ((it.sub >> (16 * h + r)) & 1u) && static_cast<unsigned>(ls0) < static_cast<unsigned>(lim);
    const int ls = has ? ls0 : kStageEntries;  // the zero row
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) op.b[h][ch] = stage_g[ch * 4 * kStageStride + ls];
  }
}

template <typename T, int NCH, int NCB>
__device__ __forceinline__ void run_item(floatx4 (&acc0)[NCB], floatx4 (&acc1)[NCB], const ItemOps<NCH, NCB>& op) {
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    mfma_block<T, NCB>(acc0, op.a[ch], op.b[0][ch]);
    mfma_block<T, NCB>(acc1, op.a[ch], op.b[1][ch]);
  }
}

// Next item of a block pair: the lowest offset left in todo (K^3 <= 32 here,
// so one 32-bit word holds the offsets).  lov and subv hold, in lane k, offset
// k's first slot for the pair (relative to the range start) and the pair's
// 32-bit row mask.
__device__ __forceinline__ Item next_item(uint32_t& todo, int lov, int subv) {
  if (todo == 0u) return Item{-1, 0, 0u};
  const int k = __builtin_ctz(todo);
  todo &= todo - 1u;
  return Item{k, lane_i32(lov, k), static_cast<uint32_t>(lane_i32(subv, k))};
}

template <typename T, int CIN, int COUT>
__global__ __launch_bounds__(kSmallWaves * 64) void k_forward_small(
    const T* __restrict__ feats, const T* __restrict__ weights, T* __restrict__ out,
    const int32_t* __restrict__ in_idx, const int32_t* __restrict__ tile_off,
    const unsigned long long* __restrict__ tile_mask, const int32_t* __restrict__ tile_rows,
    const int32_t* __restrict__ perm, int64_t n, int64_t tiles, int KV, int tw, int spin_limit) {
  using Sh = SmallShape<T, CIN, COUT>;
  constexpr int CHUNK = Sh::CHUNK, VEC = Sh::VEC, NCH = Sh::NCH, NCB = Sh::NCB, ROWV = Sh::ROWV;
  extern __shared__ uint4 smem4[];
  uint4* wl = smem4;  // [KV][NCB][NCH][64] A operands
  const int nw = static_cast<int>(blockDim.x >> 6);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int aslot = operand_slot(lane);
  const uint32_t below_r = (1u << r) - 1u;
  uint4* stage = wl + static_cast<size_t>(KV) * NCB * NCH * 64 + static_cast<size_t>(wave) * ROWV * kStageStride;
  const uint4* stage_g = stage + g * kStageStride;  // this lane's chunk (of ci-chunk 0) of the stage it reads
  const int centre = (KV - 1) / 2;
  if (lane < ROWV) stage[lane * kStageStride + kStageEntries] = make_uint4(0u, 0u, 0u, 0u);  // zero row

  // The weight loads of this thread's first block and the first tile's index
  // and row gathers are independent: issue both before waiting on either.
  constexpr int kRB = CIN / VEC, kCBK = COUT / VEC;
  const int nblk = KV * kRB * kCBK;
  WeightBlock<T, CIN, COUT> wb;
  weight_block_load<T, CIN, COUT>(wb, weights, tid, nblk);
  // Waves [0, tw) own tiles; the others are spares, which take the rows
  // [32, 64) of the workgroup's heaviest tiles, so that those end with the
  // rest.  A tile with more entries than one stage holds splits first (each
  // half then gathers its own entries instead of the tile taking a second
  // gather round); a lighter one (at least kSplitMin entries, and only when
  // its owner has no later tile) is shared: the spare computes its upper
  // half from the owner's stage once the owner flags it filled.  That wait is
  // bounded (spin_limit sleeps): a spare still waiting then gathers its half
  // tile itself, as for a heavy tile, so no wave's progress rests on another's.
  int* s_tile = reinterpret_cast<int*>(wl + static_cast<size_t>(KV) * NCB * NCH * 64 +
                                       static_cast<size_t>(nw) * ROWV * kStageStride);
  int* s_weight = s_tile + kSmallWaves;
  int* s_ready = s_weight + kSmallWaves;
  const bool spare = wave >= tw;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * tw;
  // Workgroups are dealt to the 8 XCDs in turn (b mod 8); each XCD takes a
  // contiguous eighth of the round's tiles, so neighbouring rows stay in one
  // L2, and inside it wave w of its j-th workgroup takes tile w G8 + j
  // (G8 = G / 8, the grid is a multiple of 8): dense regions, whose tiles
  // are heavy, spread over the XCD's workgroups.  Measured on the indoor
  // scene: 16.9 us against 19.8 us for consecutive tiles per workgroup.
  const int64_t g8 = gridDim.x / 8;
  int64_t t = spare ? tiles
                    : static_cast<int64_t>(blockIdx.x % 8) * g8 * tw + static_cast<int64_t>(wave) * g8 +
                          blockIdx.x / 8;
  int row_lo = 0, row_hi = kTileRows;  // rows of the tile this wave computes
  unsigned long long mk_full = 0ull;
  int lok_full = 0;
  bool deferred = false;  // first-round loads wait for the split decision
  bool publish = false;   // an owner whose stage a spare also reads
  int shared_from = -1;   // a spare: the owner wave whose stage it reads
  TileMeta tm{0ull, 0, 0, 0};
  int cntk = 0;
  StageRows<ROWV> rows;
  int pos_next[kStageRounds];
  uint4 bc[4][NCH];  // the tile's own rows (centre offset)
  auto load_centre = [&](int64_t q0) {
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int64_t q = q0 + qb * 16 + r;  // position; its row through perm
      const int64_t qp = q < n ? q : n - 1;
      const int64_t qs = perm != nullptr ? static_cast<int64_t>(perm[qp]) : qp;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        bc[qb][ch] = *reinterpret_cast<const uint4*>(feats + qs * CIN + ch * CHUNK + g * VEC);
        if (q >= n) bc[qb][ch] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  // A whole tile's first stage comes from its slot table, loaded with its
  // masks (the list positions of its entries are not needed).
  int32_t srow[kStageRounds];
  auto load_slots = [&](int64_t tt) {
#pragma unroll
    for (int rd = 0; rd < kStageRounds; ++rd) srow[rd] = tile_rows[tt * kTileSlots + lane + 64 * rd];
  };
  auto issue_slots = [&]() {
    cntk = (lane < KV && lane != centre) ? __popcll(tm.mk) : 0;
    if (tm.total > 0) load_slot_rows<T, CIN>(feats, srow, tm.total, lane, rows);
  };
  auto issue_first = [&]() {
    cntk = (lane < KV && lane != centre) ? __popcll(tm.mk) : 0;
    if (tm.total > 0) {
      int pos[kStageRounds];
      stage_positions(tm, cntk, 0, lane, pos);
      load_stage_rows<T, CIN>(feats, in_idx, pos, rows);
    }
  };
  if (t < tiles) {
    load_centre(t * kTileRows);
    load_meta(tile_mask, tile_off, t, tiles, KV, lane, mk_full, lok_full);
    load_slots(t);
    tm = window_meta(mk_full, lok_full, 0, kTileRows, KV, centre, lane);
    deferred = tm.total > kStageEntries && tw < nw;
    if (!deferred) issue_slots();
  }
  if (!spare && lane == 0) {
    int weight = -1;
    if (t < tiles && (deferred || (tm.total >= kSplitMin && t + nwaves >= tiles))) weight = tm.total;
    s_tile[wave] = static_cast<int>(t);
    s_weight[wave] = weight;
    s_ready[wave] = -1;
  }
  weight_block_store<T, CIN, COUT>(wb, wl, nblk);
  for (int b = tid + blockDim.x; b < nblk; b += blockDim.x) {
    weight_block_load<T, CIN, COUT>(wb, weights, b, nblk);
    weight_block_store<T, CIN, COUT>(wb, wl, nblk);
  }
  __syncthreads();
  if (tw < nw) {
    // Split candidates by weight (ties by wave): the i-th goes to spare i.
    const int wv = lane < tw ? s_weight[lane] : -1;
    int rank = 0;
    for (int u = 0; u < tw; ++u) {
      const int wu = lane_i32(wv, u);
      rank += (wu > wv || (wu == wv && u < lane)) ? 1 : 0;
    }
    const bool split = wv >= 0 && rank < nw - tw;
    const unsigned long long splits = __ballot(split);
    if (spare) {
      const unsigned long long mine = __ballot(split && rank == wave - tw);
      if (mine != 0ull) {
        const int w = __ffsll(static_cast<long long>(mine)) - 1;
        t = s_tile[w];
        row_lo = kTileRows / 2;
        load_centre(t * kTileRows);
        load_meta(tile_mask, tile_off, t, tiles, KV, lane, mk_full, lok_full);
        if (s_weight[w] > kStageEntries) {
          tm = window_meta(mk_full, lok_full, row_lo, row_hi, KV, centre, lane);
          issue_first();
        } else {
          // the owner's slot numbering, restricted to rows [32, 64): offset
          // k's first slot moves past its entries in rows [0, 32)
          tm = window_meta(mk_full, lok_full, 0, kTileRows, KV, centre, lane);
          tm.basek += static_cast<int>(__popcll(tm.mk & (~0ull >> (kTileRows / 2))));
          tm.mk &= ~0ull << (kTileRows / 2);
          shared_from = w;
          stage_g = wl + static_cast<size_t>(KV) * NCB * NCH * 64 + static_cast<size_t>(w) * ROWV * kStageStride +
                    g * kStageStride;
        }
      } else {
        t = tiles;
      }
    } else if ((splits >> wave) & 1ull) {
      row_hi = kTileRows / 2;
      if (deferred) {
        tm = window_meta(mk_full, lok_full, row_lo, row_hi, KV, centre, lane);
        issue_first();
      } else {
        tm.mk &= ~0ull >> (kTileRows / 2);  // rows [0, 32), same slots
        publish = true;
      }
    } else if (deferred) {
      issue_slots();
    }
  }

  bool first = true;
  for (; t < tiles; t += nwaves) {
    const int64_t q0 = t * kTileRows;
    if (!first) {
      if (spare) break;  // a spare computes one half tile
      row_lo = 0;
      row_hi = kTileRows;
      load_centre(q0);
      load_slots(t);
      tm = tile_meta<T, CIN>(tile_mask, tile_off, t, tiles, KV, centre, lane);
      issue_slots();
    }
    floatx4 acc[4][NCB];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[qb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
    // centre offset: a dense GEMM on the tile's own rows
    {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        uint4 a[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) a[cb] = wl[((static_cast<size_t>(centre) * NCB + cb) * NCH + ch) * 64 + aslot];
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) mfma_block<T, NCB>(acc[qb], a, bc[qb][ch]);
      }
    }
    for (int s0 = 0; s0 < tm.total; s0 += kStageEntries) {
      int s1 = (tm.total - s0 < kStageEntries) ? tm.total : s0 + kStageEntries;
      if (shared_from >= 0) {
        // the owner's stage: wait until its owner has filled it (the flag is
        // read into a scalar, so the loop is wave-uniform); spin_limit < 0
        // skips the wait
        bool ready = false;
        for (int spins = 0; spin_limit >= 0; ++spins) {
          ready = __builtin_amdgcn_readfirstlane(__hip_atomic_load(&s_ready[shared_from], __ATOMIC_ACQUIRE,
                                                                   __HIP_MEMORY_SCOPE_WORKGROUP)) ==
                  static_cast<int>(t);
          if (ready || spins >= spin_limit) break;
          __builtin_amdgcn_s_sleep(1);
        }
        if (!ready) {
          // gather the upper half itself, into its own stage: one stage
          // holds it (the owner's whole tile fitted one, s0 = 0)
          shared_from = -1;
          stage_g = stage + g * kStageStride;
          tm = window_meta(mk_full, lok_full, row_lo, row_hi, KV, centre, lane);
          issue_first();
          s1 = tm.total;
        }
      }
      if (shared_from < 0) {
        wave_lds_sync();  // earlier reads of the stage are done
        commit_stage<ROWV>(stage, rows, lane);
        wave_lds_sync();
        if (publish && lane == 0) {
          __hip_atomic_store(&s_ready[wave], static_cast<int>(t), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
      // the next range's rows are loaded while this one runs
      if (s1 < tm.total) {
        stage_positions(tm, cntk, s1, lane, pos_next);
        load_stage_rows<T, CIN>(feats, in_idx, pos_next, rows);
      }
      // Per pair of 16-row blocks, the offsets with entries in [s0, s1),
      // ping-ponging between two operand sets: the next item's LDS reads are
      // in flight while the current one runs on MFMA.  The pair index is
      // static, so each block's accumulators stay in place.
      const int lim = s1 - s0;
#pragma unroll
      for (int qp = 0; qp < 2; ++qp) {
        const bool mine = lane < KV && lane != centre;
        const uint32_t subv = mine ? static_cast<uint32_t>(tm.mk >> (32 * qp)) : 0u;
        const unsigned long long below = (qp == 0) ? 0ull : (tm.mk & 0xffffffffull);
        const int lov = tm.basek + static_cast<int>(__popcll(below)) - s0;
        const int c = __popc(subv);
        uint32_t todo = static_cast<uint32_t>(__ballot(c > 0 && lov + c > 0 && lov < lim));
        if (todo == 0u) continue;
        // Items go in pairs; an odd count is padded with an end item, whose
        // B operands are the zero row (it adds nothing).  One loop exit keeps
        // the LDS wait counts the same on every path.
        const int items = __popc(todo);
        ItemOps<NCH, NCB> x, y;
        load_item<T, CIN, COUT>(x, wl, stage_g, next_item(todo, lov, static_cast<int>(subv)), lim, r, below_r, aslot);
        for (int i = 0; i < items; i += 2) {
          load_item<T, CIN, COUT>(y, wl, stage_g, next_item(todo, lov, static_cast<int>(subv)), lim, r, below_r,
                                  aslot);
          // keep the scheduler from sinking these reads below the MFMAs
          // (which would reuse one operand set and wait on every item)
          __builtin_amdgcn_sched_barrier(0);
          run_item<T, NCH, NCB>(acc[2 * qp], acc[2 * qp + 1], x);
          load_item<T, CIN, COUT>(x, wl, stage_g, next_item(todo, lov, static_cast<int>(subv)), lim, r, below_r,
                                  aslot);
          __builtin_amdgcn_sched_barrier(0);
          run_item<T, NCH, NCB>(acc[2 * qp], acc[2 * qp + 1], y);
        }
      }
    }
    first = false;
    // epilogue: round to the output dtype, each row written once (only the
    // rows of this wave's window: a split tile's other half is another
    // wave's)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int64_t q = q0 + qb * 16 + r;
      const bool mine = qb * 16 >= row_lo && qb * 16 < row_hi;  // wave-uniform
      if constexpr (sizeof(T) == 2 && NCB % 2 == 0) {
        // 16-bit outputs in 16-byte pieces: each pair of column blocks is
        // regrouped between lanes l and l ^ 16 (one v_permlane16_swap per
        // dword) so that every lane holds 8 consecutive columns (an even g
        // 32 p + 4 g .. + 7, an odd g 32 p + 16 + 4 (g - 1) .. + 7), and a
        // store writes 64 contiguous bytes of each of 16 rows rather than
        // 8-byte fragments.
        if (mine) {
          const int64_t row = q < n ? (perm != nullptr ? static_cast<int64_t>(perm[q]) : q) : -1;
#pragma unroll
          for (int p = 0; p < NCB / 2; ++p) {
            const uint2 x = __builtin_bit_cast(uint2, Elem<T>::pack4(acc[qb][2 * p]));
            const uint2 y = __builtin_bit_cast(uint2, Elem<T>::pack4(acc[qb][2 * p + 1]));
            const auto s0 = __builtin_amdgcn_permlane16_swap(x.x, y.x, false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(x.y, y.y, false, false);
            if (row >= 0)
              *reinterpret_cast<uint4*>(out + row * COUT + 32 * p + 4 * (g & ~1) + 16 * (g & 1)) =
                  uint4{s0[0], s1[0], s0[1], s1[1]};
          }
        }
      } else if (q < n && mine) {
        const int64_t row = perm != nullptr ? static_cast<int64_t>(perm[q]) : q;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) Elem<T>::store4(out + row * COUT + cb * 16 + 4 * g, acc[qb][cb]);
      }
    }
  }
}

// Sleeps a spare wave waits for its owner's stage before gathering its rows
// itself (s_sleep 1 is 64 clocks: about 1.7 ms in all, far beyond the few
// microseconds an owner takes to fill its stage).  The environment variable
// SPCONV_SMALL_SPIN_LIMIT overrides it at each launch (-1: never wait), for
// tests that run the fallback.
int small_spin_limit() {
  int limit = 1 << 16;
  if (const char* v = std::getenv("SPCONV_SMALL_SPIN_LIMIT")) {
    const long x = std::strtol(v, nullptr, 10);
    if (x >= -1 && x <= (1 << 24)) limit = static_cast<int>(x);
  }
  return limit;
}

int device_cu_count() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) {
      cus = v;
    } else {
      cus = 256;
    }
  }
  return cus;
}

template <typename T, int CIN, int COUT>
hipError_t launch_small(const ForwardArgs& a, hipStream_t stream) {
  using Sh = SmallShape<T, CIN, COUT>;
  // One workgroup per CU (LDS-bound), with just enough waves for every tile to
  // have its own wave when the CUs allow it.
  // Up to kSpares more waves per workgroup take the upper halves of tiles
  // with more entries than one stage holds, when the workgroup has room.
  const int64_t cus = device_cu_count();
  int64_t tw = (a.tiles + cus - 1) / cus;
  if (tw < 1) tw = 1;
  if (tw > kSmallWaves) tw = kSmallWaves;
  int64_t waves = tw + kSpares;
  if (waves > kSmallWaves) waves = kSmallWaves;
  const size_t lds = Sh::lds_bytes(a.KV, static_cast<int>(waves));
  const int64_t want = (a.tiles + tw - 1) / tw;
  const unsigned grid = static_cast<unsigned>(((want < cus ? want : cus) + 7) / 8 * 8);
  static bool lds_raised = false;  // raise the dynamic-LDS limit once per instantiation
  if (!lds_raised) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_forward_small<T, CIN, COUT>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(kSmallLdsCap));
    if (e != hipSuccess) return e;
    lds_raised = true;
  }
  hipLaunchKernelGGL((k_forward_small<T, CIN, COUT>), dim3(grid), dim3(static_cast<unsigned>(waves) * 64), lds, stream,
                     static_cast<const T*>(a.feats), static_cast<const T*>(a.weights),
                     static_cast<T*>(a.out), a.in_idx, a.tile_off, a.tile_mask, a.tile_rows, a.perm, a.n,
                     a.tiles, a.KV, static_cast<int>(tw), small_spin_limit());
  return hipGetLastError();
}

// Small kernel shapes; returns hipErrorNotSupported when the shape has none.
template <typename T>
hipError_t try_small(const ForwardArgs& a, hipStream_t stream) {
  if (a.KV > 32) return hipErrorNotSupported;  // one 32-bit word of offsets
  // The centre runs as a dense GEMM on the tile's own rows: maps without an
  // identity offset (strided, transposed) take the generic kernel.
  if (a.centre != (a.KV - 1) / 2) return hipErrorNotSupported;
  constexpr size_t kBudget = kSmallLdsCap;
  if constexpr (sizeof(T) == 2) {
    if (a.cin == 32 && a.cout == 32 && SmallShape<T, 32, 32>::lds_bytes(a.KV, kSmallWaves) <= kBudget) return launch_small<T, 32, 32>(a, stream);
    if (a.cin == 32 && a.cout == 16 && SmallShape<T, 32, 16>::lds_bytes(a.KV, kSmallWaves) <= kBudget) return launch_small<T, 32, 16>(a, stream);
  } else {
    if (a.cin == 16 && a.cout == 16 && SmallShape<T, 16, 16>::lds_bytes(a.KV, kSmallWaves) <= kBudget) return launch_small<T, 16, 16>(a, stream);
    if (a.cin == 16 && a.cout == 32 && SmallShape<T, 16, 32>::lds_bytes(a.KV, kSmallWaves) <= kBudget) return launch_small<T, 16, 32>(a, stream);
  }
  return hipErrorNotSupported;
}

template <typename T, int CB>
hipError_t launch_typed(const ForwardArgs& a, hipStream_t stream) {
  const size_t lds = static_cast<size_t>(kOffsetsPerStage) * (kTileRows + 2) * sizeof(int32_t) +
                     static_cast<size_t>(CB) * (a.cin + Elem<T>::kPad) * sizeof(T);
  const dim3 grid(static_cast<unsigned>(a.tiles), static_cast<unsigned>((a.cout + CB - 1) / CB));
  hipLaunchKernelGGL((k_forward<T, CB>), grid, dim3(kThreads), lds, stream,
                     static_cast<const T*>(a.feats), static_cast<const T*>(a.weights),
                     static_cast<T*>(a.out), a.in_idx, a.tile_mask, a.tile_off, a.perm, a.n, a.tiles, a.KV,
                     a.cin, a.cout, a.centre);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dispatch_cb(const ForwardArgs& a, hipStream_t stream) {
  // Largest channel block whose transposed weight tile fits the LDS budget.
  const size_t budget = 48 * 1024;
  const size_t row = static_cast<size_t>(a.cin + Elem<T>::kPad) * sizeof(T);
  if (a.cout > 32 && 64 * row <= budget) return launch_typed<T, 64>(a, stream);
  if (a.cout > 16 && 32 * row <= budget) return launch_typed<T, 32>(a, stream);
  if (16 * row <= budget) return launch_typed<T, 16>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace

template <typename T>
hipError_t dispatch(const ForwardArgs& a, hipStream_t stream) {
  const hipError_t e = try_small<T>(a, stream);
  if (e != hipErrorNotSupported) return e;
  return launch_dispatch_cb<T>(a, stream);
}

bool small_supported(const ForwardArgs& a) {
  if (a.KV > 32 || a.centre != (a.KV - 1) / 2) return false;  // the centre runs as a dense GEMM on the tile's rows
  if (a.dtype == 0) {
    return a.cin == 16 && (a.cout == 16 || a.cout == 32);
  }
  return a.cin == 32 && (a.cout == 16 || a.cout == 32);
}

hipError_t launch_forward(const ForwardArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case 0: return dispatch<float>(a, stream);
    case 1: return dispatch<_Float16>(a, stream);
    case 2: return dispatch<__bf16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace spconv
