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
  __device__ static void store4(_Float16* dst, floatx4 v) {
    u16x4 o;
    for (int i = 0; i < 4; ++i) {
      const _Float16 h = static_cast<_Float16>(v[i]);  // v_cvt_f16_f32: round to nearest even
      o[i] = __builtin_bit_cast(uint16_t, h);
    }
    *reinterpret_cast<u16x4*>(dst) = o;
  }
};
template <>
struct Elem<__bf16> {
  static constexpr int kVec = 8;
  static constexpr int kChunk = 32;
  static constexpr int kPad = 8;
  __device__ static void store4(__bf16* dst, floatx4 v) {
    u16x4 o;
    for (int i = 0; i < 4; ++i) o[i] = bf16_bits_rne(v[i]);
    *reinterpret_cast<u16x4*>(dst) = o;
  }
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
    const int32_t* __restrict__ in_idx, const int32_t* __restrict__ out_idx,
    const int32_t* __restrict__ tile_off, int64_t n, int64_t tiles, int KV, int cin, int cout) {
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
  const int centre = (KV - 1) / 2;
  const int row_in_tile = wave * 16 + r;
  const int64_t q = q0 + row_in_tile;

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
    // row -> input-row table of this tile for the stage's offsets
    for (int i = 0; i < kn; ++i) {
      if (kb + i == centre) continue;
      const int lo = lo_lds[i], hi = hi_lds[i];
      for (int e = lo + tid; e < hi; e += kThreads) {
        nbr_lds[i * kTileRows + static_cast<int>(out_idx[e] - q0)] = in_idx[e];
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
      const int32_t src = (k == centre) ? (q < n ? static_cast<int32_t>(q) : -1)
                                        : nbr_lds[i * kTileRows + row_in_tile];
      if (__ballot(src >= 0) == 0ull) continue;  // none of this wave's 16 rows uses offset k
      const T* frow = feats + static_cast<int64_t>(src < 0 ? 0 : src) * cin;
      const T* wrow = wt + r * ldw;
      for (int c = 0; c < cin; c += CHUNK) {
        const int cc = c + g * (CHUNK / 4);
        const bool inside = cc < cin;
        const int ccs = inside ? cc : 0;
        Step<T, NCB>::run(acc, frow + ccs, inside && src >= 0, wrow + ccs, inside, 16 * ldw);
      }
    }
  }

  // Epilogue: fp32 -> dtype, each output row written once.
  if (q < n) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int co = co0 + cb * 16 + 4 * g;
      if (co < cout) Elem<T>::store4(out + q * cout + co, acc[cb]);
    }
  }
}

template <typename T, int CB>
hipError_t launch_typed(const ForwardArgs& a, hipStream_t stream) {
  const size_t lds = static_cast<size_t>(kOffsetsPerStage) * (kTileRows + 2) * sizeof(int32_t) +
                     static_cast<size_t>(CB) * (a.cin + Elem<T>::kPad) * sizeof(T);
  const dim3 grid(static_cast<unsigned>(a.tiles), static_cast<unsigned>((a.cout + CB - 1) / CB));
  hipLaunchKernelGGL((k_forward<T, CB>), grid, dim3(kThreads), lds, stream,
                     static_cast<const T*>(a.feats), static_cast<const T*>(a.weights),
                     static_cast<T*>(a.out), a.in_idx, a.out_idx, a.tile_off, a.n, a.tiles, a.KV,
                     a.cin, a.cout);
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

hipError_t launch_forward(const ForwardArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case 0: return launch_dispatch_cb<float>(a, stream);
    case 1: return launch_dispatch_cb<_Float16>(a, stream);
    case 2: return launch_dispatch_cb<__bf16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace spconv
