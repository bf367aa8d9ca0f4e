// Backward of a submanifold sparse convolution on gfx950.
//
// The forward adds, for every map entry (P, Q, W_d), f_in(P) x W_d to
// f_out(Q) ("Sparse convolution for point clouds", section "The map and the
// update rule").  By the chain rule each entry therefore adds
// grad_out(Q) x W_d^T to grad_in(P) and the outer product f_in(P) x
// grad_out(Q) to the gradient of W_d.
//
// Data gradient: (P, Q, d) is an entry exactly when (Q, P, -d) is ("Sparse
// inputs and sparse convolution", section "A symmetry you can check on the
// slide"), so grad_in is the forward over the same map with the weights
// W'_k = W_{K^3 - 1 - k}^T: k_mirror_transpose writes W' and any forward
// kernel runs on it.
//
// Weight gradient: per offset k, a GEMM whose reduction runs over the entries
// of list k, with both operands gathered (rows of the input features by
// in_idx, rows of the output gradient by out_idx).  A workgroup takes one
// chunk of up to kWgradChunk entries of one offset and one group of output
// columns; per step of 32 entries it stages both gathered row sets in LDS
// transposed (channel-major), so that an MFMA operand (16 channels x 32
// entries) is one 16-byte LDS read per lane, and accumulates
// grad_w[k][ci][co] on MFMA in fp32.  Each chunk writes fp32 partial sums,
// and k_wgrad_reduce adds a offset's chunks in chunk order, so the result
// does not depend on scheduling.
#include "internal.h"

namespace spconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// W'[k][co][ci] = W[KV - 1 - k][ci][co], one 32 x 32 tile (of one k) per
// workgroup, transposed through LDS with coalesced reads and writes.
template <typename T>
__global__ __launch_bounds__(256) void k_mirror_transpose(const T* __restrict__ w, T* __restrict__ wt, int KV,
                                                          int cin, int cout) {
  __shared__ T tile[32][33];
  const int tiles_ci = (cin + 31) / 32, tiles_co = (cout + 31) / 32;
  const int64_t b = blockIdx.x;
  const int tco = static_cast<int>(b % tiles_co);
  const int tci = static_cast<int>((b / tiles_co) % tiles_ci);
  const int k = static_cast<int>(b / (static_cast<int64_t>(tiles_co) * tiles_ci));
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const T* src = w + static_cast<int64_t>(KV - 1 - k) * cin * cout;
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int ci = tci * 32 + ty + i, co = tco * 32 + tx;
    if (ci < cin && co < cout) tile[ty + i][tx] = src[static_cast<int64_t>(ci) * cout + co];
  }
  __syncthreads();
  T* dst = wt + static_cast<int64_t>(k) * cin * cout;
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int co = tco * 32 + ty + i, ci = tci * 32 + tx;
    if (ci < cin && co < cout) dst[static_cast<int64_t>(co) * cin + ci] = tile[tx][ty + i];
  }
}

template <typename T>
__device__ __forceinline__ floatx4 mfma(uint4 a, uint4 b, floatx4 c) {
  if constexpr (__is_same(T, _Float16)) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// First entry of offset k and the entry after its last: the map's tile
// offsets start every offset's list at its first tile.
__device__ __forceinline__ void list_range(const int32_t* __restrict__ tile_off, int64_t tiles, int k, int KV,
                                           int64_t* lo, int64_t* hi) {
  *lo = tile_off[static_cast<int64_t>(k) * tiles];
  *hi = (k + 1 < KV) ? tile_off[static_cast<int64_t>(k + 1) * tiles] : tile_off[static_cast<int64_t>(KV) * tiles];
}

// Grid: x = chunk of kWgradChunk entries, y = offset k, z = group of COLS
// output columns; 4 waves.  Wave w owns the 16 x 16 output tiles w, w + 4,
// ... of the CIN x COLS block (tile t: channel block t / (COLS / 16), column
// block t % (COLS / 16)).  LDS: fT[CIN][32] and gT[COLS][32] of the step's
// entries (channel-major, so that lane (g, r) of an operand reads channel r
// of its block, entries 8 g .. 8 g + 7, in one 16-byte read).
constexpr int kWgradChunk = 16384;
template <typename T, int CIN, int COLS>
__global__ __launch_bounds__(256) void k_wgrad(const uint16_t* __restrict__ feats, const uint16_t* __restrict__ gout,
                                               const int32_t* __restrict__ in_idx,
                                               const int32_t* __restrict__ out_idx,
                                               const int32_t* __restrict__ tile_off, int64_t tiles, int KV, int cout,
                                               float* __restrict__ part) {
  constexpr int NT = (CIN / 16) * (COLS / 16);  // output tiles
  constexpr int TPW = (NT + 3) / 4;             // tiles per wave
  __shared__ __align__(16) uint16_t fT[CIN * 32];
  __shared__ __align__(16) uint16_t gT[COLS * 32];
  const int k = blockIdx.y;
  const int64_t chunk = blockIdx.x;
  const int col0 = blockIdx.z * COLS;
  int64_t lo, hi;
  list_range(tile_off, tiles, k, KV, &lo, &hi);
  const int64_t e0 = lo + chunk * kWgradChunk;
  if (e0 >= hi) return;  // uniform: this offset has fewer chunks
  const int64_t e1 = (hi - e0 < kWgradChunk) ? hi : e0 + kWgradChunk;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  floatx4 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  // Staging: a 16-byte piece (8 channels) of one entry's row per thread and
  // round; CIN / 8 pieces per feature row, COLS / 8 per gradient row.
  constexpr int FP = CIN / 8 * 32, GP = COLS / 8 * 32;  // pieces per step
  for (int64_t s = e0; s < e1; s += 32) {
    for (int p = tid; p < FP + GP; p += 256) {
      const bool isf = p < FP;
      const int pp = isf ? p : p - FP;
      const int per = isf ? CIN / 8 : COLS / 8;
      const int e = pp / per, c8 = (pp % per) * 8;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (s + e < e1) {
        if (isf) v = *reinterpret_cast<const uint4*>(feats + static_cast<int64_t>(in_idx[s + e]) * CIN + c8);
        else v = *reinterpret_cast<const uint4*>(gout + static_cast<int64_t>(out_idx[s + e]) * cout + col0 + c8);
      }
      uint16_t* dst = (isf ? fT : gT) + c8 * 32 + e;
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[i * 32] = static_cast<uint16_t>(w4[i >> 1] >> (16 * (i & 1)));
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wave + 4 * i;
      if (t < NT) {
        const int cb = t / (COLS / 16), ob = t % (COLS / 16);
        const uint4 a = *reinterpret_cast<const uint4*>(fT + (cb * 16 + r) * 32 + 8 * g);
        const uint4 b = *reinterpret_cast<const uint4*>(gT + (ob * 16 + r) * 32 + 8 * g);
        acc[i] = mfma<T>(a, b, acc[i]);
      }
    }
    __syncthreads();
  }
  // D element (row 4 g + j, column r) of tile (cb, ob) is grad_w[k][ci =
  // 16 cb + 4 g + j][co = col0 + 16 ob + r]: partial [chunk][k][ci][co].
  float* pk = part + (chunk * KV + k) * static_cast<int64_t>(CIN) * cout;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = wave + 4 * i;
    if (t < NT) {
      const int cb = t / (COLS / 16), ob = t % (COLS / 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) pk[static_cast<int64_t>(cb * 16 + 4 * g + j) * cout + col0 + ob * 16 + r] = acc[i][j];
    }
  }
}

// Any dtype and channel counts (fp32 features, or channels not multiples of
// 16): per step of 32 entries the rows are staged in LDS as fp32, and thread
// t accumulates the products of its (ci, co) pairs of the block of COLS
// output columns in fp32.  Same partial layout as k_wgrad.
template <typename T>
__global__ __launch_bounds__(256) void k_wgrad_generic(const T* __restrict__ feats, const T* __restrict__ gout,
                                                       const int32_t* __restrict__ in_idx,
                                                       const int32_t* __restrict__ out_idx,
                                                       const int32_t* __restrict__ tile_off, int64_t tiles, int KV,
                                                       int cin, int cout, int cols, float* __restrict__ part) {
  constexpr int kMaxPerThread = 64;
  extern __shared__ float gsm[];  // fs[32][cin], gs[32][cols]
  float* fs = gsm;
  float* gs = gsm + 32 * cin;
  const int k = blockIdx.y;
  const int64_t chunk = blockIdx.x;
  const int col0 = blockIdx.z * cols;
  const int ncols = (cout - col0 < cols) ? cout - col0 : cols;
  int64_t lo, hi;
  list_range(tile_off, tiles, k, KV, &lo, &hi);
  const int64_t e0 = lo + chunk * kWgradChunk;
  if (e0 >= hi) return;
  const int64_t e1 = (hi - e0 < kWgradChunk) ? hi : e0 + kWgradChunk;
  const int tid = threadIdx.x;
  const int pairs = cin * ncols;
  float acc[kMaxPerThread];
#pragma unroll
  for (int i = 0; i < kMaxPerThread; ++i) acc[i] = 0.f;
  for (int64_t s = e0; s < e1; s += 32) {
    for (int i = tid; i < 32 * cin; i += 256) {
      const int e = i / cin, c = i % cin;
      fs[i] = (s + e < e1) ? static_cast<float>(feats[static_cast<int64_t>(in_idx[s + e]) * cin + c]) : 0.f;
    }
    for (int i = tid; i < 32 * ncols; i += 256) {
      const int e = i / ncols, c = i % ncols;
      gs[e * cols + c] = (s + e < e1) ? static_cast<float>(gout[static_cast<int64_t>(out_idx[s + e]) * cout + col0 + c]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMaxPerThread; ++i) {
      const int pidx = tid + 256 * i;
      if (pidx < pairs) {
        const int ci = pidx / ncols, co = pidx % ncols;
        float a = acc[i];
        for (int e = 0; e < 32; ++e) a = fmaf(fs[e * cin + ci], gs[e * cols + co], a);
        acc[i] = a;
      }
    }
    __syncthreads();
  }
  float* pk = part + (chunk * KV + k) * static_cast<int64_t>(cin) * cout;
#pragma unroll
  for (int i = 0; i < kMaxPerThread; ++i) {
    const int pidx = tid + 256 * i;
    if (pidx < pairs) {
      const int ci = pidx / ncols, co = pidx % ncols;
      pk[static_cast<int64_t>(ci) * cout + col0 + co] = acc[i];
    }
  }
}

// grad_w[k][i] = sum of the partials of offset k's chunks, in chunk order.
__global__ __launch_bounds__(256) void k_wgrad_reduce(const float* __restrict__ part,
                                                      const int32_t* __restrict__ tile_off, int64_t tiles, int KV,
                                                      int64_t per_k, float* __restrict__ grad_w) {
  const int k = blockIdx.y;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= per_k) return;
  int64_t lo, hi;
  list_range(tile_off, tiles, k, KV, &lo, &hi);
  const int64_t chunks = (hi - lo + kWgradChunk - 1) / kWgradChunk;
  float s = 0.f;
  for (int64_t c = 0; c < chunks; ++c) s += part[(c * KV + k) * per_k + i];
  grad_w[static_cast<int64_t>(k) * per_k + i] = s;
}

template <typename T>
hipError_t launch_mirror(const T* w, T* wt, int KV, int cin, int cout, hipStream_t stream) {
  const int64_t grid = static_cast<int64_t>(KV) * ((cin + 31) / 32) * ((cout + 31) / 32);
  hipLaunchKernelGGL(k_mirror_transpose<T>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, w, wt, KV, cin,
                     cout);
  return hipGetLastError();
}

template <typename T, int CIN, int COLS>
hipError_t launch_wgrad_mfma(const WgradArgs& a, float* part, int64_t max_chunks, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(max_chunks), static_cast<unsigned>(a.KV), static_cast<unsigned>(a.cout / COLS));
  hipLaunchKernelGGL((k_wgrad<T, CIN, COLS>), grid, dim3(256), 0, stream, static_cast<const uint16_t*>(a.feats),
                     static_cast<const uint16_t*>(a.grad_out), a.in_idx, a.out_idx, a.tile_off, a.tiles, a.KV,
                     a.cout, part);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_wgrad_cin(const WgradArgs& a, float* part, int64_t max_chunks, hipStream_t stream) {
  const int cols = wgrad_cols(a);
  switch (a.cin * 1000 + cols) {
    case 16016: return launch_wgrad_mfma<T, 16, 16>(a, part, max_chunks, stream);
    case 16032: return launch_wgrad_mfma<T, 16, 32>(a, part, max_chunks, stream);
    case 16064: return launch_wgrad_mfma<T, 16, 64>(a, part, max_chunks, stream);
    case 32016: return launch_wgrad_mfma<T, 32, 16>(a, part, max_chunks, stream);
    case 32032: return launch_wgrad_mfma<T, 32, 32>(a, part, max_chunks, stream);
    case 32064: return launch_wgrad_mfma<T, 32, 64>(a, part, max_chunks, stream);
    case 64016: return launch_wgrad_mfma<T, 64, 16>(a, part, max_chunks, stream);
    case 64032: return launch_wgrad_mfma<T, 64, 32>(a, part, max_chunks, stream);
    case 64064: return launch_wgrad_mfma<T, 64, 64>(a, part, max_chunks, stream);
    case 128016: return launch_wgrad_mfma<T, 128, 16>(a, part, max_chunks, stream);
    case 128032: return launch_wgrad_mfma<T, 128, 32>(a, part, max_chunks, stream);
    case 128064: return launch_wgrad_mfma<T, 128, 64>(a, part, max_chunks, stream);
    case 256016: return launch_wgrad_mfma<T, 256, 16>(a, part, max_chunks, stream);
    case 256032: return launch_wgrad_mfma<T, 256, 32>(a, part, max_chunks, stream);
    case 256064: return launch_wgrad_mfma<T, 256, 64>(a, part, max_chunks, stream);
    default: return hipErrorNotSupported;
  }
}

template <typename T>
hipError_t launch_wgrad_generic(const WgradArgs& a, float* part, int64_t max_chunks, hipStream_t stream) {
  // columns per workgroup: at most 64 (cin x cols) pairs per thread
  int cols = a.cout;
  while (static_cast<int64_t>(a.cin) * cols > 64 * 256) cols = (cols + 1) / 2;
  const dim3 grid(static_cast<unsigned>(max_chunks), static_cast<unsigned>(a.KV),
                  static_cast<unsigned>((a.cout + cols - 1) / cols));
  const size_t lds = static_cast<size_t>(32) * (a.cin + cols) * sizeof(float);
  static bool raised = false;
  if (!raised) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_wgrad_generic<T>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    raised = true;
  }
  hipLaunchKernelGGL(k_wgrad_generic<T>, grid, dim3(256), lds, stream, static_cast<const T*>(a.feats),
                     static_cast<const T*>(a.grad_out), a.in_idx, a.out_idx, a.tile_off, a.tiles, a.KV, a.cin,
                     a.cout, cols, part);
  return hipGetLastError();
}

bool wgrad_mfma_shape(const WgradArgs& a) {
  if (a.dtype != 1 && a.dtype != 2) return false;
  if (a.cin != 16 && a.cin != 32 && a.cin != 64 && a.cin != 128 && a.cin != 256) return false;
  return a.cout % 16 == 0;
}

}  // namespace

// Output columns of one weight-gradient workgroup (MFMA path): the widest of
// 64, 32, 16 that divides C_out.
int wgrad_cols(const WgradArgs& a) {
  if (a.cout % 64 == 0) return 64;
  if (a.cout % 32 == 0) return 32;
  return 16;
}

int64_t wgrad_max_chunks(const WgradArgs& a) {
  // the centre list holds every row, and no list holds more
  return (a.n + kWgradChunk - 1) / kWgradChunk;
}

size_t wgrad_workspace_bytes(const WgradArgs& a) {
  return static_cast<size_t>(wgrad_max_chunks(a)) * a.KV * a.cin * a.cout * sizeof(float);
}

size_t mirror_workspace_bytes(int KV, int cin, int cout, int dtype) {
  const size_t es = dtype == 0 ? 4 : 2;
  return (static_cast<size_t>(KV) * cin * cout * es + 255) / 256 * 256;
}

hipError_t launch_mirror_transpose(const void* w, void* wt, int KV, int cin, int cout, int dtype,
                                   hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_mirror(static_cast<const float*>(w), static_cast<float*>(wt), KV, cin, cout, stream);
    case 1: return launch_mirror(static_cast<const _Float16*>(w), static_cast<_Float16*>(wt), KV, cin, cout, stream);
    case 2: return launch_mirror(static_cast<const __bf16*>(w), static_cast<__bf16*>(wt), KV, cin, cout, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_wgrad(const WgradArgs& a, void* workspace, hipStream_t stream) {
  float* part = static_cast<float*>(workspace);
  const int64_t max_chunks = wgrad_max_chunks(a);
  hipError_t e;
  if (wgrad_mfma_shape(a)) {
    e = (a.dtype == 1) ? launch_wgrad_cin<_Float16>(a, part, max_chunks, stream)
                       : launch_wgrad_cin<__bf16>(a, part, max_chunks, stream);
  } else if (a.dtype == 0) {
    e = launch_wgrad_generic<float>(a, part, max_chunks, stream);
  } else if (a.dtype == 1) {
    e = launch_wgrad_generic<_Float16>(a, part, max_chunks, stream);
  } else {
    e = launch_wgrad_generic<__bf16>(a, part, max_chunks, stream);
  }
  if (e != hipSuccess) return e;
  const int64_t per_k = static_cast<int64_t>(a.cin) * a.cout;
  hipLaunchKernelGGL(k_wgrad_reduce, dim3(static_cast<unsigned>((per_k + 255) / 256), static_cast<unsigned>(a.KV)),
                     dim3(256), 0, stream, part, a.tile_off, a.tiles, a.KV, per_k, a.grad_w);
  return hipGetLastError();
}

}  // namespace spconv
