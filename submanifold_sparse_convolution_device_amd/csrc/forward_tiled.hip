// Forward of a submanifold sparse convolution for mid and large channel
// counts (C_in in {32, 64, 128, 256}) on gfx950.
//
// Same computation as the small-channel kernel (forward.hip): for every output
// row Q, f_out(Q) = sum over map entries (P, Q, W_d) of f_in(P) x W_d
// ("Sparse convolution for point clouds", section "The map and the update
// rule"), accumulated on chip per output row and written once.
//
// Here W_d does not fit in LDS all at once, so a workgroup walks the offsets
// present in its rows and shares one W_d slice (C_in x CB output channels) in
// LDS per offset, double-buffered: while the MFMAs of offset d run, the slice
// of the next offset is copied in.  The slices come from a copy of the weights
// already in MFMA operand order (k_prep_weights, one small launch), so staging
// is a straight 16-byte copy.  Each wave owns 16 x QB output rows and keeps
// their CB-column accumulators in registers.  A wave's gathered input rows
// (B operands, 16 bytes per lane and chunk) for the next offset are loaded
// from global memory while the current offset runs, and their row indices two
// offsets ahead.  A 16-row block without a neighbour at offset d skips that
// offset's MFMAs; the offsets of the workgroup are the union of its rows'.
#include "internal.h"

namespace spconv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

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

// Weights in MFMA operand order: block (k, cbg, ch) holds, for lane
// (g, r) = (l / 16, l mod 16), the 8 values W[k][ch * 32 + 8 g + i][16 cbg + r].
// One workgroup per (k, ch, group of 64 output channels): its 32 x 64 slice
// of W_k is read in 16-byte pieces along the output channels (one per
// thread, whole rows coalesced), transposed through LDS, and written as up
// to four whole operand blocks (1 KB each, one per wave).  The first
// workgroup also clears the 512-byte zero row.
template <typename T>
__global__ __launch_bounds__(256) void k_prep_weights(const T* __restrict__ w, uint4* __restrict__ wop,
                                                      uint4* __restrict__ zero, int KV, int cin, int cout) {
  constexpr int kCols = 64, kStride = kCols + 8;  // row stride of 144 bytes: 16-byte aligned rows
  __shared__ __align__(16) uint16_t tile[32 * kStride];
  const int t = threadIdx.x;
  if (blockIdx.x == 0 && t < 32) zero[t] = make_uint4(0u, 0u, 0u, 0u);
  const int nch = cin / 32, ncbg = cout / 16, ngrp = (cout + kCols - 1) / kCols;
  const int64_t b = blockIdx.x;
  const int grp = static_cast<int>(b % ngrp);
  const int ch = static_cast<int>((b / ngrp) % nch);
  const int k = static_cast<int>(b / (static_cast<int64_t>(ngrp) * nch));
  if (k >= KV) return;  // uniform over the workgroup
  const int co0 = grp * kCols;
  {
    const int row = t >> 3, c8 = (t & 7) * 8;  // C_out is a multiple of 16: a piece is all in or all out
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (co0 + c8 < cout) {
      v = *reinterpret_cast<const uint4*>(w + (static_cast<int64_t>(k) * cin + ch * 32 + row) * cout + co0 + c8);
    }
    *reinterpret_cast<uint4*>(&tile[row * kStride + c8]) = v;
  }
  __syncthreads();
  const int cb = t >> 6, lane = t & 63, r = lane & 15, g = lane >> 4;
  const int cbg = grp * (kCols / 16) + cb;
  if (cbg < ncbg) {
    uint16_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = tile[(8 * g + i) * kStride + 16 * cb + r];
    uint4 out;
    __builtin_memcpy(&out, o, sizeof(out));
    wop[((static_cast<int64_t>(k) * ncbg + cbg) * nch + ch) * 64 + lane] = out;
  }
}

template <int CIN, int CB, int QB>
struct TiledShape {
  static constexpr int NCH = CIN / 32;   // ci chunks of one MFMA
  static constexpr int NCB = CB / 16;    // 16-wide output blocks per wave
  static constexpr int WSLICE = NCB * NCH * 64;  // uint4 per W slice
};

// Row index (or -1) of each of the wave's QB 16-row blocks at offset k.
template <int QB>
struct Src {
  int v[QB];
};

template <typename T, int CIN, int CB, int QB>
__global__ __launch_bounds__(512) void k_forward_tiled(
    const T* __restrict__ feats, const uint4* __restrict__ wop, T* __restrict__ out,
    const int32_t* __restrict__ in_idx, const int32_t* __restrict__ tile_off,
    const unsigned long long* __restrict__ tile_mask, const int32_t* __restrict__ perm, int64_t n, int64_t tiles,
    int KV, int cout, int centre) {
  using Sh = TiledShape<CIN, CB, QB>;
  constexpr int NCH = Sh::NCH, NCB = Sh::NCB, WSLICE = Sh::WSLICE;
  constexpr int UNITS_PER_TILE = 4 / QB;  // waves per 64-row tile
  extern __shared__ uint4 smem[];
  uint4* wbuf = smem;  // [2][WSLICE]
  unsigned long long* pres = reinterpret_cast<unsigned long long*>(smem + 2 * WSLICE);  // [waves][2]

  const int nw = blockDim.x >> 6;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * nw + wave;  // 16 QB rows
  const int64_t t = unit / UNITS_PER_TILE;
  const int qb0 = static_cast<int>(unit % UNITS_PER_TILE) * QB;  // first 16-row block in the tile
  const int64_t q_first = t * kTileRows + qb0 * 16;
  const bool active = (t < tiles) && (q_first < n);
  const int cbg0 = blockIdx.y * NCB;  // first 16-column block
  const int ncbg = cout / 16;

  // Offset k's tile mask (all 64 rows of the tile: list ranks count every
  // earlier row) and list start, in lane k (k < 64) or lane k - 64 (k >= 64).
  const unsigned long long rows_mask =
      (QB == 4) ? ~0ull : (((1ull << (16 * QB)) - 1ull) << (16 * qb0));
  unsigned long long m0 = 0ull, m1 = 0ull;
  int lo0 = 0, lo1 = 0;
  if (active) {
    if (lane < KV) {
      m0 = tile_mask[static_cast<int64_t>(lane) * tiles + t];
      lo0 = tile_off[static_cast<int64_t>(lane) * tiles + t];
    }
    if (lane + 64 < KV) {
      m1 = tile_mask[static_cast<int64_t>(lane + 64) * tiles + t];
      lo1 = tile_off[static_cast<int64_t>(lane + 64) * tiles + t];
    }
  }
  // offsets present in this wave's rows, then anywhere in the workgroup
  {
    const unsigned long long p0 = __ballot((m0 & rows_mask) != 0ull);
    const unsigned long long p1 = __ballot((m1 & rows_mask) != 0ull);
    if (lane == 0) {
      pres[2 * wave] = p0;
      pres[2 * wave + 1] = p1;
    }
  }
  __syncthreads();
  unsigned long long todo0 = 0ull, todo1 = 0ull;
  for (int w = 0; w < nw; ++w) {
    todo0 |= pres[2 * w];
    todo1 |= pres[2 * w + 1];
  }

  auto mask_of = [&](int k) -> unsigned long long {
    const unsigned long long v = (k < 64) ? m0 : m1;
    const int src = k & 63;
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), src));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), src));
    return (static_cast<unsigned long long>(hi) << 32) | lo;
  };
  auto lo_of = [&](int k) -> int { return __builtin_amdgcn_readlane((k < 64) ? lo0 : lo1, k & 63); };
  auto next_offset = [&]() -> int {
    if (todo0) {
      const int k = __ffsll(static_cast<long long>(todo0)) - 1;
      todo0 &= todo0 - 1ull;
      return k;
    }
    if (todo1) {
      const int k = 64 + __ffsll(static_cast<long long>(todo1)) - 1;
      todo1 &= todo1 - 1ull;
      return k;
    }
    return -1;
  };
  // Row index of this lane's row in each block at offset k (centre: itself).
  auto load_src = [&](int k) -> Src<QB> {
    Src<QB> s;
#pragma unroll
    for (int b = 0; b < QB; ++b) s.v[b] = -1;
    if (k < 0 || !active) return s;
    const unsigned long long m = mask_of(k);
    if ((m & rows_mask) == 0ull) return s;
    const int lk = lo_of(k);
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int row = (qb0 + b) * 16 + r;
      const bool has = (m >> row) & 1ull;
      if (k == centre) {  // the row at this position (the list of the centre is the identity)
        const int64_t q = t * kTileRows + row;
        s.v[b] = has ? (perm != nullptr ? perm[q] : static_cast<int>(q)) : -1;
      } else {
        const int rank = __popcll(m & ((1ull << row) - 1ull));
        s.v[b] = has ? in_idx[static_cast<int64_t>(lk) + rank] : -1;
      }
    }
    return s;
  };
  auto load_b = [&](const Src<QB>& s, uint4 (&b)[QB][NCH]) {
#pragma unroll
    for (int bb = 0; bb < QB; ++bb) {
      const T* rowp = feats + static_cast<int64_t>(s.v[bb] < 0 ? 0 : s.v[bb]) * CIN + g * 8;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        b[bb][ch] = make_uint4(0u, 0u, 0u, 0u);
        if (s.v[bb] >= 0) b[bb][ch] = *reinterpret_cast<const uint4*>(rowp + ch * 32);
      }
    }
  };
  // The W slice of offset k in the prepared weights.
  auto wsrc = [&](int k) -> const uint4* {
    return wop + (static_cast<int64_t>(k) * ncbg + cbg0) * NCH * 64;
  };

  floatx4 acc[QB][NCB];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[b][cb] = floatx4{0.f, 0.f, 0.f, 0.f};

  int kc = next_offset();
  if (kc < 0) return;  // uniform: nothing in this workgroup (never the case for a valid tile)
  const int stride = blockDim.x;
  // stage W of the first offset
  {
    const uint4* src = wsrc(kc);
    for (int i = tid; i < WSLICE; i += stride) wbuf[i] = src[i];
  }
  int kn = next_offset();
  Src<QB> s_cur = load_src(kc);
  Src<QB> s_nxt = load_src(kn);
  uint4 b_cur[QB][NCH];
  load_b(s_cur, b_cur);
  __syncthreads();
  int buf = 0;
  while (kc >= 0) {
    // 1. next offset's W slice into registers (copied to LDS after the MFMAs)
    constexpr int WPT_MAX = 8;  // uint4 per thread for nw >= WSLICE / (64 * 8)
    uint4 wreg[WPT_MAX];
    const int wpt = (WSLICE + stride - 1) / stride;
    if (kn >= 0) {
      const uint4* src = wsrc(kn);
#pragma unroll
      for (int j = 0; j < WPT_MAX; ++j) {
        const int i = tid + j * stride;
        if (j < wpt && i < WSLICE) wreg[j] = src[i];
      }
    }
    // 2. next offset's B operands and the row indices of the one after
    uint4 b_nxt[QB][NCH];
    load_b(s_nxt, b_nxt);
    const int kn2 = next_offset();
    const Src<QB> s_nxt2 = load_src(kn2);
    // 3. MFMAs of offset kc
    const uint4* wl = wbuf + buf * WSLICE;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      if (__ballot(s_cur.v[b] >= 0) == 0ull) continue;  // no row of this block has offset kc
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const uint4 a = wl[(cb * NCH + ch) * 64 + lane];
          acc[b][cb] = mfma<T>(a, b_cur[b][ch], acc[b][cb]);
        }
      }
    }
    // 4. publish the next slice
    if (kn >= 0) {
      uint4* dst = wbuf + (buf ^ 1) * WSLICE;
#pragma unroll
      for (int j = 0; j < WPT_MAX; ++j) {
        const int i = tid + j * stride;
        if (j < wpt && i < WSLICE) dst[i] = wreg[j];
      }
    }
    __syncthreads();
    buf ^= 1;
    kc = kn;
    kn = kn2;
    s_cur = s_nxt;
    s_nxt = s_nxt2;
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) b_cur[b][ch] = b_nxt[b][ch];
  }
  // epilogue
  if (active) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int64_t q = q_first + b * 16 + r;
      if (q < n) {
        const int64_t row = perm != nullptr ? static_cast<int64_t>(perm[q]) : q;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          store4<T>(out + row * cout + (cbg0 + cb) * 16 + 4 * g, acc[b][cb]);
        }
      }
    }
  }
}

int cu_count() {
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

template <typename T, int CIN, int CB, int QB>
hipError_t launch_tiled_shape(const ForwardArgs& a, const uint4* wop, int nw, hipStream_t stream) {
  using Sh = TiledShape<CIN, CB, QB>;
  const int64_t units = a.tiles * (4 / QB);
  const dim3 grid(static_cast<unsigned>((units + nw - 1) / nw), static_cast<unsigned>(a.cout / CB));
  const size_t lds = 2 * Sh::WSLICE * sizeof(uint4) + 2 * 8 * 8;
  static bool raised = false;
  if (!raised) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_forward_tiled<T, CIN, CB, QB>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    raised = true;
  }
  hipLaunchKernelGGL((k_forward_tiled<T, CIN, CB, QB>), grid, dim3(64 * nw), lds, stream,
                     static_cast<const T*>(a.feats), wop, static_cast<T*>(a.out), a.in_idx, a.tile_off,
                     a.tile_mask, a.perm, a.n, a.tiles, a.KV, a.cout, a.centre);
  return hipGetLastError();
}

template <typename T, int CIN, int QB>
hipError_t launch_tiled_cin(const ForwardArgs& a, const uint4* wop, hipStream_t stream) {
  // Output-channel block: the widest that still gives every SIMD two waves.
  const int64_t row_units = a.tiles * (4 / QB);
  const int64_t want = 8LL * cu_count();
  int cb = 64;
  while (cb > 16 && (a.cout % cb != 0 || row_units * (a.cout / cb) < want)) cb >>= 1;
  if (a.cout % cb != 0) cb = 16;
  // waves per workgroup: as many as keep two workgroups per CU
  const int64_t waves = row_units * (a.cout / cb);
  int nw = 8;
  while (nw > 1 && waves / nw < 2LL * cu_count()) nw >>= 1;
  // every thread must hold at most 8 uint4 of the W slice
  const int wslice = (cb / 16) * (CIN / 32) * 64;
  while (nw < 8 && (wslice + 64 * nw - 1) / (64 * nw) > 8) nw <<= 1;
  switch (cb) {
    case 64: return launch_tiled_shape<T, CIN, 64, QB>(a, wop, nw, stream);
    case 32: return launch_tiled_shape<T, CIN, 32, QB>(a, wop, nw, stream);
    default: return launch_tiled_shape<T, CIN, 16, QB>(a, wop, nw, stream);
  }
}

template <typename T>
hipError_t launch_tiled_typed(const ForwardArgs& a, const uint4* wop, hipStream_t stream) {
  switch (a.cin) {
    case 32: return launch_tiled_cin<T, 32, 4>(a, wop, stream);
    case 64: return launch_tiled_cin<T, 64, 4>(a, wop, stream);
    case 128: return launch_tiled_cin<T, 128, 4>(a, wop, stream);
    case 256: return launch_tiled_cin<T, 256, 2>(a, wop, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

bool tiled_supported(const ForwardArgs& a) {
  if (a.dtype != 1 && a.dtype != 2) return false;
  if (a.KV > 128) return false;
  if (a.cin != 32 && a.cin != 64 && a.cin != 128 && a.cin != 256) return false;
  return a.cout % 16 == 0;
}

// Operand-order weights, then a 512-byte zero row (aligned to 256 bytes).
size_t tiled_workspace_bytes(const ForwardArgs& a) {
  return (static_cast<size_t>(a.KV) * a.cin * a.cout * 2 + 255) / 256 * 256 + 512;
}

const uint4* workspace_zero_row(const ForwardArgs& a, const void* workspace) {
  return reinterpret_cast<const uint4*>(static_cast<const char*>(workspace) +
                                        (static_cast<size_t>(a.KV) * a.cin * a.cout * 2 + 255) / 256 * 256);
}

hipError_t launch_prep_weights(const ForwardArgs& a, void* workspace, hipStream_t stream) {
  uint4* wop = static_cast<uint4*>(workspace);
  uint4* zero = const_cast<uint4*>(workspace_zero_row(a, workspace));
  const int64_t groups = static_cast<int64_t>(a.KV) * (a.cin / 32) * ((a.cout + 63) / 64);
  const unsigned grid = static_cast<unsigned>(groups);
  if (a.dtype == 1) {
    hipLaunchKernelGGL(k_prep_weights<_Float16>, dim3(grid), dim3(256), 0, stream,
                       static_cast<const _Float16*>(a.weights), wop, zero, a.KV, a.cin, a.cout);
  } else {
    hipLaunchKernelGGL(k_prep_weights<__bf16>, dim3(grid), dim3(256), 0, stream,
                       static_cast<const __bf16*>(a.weights), wop, zero, a.KV, a.cin, a.cout);
  }
  return hipGetLastError();
}

hipError_t launch_forward_tiled(const ForwardArgs& a, void* workspace, hipStream_t stream) {
  if (a.prepared == nullptr) {
    const hipError_t e = launch_prep_weights(a, workspace, stream);
    if (e != hipSuccess) return e;
  }
  const uint4* wop = static_cast<const uint4*>(a.prepared != nullptr ? a.prepared : workspace);
  if (a.dtype == 1) return launch_tiled_typed<_Float16>(a, wop, stream);
  return launch_tiled_typed<__bf16>(a, wop, stream);
}

}  // namespace spconv
