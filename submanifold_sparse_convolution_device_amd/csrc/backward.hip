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
// in_idx, rows of the output gradient by out_idx).  The work is cut by tile
// ranges: one workgroup takes the entries of one offset inside one range of
// output tiles, so the workgroups of all offsets for a range read the same
// neighbourhood of rows, and the grid keeps them on one XCD, where those rows
// stay in its L2.  Per round of entries, the gathered rows are copied whole
// from global memory straight into LDS (row-major, 16-byte pieces
// XOR-swizzled), a few rounds ahead of the MFMAs; the MFMA operands, which
// run along the entries, come out of LDS with transposing reads
// (ds_read_b64_tr_b16: in each 16-lane block, lanes 4j .. 4j + 3 give 4
// consecutive values each of row j, and lane i receives value i of the four
// rows).  Each workgroup writes fp32 partial sums for its tile range, and
// k_wgrad_reduce adds an offset's ranges in range order, so the result does
// not depend on scheduling.
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

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier that orders only what the kernel orders by hand: the
// copies into LDS a round needs are waited for by count before it, and the
// LDS reads complete inside their own asm, so no memory fence (which would
// drain the copies still in flight for later rounds) is wanted.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt with only a vector-memory count (the other counters unconstrained).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One transposing LDS read (see the top of the file), left in flight.  Asm,
// because the compiler cannot tell the stage buffers apart and would wait for
// every copy into LDS still in flight before a visible LDS read.
template <int OFF>
__device__ __forceinline__ void read_tr(uint32_t addr, u32x2& v) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
}

// Rounds of 32 x SUB entries: SUB is the smallest power of two (at least WK)
// that brings a round to about 16 KB of staged rows, rounded up so that its
// 1 KB copies split evenly over the 4 waves.
constexpr int wgrad_sub(int c, int wk) {
  int s = 1;
  while (2 * s * c <= 256) s *= 2;
  if (s < wk) s = wk;
  while ((s * c / 16) % 4 != 0) s *= 2;
  return s;
}

// Shape of the MFMA weight-gradient kernel for CIN input channels and a group
// of COLS output columns: CB x OB blocks of 16 x 16 accumulators, split over
// the 4 waves as WA (input-channel blocks) x WB (column blocks) x WK (rounds'
// 32-entry steps, for blocks too small to split).
template <int CIN, int COLS>
struct WgradShape {
  static constexpr int CB = CIN / 16, OB = COLS / 16, NT = CB * OB;
  static constexpr int WA = NT >= 4 ? ((CB >= 2 && OB >= 2) ? 2 : (OB == 1 ? 4 : 1)) : (CB == 2 ? 2 : 1);
  static constexpr int WB = NT >= 4 ? ((CB >= 2 && OB >= 2) ? 2 : (OB == 1 ? 1 : 4)) : (OB == 2 ? 2 : 1);
  static constexpr int WK = 4 / (WA * WB);
  static constexpr int CBW = CB / WA, OBW = OB / WB;
  static constexpr int SUB = wgrad_sub(CIN + COLS, WK);
  static constexpr int ROWS = 32 * SUB;  // entries per round
  // 16-byte pieces per staged row; a copy (64 lanes x 16 bytes) moves
  // 64 / SEG whole rows.
  static constexpr int SEGF = CIN / 8, SEGG = COLS / 8;
  static constexpr int NF = ROWS * SEGF / 64, NG = ROWS * SEGG / 64, NL = NF + NG, NLW = NL / 4;
  static constexpr int F_BYTES = ROWS * CIN * 2;
  static constexpr int STAGE_BYTES = NL * 1024;
  static constexpr int STAGES = NL <= 24 ? 3 : 2;
  // A round's 2 ROWS row indices (feature rows, then gradient rows) are also
  // copied into LDS, a quarter by each wave: IPW of them, in NI copies of
  // 64 lanes; wave w's share sits at IDX_WAVE x w of the round's index area
  // (lanes past IPW load a clamped index into padding).  Three areas rotate.
  static constexpr int IPW = ROWS / 2;
  static constexpr int NI = (IPW + 63) / 64;
  static constexpr int IDX_WAVE = 256 * NI;  // bytes
  static constexpr int IDX_AREA = 4 * IDX_WAVE;
  // Loads of one wave issued after round r's row copies: one step's index and
  // row copies for each of the STAGES - 2 steps in between.
  static constexpr int FULL_WAIT = (NI + NLW) * (STAGES - 2);
  static constexpr size_t lds_bytes() { return static_cast<size_t>(STAGES) * STAGE_BYTES + 3 * IDX_AREA; }
  static_assert(NL % 4 == 0, "copies split evenly over the waves");
  static_assert(WA * WB * WK == 4 && SUB % WK == 0, "wave split");
  static_assert(FULL_WAIT < 64, "vmcnt range");
};

// Position of 16-byte piece c of staged row i: c ^ wg_swz<SEG>(i).  The 16
// rows one transposing read touches (rows 8 g + 4 h + j of a 32-row step,
// g, j in 0..3) then fall on distinct banks in pairs of pieces: the swizzle
// uses only bits 0, 1 and 3 of the row (not h or the step), so a lane's
// swizzle is the same for all its reads.
template <int SEG>
__device__ __forceinline__ int wg_swz(int i) {
  if constexpr (SEG >= 16) return 2 * ((i & 3) + 4 * ((i >> 3) & 1));
  else if constexpr (SEG == 8) return 2 * (((i >> 1) & 1) + 2 * ((i >> 3) & 1));
  else if constexpr (SEG == 4) return 2 * ((i >> 3) & 1);
  else return 0;
}

// Buffer resource word 3 for raw 32-bit-element loads (gfx9 data format 32,
// no swizzle): the bounds check compares each byte offset with the record
// count, the buffer's size in bytes.
constexpr int kBufferWord3 = 0x00020000;
// Largest feature or gradient buffer the row copies address with 32-bit
// byte offsets (a missing row's offset, just below 2^32, must stay past its
// end).
constexpr int64_t kWgradMaxBytes = (int64_t{1} << 32) - 4096;

// Grid: units (tile range p, column group cg, offset k), k fastest, dealt so
// that consecutive units run on one XCD.  Each unit writes the fp32 partial
// part[p][k][ci][col0 + co] of its CIN x COLS block (zeros for no entries).
template <typename T, int CIN, int COLS>
__global__ __launch_bounds__(256) void k_wgrad(const uint16_t* __restrict__ feats, const uint16_t* __restrict__ gout,
                                               const int32_t* __restrict__ in_idx,
                                               const int32_t* __restrict__ out_idx,
                                               const int32_t* __restrict__ tile_off, int64_t tiles, int tpc,
                                               int chunks, int groups, int KV, int cout, int f_rows,
                                               int g_rows, float* __restrict__ part) {
  using S = WgradShape<CIN, COLS>;
  constexpr int NLW = S::NLW, CBW = S::CBW, OBW = S::OBW, SEGF = S::SEGF, SEGG = S::SEGG;
  extern __shared__ uint4 wstage[];  // [STAGES][F rows | G rows]
  const int64_t per_xcd = gridDim.x / 8;
  const int64_t bid = blockIdx.x;
  const int64_t unit = (bid % 8) * per_xcd + bid / 8;
  if (unit >= static_cast<int64_t>(chunks) * groups * KV) return;  // uniform
  const int k = static_cast<int>(unit % KV);
  const int64_t pg = unit / KV;
  const int cg = static_cast<int>(pg % groups);
  const int p = static_cast<int>(pg / groups);
  const int64_t t0 = static_cast<int64_t>(p) * tpc;
  const int64_t t1 = (t0 + tpc < tiles) ? t0 + tpc : tiles;
  const int e0 = tile_off[static_cast<int64_t>(k) * tiles + t0];
  const int e1 = tile_off[static_cast<int64_t>(k) * tiles + t1];
  const int col0 = cg * COLS;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int wk = wave % S::WK, wab = wave / S::WK, wa = wab / S::WB, wb = wab % S::WB;
  const int rounds = (e1 - e0 + S::ROWS - 1) / S::ROWS;

  // This wave's row copies: copy j = wave + 4 ii of a round (the NF
  // feature-row copies first).  Lane l of a copy moves piece (l % SEG) ^
  // swizzle of row (copy's first row) + l / SEG into LDS position l x 16 of
  // the copy's 1 KB.  Per copy: the lane's row in the round, the byte offset
  // of its piece in a source row, the LDS byte offset of its row's index in
  // an index area, and (wave-uniform) the source array, its row pitch and
  // the copy's LDS offset in a stage.
  int c_row[NLW];
  uint32_t c_off[NLW], c_ix[NLW];
  bool c_isf[NLW];
  uint32_t c_pitch[NLW];
  uint32_t c_lds[NLW];
#pragma unroll
  for (int ii = 0; ii < NLW; ++ii) {
    const int j = wave + 4 * ii;
    const bool isf = j < S::NF;
    const int jj = isf ? j : j - S::NF;
    const int rowf = jj * (64 / SEGF) + lane / SEGF, rowg = jj * (64 / SEGG) + lane / SEGG;
    const int cf = (lane % SEGF) ^ wg_swz<SEGF>(rowf), cgp = (lane % SEGG) ^ wg_swz<SEGG>(rowg);
    const int row = isf ? rowf : rowg;
    const int t = isf ? row : S::ROWS + row;  // position in the round's index list
    c_row[ii] = row;
    c_off[ii] = static_cast<uint32_t>(16 * (isf ? cf : cgp));
    c_ix[ii] = static_cast<uint32_t>((t / S::IPW) * S::IDX_WAVE + 4 * (t % S::IPW));
    c_isf[ii] = isf;
    c_pitch[ii] = isf ? 2u * CIN : 2u * static_cast<uint32_t>(cout);
    c_lds[ii] = static_cast<uint32_t>((isf ? 0 : S::F_BYTES) + jj * 1024);
  }
  // Buffer resources over the two sources (32-bit byte offsets; the host
  // keeps both below 2^32 - 4096 bytes): a row past the range's end gets
  // index -1, whose offset wraps past the buffer's end, where the load's
  // bounds check returns zeros.
  const __amdgpu_buffer_rsrc_t frsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(feats), 0, static_cast<int>(static_cast<uint32_t>(f_rows) * (2u * CIN)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t grsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(gout + col0), 0,
      static_cast<int>(static_cast<uint32_t>(g_rows) * (2u * static_cast<uint32_t>(cout)) - 2u * col0), kBufferWord3);
  typedef __attribute__((address_space(3))) uint4 lds_uint4;
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_uint4*)wstage));
  const uint32_t idx_base = lds_base + static_cast<uint32_t>(S::STAGES * S::STAGE_BYTES);
  // Index copies of round r into area `area`: lane l of copy d takes
  // position t = wave x IPW + 64 d + l of the round's list (feature rows'
  // in_idx, then gradient rows' out_idx), its list position clamped to the
  // range (rows past the end are told apart at the row copy).
  auto load_idx = [&](int r, int area) {
#pragma unroll
    for (int d = 0; d < S::NI; ++d) {
      const int l = 64 * d + lane;
      const int t = wave * S::IPW + (l < S::IPW ? l : 0);
      const bool isf = t < S::ROWS;
      const int e = e0 + r * S::ROWS + (isf ? t : t - S::ROWS);
      const int32_t* src = (isf ? in_idx : out_idx) + (e < e1 ? e : e1 - 1);
      uint4* dst = wstage + (static_cast<uint32_t>(S::STAGES * S::STAGE_BYTES + area * S::IDX_AREA +
                                                   wave * S::IDX_WAVE + 256 * d)) / 16;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 4, 0, 0);
    }
  };
  // Row copies of round r into `stage`, their indices read from area `area`
  // (complete and visible: see the pipeline); a row past the range's end
  // takes index -1, which the buffer load's bounds check turns into zeros,
  // as it does any index outside the source, so no copy can leave the
  // arrays.
  auto copy = [&](int r, int stage, int area) {
    int32_t rows[NLW];
    const uint32_t ia = idx_base + static_cast<uint32_t>(area * S::IDX_AREA);
#pragma unroll
    for (int ii = 0; ii < NLW; ++ii)
      asm volatile("ds_read_b32 %0, %1" : "=v"(rows[ii]) : "v"(ia + c_ix[ii]) : "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int ii = 0; ii < NLW; ++ii) asm volatile("" : "+v"(rows[ii]));
#pragma unroll
    for (int ii = 0; ii < NLW; ++ii) {
      const int e = e0 + r * S::ROWS + c_row[ii];
      const int32_t row = e < e1 ? rows[ii] : -1;
      const uint32_t voff = static_cast<uint32_t>(row) * c_pitch[ii] + c_off[ii];
      uint4* dst = wstage + (static_cast<uint32_t>(stage * S::STAGE_BYTES) + c_lds[ii]) / 16;
      if (c_isf[ii]) __builtin_amdgcn_raw_ptr_buffer_load_lds(frsrc, (lds_void*)dst, 16, static_cast<int>(voff), 0, 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(grsrc, (lds_void*)dst, 16, static_cast<int>(voff), 0, 0, 0);
    }
  };

  // Transposing reads: lane (g, i4), j = i4 / 4, q = i4 % 4, reads 4 values
  // at row 32 s + 8 g + 4 h + j, channels 16 blk + 4 q .. + 3 of its area;
  // h = 0, 1 give entries 8 g .. 8 g + 3 and 8 g + 4 .. 8 g + 7 of the MFMA
  // operand of channel (row of A, column of B) 16 blk + i4.
  const int i4 = lane & 15, g = lane >> 4;
  const int rowr = 8 * g + (i4 >> 2);
  const int qq = i4 & 3;
  uint32_t a_off[CBW], b_off[OBW];
  {
    const int swf = wg_swz<SEGF>(rowr) >> 1, swg = wg_swz<SEGG>(rowr) >> 1;
    const uint32_t fa = static_cast<uint32_t>((rowr + 32 * wk) * SEGF * 16 + 8 * qq);
    const uint32_t gb = static_cast<uint32_t>(S::F_BYTES + (rowr + 32 * wk) * SEGG * 16 + 8 * qq);
#pragma unroll
    for (int a = 0; a < CBW; ++a) a_off[a] = lds_base + fa + (static_cast<uint32_t>((wa * CBW + a) ^ swf) << 5);
#pragma unroll
    for (int b = 0; b < OBW; ++b) b_off[b] = lds_base + gb + (static_cast<uint32_t>((wb * OBW + b) ^ swg) << 5);
  }
  floatx4 acc[CBW][OBW];
#pragma unroll
  for (int a = 0; a < CBW; ++a)
#pragma unroll
    for (int b = 0; b < OBW; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int stage) {
    const uint32_t so = static_cast<uint32_t>(stage * S::STAGE_BYTES);
#pragma unroll
    for (int m = 0; m < S::SUB / S::WK; ++m) {
      u32x2 av[CBW][2], bv[OBW][2];
#pragma unroll
      for (int a = 0; a < CBW; ++a) {
        read_tr<0>(a_off[a] + so + (32 * S::WK * m) * SEGF * 16, av[a][0]);
        read_tr<4 * SEGF * 16>(a_off[a] + so + (32 * S::WK * m) * SEGF * 16, av[a][1]);
      }
#pragma unroll
      for (int b = 0; b < OBW; ++b) {
        read_tr<0>(b_off[b] + so + (32 * S::WK * m) * SEGG * 16, bv[b][0]);
        read_tr<4 * SEGG * 16>(b_off[b] + so + (32 * S::WK * m) * SEGG * 16, bv[b][1]);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int a = 0; a < CBW; ++a) asm volatile("" : "+v"(av[a][0]), "+v"(av[a][1]));
#pragma unroll
      for (int b = 0; b < OBW; ++b) asm volatile("" : "+v"(bv[b][0]), "+v"(bv[b][1]));
#pragma unroll
      for (int a = 0; a < CBW; ++a) {
        const uint4 A = make_uint4(av[a][0].x, av[a][0].y, av[a][1].x, av[a][1].y);
#pragma unroll
        for (int b = 0; b < OBW; ++b) {
          const uint4 B = make_uint4(bv[b][0].x, bv[b][0].y, bv[b][1].x, bv[b][1].y);
          acc[a][b] = mfma<T>(A, B, acc[a][b]);
        }
      }
    }
  };

  // Pipeline: round x's rows go to stage x % STAGES and its indices to area
  // x % 3.  Step r waits for round r's rows by count and syncs; that also
  // completes (and, through the barrier, shows every wave) the indices of
  // round r + STAGES - 1, which were issued before round r's rows.  It then
  // copies the indices of round r + STAGES + 1 and the rows of round r +
  // STAGES - 1, and runs round r.  Every step issues the same loads, also for
  // rounds past the end (clamped index copies; zero-row copies into a stage
  // that is not read again), so the count is always exact.  The prologue
  // issues the same sequence as the steps before round 0 would have.
  constexpr int SG = S::STAGES;
  int stage = 0, area = 0;  // stage r % STAGES and area r % 3 of the step's round r
  auto wrap3 = [](int a) { return a >= 3 ? a - 3 : a; };
  if (rounds > 0) {  // (no entries: no loads, a zero partial)
    // indices of rounds 0 .. STAGES, rows of rounds 0 .. STAGES - 2
    load_idx(0, 0);
    load_idx(1, 1);
    wait_vm<0>();
    lds_barrier();
    load_idx(2, 2);
    copy(0, 0, 0);
    if constexpr (SG == 3) {
      lds_barrier();  // every wave's reads of area 0 are done before round 3's indices overwrite it
      load_idx(3, 0);
      copy(1, 1, 1);
    }
  }
  auto step = [&](int r) {
    wait_vm<S::FULL_WAIT>();
    lds_barrier();
    load_idx(r + SG + 1, wrap3(area + SG + 1 - 3 * ((SG + 1) / 3)));
    int st = stage + SG - 1;
    if (st >= SG) st -= SG;
    copy(r + SG - 1, st, wrap3(area + SG - 1));
    compute(stage);
    stage = stage + 1 == SG ? 0 : stage + 1;
    area = area + 1 == 3 ? 0 : area + 1;
  };
  for (int r = 0; r < rounds; ++r) step(r);
  wait_vm<0>();  // no copy into LDS may be left in flight

  // Waves that split the steps (WK > 1) add their sums through LDS, in wave
  // order, into wave wk = 0 of their block.
  if constexpr (S::WK > 1) {
    lds_barrier();  // every wave is done with the stages
    floatx4* red = reinterpret_cast<floatx4*>(wstage);
    if (wk > 0) {
#pragma unroll
      for (int a = 0; a < CBW; ++a)
#pragma unroll
        for (int b = 0; b < OBW; ++b) red[((((wk - 1) * S::WA * S::WB + wab) * CBW + a) * OBW + b) * 64 + lane] = acc[a][b];
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int w = 1; w < S::WK; ++w)
#pragma unroll
      for (int a = 0; a < CBW; ++a)
#pragma unroll
        for (int b = 0; b < OBW; ++b) acc[a][b] += red[((((w - 1) * S::WA * S::WB + wab) * CBW + a) * OBW + b) * 64 + lane];
  }
  // D element (row 4 g + jj, column i4) of block (a, b) is grad_w[k][ci =
  // 16 (wa CBW + a) + 4 g + jj][co = col0 + 16 (wb OBW + b) + i4].
  float* pk = part + (static_cast<int64_t>(p) * KV + k) * CIN * cout;
#pragma unroll
  for (int a = 0; a < CBW; ++a)
#pragma unroll
    for (int b = 0; b < OBW; ++b)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        pk[static_cast<int64_t>(16 * (wa * CBW + a) + 4 * g + jj) * cout + col0 + 16 * (wb * OBW + b) + i4] = acc[a][b][jj];
}

// Any dtype and channel counts (fp32 features, or channels not multiples of
// 16): per step of 32 entries the rows are staged in LDS as fp32, and thread
// t accumulates the products of its (ci, co) pairs of the block of `cols`
// output columns in fp32.  Grid: (tile range, offset, column group); same
// partial layout as k_wgrad.
template <typename T>
__global__ __launch_bounds__(256) void k_wgrad_generic(const T* __restrict__ feats, const T* __restrict__ gout,
                                                       const int32_t* __restrict__ in_idx,
                                                       const int32_t* __restrict__ out_idx,
                                                       const int32_t* __restrict__ tile_off, int64_t tiles, int tpc,
                                                       int KV, int cin, int cout, int cols, float* __restrict__ part) {
  constexpr int kMaxPerThread = 64;
  extern __shared__ float gsm[];  // fs[32][cin], gs[32][cols]
  float* fs = gsm;
  float* gs = gsm + 32 * cin;
  const int k = blockIdx.y;
  const int p = blockIdx.x;
  const int col0 = blockIdx.z * cols;
  const int ncols = (cout - col0 < cols) ? cout - col0 : cols;
  const int64_t t0 = static_cast<int64_t>(p) * tpc;
  const int64_t t1 = (t0 + tpc < tiles) ? t0 + tpc : tiles;
  const int64_t e0 = tile_off[static_cast<int64_t>(k) * tiles + t0];
  const int64_t e1 = tile_off[static_cast<int64_t>(k) * tiles + t1];
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
  float* pk = part + (static_cast<int64_t>(p) * KV + k) * cin * cout;
#pragma unroll
  for (int i = 0; i < kMaxPerThread; ++i) {
    const int pidx = tid + 256 * i;
    if (pidx < pairs) {
      const int ci = pidx / ncols, co = pidx % ncols;
      pk[static_cast<int64_t>(ci) * cout + col0 + co] = acc[i];
    }
  }
}

// grad_w[k][i] = sum over the tile ranges p of part[p][k][i], in range order.
__global__ __launch_bounds__(256) void k_wgrad_reduce(const float* __restrict__ part, int chunks, int KV,
                                                      int64_t per_k, float* __restrict__ grad_w) {
  const int k = blockIdx.y;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= per_k) return;
  float s = 0.f;
  for (int c = 0; c < chunks; ++c) s += part[(static_cast<int64_t>(c) * KV + k) * per_k + i];
  grad_w[static_cast<int64_t>(k) * per_k + i] = s;
}

template <typename T>
hipError_t launch_mirror(const T* w, T* wt, int KV, int cin, int cout, hipStream_t stream) {
  const int64_t grid = static_cast<int64_t>(KV) * ((cin + 31) / 32) * ((cout + 31) / 32);
  hipLaunchKernelGGL(k_mirror_transpose<T>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, w, wt, KV, cin,
                     cout);
  return hipGetLastError();
}

// How a weight gradient is cut: the kernel, its group of output columns, and
// the tile ranges (tpc tiles each, `chunks` of them).
struct WgradPlan {
  bool mfma = false;
  int cols = 0;
  int groups = 0;
  int tpc = 0;
  int chunks = 0;
};

// About this many (range, column group, offset) units per launch: several
// per CU in flight, few enough that the partial sums stay small next to the
// gathered rows.
constexpr int64_t kWgradUnits = 2048;

bool wgrad_mfma_shape(const WgradArgs& a, int cols) {
  if (a.dtype != 1 && a.dtype != 2) return false;
  if (a.cin != 16 && a.cin != 32 && a.cin != 64 && a.cin != 128 && a.cin != 256) return false;
  if (a.cout % 16 != 0) return false;
  if (a.n_in * a.cin * 2 > kWgradMaxBytes || a.n * a.cout * 2 > kWgradMaxBytes) return false;
  return !(a.cin == 256 && cols == 16);
}

WgradPlan wgrad_plan(const WgradArgs& a) {
  WgradPlan pl;
  int cols = 16;
  for (int c : {128, 64, 32}) {
    if (a.cout % c == 0) {
      cols = c;
      break;
    }
  }
  pl.mfma = wgrad_mfma_shape(a, cols);
  if (!pl.mfma) {
    // at most 64 (ci, co) pairs per thread
    cols = a.cout;
    while (static_cast<int64_t>(a.cin) * cols > 64 * 256) cols = (cols + 1) / 2;
  }
  pl.cols = cols;
  pl.groups = (a.cout + cols - 1) / cols;
  const int64_t tiles = a.tiles > 0 ? a.tiles : 1;
  int64_t chunks = kWgradUnits / (static_cast<int64_t>(a.KV) * pl.groups);
  if (chunks < 1) chunks = 1;
  if (chunks > tiles) chunks = tiles;
  pl.tpc = static_cast<int>((tiles + chunks - 1) / chunks);
  pl.chunks = static_cast<int>((tiles + pl.tpc - 1) / pl.tpc);
  return pl;
}

template <typename T, int CIN, int COLS>
hipError_t launch_wgrad_mfma(const WgradArgs& a, const WgradPlan& pl, float* part, hipStream_t stream) {
  using S = WgradShape<CIN, COLS>;
  static bool raised = false;  // launches run under the library's cache lock
  if (!raised) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_wgrad<T, CIN, COLS>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(S::lds_bytes()));
    if (e != hipSuccess) return e;
    raised = true;
  }
  const int64_t units = static_cast<int64_t>(pl.chunks) * pl.groups * a.KV;
  const int64_t grid = (units + 7) / 8 * 8;  // a multiple of 8 (the XCD remapping)
  hipLaunchKernelGGL((k_wgrad<T, CIN, COLS>), dim3(static_cast<unsigned>(grid)), dim3(256), S::lds_bytes(), stream,
                     static_cast<const uint16_t*>(a.feats), static_cast<const uint16_t*>(a.grad_out), a.in_idx,
                     a.out_idx, a.tile_off, a.tiles, pl.tpc, pl.chunks, pl.groups, a.KV, a.cout,
                     static_cast<int>(a.n_in), static_cast<int>(a.n), part);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_wgrad_cin(const WgradArgs& a, const WgradPlan& pl, float* part, hipStream_t stream) {
  switch (a.cin * 1000 + pl.cols) {
    case 16016: return launch_wgrad_mfma<T, 16, 16>(a, pl, part, stream);
    case 16032: return launch_wgrad_mfma<T, 16, 32>(a, pl, part, stream);
    case 16064: return launch_wgrad_mfma<T, 16, 64>(a, pl, part, stream);
    case 16128: return launch_wgrad_mfma<T, 16, 128>(a, pl, part, stream);
    case 32016: return launch_wgrad_mfma<T, 32, 16>(a, pl, part, stream);
    case 32032: return launch_wgrad_mfma<T, 32, 32>(a, pl, part, stream);
    case 32064: return launch_wgrad_mfma<T, 32, 64>(a, pl, part, stream);
    case 32128: return launch_wgrad_mfma<T, 32, 128>(a, pl, part, stream);
    case 64016: return launch_wgrad_mfma<T, 64, 16>(a, pl, part, stream);
    case 64032: return launch_wgrad_mfma<T, 64, 32>(a, pl, part, stream);
    case 64064: return launch_wgrad_mfma<T, 64, 64>(a, pl, part, stream);
    case 64128: return launch_wgrad_mfma<T, 64, 128>(a, pl, part, stream);
    case 128016: return launch_wgrad_mfma<T, 128, 16>(a, pl, part, stream);
    case 128032: return launch_wgrad_mfma<T, 128, 32>(a, pl, part, stream);
    case 128064: return launch_wgrad_mfma<T, 128, 64>(a, pl, part, stream);
    case 128128: return launch_wgrad_mfma<T, 128, 128>(a, pl, part, stream);
    case 256032: return launch_wgrad_mfma<T, 256, 32>(a, pl, part, stream);
    case 256064: return launch_wgrad_mfma<T, 256, 64>(a, pl, part, stream);
    case 256128: return launch_wgrad_mfma<T, 256, 128>(a, pl, part, stream);
    default: return hipErrorNotSupported;
  }
}

template <typename T>
hipError_t launch_wgrad_generic(const WgradArgs& a, const WgradPlan& pl, float* part, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(pl.chunks), static_cast<unsigned>(a.KV), static_cast<unsigned>(pl.groups));
  const size_t lds = static_cast<size_t>(32) * (a.cin + pl.cols) * sizeof(float);
  static bool raised = false;
  if (!raised) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_wgrad_generic<T>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    raised = true;
  }
  hipLaunchKernelGGL(k_wgrad_generic<T>, grid, dim3(256), lds, stream, static_cast<const T*>(a.feats),
                     static_cast<const T*>(a.grad_out), a.in_idx, a.out_idx, a.tile_off, a.tiles, pl.tpc, a.KV,
                     a.cin, a.cout, pl.cols, part);
  return hipGetLastError();
}

}  // namespace

size_t wgrad_workspace_bytes(const WgradArgs& a) {
  const WgradPlan pl = wgrad_plan(a);
  return static_cast<size_t>(pl.chunks) * a.KV * a.cin * a.cout * sizeof(float);
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
  const WgradPlan pl = wgrad_plan(a);
  hipError_t e;
  if (pl.mfma) {
    e = (a.dtype == 1) ? launch_wgrad_cin<_Float16>(a, pl, part, stream)
                       : launch_wgrad_cin<__bf16>(a, pl, part, stream);
  } else if (a.dtype == 0) {
    e = launch_wgrad_generic<float>(a, pl, part, stream);
  } else if (a.dtype == 1) {
    e = launch_wgrad_generic<_Float16>(a, pl, part, stream);
  } else {
    e = launch_wgrad_generic<__bf16>(a, pl, part, stream);
  }
  if (e != hipSuccess) return e;
  const int64_t per_k = static_cast<int64_t>(a.cin) * a.cout;
  hipLaunchKernelGGL(k_wgrad_reduce, dim3(static_cast<unsigned>((per_k + 255) / 256), static_cast<unsigned>(a.KV)),
                     dim3(256), 0, stream, part, pl.chunks, a.KV, per_k, a.grad_w);
  return hipGetLastError();
}

}  // namespace spconv
