// TEST INFRASTRUCTURE ONLY — the oracle for submanifold sparse convolution.
//
// A plain, slow, obviously correct CPU implementation of what the GPU path
// computes.  Only the tests, the smoke check and the bench's CPU-baseline leg
// load it; the product path never does.  It shares no code, header, table or
// helper with the GPU library.
//
// What it follows (page titles as published; sections named on each page):
//  * Map ("kernel map" / "rulebook"): "Sparse inputs and sparse convolution",
//    sections "The map is the computation" (for each output q and offset d,
//    look up q + d; a hit p joins the map as (p, q, W_d)) and "The fix: compute
//    only where an input exists" (submanifold rule: the outputs are exactly the
//    inputs).  Offset sign from "Sparse convolution for point clouds", section
//    "The map and the update rule" (input P = output Q + offset), which is also
//    the GetOffset result of section 3 of the SparseConvNet blog
//    ("编织计算规则：Rulebook的生成与核心作用": offset = input - output).
//  * Coordinate table: SparseConvNet blog, section 2 ("构建计算地图"): one
//    increasing index per unique coordinate.  Here an ordered tree, on purpose
//    not a hash, so it cannot share the GPU's packing or probing.
//  * Forward: "Sparse convolution for point clouds", section "The map and the
//    update rule": for every entry, f_out(Q) += f_in(P) x W_d, starting from
//    zero, no bias.  Evaluated in fp64 on the exactly widened stored inputs.
//
// Conventions (the readings the pages leave open):
//  * coordinates are (b, z, y, x); b in [0, 2^15), z, y, x in [0, 2^16);
//  * offset index k = ((dz + r) K + (dy + r)) K + (dx + r), r = (K - 1) / 2;
//  * entries never cross batch index b;
//  * a neighbour coordinate outside the active set is a miss (no wrap);
//  * duplicate coordinates are an error, not merged.
//
// Build: g++ -O2 -std=c++17 -fopenmp -shared -fPIC (no fast-math: the fp64
// sums keep their written order).

#include <omp.h>

#include <algorithm>
#include <array>
#include <cstddef>
#include <cstdint>
#include <map>
#include <new>
#include <vector>

namespace {

enum OracleStatus : int {
  kOk = 0,
  kInvalidArg = 1,
  kDuplicateCoord = 2,
  kCoordRange = 3,
};

using Coord = std::array<int64_t, 4>;  // (b, z, y, x)

struct OracleMap {
  int32_t K = 0;
  int64_t N = 0;      // rows of the input side
  int64_t N_out = 0;  // rows of the output side (N for a submanifold map)
  int32_t stride = 1;
  int32_t kind = 0;   // 0 submanifold, 1 strided, 2 transposed strided
  std::vector<Coord> coords;                     // input side
  std::map<Coord, int64_t> row_of;               // input coordinate -> row index
  std::vector<Coord> out_coords;                 // output side (strided and transposed maps)
  std::map<Coord, int64_t> out_row_of;           // output coordinate -> row index
  std::vector<std::vector<int32_t>> in_idx;      // per offset k
  std::vector<std::vector<int32_t>> out_idx;     // per offset k
};

// Offset (dz, dy, dx) of index k for an odd kernel size K.
void offset_of(int32_t k, int32_t K, int64_t* dz, int64_t* dy, int64_t* dx) {
  const int32_t r = (K - 1) / 2;
  *dz = k / (K * K) - r;
  *dy = (k / K) % K - r;
  *dx = k % K - r;
}

// Offset (dz, dy, dx) of index k for any kernel size K: each component runs
// over lo .. lo + K - 1 with lo = -floor((K - 1) / 2), so odd sizes are
// centred (the same offsets as offset_of) and K = 2 covers 0 and 1.
int64_t offset_low(int32_t K) { return -static_cast<int64_t>((K - 1) / 2); }
void offset_of_any(int32_t k, int32_t K, int64_t* dz, int64_t* dy, int64_t* dx) {
  const int64_t lo = offset_low(K);
  *dz = k / (K * K) + lo;
  *dy = (k / K) % K + lo;
  *dx = k % K + lo;
}

// Validates coordinates and fills a coordinate -> row table; 0 or a status.
int fill_table(const int32_t* coords, int64_t N, std::vector<Coord>* rows, std::map<Coord, int64_t>* table) {
  rows->resize(static_cast<size_t>(N));
  for (int64_t i = 0; i < N; ++i) {
    Coord c = {coords[4 * i + 0], coords[4 * i + 1], coords[4 * i + 2], coords[4 * i + 3]};
    if (c[0] < 0 || c[0] >= (int64_t(1) << 15)) return kCoordRange;
    for (int d = 1; d < 4; ++d) {
      if (c[d] < 0 || c[d] >= (int64_t(1) << 16)) return kCoordRange;
    }
    (*rows)[static_cast<size_t>(i)] = c;
  }
  for (int64_t i = 0; i < N; ++i) {
    if (!table->emplace((*rows)[static_cast<size_t>(i)], i).second) return kDuplicateCoord;
  }
  return kOk;
}

}  // namespace

extern "C" {

// Builds the map of a submanifold convolution with a K^3 kernel over the N
// voxels in coords (row-major int32 [N][4], (b, z, y, x)).  Returns a status;
// on success *out holds an opaque handle to release with oracle_map_free.
int oracle_build_map_impl(const int32_t* coords, int64_t N, int32_t K, bool with_lists, void** out);

int oracle_build_map(const int32_t* coords, int64_t N, int32_t K, void** out) {
  return oracle_build_map_impl(coords, N, K, true, out);
}

// The coordinate table only (step 1 below), for row-at-a-time evaluation with
// oracle_forward_rows / oracle_neighbours on inputs too large for the full
// double loop; the per-offset lists stay empty.
int oracle_build_table(const int32_t* coords, int64_t N, int32_t K, void** out) {
  return oracle_build_map_impl(coords, N, K, false, out);
}

int oracle_build_map_impl(const int32_t* coords, int64_t N, int32_t K, bool with_lists, void** out) {
  if (out == nullptr) return kInvalidArg;
  *out = nullptr;
  if (coords == nullptr || N <= 0 || K < 1 || K % 2 == 0) return kInvalidArg;
  OracleMap* m = new (std::nothrow) OracleMap;
  if (m == nullptr) return kInvalidArg;
  m->K = K;
  m->N = N;
  m->N_out = N;
  m->coords.resize(static_cast<size_t>(N));
  // Step 1: validate ranges and fill the coordinate -> row table.
  for (int64_t i = 0; i < N; ++i) {
    Coord c = {coords[4 * i + 0], coords[4 * i + 1], coords[4 * i + 2], coords[4 * i + 3]};
    if (c[0] < 0 || c[0] >= (int64_t(1) << 15)) { delete m; return kCoordRange; }
    for (int d = 1; d < 4; ++d) {
      if (c[d] < 0 || c[d] >= (int64_t(1) << 16)) { delete m; return kCoordRange; }
    }
    m->coords[static_cast<size_t>(i)] = c;
  }
  for (int64_t i = 0; i < N; ++i) {
    auto ins = m->row_of.emplace(m->coords[static_cast<size_t>(i)], i);
    if (!ins.second) { delete m; return kDuplicateCoord; }
  }
  // Step 2: the double loop over outputs q and offsets k with a lookup of
  // q + d; a hit p adds (in = p, out = q) to list k.
  const int32_t KV = K * K * K;
  m->in_idx.assign(static_cast<size_t>(KV), {});
  m->out_idx.assign(static_cast<size_t>(KV), {});
  for (int64_t q = 0; with_lists && q < N; ++q) {
    const Coord& cq = m->coords[static_cast<size_t>(q)];
    for (int32_t k = 0; k < KV; ++k) {
      int64_t dz, dy, dx;
      offset_of(k, K, &dz, &dy, &dx);
      const Coord p = {cq[0], cq[1] + dz, cq[2] + dy, cq[3] + dx};
      auto it = m->row_of.find(p);
      if (it != m->row_of.end()) {
        m->in_idx[static_cast<size_t>(k)].push_back(static_cast<int32_t>(it->second));
        m->out_idx[static_cast<size_t>(k)].push_back(static_cast<int32_t>(q));
      }
    }
  }
  *out = m;
  return kOk;
}

void oracle_map_free(void* h) { delete static_cast<OracleMap*>(h); }

int32_t oracle_map_kernel(const void* h) { return static_cast<const OracleMap*>(h)->K; }

// Number of entries in the list of offset k (-1 if k is out of range).
int64_t oracle_map_count(const void* h, int32_t k) {
  const OracleMap* m = static_cast<const OracleMap*>(h);
  if (k < 0 || k >= static_cast<int32_t>(m->in_idx.size())) return -1;
  return static_cast<int64_t>(m->in_idx[static_cast<size_t>(k)].size());
}

// Copies list k into caller buffers of oracle_map_count(h, k) entries each.
// The list is ordered by output row (the order of the double loop).
int oracle_map_list(const void* h, int32_t k, int32_t* in_idx, int32_t* out_idx) {
  const OracleMap* m = static_cast<const OracleMap*>(h);
  if (k < 0 || k >= static_cast<int32_t>(m->in_idx.size())) return kInvalidArg;
  const auto& a = m->in_idx[static_cast<size_t>(k)];
  const auto& b = m->out_idx[static_cast<size_t>(k)];
  for (size_t e = 0; e < a.size(); ++e) { in_idx[e] = a[e]; out_idx[e] = b[e]; }
  return kOk;
}

// The forward over the whole map: out[N][Cout] = sum over k, over entries
// (j, q) of list k, of feats[j][:] x W[k] (W[k] is Cin x Cout, row-major), in
// fp64, from zero.  feats is [N][Cin], weights is [K^3][Cin][Cout].
int oracle_forward(const void* h, const double* feats, const double* weights,
                   int32_t Cin, int32_t Cout, double* out) {
  const OracleMap* m = static_cast<const OracleMap*>(h);
  if (feats == nullptr || weights == nullptr || out == nullptr || Cin <= 0 || Cout <= 0) {
    return kInvalidArg;
  }
  for (int64_t i = 0; i < m->N_out * Cout; ++i) out[i] = 0.0;
  const int32_t KV = m->K * m->K * m->K;
  for (int32_t k = 0; k < KV; ++k) {
    const auto& ins = m->in_idx[static_cast<size_t>(k)];
    const auto& outs = m->out_idx[static_cast<size_t>(k)];
    const double* Wk = weights + static_cast<int64_t>(k) * Cin * Cout;
    for (size_t e = 0; e < ins.size(); ++e) {
      const double* fj = feats + static_cast<int64_t>(ins[e]) * Cin;
      double* oq = out + static_cast<int64_t>(outs[e]) * Cout;
      for (int32_t ci = 0; ci < Cin; ++ci) {
        for (int32_t co = 0; co < Cout; ++co) {
          oq[co] += fj[ci] * Wk[static_cast<int64_t>(ci) * Cout + co];
        }
      }
    }
  }
  return kOk;
}

// The timing variant of oracle_forward: the same sums, split over output rows
// across `threads` OpenMP threads (0: the runtime's default).  Each thread owns
// a contiguous range of output rows and writes only those, so the variant is
// write-disjoint, and every output value receives the same terms in the same
// order as in oracle_forward (offsets ascending; an output row has at most one
// entry per offset), so the two agree bit for bit.  Within offset k the
// thread's entries are a contiguous run of list k, found by binary search on
// the list's increasing output rows.
int oracle_forward_parallel(const void* h, const double* feats, const double* weights,
                            int32_t Cin, int32_t Cout, double* out, int32_t threads) {
  const OracleMap* m = static_cast<const OracleMap*>(h);
  if (feats == nullptr || weights == nullptr || out == nullptr || Cin <= 0 || Cout <= 0 ||
      threads < 0) {
    return kInvalidArg;
  }
  const int32_t KV = m->K * m->K * m->K;
  const int64_t N = m->N_out;  // output rows, split over the threads
  const int nt = threads > 0 ? threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
  {
    const int64_t t = omp_get_thread_num(), T = omp_get_num_threads();
    const int64_t q_lo = N * t / T, q_hi = N * (t + 1) / T;
    for (int64_t i = q_lo * Cout; i < q_hi * Cout; ++i) out[i] = 0.0;
    for (int32_t k = 0; k < KV; ++k) {
      const auto& ins = m->in_idx[static_cast<size_t>(k)];
      const auto& outs = m->out_idx[static_cast<size_t>(k)];
      const auto first = std::lower_bound(outs.begin(), outs.end(), q_lo);
      const auto last = std::lower_bound(first, outs.end(), q_hi);
      const double* Wk = weights + static_cast<int64_t>(k) * Cin * Cout;
      for (auto it = first; it != last; ++it) {
        const size_t e = static_cast<size_t>(it - outs.begin());
        const double* fj = feats + static_cast<int64_t>(ins[e]) * Cin;
        double* oq = out + static_cast<int64_t>(outs[e]) * Cout;
        for (int32_t ci = 0; ci < Cin; ++ci) {
          for (int32_t co = 0; co < Cout; ++co) {
            oq[co] += fj[ci] * Wk[static_cast<int64_t>(ci) * Cout + co];
          }
        }
      }
    }
  }
  return kOk;
}

// Gradient of the forward with respect to its input features, by the chain
// rule of the forward's sum ("Sparse convolution for point clouds", section
// "The map and the update rule": each entry (P, Q, W_d) adds f_in(P) x W_d to
// f_out(Q), so it adds grad_out(Q) x W_d^T to grad_in(P)):
//   grad_in[j][ci] = sum over k, over entries (j, q) of list k, over co of
//                    grad_out[q][co] x W[k][ci][co]
// in fp64, from zero.  grad_out is [N][Cout], grad_in [N][Cin].
int oracle_backward_data(const void* h, const double* grad_out, const double* weights,
                         int32_t Cin, int32_t Cout, double* grad_in) {
  const OracleMap* m = static_cast<const OracleMap*>(h);
  if (grad_out == nullptr || weights == nullptr || grad_in == nullptr || Cin <= 0 || Cout <= 0) {
    return kInvalidArg;
  }
  for (int64_t i = 0; i < m->N * Cin; ++i) grad_in[i] = 0.0;
  const int32_t KV = m->K * m->K * m->K;
  for (int32_t k = 0; k < KV; ++k) {
    const auto& ins = m->in_idx[static_cast<size_t>(k)];
    const auto& outs = m->out_idx[static_cast<size_t>(k)];
    const double* Wk = weights + static_cast<int64_t>(k) * Cin * Cout;
    for (size_t e = 0; e < ins.size(); ++e) {
      const double* gq = grad_out + static_cast<int64_t>(outs[e]) * Cout;
      double* gj = grad_in + static_cast<int64_t>(ins[e]) * Cin;
      for (int32_t ci = 0; ci < Cin; ++ci) {
        for (int32_t co = 0; co < Cout; ++co) {
          gj[ci] += gq[co] * Wk[static_cast<int64_t>(ci) * Cout + co];
        }
      }
    }
  }
  return kOk;
}

// Gradient of the forward with respect to the weights, by the same chain
// rule: each entry (j, q) of list k adds the outer product f_in[j] x
// grad_out[q] to W[k]'s gradient:
//   grad_w[k][ci][co] = sum over entries (j, q) of list k of
//                       feats[j][ci] x grad_out[q][co]
// in fp64, from zero.  feats is [N][Cin], grad_out [N][Cout], grad_w
// [K^3][Cin][Cout].
int oracle_backward_weights(const void* h, const double* feats, const double* grad_out,
                            int32_t Cin, int32_t Cout, double* grad_w) {
  const OracleMap* m = static_cast<const OracleMap*>(h);
  if (feats == nullptr || grad_out == nullptr || grad_w == nullptr || Cin <= 0 || Cout <= 0) {
    return kInvalidArg;
  }
  const int32_t KV = m->K * m->K * m->K;
  for (int64_t i = 0; i < static_cast<int64_t>(KV) * Cin * Cout; ++i) grad_w[i] = 0.0;
  for (int32_t k = 0; k < KV; ++k) {
    const auto& ins = m->in_idx[static_cast<size_t>(k)];
    const auto& outs = m->out_idx[static_cast<size_t>(k)];
    double* Gk = grad_w + static_cast<int64_t>(k) * Cin * Cout;
    for (size_t e = 0; e < ins.size(); ++e) {
      const double* fj = feats + static_cast<int64_t>(ins[e]) * Cin;
      const double* gq = grad_out + static_cast<int64_t>(outs[e]) * Cout;
      for (int32_t ci = 0; ci < Cin; ++ci) {
        for (int32_t co = 0; co < Cout; ++co) {
          Gk[static_cast<int64_t>(ci) * Cout + co] += fj[ci] * gq[co];
        }
      }
    }
  }
  return kOk;
}

// The timing and large-input variant of oracle_backward_weights: the offsets
// split over `threads` OpenMP threads (0: the runtime's default), each
// thread writing only its offsets' gradients with the same terms in the same
// order, so the result is bit-identical to oracle_backward_weights.
int oracle_backward_weights_parallel(const void* h, const double* feats, const double* grad_out,
                                     int32_t Cin, int32_t Cout, double* grad_w, int32_t threads) {
  const OracleMap* m = static_cast<const OracleMap*>(h);
  if (feats == nullptr || grad_out == nullptr || grad_w == nullptr || Cin <= 0 || Cout <= 0 || threads < 0) {
    return kInvalidArg;
  }
  const int32_t KV = m->K * m->K * m->K;
  const int nt = threads > 0 ? threads : omp_get_max_threads();
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
  for (int32_t k = 0; k < KV; ++k) {
    const auto& ins = m->in_idx[static_cast<size_t>(k)];
    const auto& outs = m->out_idx[static_cast<size_t>(k)];
    double* Gk = grad_w + static_cast<int64_t>(k) * Cin * Cout;
    for (int64_t i = 0; i < static_cast<int64_t>(Cin) * Cout; ++i) Gk[i] = 0.0;
    for (size_t e = 0; e < ins.size(); ++e) {
      const double* fj = feats + static_cast<int64_t>(ins[e]) * Cin;
      const double* gq = grad_out + static_cast<int64_t>(outs[e]) * Cout;
      for (int32_t ci = 0; ci < Cin; ++ci) {
        for (int32_t co = 0; co < Cout; ++co) {
          Gk[static_cast<int64_t>(ci) * Cout + co] += fj[ci] * gq[co];
        }
      }
    }
  }
  return kOk;
}

// Threads oracle_forward_parallel uses when asked for the default.
int32_t oracle_max_threads(void) { return omp_get_max_threads(); }

// The same definition evaluated for selected output rows only, straight from
// the coordinate table: out[i][:] = sum over offsets d with q_i + d active of
// feats[row(q_i + d)][:] x W[k(d)].  Used where the whole map is too large to
// evaluate in seconds.  rows holds n_rows output row indices.
int oracle_forward_rows(const void* h, const double* feats, const double* weights,
                        int32_t Cin, int32_t Cout, const int64_t* rows, int64_t n_rows,
                        double* out) {
  const OracleMap* m = static_cast<const OracleMap*>(h);
  if (feats == nullptr || weights == nullptr || out == nullptr || rows == nullptr ||
      Cin <= 0 || Cout <= 0 || n_rows < 0) {
    return kInvalidArg;
  }
  const int32_t KV = m->K * m->K * m->K;
  for (int64_t i = 0; i < n_rows; ++i) {
    const int64_t q = rows[i];
    if (q < 0 || q >= m->N) return kInvalidArg;
    double* oq = out + i * Cout;
    for (int32_t co = 0; co < Cout; ++co) oq[co] = 0.0;
    const Coord& cq = m->coords[static_cast<size_t>(q)];
    for (int32_t k = 0; k < KV; ++k) {
      int64_t dz, dy, dx;
      offset_of(k, m->K, &dz, &dy, &dx);
      auto it = m->row_of.find(Coord{cq[0], cq[1] + dz, cq[2] + dy, cq[3] + dx});
      if (it == m->row_of.end()) continue;
      const double* fj = feats + it->second * Cin;
      const double* Wk = weights + static_cast<int64_t>(k) * Cin * Cout;
      for (int32_t ci = 0; ci < Cin; ++ci) {
        for (int32_t co = 0; co < Cout; ++co) {
          oq[co] += fj[ci] * Wk[static_cast<int64_t>(ci) * Cout + co];
        }
      }
    }
  }
  return kOk;
}

// Neighbour rows of selected outputs: nbr[i][k] = row of q_i + d(k), or -1.
int oracle_neighbours(const void* h, const int64_t* rows, int64_t n_rows, int32_t* nbr) {
  const OracleMap* m = static_cast<const OracleMap*>(h);
  if (rows == nullptr || nbr == nullptr || n_rows < 0) return kInvalidArg;
  const int32_t KV = m->K * m->K * m->K;
  for (int64_t i = 0; i < n_rows; ++i) {
    const int64_t q = rows[i];
    if (q < 0 || q >= m->N) return kInvalidArg;
    const Coord& cq = m->coords[static_cast<size_t>(q)];
    for (int32_t k = 0; k < KV; ++k) {
      int64_t dz, dy, dx;
      offset_of(k, m->K, &dz, &dy, &dx);
      auto it = m->row_of.find(Coord{cq[0], cq[1] + dz, cq[2] + dy, cq[3] + dx});
      nbr[i * KV + k] = (it == m->row_of.end()) ? -1 : static_cast<int32_t>(it->second);
    }
  }
  return kOk;
}

// ---- Strided maps ("Sparse inputs and sparse convolution", section "The map
// is the computation": for each output q and offset d, look up s q + d; a hit
// p joins the map as (p, q, W_d)) with the regular output definition of the
// SparseConvNet blog, section 2 ("常规输出定义": an output is computed where
// the kernel covers at least one active input).  Here the outputs are the
// q >= 0 (in z, y, x; same batch) with an input at s q + d for some offset d
// of the K^3 kernel (components lo .. lo + K - 1, offset_of_any), in
// lexicographic (b, z, y, x) order; q must be representable (< 2^16).
int oracle_build_map_strided(const int32_t* coords, int64_t N, int32_t K, int32_t stride, void** out) {
  if (out == nullptr) return kInvalidArg;
  *out = nullptr;
  if (coords == nullptr || N <= 0 || K < 1 || K > 7 || stride < 1 || stride > 16) return kInvalidArg;
  OracleMap* m = new (std::nothrow) OracleMap;
  if (m == nullptr) return kInvalidArg;
  m->K = K;
  m->N = N;
  m->stride = stride;
  m->kind = 1;
  // Step 1: the input table.
  const int st = fill_table(coords, N, &m->coords, &m->row_of);
  if (st != kOk) { delete m; return st; }
  // Step 2: the output set, from every (input, offset) pair that lands on a
  // grid point s q: q = (p - d) / s when that divides and is >= 0.
  const int32_t KV = K * K * K;
  std::map<Coord, int64_t> outs;
  for (const Coord& p : m->coords) {
    for (int32_t k = 0; k < KV; ++k) {
      int64_t d[3];
      offset_of_any(k, K, &d[0], &d[1], &d[2]);
      Coord q = {p[0], 0, 0, 0};
      bool ok = true;
      for (int i = 0; i < 3; ++i) {
        const int64_t v = p[1 + i] - d[i];
        if (v < 0 || v % stride != 0 || v / stride >= (int64_t(1) << 16)) { ok = false; break; }
        q[1 + i] = v / stride;
      }
      if (ok) outs.emplace(q, 0);
    }
  }
  int64_t row = 0;
  for (auto& kv : outs) {
    kv.second = row++;
    m->out_coords.push_back(kv.first);
  }
  m->out_row_of = std::move(outs);
  m->N_out = row;
  // Step 3: the double loop over outputs q (in order) and offsets k with a
  // lookup of s q + d; a hit p adds (in = p, out = q) to list k.
  m->in_idx.assign(static_cast<size_t>(KV), {});
  m->out_idx.assign(static_cast<size_t>(KV), {});
  for (int64_t q = 0; q < m->N_out; ++q) {
    const Coord& cq = m->out_coords[static_cast<size_t>(q)];
    for (int32_t k = 0; k < KV; ++k) {
      int64_t dz, dy, dx;
      offset_of_any(k, K, &dz, &dy, &dx);
      const Coord p = {cq[0], stride * cq[1] + dz, stride * cq[2] + dy, stride * cq[3] + dx};
      auto it = m->row_of.find(p);
      if (it != m->row_of.end()) {
        m->in_idx[static_cast<size_t>(k)].push_back(static_cast<int32_t>(it->second));
        m->out_idx[static_cast<size_t>(k)].push_back(static_cast<int32_t>(q));
      }
    }
  }
  *out = m;
  return kOk;
}

// The transpose of a strided map (the upsampling convolution): its outputs
// are the strided map's inputs (in their order) and its inputs the strided
// map's outputs.  Built from its own definition, not by swapping the lists:
// for each output j (input p_j of the strided map) and offset k, the input is
// the strided output q with s q + d = p_j, i.e. q = (p_j - d) / s when that
// divides, is >= 0 and is an output; the entry is (in = q, out = j).
int oracle_transpose_map(const void* h, void** out) {
  if (out == nullptr) return kInvalidArg;
  *out = nullptr;
  const OracleMap* m = static_cast<const OracleMap*>(h);
  if (m == nullptr || m->kind != 1) return kInvalidArg;
  OracleMap* t = new (std::nothrow) OracleMap;
  if (t == nullptr) return kInvalidArg;
  t->K = m->K;
  t->stride = m->stride;
  t->kind = 2;
  t->N = m->N_out;
  t->N_out = m->N;
  t->coords = m->out_coords;
  t->row_of = m->out_row_of;
  t->out_coords = m->coords;
  t->out_row_of = m->row_of;
  const int32_t K = m->K, KV = K * K * K, s = m->stride;
  t->in_idx.assign(static_cast<size_t>(KV), {});
  t->out_idx.assign(static_cast<size_t>(KV), {});
  for (int64_t j = 0; j < t->N_out; ++j) {
    const Coord& pj = t->out_coords[static_cast<size_t>(j)];
    for (int32_t k = 0; k < KV; ++k) {
      int64_t d[3];
      offset_of_any(k, K, &d[0], &d[1], &d[2]);
      Coord q = {pj[0], 0, 0, 0};
      bool ok = true;
      for (int i = 0; i < 3; ++i) {
        const int64_t v = pj[1 + i] - d[i];
        if (v < 0 || v % s != 0) { ok = false; break; }
        q[1 + i] = v / s;
      }
      if (!ok) continue;
      auto it = t->row_of.find(q);
      if (it != t->row_of.end()) {
        t->in_idx[static_cast<size_t>(k)].push_back(static_cast<int32_t>(it->second));
        t->out_idx[static_cast<size_t>(k)].push_back(static_cast<int32_t>(j));
      }
    }
  }
  *out = t;
  return kOk;
}

// Rows of the input and output sides, and the stride.
int64_t oracle_map_rows_in(const void* h) { return static_cast<const OracleMap*>(h)->N; }
int64_t oracle_map_rows_out(const void* h) { return static_cast<const OracleMap*>(h)->N_out; }
int32_t oracle_map_stride(const void* h) { return static_cast<const OracleMap*>(h)->stride; }

// Output coordinates of a strided or transposed map into [N_out][4] (b, z, y, x).
int oracle_map_out_coords(const void* h, int32_t* out) {
  const OracleMap* m = static_cast<const OracleMap*>(h);
  if (out == nullptr || m->kind == 0) return kInvalidArg;
  for (size_t i = 0; i < m->out_coords.size(); ++i) {
    for (int d = 0; d < 4; ++d) out[4 * i + d] = static_cast<int32_t>(m->out_coords[i][static_cast<size_t>(d)]);
  }
  return kOk;
}

}  // extern "C"
