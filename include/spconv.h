/*
 * spconv.h — C ABI of the MI355X (gfx950) submanifold sparse convolution library.
 *
 * The operation (page titles as published, section names on each page):
 *
 *   Sparse tensor: a coordinate list of active voxels (b, z, y, x) and a
 *   feature list with one row per voxel — SparseConvNet blog
 *   ("图解稀疏卷积SparseConvNet：从哈希表到Rulebook的完整实现原理"), section 1.
 *
 *   Submanifold rule: an output exists exactly where an input exists
 *   (P_out = P_in; odd kernel, stride 1, same padding) — "Sparse inputs and
 *   sparse convolution", section "The fix: compute only where an input
 *   exists"; "Sparse convolution for point clouds", section "Submanifold
 *   sparse convolution".
 *
 *   Map (rulebook): for each output Q and offset d, the input P = Q + d, if
 *   active, adds the entry (P, Q, W_d) — "Sparse inputs and sparse
 *   convolution", section "The map is the computation"; offset sign as in
 *   "Sparse convolution for point clouds", section "The map and the update
 *   rule" (P = Q + offset), and in the GetOffset derivation of the blog's
 *   section 3 (offset = input - output).  Entries are grouped by offset
 *   ("sorted by weight offset", section "Nine entries become two").
 *
 *   Forward: f_out(Q) = sum over the map's entries (P, Q, W_d) of
 *   f_in(P) x W_d, from zero, no bias — "Sparse convolution for point clouds",
 *   section "The map and the update rule".
 *
 * Conventions of this ABI:
 *   - coordinates: int32 [N][4] rows (b, z, y, x), row-major, b in [0, 2^15),
 *     z, y, x in [0, 2^16); rows must be unique; entries never cross b;
 *   - kernel size K in {1, 3, 5, 7}; r = (K - 1) / 2;
 *   - offset index k(dz, dy, dx) = ((dz + r) K + (dy + r)) K + (dx + r), so the
 *     centre is k = (K^3 - 1) / 2 and k(-d) = K^3 - 1 - k(d);
 *   - weights: [K^3][C_in][C_out] row-major, the same dtype as the features;
 *     W[k] multiplies the input at Q + d(k) (cross-correlation);
 *   - a neighbour coordinate outside [0, 2^16) or not in the set is a miss.
 *
 * Memory and streams: every d_ pointer is device memory owned by the caller,
 * except the map's lists, which the map owns.  hip_stream is a hipStream_t
 * (NULL = the null stream).  spconv_build_map synchronises hip_stream once (to
 * read the per-offset counts and the device-side error flags);
 * spconv_build_map_async only enqueues, and the counts and device errors are
 * read by the first call that needs them.  spconv_forward is asynchronous on
 * its stream.  The map's device buffers come from a library-owned
 * stream-ordered memory pool on the current device.  The library also keeps,
 * per (device, stream), a build workspace, a forward workspace and up to four
 * released map blocks, and reuses them for later calls on the same stream
 * (stream order makes the reuse safe); they are held until the process ends.
 * A stream that the library has used must not be destroyed while library
 * work on it is still pending.
 *
 * Errors: functions return a status; nothing throws across the ABI.  Host-
 * checkable errors are reported before any device work.  On error, output
 * handles are set to NULL and nothing leaks.  spconv_last_error() returns a
 * thread-local message describing the last failure.
 */
#ifndef SPCONV_H_
#define SPCONV_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations are 32-bit integers on the ABI.  C++ gives them that
 * underlying type explicitly, so that any int32 a caller passes is a value
 * of the type (and an unknown one is rejected, not undefined). */
#ifdef __cplusplus
#define SPCONV_ENUM(name) enum name : int32_t
#else
#define SPCONV_ENUM(name) enum name
#endif

typedef SPCONV_ENUM(spconv_status) {
  SPCONV_OK = 0,
  SPCONV_ERR_INVALID_ARG = 1,     /* null pointer, bad size, misaligned buffer, K/C mismatch   */
  SPCONV_ERR_DUPLICATE_COORD = 2, /* two rows share one (b, z, y, x) (detected on the device)  */
  SPCONV_ERR_COORD_RANGE = 3,     /* a coordinate outside the ranges above (device-detected)   */
  SPCONV_ERR_UNSUPPORTED = 4,     /* K not in {1,3,5,7}, dtype or channel count not supported  */
  SPCONV_ERR_OUT_OF_MEMORY = 5,   /* device allocation failed                                  */
  SPCONV_ERR_DEVICE = 6           /* a HIP runtime call failed                                 */
} spconv_status;

typedef SPCONV_ENUM(spconv_dtype) {
  SPCONV_F32 = 0,  /* fp32 features and weights, fp32 products and accumulation                */
  SPCONV_F16 = 1,  /* fp16 features and weights, fp32 accumulation, output rounded to nearest even */
  SPCONV_BF16 = 2  /* bf16 features and weights, fp32 accumulation, output rounded to nearest even */
} spconv_dtype;

/* Opaque kernel map.  Owns its device buffers until spconv_map_free. */
typedef struct spconv_map spconv_map;

/* Opaque copy of one layer's weights, prepared for repeated forwards
 * (spconv_weights_prepare).  Owns its device buffers until
 * spconv_weights_free. */
typedef struct spconv_weights spconv_weights;

/* Kinds of map (spconv_map_geometry). */
typedef SPCONV_ENUM(spconv_map_kind) {
  SPCONV_MAP_SUBMANIFOLD = 0, /* outputs = inputs (spconv_build_map)            */
  SPCONV_MAP_STRIDED = 1,     /* downsampling (spconv_build_map_strided)          */
  SPCONV_MAP_TRANSPOSED = 2   /* upsampling, a strided map's transpose            */
} spconv_map_kind;

/* Version of this ABI (incremented on any incompatible change; 2: lists in
 * the map's row order instead of increasing out_idx; 3: strided and
 * transposed maps, whose input and output rows differ; 4: the grouped
 * dataflow, its plan and the dataflow selector; 5: prepared weights). */
int32_t spconv_abi_version(void);

/*
 * Builds the kernel map of a submanifold convolution with a K x K x K kernel
 * over the N voxels at d_coords (device int32 [N][4], (b, z, y, x)).
 *
 * The map holds, for every offset k, the list of entries (in_idx, out_idx)
 * with coords[in_idx] = coords[out_idx] + d(k) (same b).  The centre list is
 * the identity (q, q) for every row.  Within one offset the entries follow
 * the map's row order, the order in which the forward computes its rows: for
 * K > 1 and N >= 262144, the rows of each window of 4096 consecutive input
 * rows sorted stably by a 16-bit key of their neighbour set (bit 15 - i set
 * when the row has a neighbour at the i-th of: the offsets with every
 * coordinate within one step of the centre, in index order, then the others
 * in index order), so that rows computed together need the same weights
 * ("TorchSparse: regular computation from irregular sparsity", section
 * "TorchSparse++: overlap memory with computation"); otherwise the input
 * order.  The centre list therefore lists every row once, in that order.
 * Work: a device hash insert of all N keys, a probe of the (K^3 - 1) / 2
 * offsets with k > centre for every voxel, each hit also emitting its mirror
 * entry (P, Q, d) <-> (Q, P, -d) ("Sparse inputs and sparse convolution",
 * section "A symmetry you can check on the slide"), the per-window sort, and
 * a prefix-scan compaction per offset.
 *
 * Errors: INVALID_ARG (d_coords or out_map NULL, N <= 0, N x K^3 >= 2^31),
 * UNSUPPORTED (K not in {1,3,5,7}), DUPLICATE_COORD, COORD_RANGE,
 * OUT_OF_MEMORY, DEVICE.  On success *out_map is a new map, else NULL.
 */
spconv_status spconv_build_map(const int32_t* d_coords, int64_t n, int32_t kernel_size,
                               void* hip_stream, spconv_map** out_map);

/*
 * The same map build, without the wait: returns as soon as the work is
 * enqueued on hip_stream, so that a forward can follow on the device without
 * an idle gap.  Host-checkable errors are returned as by spconv_build_map.
 * The device-detected ones (DUPLICATE_COORD, COORD_RANGE) and the counts
 * become known when the build completes; spconv_map_wait, spconv_map_info
 * (for total_entries) and spconv_map_counts wait for that and return such an
 * error.  A forward over a map whose build reports an error is memory-safe
 * but its output is meaningless.  On success *out_map is a new map (to be
 * freed with spconv_map_free whatever its build reports), else NULL.
 */
spconv_status spconv_build_map_async(const int32_t* d_coords, int64_t n, int32_t kernel_size,
                                     void* hip_stream, spconv_map** out_map);

/* Waits until the map's build has completed on the device (no-op for a map
 * from spconv_build_map) and returns its device status: OK, DUPLICATE_COORD,
 * COORD_RANGE or DEVICE.  The map stays valid either way. */
spconv_status spconv_map_wait(spconv_map* map);

/* Kernel size, number of voxels and total entries (sum of all counts,
 * including the N centre entries).  Any output pointer may be NULL. */
spconv_status spconv_map_info(spconv_map* map, int32_t* kernel_size, int64_t* n,
                              int64_t* total_entries);

/* Copies the per-offset entry counts h_counts[K^3] and list offsets
 * h_offsets[K^3 + 1] (host arrays; either may be NULL).  The entries of
 * offset k lie at [h_offsets[k], h_offsets[k+1]) of the lists. */
spconv_status spconv_map_counts(spconv_map* map, int64_t* h_counts, int64_t* h_offsets);

/* Borrowed device pointers to the map's int32 lists (total_entries each),
 * valid until spconv_map_free.  Reading them is ordered after the build on the
 * build's stream. */
spconv_status spconv_map_lists(const spconv_map* map, const int32_t** d_in_idx,
                               const int32_t** d_out_idx);

/*
 * Forward of one submanifold convolution over a map:
 *   d_out[q][:] = sum_k sum_{(j, q) in list k} d_feats[j][:] x W[k]
 * with d_feats [N][c_in], d_weights [K^3][c_in][c_out] and d_out [N][c_out]
 * (caller-allocated, overwritten), all row-major in dtype and 16-byte aligned.
 * Products accumulate in fp32; the result is rounded to dtype (to nearest
 * even).  The work is one fused kernel: the centre offset is a dense
 * (identity-indexed) GEMM and every other offset gathers its input rows by
 * index; each output row is accumulated on chip and written once.  For
 * F16/BF16 with c_in in {32, 64, 128, 256} outside the small-channel shapes,
 * a short kernel first copies W into MFMA operand order in the stream's
 * forward workspace.
 *
 * The forward is ordered after the map's build: by stream order on the
 * build's stream; on another stream the library makes that stream wait for
 * the build first.
 *
 * Requirements: c_in, c_out multiples of 8 in [8, 1024] (F16/BF16), or
 * multiples of 4 in [4, 512] (F32); d_out shares no byte with d_feats or
 * d_weights (no in-place forward).  Errors: INVALID_ARG (NULL or misaligned
 * pointers, channel counts out of range, d_out overlapping an input),
 * UNSUPPORTED (dtype, channel multiple), OUT_OF_MEMORY (workspace), DEVICE.
 */
spconv_status spconv_forward(const void* d_feats, const void* d_weights, const spconv_map* map,
                             int32_t c_in, int32_t c_out, spconv_dtype dtype, void* d_out,
                             void* hip_stream);

/*
 * Gradient of the forward with respect to its input features:
 *   d_grad_in[j][:] = sum_k sum_{(j, q) in list k} d_grad_out[q][:] x W[k]^T
 * with d_grad_out [N][c_out], d_weights [K^3][c_in][c_out] (the forward's
 * weights, unchanged) and d_grad_in [N][c_in] (caller-allocated,
 * overwritten), all in dtype; fp32 accumulation, rounded to dtype (to
 * nearest even).  By the chain rule of the forward's sum, each entry
 * (P, Q, W_d) sends grad_out(Q) x W_d^T back to P ("Sparse convolution for
 * point clouds", section "The map and the update rule"), and since
 * (P, Q, d) is an entry exactly when (Q, P, -d) is ("Sparse inputs and
 * sparse convolution", section "A symmetry you can check on the slide"),
 * this is the forward over the same map with the weights
 * W'_k = W_{K^3 - 1 - k}^T: a short kernel writes W' into the stream's
 * workspace and the forward's kernels run on it.  Requirements, ordering
 * and errors as for spconv_forward with c_in and c_out exchanged
 * (d_grad_in shares no byte with d_grad_out or d_weights).  Submanifold maps
 * only (UNSUPPORTED otherwise): the data gradient of a strided map is the
 * forward over its transpose (spconv_map_transpose) with the weights W[k]^T,
 * and that of a transposed map the forward over the strided map with W[k]^T.
 */
spconv_status spconv_backward_data(const void* d_grad_out, const void* d_weights, const spconv_map* map,
                                   int32_t c_in, int32_t c_out, spconv_dtype dtype, void* d_grad_in,
                                   void* hip_stream);

/*
 * Gradient of the forward with respect to the weights:
 *   d_grad_w[k][ci][co] = sum_{(j, q) in list k} d_feats[j][ci] x d_grad_out[q][co]
 * with d_feats [N][c_in] and d_grad_out [N][c_out] in dtype, and d_grad_w
 * [K^3][c_in][c_out] in fp32 (caller-allocated, overwritten): each entry
 * (P, Q, W_d) adds the outer product f_in(P) x grad_out(Q) to W_d's gradient
 * (the chain rule of the same sum).  Products and sums are fp32: each
 * offset's entries are cut by ranges of consecutive 64-row output tiles
 * (about 2048 (range, column group, offset) units per call), each range
 * summed on MFMA (F16/BF16 with c_in in {16, 32, 64, 128, 256} and c_out a
 * multiple of 16, except c_in = 256 with c_out not a multiple of 32; other
 * shapes on the vector units), and the ranges' sums are added in range
 * order, so the result does not depend on scheduling.  The partial sums live
 * in the stream's workspace (K^3 x c_in x c_out x 4 bytes per range).  Any
 * map kind: d_feats has the map's input rows, d_grad_out its output rows
 * (spconv_map_geometry).  Requirements as for spconv_forward; d_grad_w
 * shares no byte with the inputs.  Errors: INVALID_ARG, UNSUPPORTED,
 * OUT_OF_MEMORY, DEVICE.
 */
spconv_status spconv_backward_weights(const void* d_feats, const void* d_grad_out, const spconv_map* map,
                                      int32_t c_in, int32_t c_out, spconv_dtype dtype, float* d_grad_w,
                                      void* hip_stream);

/*
 * The same forward as spconv_forward, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  It calls no device allocator.  Where spconv_forward
 * would take its workspace from the stream's cache (F16/BF16 shapes with
 * c_in in {32, 64, 128, 256} outside the small-channel ones: the weights in
 * MFMA operand order, a zero row and any fp32 partial outputs), this variant
 * uses a fixed scratch array of 32 MiB per device instead, held by the
 * library from its first use on a device until the process ends.  The
 * caller still passes the inputs and the output.
 *
 * Every call on one device shares that device's scratch: calls whose work
 * overlaps on one device (on different streams, or on one stream while an
 * earlier call of this variant is still using it from another) race and may
 * return wrong results.  Calls ordered one after another are safe: each
 * overwrites everything it reads of the scratch.
 *
 * Arguments, ordering after the map's build, outputs and errors as for
 * spconv_forward, plus UNSUPPORTED when the forward needs more workspace
 * than the scratch holds (the message states both sizes) and INVALID_ARG
 * when the current device is not the map's.
 */
spconv_status spconv_forward_noalloc(const void* d_feats, const void* d_weights, const spconv_map* map,
                                     int32_t c_in, int32_t c_out, spconv_dtype dtype, void* d_out,
                                     void* hip_stream);

/*
 * Prepares one layer's weights for repeated forwards (spconv_forward_prepared)
 * with the same weights, as in inference, where a layer's W_d stay fixed over
 * many calls ("Sparse convolution for point clouds", section "The map and the
 * update rule": the update applies W_d to every entry of offset d).  The
 * forward's wide and tiled kernels read W_d in MFMA operand order, a layout
 * spconv_forward writes into its workspace on every call (one small launch);
 * here it is written once.
 *
 * d_weights: device [kernel_volume][c_in][c_out] of dtype, 16-byte aligned,
 * only read, and copied: later changes to it do not reach the handle.
 * kernel_volume: K^3 of the maps the handle will be used with, in [1, 343].
 * c_in, c_out, dtype: as for spconv_forward.  On SPCONV_OK *out is a handle
 * that holds a device copy of the weights and, for F16/BF16 with c_in in
 * {32, 64, 128, 256}, c_out a multiple of 16 and kernel_volume <= 128, the
 * operand-order copy (the shapes whose forward uses it).  Device memory is
 * allocated on the current device (which the handle is bound to); the copies
 * are enqueued on hip_stream (NULL: the legacy default stream), so work on
 * another stream that uses the handle must be ordered after it.
 * Errors: INVALID_ARG (NULL pointer, misaligned weights, kernel_volume or
 * channels out of range), UNSUPPORTED (dtype, channel multiples),
 * OUT_OF_MEMORY, DEVICE.  On error *out is NULL.
 */
spconv_status spconv_weights_prepare(const void* d_weights, int32_t kernel_volume, int32_t c_in, int32_t c_out,
                                     spconv_dtype dtype, void* hip_stream, spconv_weights** out);

/*
 * The forward of spconv_forward with prepared weights: c_in, c_out and dtype
 * are the handle's, and the wide and tiled paths read its operand-order copy
 * instead of writing one.  The output is bit-identical to spconv_forward with
 * the weights the handle copied.  Requirements, ordering after the map's
 * build and the stream's workspace as for spconv_forward; the map's kernel
 * volume and device must be the handle's.  Errors: INVALID_ARG (NULL handle
 * or map, kernel volume or device mismatch, and those of spconv_forward),
 * UNSUPPORTED, OUT_OF_MEMORY, DEVICE.
 */
spconv_status spconv_forward_prepared(const void* d_feats, const spconv_weights* weights, const spconv_map* map,
                                      void* d_out, void* hip_stream);

/* Frees a handle from spconv_weights_prepare (NULL is ignored).  Waits for
 * the device's work in flight, which may still read it. */
void spconv_weights_free(spconv_weights* weights);

/*
 * Builds the kernel map of a strided (downsampling) sparse convolution with a
 * K x K x K kernel and stride `stride` over the n_in voxels at d_coords
 * (device int32 [n_in][4], (b, z, y, x), unique).
 *
 * Offsets: each component of d runs over lo .. lo + K - 1 with
 * lo = -floor((K - 1) / 2) (centred for odd K; K = 2 covers 0 and 1), index
 * k(d) = ((dz - lo) K + (dy - lo)) K + (dx - lo); weights [K^3][c_in][c_out].
 * Outputs: the regular output definition (SparseConvNet blog, section 2: an
 * output is computed where the kernel covers at least one active input) on
 * the grid of stride `stride`: every q >= 0 (same b) with an input at
 * stride x q + d for some offset d, in lexicographic (b, z, y, x) order
 * (spconv_map_out_coords; K = 2, stride 2 gives unique(coords // 2)).
 * Entries: for each output q and offset d, the input at stride x q + d, if
 * active, adds (in, q, W_d) ("Sparse inputs and sparse convolution", section
 * "The map is the computation": look up s q + d).  There is no identity
 * offset; the forward (spconv_forward) reads d_feats [n_in][c_in] and writes
 * d_out [n_out][c_out].  Lists are grouped by offset, in increasing output
 * row within an offset.
 *
 * Work: the input table (the same device hash as spconv_build_map), every
 * (input, offset) candidate output key, a device radix sort and unique of
 * the keys, a host read of the number of outputs (one wait), then a probe of
 * every offset for every output and the per-offset compaction.  The build
 * synchronises hip_stream twice.
 *
 * Errors: INVALID_ARG (NULL or misaligned pointers, n_in <= 0, n_in x
 * ceil(K / stride)^3 >= 2^31, n_out x K^3 >= 2^31), UNSUPPORTED (K not in
 * [1, 5], stride not in [1, 16]), DUPLICATE_COORD, COORD_RANGE,
 * OUT_OF_MEMORY, DEVICE.  On success *out_map is a new map (it may have no
 * outputs: then every forward over it writes nothing), else NULL.
 */
spconv_status spconv_build_map_strided(const int32_t* d_coords, int64_t n_in, int32_t kernel_size, int32_t stride,
                                       void* hip_stream, spconv_map** out_map);

/*
 * The transpose of a strided map: the upsampling convolution from the
 * strided map's outputs back onto its inputs.  Its outputs are the strided
 * map's inputs (in their order; spconv_map_out_coords) and its entries the
 * strided map's, reversed: (q, p, W_d) for every (p, q, W_d), found by
 * probing, for each of its outputs p and offsets d, the strided output q
 * with stride x q + d = p.  Lists in increasing output row within an offset.
 * The forward over it reads d_feats [n_out of the strided map][c_in] and
 * writes d_out [n_in of the strided map][c_out] with weights
 * [K^3][c_in][c_out].  Synchronises hip_stream once.
 *
 * Errors: INVALID_ARG (NULL pointers, not on the map's device), UNSUPPORTED
 * (map not strided), OUT_OF_MEMORY, DEVICE.  The strided map stays valid and
 * independent of the new one.
 */
spconv_status spconv_map_transpose(spconv_map* map, void* hip_stream, spconv_map** out_map);

/* Input rows, output rows, stride (1 for a submanifold map) and kind
 * (spconv_map_kind) of a map; any output pointer may be NULL. */
spconv_status spconv_map_geometry(const spconv_map* map, int64_t* n_in, int64_t* n_out, int32_t* stride,
                                  int32_t* kind);

/* Borrowed device pointer to the output coordinates (int32 [n_out][4]) of a
 * strided or transposed map, valid until spconv_map_free.  UNSUPPORTED for a
 * submanifold map, whose outputs are its inputs. */
spconv_status spconv_map_out_coords(const spconv_map* map, const int32_t** d_out_coords);

/* ---- Weight-stationary forward with adaptive grouping ----
 *
 * The comparison dataflow of "TorchSparse: regular computation from
 * irregular sparsity", sections "The spectrum: separate, dense, grouped" and
 * "How the groups are chosen": gather the input rows of each offset into a
 * batch, multiply each batch by its W_d, scatter the products back onto the
 * output rows.  Offsets run in groups, one batched product each, every
 * member padded with zero rows to the group's largest map; the padded rows
 * are computed (the redundant work the grouping trades for fewer, larger
 * products) and their products dropped.
 *
 * The groups for (epsilon, S): the offsets with entries, the identity offset
 * of a submanifold map apart (it forms a group of its own, first), walked in
 * decreasing map size (ties by lower index) and cut into runs; a run takes
 * the next offset while its redundant ratio (m x max - sum) / (m x max) over
 * its m maps stays at most epsilon (computed in double precision), else that
 * offset starts the next run.  A run whose largest map is at least S runs as
 * separate products, one per offset; every other run is one group.  So
 * epsilon = 1 with S = +inf is one dense batch of the non-identity offsets,
 * S = 0 is fully separate computation, and epsilon = 0 groups equal map
 * sizes only (the mirror pairs of a submanifold map).
 */
typedef SPCONV_ENUM(spconv_dataflow_kind) {
  SPCONV_DATAFLOW_FUSED = 0,   /* spconv_forward's output-stationary kernels */
  SPCONV_DATAFLOW_GROUPED = 1  /* spconv_forward_grouped with (epsilon, S) */
} spconv_dataflow_kind;

/* The choice spconv_select_dataflow makes for one layer configuration. */
typedef struct spconv_dataflow {
  int32_t kind;        /* spconv_dataflow_kind */
  int32_t groups;      /* groups of the chosen plan (0 for the fused dataflow) */
  double epsilon;      /* the chosen plan's epsilon and S (grouped only) */
  double S;
  float ms;            /* measured time per call of the chosen dataflow */
  float fused_ms;      /* measured time per call of the fused dataflow */
  int32_t candidates;  /* distinct candidates timed (the fused one included) */
  int32_t reserved;
} spconv_dataflow;

/*
 * The groups of (epsilon, S) over `map` (see above), in execution order:
 * h_offsets[i] is the offset index of entry i and h_groups[i] its group
 * (0, 1, ...; the entries of a group are consecutive, in decreasing map
 * size).  Offsets without entries are in no group.  capacity is the length
 * of h_offsets and h_groups (K^3 always suffices); either may be NULL, as
 * may any of n_entries, n_groups and padded_rows (sum over entries of their
 * group's largest map: the rows the batched products run).
 *
 * Waits for the map's build if it is still running.  Errors: INVALID_ARG
 * (NULL map, epsilon or S negative or NaN, capacity below the entries), and
 * the build's own errors.
 */
spconv_status spconv_group_plan(spconv_map* map, double epsilon, double S, int32_t capacity, int32_t* h_offsets,
                                int32_t* h_groups, int32_t* n_entries, int32_t* n_groups, int64_t* padded_rows);

/*
 * The same plan from per-offset map sizes the caller supplies (host memory,
 * h_counts[k] for k < kernel_volume; centre is the identity offset that runs
 * on its own, or -1 for none): no map and no device involved.  Errors:
 * INVALID_ARG (NULL h_counts, kernel_volume not in [1, 343], centre not in
 * [-1, kernel_volume), a count not in [0, 2^40), epsilon or S negative or
 * NaN, capacity below the entries).
 */
spconv_status spconv_group_plan_counts(const int64_t* h_counts, int32_t kernel_volume, int32_t centre,
                                       double epsilon, double S, int32_t capacity, int32_t* h_offsets,
                                       int32_t* h_groups, int32_t* n_entries, int32_t* n_groups,
                                       int64_t* padded_rows);

/*
 * Forward over `map` in the grouped weight-stationary dataflow: the same
 * result as spconv_forward (same arguments, layouts and aliasing rules),
 * computed as one gather of every offset's padded batch, one MFMA batched
 * product per group (fp32 products) and one deterministic reduction of the
 * products in offset order per output row, rounded once to the dtype.
 * Needs f16 or bf16, c_in % 32 == 0, c_out % 16 == 0.  Its workspace
 * (weights in operand order, the padded batches, one fp32 row of c_out per
 * map entry) comes from the stream's cached forward workspace.
 *
 * Waits for the map's build if it is still running (the plan is made on the
 * host from the counts).  Errors: those of spconv_forward, INVALID_ARG
 * (epsilon or S negative or NaN), UNSUPPORTED (dtype or channel counts).
 */
spconv_status spconv_forward_grouped(const void* d_feats, const void* d_weights, spconv_map* map, int32_t c_in,
                                     int32_t c_out, spconv_dtype dtype, double epsilon, double S, void* d_out,
                                     void* hip_stream);

/*
 * Per-configuration dataflow selector, after the Sparse Autotuner of
 * "TorchSparse: regular computation from irregular sparsity", section
 * "TorchSparse++: overlap memory with computation" (one configuration chosen
 * per layer from a design space holding gather-GEMM-scatter with grouping
 * and the fused dataflow): times, on the caller's buffers, the
 * fused forward and the grouped forward for every (epsilon, S) of the grid
 * (plans equal to an earlier one skipped), each once untimed and then
 * `reps` times between two events on hip_stream, and reports the fastest
 * in *best (ties go to the earlier candidate; the fused one is first).  A
 * NULL grid takes the default: epsilon in {0, 0.1, 0.2, 0.3, 0.5, 1}, S in
 * {+inf, 65536, 16384, 0}.  The grouped candidates are skipped where the
 * grouped forward is unsupported (fp32, channel counts).  On return d_out
 * holds the chosen dataflow's output.  Synchronises hip_stream once per
 * candidate.
 *
 * Errors: those of spconv_forward, INVALID_ARG (NULL best, reps not in
 * [1, 1000], a grid longer than 64 or holding a negative or NaN value).
 */
spconv_status spconv_select_dataflow(const void* d_feats, const void* d_weights, spconv_map* map, int32_t c_in,
                                     int32_t c_out, spconv_dtype dtype, const double* epsilons, int32_t n_epsilons,
                                     const double* thresholds, int32_t n_thresholds, int32_t reps, void* d_out,
                                     void* hip_stream, spconv_dataflow* best);

/* Releases a map.  Its buffers go back, in the order of the build's stream,
 * to that stream's cache of map blocks (or to the pool); the caller must not
 * free a map while work on another stream still reads it.  NULL is ignored. */
void spconv_map_free(spconv_map* map);

/* Static name of a status ("SPCONV_OK", ...). */
const char* spconv_status_string(spconv_status status);

/* Thread-local detail of the last error on this thread ("" if none). */
const char* spconv_last_error(void);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif /* SPCONV_H_ */
