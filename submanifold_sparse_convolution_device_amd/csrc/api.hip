// Host side of the C ABI declared in include/spconv.h: argument validation,
// stream-ordered memory, the single read-back of the map build, and kernel
// launches.  No compute happens here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "../../include/spconv.h"
#include "internal.h"

namespace {

// Pinned host slot that receives one build's summary (written by the build's
// last kernel), with the event that marks its arrival.  Slots are reused; a
// slot released while its build may still be running is reclaimed only once
// its event has completed.
struct SummarySlot {
  long long* host = nullptr;
  long long* device = nullptr;  // the same memory, as the device addresses it
  hipEvent_t done = nullptr;
};

}  // namespace

struct spconv_map {
  int device = 0;
  hipStream_t stream = nullptr;
  int32_t K = 0;
  int32_t KV = 0;
  int64_t n = 0;      // output rows (the forward's rows and tiles)
  int64_t n_in = 0;   // input rows (n for a submanifold map)
  int32_t centre = 0;  // offset whose list is the identity, -1 for none
  int32_t stride = 1;
  int32_t kind = 0;    // SPCONV_MAP_SUBMANIFOLD, _STRIDED or _TRANSPOSED
  int32_t* out_coords = nullptr;  // [n][4] (strided and transposed maps; in the block)
  int32_t* in_coords = nullptr;   // [n_in][4] copy (strided and transposed maps; in the block)
  int64_t tiles = 0;
  void* block = nullptr;  // one pool allocation holding the MapBuffers
  size_t block_bytes = 0;
  spconv::MapBuffers buf;
  // Filled when the build's summary has been read (see finish_build).
  SummarySlot* slot = nullptr;   // non-null while the summary is not yet read
  spconv_status status = SPCONV_OK;
  std::string error;             // detail of a device-detected error
  int64_t total = 0;
  std::vector<int64_t> counts;   // KV
  std::vector<int64_t> offsets;  // KV + 1
};

// A copy of one layer's weights made for repeated forwards: the raw
// [K^3][C_in][C_out] copy and, for the shapes the wide and tiled paths take,
// the same weights in MFMA operand order with the zero row after them.
struct spconv_weights {
  int device = 0;
  int32_t KV = 0, c_in = 0, c_out = 0;
  spconv_dtype dtype = SPCONV_F32;
  void* raw = nullptr;
  void* prepared = nullptr;  // NULL for shapes that never use it
};

namespace {

thread_local std::string g_last_error;

spconv_status fail(spconv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

spconv_status hip_fail(hipError_t e, const char* what) {
  const spconv_status st =
      (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) ? SPCONV_ERR_OUT_OF_MEMORY
                                                                   : SPCONV_ERR_DEVICE;
  return fail(st, "%s: %s (%d)", what, hipGetErrorString(e), static_cast<int>(e));
}

#define SPCONV_HIP(call, what)                 \
  do {                                         \
    const hipError_t e_ = (call);              \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

// One stream-ordered pool per device, kept warm (no release at sync points),
// so per-build workspace and map buffers cost no driver allocation once the
// pool has grown.
std::mutex g_pool_mu;
std::vector<hipMemPool_t> g_pools;

spconv_status pool_for(int device, hipMemPool_t* out) {
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if (static_cast<int>(g_pools.size()) <= device) g_pools.resize(device + 1, nullptr);
  if (g_pools[device] == nullptr) {
    hipMemPoolProps props;
    std::memset(&props, 0, sizeof(props));
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = device;
    hipMemPool_t pool = nullptr;
    SPCONV_HIP(hipMemPoolCreate(&pool, &props), "hipMemPoolCreate");
    uint64_t keep = ~0ull;
    SPCONV_HIP(hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep),
               "hipMemPoolSetAttribute");
    g_pools[device] = pool;
  }
  *out = g_pools[device];
  return SPCONV_OK;
}

// Device buffers kept per (device, stream) between calls.  Work on one stream
// runs in order, so a buffer that earlier work on a stream has released can
// be handed to later work on the same stream with no allocator call (the
// pool's asynchronous malloc and free cost several microseconds of host time
// each, on every build and forward otherwise).  Buffers leave a stream only
// through the pool's stream-ordered free.
struct StreamCache {
  int device = 0;
  hipStream_t stream = nullptr;
  void* scratch = nullptr;  // map build workspace
  size_t scratch_bytes = 0;
  // Table slots of the last build launched on the scratch, whose table and
  // occupancy map it leaves clear (0: not known clear).
  int64_t clear_slots = 0;
  void* fwd = nullptr;  // forward workspace
  size_t fwd_bytes = 0;
  std::vector<std::pair<void*, size_t>> blocks;  // map blocks released on this stream
};
constexpr size_t kCachedBlocks = 4;
std::mutex g_cache_mu;
std::vector<StreamCache*> g_caches;

StreamCache* cache_for(int device, hipStream_t stream) {
  for (StreamCache* c : g_caches)
    if (c->device == device && c->stream == stream) return c;
  StreamCache* c = new StreamCache;
  c->device = device;
  c->stream = stream;
  g_caches.push_back(c);
  return c;
}

// Makes `buf` hold at least `need` bytes (grown with 25% headroom).
spconv_status grow_buffer(void*& buf, size_t& have, size_t need, hipMemPool_t pool, hipStream_t stream,
                          const char* what) {
  if (have >= need && buf != nullptr) return SPCONV_OK;
  if (buf != nullptr) (void)hipFreeAsync(buf, stream);
  buf = nullptr;
  have = 0;
  const size_t want = need + need / 4;
  SPCONV_HIP(hipMallocFromPoolAsync(&buf, want, pool, stream), what);
  have = want;
  return SPCONV_OK;
}

// A released map block of at least `need` bytes (and at most twice that),
// else a new one.
spconv_status take_block(StreamCache* c, size_t need, hipMemPool_t pool, void** out, size_t* bytes) {
  size_t best = c->blocks.size();
  for (size_t i = 0; i < c->blocks.size(); ++i) {
    const size_t b = c->blocks[i].second;
    if (b >= need && b <= 2 * need && (best == c->blocks.size() || b < c->blocks[best].second)) best = i;
  }
  if (best < c->blocks.size()) {
    *out = c->blocks[best].first;
    *bytes = c->blocks[best].second;
    c->blocks.erase(c->blocks.begin() + static_cast<std::ptrdiff_t>(best));
    return SPCONV_OK;
  }
  SPCONV_HIP(hipMallocFromPoolAsync(out, need, pool, c->stream), "map allocation");
  *bytes = need;
  return SPCONV_OK;
}

void release_block(int device, hipStream_t stream, void* block, size_t bytes) {
  std::lock_guard<std::mutex> lock(g_cache_mu);
  StreamCache* c = cache_for(device, stream);
  if (c->blocks.size() < kCachedBlocks) {
    c->blocks.emplace_back(block, bytes);
  } else {
    (void)hipFreeAsync(block, stream);
  }
}

// Summary slots, one free list per device.  A slot holds enough for the
// largest kernel (K = 7).
constexpr size_t kSlotBytes = sizeof(long long) * (spconv::kSummaryHead + 343);
constexpr int kSlotsPerBatch = 16;

struct SlotPool {
  std::vector<SummarySlot*> free;
  std::vector<SummarySlot*> pending;  // released while their build may still write them
};
std::mutex g_slot_mu;
std::vector<SlotPool> g_slots;

spconv_status acquire_slot(int device, SummarySlot** out) {
  std::lock_guard<std::mutex> lock(g_slot_mu);
  if (static_cast<int>(g_slots.size()) <= device) g_slots.resize(device + 1);
  SlotPool& pool = g_slots[device];
  for (size_t i = 0; i < pool.pending.size();) {
    if (hipEventQuery(pool.pending[i]->done) == hipSuccess) {
      pool.free.push_back(pool.pending[i]);
      pool.pending[i] = pool.pending.back();
      pool.pending.pop_back();
    } else {
      ++i;
    }
  }
  if (pool.free.empty()) {
    void* p = nullptr;
    SPCONV_HIP(hipHostMalloc(&p, kSlotBytes * kSlotsPerBatch,
                             hipHostMallocPortable | hipHostMallocMapped | hipHostMallocCoherent),
               "hipHostMalloc");
    for (int i = 0; i < kSlotsPerBatch; ++i) {
      SummarySlot* slot = new (std::nothrow) SummarySlot;
      if (slot == nullptr) return fail(SPCONV_ERR_OUT_OF_MEMORY, "host allocation");
      slot->host = reinterpret_cast<long long*>(static_cast<char*>(p) + kSlotBytes * i);
      void* dp = nullptr;
      SPCONV_HIP(hipHostGetDevicePointer(&dp, slot->host, 0), "hipHostGetDevicePointer");
      slot->device = static_cast<long long*>(dp);
      SPCONV_HIP(hipEventCreateWithFlags(&slot->done, hipEventDisableTiming), "hipEventCreateWithFlags");
      pool.free.push_back(slot);
    }
  }
  *out = pool.free.back();
  pool.free.pop_back();
  return SPCONV_OK;
}

void release_slot(int device, SummarySlot* slot) {
  std::lock_guard<std::mutex> lock(g_slot_mu);
  g_slots[device].pending.push_back(slot);
}

// Waits for the build's summary (once) and records the counts or the device
// error it reports.
spconv_status finish_build(spconv_map* m) {
  if (m->slot != nullptr) {
    hipError_t e;
    // Spinning keeps the wake-up latency of a blocking wait off the critical path.
    while ((e = hipEventQuery(m->slot->done)) == hipErrorNotReady) {
    }
    const long long* sum = m->slot->host;
    if (e != hipSuccess) {
      m->status = hip_fail(e, "map build");
      m->error = g_last_error;
    } else {
      const unsigned long long flags = static_cast<unsigned long long>(sum[0]);
      if (flags & spconv::kFlagRange) {
        m->status = SPCONV_ERR_COORD_RANGE;
        m->error = "a coordinate is outside b in [0, 2^15), z, y, x in [0, 2^16)";
      } else if (flags & spconv::kFlagDuplicate) {
        m->status = SPCONV_ERR_DUPLICATE_COORD;
        m->error = "two rows share one (b, z, y, x) coordinate";
      } else if (flags & spconv::kFlagTableFull) {
        m->status = SPCONV_ERR_DEVICE;
        m->error = "internal: hash table probe exceeded its bound";
      } else {
        m->counts.assign(sum + spconv::kSummaryHead, sum + spconv::kSummaryHead + m->KV);
        m->offsets.resize(m->KV + 1);
        m->offsets[0] = 0;
        for (int k = 0; k < m->KV; ++k) m->offsets[k + 1] = m->offsets[k] + m->counts[k];
        m->total = m->offsets[m->KV];
      }
    }
    release_slot(m->device, m->slot);
    m->slot = nullptr;
  }
  if (m->status != SPCONV_OK) return fail(m->status, "%s", m->error.c_str());
  return SPCONV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Fixed scratch of spconv_forward_noalloc: one array per device, held until
// the process ends, for the forward workspace (weights in MFMA operand order,
// the zero row and any fp32 partial outputs).  Host code never uses the
// array's name as an address: each device's address comes from
// hipGetSymbolAddress, taken once with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

spconv_status noalloc_scratch(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) {
    return fail(SPCONV_ERR_UNSUPPORTED, "device %d beyond the %d the fixed scratch covers", device, kMaxDevices);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    void* ptr = nullptr;
    SPCONV_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(SPCONV_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return SPCONV_OK;
}

// Validates a forward call and fills its launch arguments.
spconv_status forward_args(const void* d_feats, const void* d_weights, const spconv_map* map, int32_t c_in,
                           int32_t c_out, spconv_dtype dtype, void* d_out, spconv::ForwardArgs* out) {
  // Checks that need no map first, then those that read it.
  if (map == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "map is NULL");
  if (d_weights == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "NULL weight pointer");
  if (!aligned16(d_feats) || !aligned16(d_weights) || !aligned16(d_out)) {
    return fail(SPCONV_ERR_INVALID_ARG, "feature, weight and output buffers must be 16-byte aligned");
  }
  if (dtype != SPCONV_F32 && dtype != SPCONV_F16 && dtype != SPCONV_BF16) {
    return fail(SPCONV_ERR_UNSUPPORTED, "dtype %d not supported", static_cast<int>(dtype));
  }
  const int32_t cmax = (dtype == SPCONV_F32) ? 512 : 1024;
  if (c_in < 1 || c_out < 1 || c_in > cmax || c_out > cmax) {
    return fail(SPCONV_ERR_INVALID_ARG, "c_in = %d, c_out = %d must lie in [1, %d]", c_in, c_out, cmax);
  }
  const int32_t mult = (dtype == SPCONV_F32) ? 4 : 8;
  if (c_in % mult != 0 || c_out % mult != 0) {
    return fail(SPCONV_ERR_UNSUPPORTED, "c_in = %d and c_out = %d must be multiples of %d", c_in,
                c_out, mult);
  }
  // A side with no rows (a strided map without outputs, or its transpose)
  // may be NULL: nothing of it is read or written.
  if ((d_feats == nullptr && map->n_in > 0) || (d_out == nullptr && map->n > 0)) {
    return fail(SPCONV_ERR_INVALID_ARG, "NULL feature or output pointer");
  }
  {
    // The output is written while other workgroups still read input rows and
    // weights: it must not share a byte with either.
    const uint64_t es = (dtype == SPCONV_F32) ? 4u : 2u;
    const uint64_t out_b = static_cast<uint64_t>(map->n) * c_out * es;
    const uint64_t in_b = static_cast<uint64_t>(map->n_in) * c_in * es;
    const uint64_t w_b = static_cast<uint64_t>(map->KV) * c_in * c_out * es;
    auto overlap = [](const void* p, uint64_t np, const void* q, uint64_t nq) {
      const uint64_t a0 = reinterpret_cast<uintptr_t>(p), b0 = reinterpret_cast<uintptr_t>(q);
      return a0 < b0 + nq && b0 < a0 + np;
    };
    if (overlap(d_out, out_b, d_feats, in_b) || overlap(d_out, out_b, d_weights, w_b)) {
      return fail(SPCONV_ERR_INVALID_ARG, "d_out overlaps the features or the weights");
    }
  }
  spconv::ForwardArgs& a = *out;
  a.feats = d_feats;
  a.weights = d_weights;
  a.out = d_out;
  a.in_idx = map->buf.in_idx;
  a.out_idx = map->buf.out_idx;
  a.tile_off = map->buf.tile_off;
  a.tile_mask = map->buf.tile_mask;
  a.tile_rows = map->buf.tile_rows;
  a.perm = map->buf.perm;
  a.n = map->n;
  a.tiles = map->tiles;
  a.KV = map->KV;
  a.cin = c_in;
  a.cout = c_out;
  a.dtype = static_cast<int32_t>(dtype);
  a.centre = map->centre;
  a.n_in = map->n_in;
  return SPCONV_OK;
}

// A map known to hold no entries (a strided map with no outputs, or its
// transpose): the forward writes zeros and launches no kernel.
bool known_empty(const spconv_map* map) { return map->slot == nullptr && map->total == 0; }

spconv_status zero_output(void* d_out, int64_t rows, int32_t c_out, spconv_dtype dtype, hipStream_t stream) {
  const size_t es = (dtype == SPCONV_F32) ? 4u : 2u;
  if (rows > 0) SPCONV_HIP(hipMemsetAsync(d_out, 0, static_cast<size_t>(rows) * c_out * es, stream), "hipMemsetAsync");
  return SPCONV_OK;
}

// Orders `stream` after the map's build when it is another stream than the
// build's and the build is not yet known complete.
spconv_status order_after_build(const spconv_map* map, hipStream_t stream) {
  if (stream != map->stream && map->slot != nullptr) {
    const hipError_t ew = hipStreamWaitEvent(stream, map->slot->done, 0);
    if (ew != hipSuccess) return hip_fail(ew, "hipStreamWaitEvent");
  }
  return SPCONV_OK;
}

enum class ForwardPath { kSmall, kWide, kTiled, kGeneric };

ForwardPath forward_path(const spconv::ForwardArgs& a) {
  if (spconv::small_supported(a)) return ForwardPath::kSmall;
  if (spconv::wide_supported(a)) return ForwardPath::kWide;
  if (spconv::tiled_supported(a)) return ForwardPath::kTiled;
  return ForwardPath::kGeneric;
}

size_t forward_workspace_bytes(ForwardPath path, const spconv::ForwardArgs& a) {
  if (path == ForwardPath::kWide) return spconv::wide_workspace_bytes(a);
  if (path == ForwardPath::kTiled) return a.prepared != nullptr ? 0 : spconv::tiled_workspace_bytes(a);
  return 0;
}

// Launches the forward's kernels; `ws` holds forward_workspace_bytes(path, a)
// bytes (unused by the small and generic paths).
spconv_status launch_forward_path(ForwardPath path, const spconv::ForwardArgs& a, void* ws, hipStream_t stream) {
  hipError_t e;
  switch (path) {
    case ForwardPath::kWide:
      e = a.prepared != nullptr ? hipSuccess : spconv::launch_prep_weights(a, ws, stream);
      if (e == hipSuccess) e = spconv::launch_forward_wide(a, ws, stream);
      break;
    case ForwardPath::kTiled:
      e = spconv::launch_forward_tiled(a, ws, stream);
      break;
    default:
      e = spconv::launch_forward(a, stream);
      break;
  }
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return SPCONV_OK;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Block layout of a strided or transposed map: the lists (cap entries), tile
// offsets, masks and slot table over `tiles` output tiles, then the output
// and input coordinates.
struct GeneralLayout {
  size_t list_b, tile_off_b, mask_b, rows_b, out_c_b, in_c_b;
};
GeneralLayout general_layout(int64_t tiles, int32_t KV, int64_t cap, int64_t n_out, int64_t n_in, size_t* total) {
  GeneralLayout l;
  const size_t t = static_cast<size_t>(KV) * tiles;
  l.list_b = align256(static_cast<size_t>(cap) * sizeof(int32_t));
  l.tile_off_b = align256((t + 1) * sizeof(int32_t));
  l.mask_b = align256(std::max<size_t>(t, 1) * sizeof(unsigned long long));
  l.rows_b = align256(std::max<size_t>(static_cast<size_t>(tiles), 1) * spconv::kTileSlots * sizeof(int32_t));
  l.out_c_b = align256(std::max<size_t>(static_cast<size_t>(n_out), 1) * 4 * sizeof(int32_t));
  l.in_c_b = align256(std::max<size_t>(static_cast<size_t>(n_in), 1) * 4 * sizeof(int32_t));
  *total = 2 * l.list_b + l.tile_off_b + l.mask_b + l.rows_b + l.out_c_b + l.in_c_b;
  return l;
}
void carve_general(const GeneralLayout& l, spconv_map* m) {
  char* c = static_cast<char*>(m->block);
  m->buf.in_idx = reinterpret_cast<int32_t*>(c);
  c += l.list_b;
  m->buf.out_idx = reinterpret_cast<int32_t*>(c);
  c += l.list_b;
  m->buf.tile_off = reinterpret_cast<int32_t*>(c);
  c += l.tile_off_b;
  m->buf.tile_mask = reinterpret_cast<unsigned long long*>(c);
  c += l.mask_b;
  m->buf.tile_rows = reinterpret_cast<int32_t*>(c);
  c += l.rows_b;
  m->buf.perm = nullptr;
  m->out_coords = reinterpret_cast<int32_t*>(c);
  c += l.out_c_b;
  m->in_coords = reinterpret_cast<int32_t*>(c);
}

// A map with no entries: complete at once (no summary to wait for).
void mark_empty(spconv_map* m) {
  if (m->slot != nullptr) {
    release_slot(m->device, m->slot);
    m->slot = nullptr;
  }
  m->counts.assign(static_cast<size_t>(m->KV), 0);
  m->offsets.assign(static_cast<size_t>(m->KV) + 1, 0);
  m->total = 0;
}


// ---- grouped (weight-stationary) forward ----

spconv_status check_plan_args(double epsilon, double S) {
  if (!(epsilon >= 0.0) || !(S >= 0.0)) {
    return fail(SPCONV_ERR_INVALID_ARG, "epsilon = %g and S = %g must be >= 0 (S may be +inf)", epsilon, S);
  }
  return SPCONV_OK;
}

// Launches the grouped forward of `a` with `plan` from the stream's cached
// forward workspace.
spconv_status launch_grouped(const spconv_map* map, const spconv::ForwardArgs& a, const spconv::GroupPlan& plan,
                             hipStream_t stream) {
  hipMemPool_t pool = nullptr;
  spconv_status st = pool_for(map->device, &pool);
  if (st != SPCONV_OK) return st;
  std::lock_guard<std::mutex> lock(g_cache_mu);
  StreamCache* c = cache_for(map->device, stream);
  st = grow_buffer(c->fwd, c->fwd_bytes, spconv::grouped_workspace_bytes(a, plan), pool, stream,
                   "forward workspace allocation");
  if (st != SPCONV_OK) return st;
  const hipError_t e = spconv::launch_forward_grouped(a, plan, c->fwd, stream);
  if (e != hipSuccess) return hip_fail(e, "grouped forward launch");
  return SPCONV_OK;
}

// The fused forward (the path spconv_forward takes) from the stream's cache.
spconv_status launch_fused(const spconv_map* map, const spconv::ForwardArgs& a, hipStream_t stream) {
  const ForwardPath path = forward_path(a);
  const size_t ws_bytes = forward_workspace_bytes(path, a);
  if (ws_bytes == 0) return launch_forward_path(path, a, nullptr, stream);
  hipMemPool_t pool = nullptr;
  spconv_status st = pool_for(map->device, &pool);
  if (st != SPCONV_OK) return st;
  std::lock_guard<std::mutex> lock(g_cache_mu);
  StreamCache* c = cache_for(map->device, stream);
  st = grow_buffer(c->fwd, c->fwd_bytes, ws_bytes, pool, stream, "forward workspace allocation");
  if (st != SPCONV_OK) return st;
  return launch_forward_path(path, a, c->fwd, stream);
}

bool same_plan(const spconv::GroupPlan& x, const spconv::GroupPlan& y) {
  return x.entries == y.entries && x.entry_group == y.entry_group;
}
}  // namespace

extern "C" {

int32_t spconv_abi_version(void) { return 5; }

const char* spconv_status_string(spconv_status s) {
  switch (s) {
    case SPCONV_OK: return "SPCONV_OK";
    case SPCONV_ERR_INVALID_ARG: return "SPCONV_ERR_INVALID_ARG";
    case SPCONV_ERR_DUPLICATE_COORD: return "SPCONV_ERR_DUPLICATE_COORD";
    case SPCONV_ERR_COORD_RANGE: return "SPCONV_ERR_COORD_RANGE";
    case SPCONV_ERR_UNSUPPORTED: return "SPCONV_ERR_UNSUPPORTED";
    case SPCONV_ERR_OUT_OF_MEMORY: return "SPCONV_ERR_OUT_OF_MEMORY";
    case SPCONV_ERR_DEVICE: return "SPCONV_ERR_DEVICE";
  }
  return "SPCONV_ERR_UNKNOWN";
}

const char* spconv_last_error(void) { return g_last_error.c_str(); }

spconv_status spconv_build_map_async(const int32_t* d_coords, int64_t n, int32_t kernel_size,
                                     void* hip_stream, spconv_map** out_map) {
  g_last_error.clear();
  if (out_map == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "out_map is NULL");
  *out_map = nullptr;
  if (d_coords == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "d_coords is NULL");
  if (!aligned16(d_coords)) return fail(SPCONV_ERR_INVALID_ARG, "d_coords is not 16-byte aligned");
  if (n <= 0) return fail(SPCONV_ERR_INVALID_ARG, "n = %lld must be positive", (long long)n);
  if (kernel_size != 1 && kernel_size != 3 && kernel_size != 5 && kernel_size != 7) {
    return fail(SPCONV_ERR_UNSUPPORTED, "kernel_size = %d not in {1, 3, 5, 7}", kernel_size);
  }
  const int32_t KV = kernel_size * kernel_size * kernel_size;
  if (n >= (int64_t(1) << 31) / KV) {
    return fail(SPCONV_ERR_INVALID_ARG, "n x K^3 = %lld x %d must stay below 2^31",
                (long long)n, KV);
  }
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);

  const spconv::BuildPlan p = spconv::make_plan(n, kernel_size);

  int device = 0;
  SPCONV_HIP(hipGetDevice(&device), "hipGetDevice");
  hipMemPool_t pool = nullptr;
  spconv_status st = pool_for(device, &pool);
  if (st != SPCONV_OK) return st;

  spconv_map* m = new (std::nothrow) spconv_map;
  if (m == nullptr) return fail(SPCONV_ERR_OUT_OF_MEMORY, "host allocation");
  st = acquire_slot(device, &m->slot);
  if (st != SPCONV_OK) {
    delete m;
    return st;
  }
  // The stream's build workspace and a map block (both reused across builds
  // on this stream); the cache lock also serialises enqueueing on a stream.
  std::lock_guard<std::mutex> lock(g_cache_mu);
  StreamCache* c = cache_for(device, stream);
  void* const scratch_before = c->scratch;
  st = grow_buffer(c->scratch, c->scratch_bytes, spconv::build_scratch_bytes(p), pool, stream,
                   "workspace allocation");
  if (c->scratch != scratch_before) c->clear_slots = 0;  // new memory
  if (st == SPCONV_OK) st = take_block(c, spconv::map_buffer_bytes(p), pool, &m->block, &m->block_bytes);
  if (st != SPCONV_OK) {
    release_slot(device, m->slot);
    delete m;
    return st;
  }
  spconv::BuildScratch s;
  spconv::carve_build_scratch(p, c->scratch, &s);
  spconv::carve_map_buffers(p, m->block, &m->buf);
  auto discard = [&](spconv_status st) {
    (void)hipFreeAsync(m->block, stream);
    release_slot(device, m->slot);
    delete m;
    return st;
  };

  // The table sits at the start of the scratch, so a clear table of the same
  // size is this build's table.  Until the launches succeed it is not known
  // clear.
  const bool table_clear = c->clear_slots == p.table_slots;
  c->clear_slots = 0;
  hipError_t e = spconv::launch_build(p, d_coords, s, m->buf, m->slot->device, table_clear, stream);
  if (e != hipSuccess) return discard(hip_fail(e, "map build launch"));
  c->clear_slots = p.ordered ? 0 : p.table_slots;  // k_compact leaves an unordered map's table clear
  e = hipEventRecord(m->slot->done, stream);
  if (e != hipSuccess) return discard(hip_fail(e, "hipEventRecord"));

  m->device = device;
  m->stream = stream;
  m->K = kernel_size;
  m->KV = KV;
  m->n = n;
  m->n_in = n;
  m->centre = (KV - 1) / 2;
  m->tiles = p.tiles;
  *out_map = m;
  return SPCONV_OK;
}

spconv_status spconv_build_map(const int32_t* d_coords, int64_t n, int32_t kernel_size,
                               void* hip_stream, spconv_map** out_map) {
  spconv_status st = spconv_build_map_async(d_coords, n, kernel_size, hip_stream, out_map);
  if (st != SPCONV_OK) return st;
  st = finish_build(*out_map);
  if (st != SPCONV_OK) {
    spconv_map_free(*out_map);
    *out_map = nullptr;
  }
  return st;
}

spconv_status spconv_map_wait(spconv_map* map) {
  if (map == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "map is NULL");
  return finish_build(map);
}

spconv_status spconv_map_info(spconv_map* map, int32_t* kernel_size, int64_t* n,
                              int64_t* total_entries) {
  if (map == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "map is NULL");
  if (kernel_size) *kernel_size = map->K;
  if (n) *n = map->n;
  if (total_entries) {
    const spconv_status st = finish_build(map);
    if (st != SPCONV_OK) return st;
    *total_entries = map->total;
  }
  return SPCONV_OK;
}

spconv_status spconv_map_counts(spconv_map* map, int64_t* h_counts, int64_t* h_offsets) {
  if (map == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "map is NULL");
  const spconv_status st = finish_build(map);
  if (st != SPCONV_OK) return st;
  if (h_counts) std::memcpy(h_counts, map->counts.data(), sizeof(int64_t) * map->KV);
  if (h_offsets) std::memcpy(h_offsets, map->offsets.data(), sizeof(int64_t) * (map->KV + 1));
  return SPCONV_OK;
}

spconv_status spconv_map_lists(const spconv_map* map, const int32_t** d_in_idx,
                               const int32_t** d_out_idx) {
  if (map == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "map is NULL");
  if (d_in_idx) *d_in_idx = map->buf.in_idx;
  if (d_out_idx) *d_out_idx = map->buf.out_idx;
  return SPCONV_OK;
}

spconv_status spconv_forward(const void* d_feats, const void* d_weights, const spconv_map* map,
                             int32_t c_in, int32_t c_out, spconv_dtype dtype, void* d_out,
                             void* hip_stream) {
  g_last_error.clear();
  spconv::ForwardArgs a;
  spconv_status st = forward_args(d_feats, d_weights, map, c_in, c_out, dtype, d_out, &a);
  if (st != SPCONV_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  st = order_after_build(map, stream);
  if (st != SPCONV_OK) return st;
  if (known_empty(map)) return zero_output(d_out, map->n, c_out, dtype, stream);
  const ForwardPath path = forward_path(a);
  const size_t ws_bytes = forward_workspace_bytes(path, a);
  if (ws_bytes == 0) return launch_forward_path(path, a, nullptr, stream);
  hipMemPool_t pool = nullptr;
  st = pool_for(map->device, &pool);
  if (st != SPCONV_OK) return st;
  // The stream's forward workspace (prepared weights, zero row, partials),
  // reused by later forwards on the stream.
  std::lock_guard<std::mutex> lock(g_cache_mu);
  StreamCache* c = cache_for(map->device, stream);
  st = grow_buffer(c->fwd, c->fwd_bytes, ws_bytes, pool, stream, "forward workspace allocation");
  if (st != SPCONV_OK) return st;
  return launch_forward_path(path, a, c->fwd, stream);
}

spconv_status spconv_forward_noalloc(const void* d_feats, const void* d_weights, const spconv_map* map,
                                     int32_t c_in, int32_t c_out, spconv_dtype dtype, void* d_out,
                                     void* hip_stream) {
  g_last_error.clear();
  spconv::ForwardArgs a;
  spconv_status st = forward_args(d_feats, d_weights, map, c_in, c_out, dtype, d_out, &a);
  if (st != SPCONV_OK) return st;
  const ForwardPath path = forward_path(a);
  const size_t ws_bytes = forward_workspace_bytes(path, a);
  if (ws_bytes > kNoAllocScratchBytes) {
    return fail(SPCONV_ERR_UNSUPPORTED,
                "this forward needs %zu bytes of workspace; the fixed scratch of spconv_forward_noalloc holds %zu",
                ws_bytes, kNoAllocScratchBytes);
  }
  int device = 0;
  SPCONV_HIP(hipGetDevice(&device), "hipGetDevice");
  if (device != map->device) {
    return fail(SPCONV_ERR_INVALID_ARG, "the current device (%d) is not the map's (%d)", device, map->device);
  }
  void* ws = nullptr;
  if (ws_bytes > 0) {
    st = noalloc_scratch(device, &ws);
    if (st != SPCONV_OK) return st;
  }
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  st = order_after_build(map, stream);
  if (st != SPCONV_OK) return st;
  if (known_empty(map)) return zero_output(d_out, map->n, c_out, dtype, stream);
  return launch_forward_path(path, a, ws, stream);
}

spconv_status spconv_weights_prepare(const void* d_weights, int32_t kernel_volume, int32_t c_in, int32_t c_out,
                                     spconv_dtype dtype, void* hip_stream, spconv_weights** out) {
  g_last_error.clear();
  if (out == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (d_weights == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "NULL weight pointer");
  if (!aligned16(d_weights)) return fail(SPCONV_ERR_INVALID_ARG, "the weights must be 16-byte aligned");
  if (dtype != SPCONV_F32 && dtype != SPCONV_F16 && dtype != SPCONV_BF16) {
    return fail(SPCONV_ERR_UNSUPPORTED, "dtype %d not supported", static_cast<int>(dtype));
  }
  if (kernel_volume < 1 || kernel_volume > 343) {
    return fail(SPCONV_ERR_INVALID_ARG, "kernel_volume = %d must lie in [1, 343]", kernel_volume);
  }
  const int32_t cmax = (dtype == SPCONV_F32) ? 512 : 1024;
  if (c_in < 1 || c_out < 1 || c_in > cmax || c_out > cmax) {
    return fail(SPCONV_ERR_INVALID_ARG, "c_in = %d, c_out = %d must lie in [1, %d]", c_in, c_out, cmax);
  }
  const int32_t mult = (dtype == SPCONV_F32) ? 4 : 8;
  if (c_in % mult != 0 || c_out % mult != 0) {
    return fail(SPCONV_ERR_UNSUPPORTED, "c_in = %d and c_out = %d must be multiples of %d", c_in, c_out, mult);
  }
  int device = 0;
  SPCONV_HIP(hipGetDevice(&device), "hipGetDevice");
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  auto* w = new (std::nothrow) spconv_weights;
  if (w == nullptr) return fail(SPCONV_ERR_OUT_OF_MEMORY, "host allocation of the weight handle");
  w->device = device;
  w->KV = kernel_volume;
  w->c_in = c_in;
  w->c_out = c_out;
  w->dtype = dtype;
  const size_t raw_b = static_cast<size_t>(kernel_volume) * c_in * c_out * (dtype == SPCONV_F32 ? 4 : 2);
  // The operand-order copy exists for the shapes of the wide and tiled paths
  // (F16/BF16, C_in in {32, 64, 128, 256}, C_out a multiple of 16, K^3 <= 128).
  spconv::ForwardArgs a;
  a.weights = d_weights;
  a.KV = kernel_volume;
  a.cin = c_in;
  a.cout = c_out;
  a.dtype = static_cast<int32_t>(dtype);
  const bool with_prepared = dtype != SPCONV_F32 && kernel_volume <= 128 && c_out % 16 == 0 &&
                             (c_in == 32 || c_in == 64 || c_in == 128 || c_in == 256);
  hipError_t e = hipMalloc(&w->raw, raw_b);
  if (e == hipSuccess && with_prepared) e = hipMalloc(&w->prepared, spconv::tiled_workspace_bytes(a));
  if (e != hipSuccess) {
    spconv_weights_free(w);
    return e == hipErrorOutOfMemory ? fail(SPCONV_ERR_OUT_OF_MEMORY, "weight copy allocation")
                                    : hip_fail(e, "weight copy allocation");
  }
  e = hipMemcpyAsync(w->raw, d_weights, raw_b, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess && with_prepared) e = spconv::launch_prep_weights(a, w->prepared, stream);
  if (e != hipSuccess) {
    spconv_weights_free(w);
    return hip_fail(e, "weight preparation");
  }
  *out = w;
  return SPCONV_OK;
}

spconv_status spconv_forward_prepared(const void* d_feats, const spconv_weights* weights, const spconv_map* map,
                                      void* d_out, void* hip_stream) {
  g_last_error.clear();
  if (weights == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "weights is NULL");
  if (map != nullptr && map->KV != weights->KV) {
    return fail(SPCONV_ERR_INVALID_ARG, "the map has %d offsets, the weights %d", map->KV, weights->KV);
  }
  if (map != nullptr && map->device != weights->device) {
    return fail(SPCONV_ERR_INVALID_ARG, "the map is on device %d, the weights on %d", map->device, weights->device);
  }
  spconv::ForwardArgs a;
  spconv_status st = forward_args(d_feats, weights->raw, map, weights->c_in, weights->c_out, weights->dtype, d_out,
                                  &a);
  if (st != SPCONV_OK) return st;
  a.prepared = weights->prepared;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  st = order_after_build(map, stream);
  if (st != SPCONV_OK) return st;
  if (known_empty(map)) return zero_output(d_out, map->n, weights->c_out, weights->dtype, stream);
  return launch_fused(map, a, stream);
}

void spconv_weights_free(spconv_weights* weights) {
  if (weights == nullptr) return;
  // hipFree waits for the device's work in flight, which may still read them.
  if (weights->raw != nullptr) (void)hipFree(weights->raw);
  if (weights->prepared != nullptr) (void)hipFree(weights->prepared);
  delete weights;
}

spconv_status spconv_backward_data(const void* d_grad_out, const void* d_weights, const spconv_map* map,
                                   int32_t c_in, int32_t c_out, spconv_dtype dtype, void* d_grad_in,
                                   void* hip_stream) {
  g_last_error.clear();
  if (map != nullptr && map->kind != SPCONV_MAP_SUBMANIFOLD) {
    return fail(SPCONV_ERR_UNSUPPORTED,
                "the data gradient of a strided or transposed map is the forward over its transpose "
                "(spconv_map_transpose) with the weights W[k]^T");
  }
  // The data gradient is the forward of grad_out over the same map with the
  // mirrored, transposed weights: C_out channels in, C_in out.
  spconv::ForwardArgs a;
  spconv_status st = forward_args(d_grad_out, d_weights, map, c_out, c_in, dtype, d_grad_in, &a);
  if (st != SPCONV_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  st = order_after_build(map, stream);
  if (st != SPCONV_OK) return st;
  const size_t mirror_bytes = spconv::mirror_workspace_bytes(map->KV, c_in, c_out, static_cast<int>(dtype));
  const ForwardPath path = forward_path(a);
  const size_t ws_bytes = mirror_bytes + forward_workspace_bytes(path, a);
  hipMemPool_t pool = nullptr;
  st = pool_for(map->device, &pool);
  if (st != SPCONV_OK) return st;
  std::lock_guard<std::mutex> lock(g_cache_mu);
  StreamCache* c = cache_for(map->device, stream);
  st = grow_buffer(c->fwd, c->fwd_bytes, ws_bytes, pool, stream, "backward workspace allocation");
  if (st != SPCONV_OK) return st;
  const hipError_t e = spconv::launch_mirror_transpose(d_weights, c->fwd, map->KV, c_in, c_out,
                                                       static_cast<int>(dtype), stream);
  if (e != hipSuccess) return hip_fail(e, "weight mirror launch");
  a.weights = c->fwd;
  return launch_forward_path(path, a, static_cast<char*>(c->fwd) + mirror_bytes, stream);
}

spconv_status spconv_backward_weights(const void* d_feats, const void* d_grad_out, const spconv_map* map,
                                      int32_t c_in, int32_t c_out, spconv_dtype dtype, float* d_grad_w,
                                      void* hip_stream) {
  g_last_error.clear();
  if (map == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "map is NULL");
  if ((d_feats == nullptr && map->n_in > 0) || (d_grad_out == nullptr && map->n > 0) || d_grad_w == nullptr) {
    return fail(SPCONV_ERR_INVALID_ARG, "NULL feature, gradient or weight-gradient pointer");
  }
  if (!aligned16(d_feats) || !aligned16(d_grad_out) || !aligned16(d_grad_w)) {
    return fail(SPCONV_ERR_INVALID_ARG, "feature and gradient buffers must be 16-byte aligned");
  }
  if (dtype != SPCONV_F32 && dtype != SPCONV_F16 && dtype != SPCONV_BF16) {
    return fail(SPCONV_ERR_UNSUPPORTED, "dtype %d not supported", static_cast<int>(dtype));
  }
  const int32_t cmax = (dtype == SPCONV_F32) ? 512 : 1024;
  if (c_in < 1 || c_out < 1 || c_in > cmax || c_out > cmax) {
    return fail(SPCONV_ERR_INVALID_ARG, "c_in = %d, c_out = %d must lie in [1, %d]", c_in, c_out, cmax);
  }
  const int32_t mult = (dtype == SPCONV_F32) ? 4 : 8;
  if (c_in % mult != 0 || c_out % mult != 0) {
    return fail(SPCONV_ERR_UNSUPPORTED, "c_in = %d and c_out = %d must be multiples of %d", c_in, c_out, mult);
  }
  {
    const uint64_t es = (dtype == SPCONV_F32) ? 4u : 2u;
    const uint64_t gw_b = static_cast<uint64_t>(map->KV) * c_in * c_out * sizeof(float);
    auto overlap = [](const void* p, uint64_t np, const void* q, uint64_t nq) {
      const uint64_t a0 = reinterpret_cast<uintptr_t>(p), b0 = reinterpret_cast<uintptr_t>(q);
      return a0 < b0 + nq && b0 < a0 + np;
    };
    if (overlap(d_grad_w, gw_b, d_feats, static_cast<uint64_t>(map->n_in) * c_in * es) ||
        overlap(d_grad_w, gw_b, d_grad_out, static_cast<uint64_t>(map->n) * c_out * es)) {
      return fail(SPCONV_ERR_INVALID_ARG, "d_grad_w overlaps the features or the output gradient");
    }
  }
  spconv::WgradArgs a;
  a.feats = d_feats;
  a.grad_out = d_grad_out;
  a.grad_w = d_grad_w;
  a.in_idx = map->buf.in_idx;
  a.out_idx = map->buf.out_idx;
  a.tile_off = map->buf.tile_off;
  a.n = map->n;
  a.n_in = map->n_in;
  a.tiles = map->tiles;
  a.KV = map->KV;
  a.cin = c_in;
  a.cout = c_out;
  a.dtype = static_cast<int32_t>(dtype);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  spconv_status st = order_after_build(map, stream);
  if (st != SPCONV_OK) return st;
  if (known_empty(map)) {
    SPCONV_HIP(hipMemsetAsync(d_grad_w, 0, static_cast<size_t>(map->KV) * c_in * c_out * sizeof(float), stream),
               "hipMemsetAsync");
    return SPCONV_OK;
  }
  hipMemPool_t pool = nullptr;
  st = pool_for(map->device, &pool);
  if (st != SPCONV_OK) return st;
  std::lock_guard<std::mutex> lock(g_cache_mu);
  StreamCache* c = cache_for(map->device, stream);
  st = grow_buffer(c->fwd, c->fwd_bytes, spconv::wgrad_workspace_bytes(a), pool, stream,
                   "weight-gradient workspace allocation");
  if (st != SPCONV_OK) return st;
  const hipError_t e = spconv::launch_wgrad(a, c->fwd, stream);
  if (e != hipSuccess) return hip_fail(e, "weight-gradient launch");
  return SPCONV_OK;
}

spconv_status spconv_build_map_strided(const int32_t* d_coords, int64_t n_in, int32_t kernel_size, int32_t stride,
                                       void* hip_stream, spconv_map** out_map) {
  g_last_error.clear();
  if (out_map == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "out_map is NULL");
  *out_map = nullptr;
  if (d_coords == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "d_coords is NULL");
  if (!aligned16(d_coords)) return fail(SPCONV_ERR_INVALID_ARG, "d_coords is not 16-byte aligned");
  if (n_in <= 0) return fail(SPCONV_ERR_INVALID_ARG, "n_in = %lld must be positive", (long long)n_in);
  if (kernel_size < 1 || kernel_size > 5) {
    return fail(SPCONV_ERR_UNSUPPORTED, "kernel_size = %d not in [1, 5] for a strided map", kernel_size);
  }
  if (stride < 1 || stride > 16) return fail(SPCONV_ERR_UNSUPPORTED, "stride = %d not in [1, 16]", stride);
  const spconv::OutCoordPlan op = spconv::out_coord_plan(n_in, kernel_size, stride);
  if (op.m >= (int64_t(1) << 31)) {
    return fail(SPCONV_ERR_INVALID_ARG, "n_in x ceil(K / stride)^3 = %lld must stay below 2^31", (long long)op.m);
  }
  const int32_t KV = kernel_size * kernel_size * kernel_size;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  int device = 0;
  SPCONV_HIP(hipGetDevice(&device), "hipGetDevice");
  hipMemPool_t pool = nullptr;
  spconv_status st = pool_for(device, &pool);
  if (st != SPCONV_OK) return st;
  spconv_map* m = new (std::nothrow) spconv_map;
  if (m == nullptr) return fail(SPCONV_ERR_OUT_OF_MEMORY, "host allocation");
  m->device = device;
  m->stream = stream;
  m->K = kernel_size;
  m->KV = KV;
  m->n_in = n_in;
  m->centre = -1;
  m->stride = stride;
  m->kind = SPCONV_MAP_STRIDED;
  st = acquire_slot(device, &m->slot);
  if (st != SPCONV_OK) {
    delete m;
    return st;
  }
  // Phase 1: the input table, the outputs' keys sorted and counted; the host
  // reads the flags and the number of outputs (the map's size depends on it).
  const int64_t slots = spconv::table_slots_for(n_in);
  const size_t table_b = align256(static_cast<size_t>(slots) * sizeof(ulonglong2));
  const size_t occ_b = align256(static_cast<size_t>(slots / 4) * sizeof(uint4));
  const size_t sum_b = align256(static_cast<size_t>(spconv::kSummaryHead + KV) * sizeof(long long));
  const size_t a_bytes = table_b + occ_b + sum_b + spconv::out_coord_scratch_bytes(op);
  void* a_buf = nullptr;
  void* b_buf = nullptr;
  auto discard = [&](spconv_status s2) {
    if (m->block != nullptr) (void)hipFreeAsync(m->block, stream);
    if (a_buf != nullptr) (void)hipFreeAsync(a_buf, stream);
    if (b_buf != nullptr) (void)hipFreeAsync(b_buf, stream);
    if (m->slot != nullptr) release_slot(device, m->slot);
    delete m;
    return s2;
  };
  hipError_t e = hipMallocFromPoolAsync(&a_buf, a_bytes, pool, stream);
  if (e != hipSuccess) return discard(hip_fail(e, "strided map workspace allocation"));
  char* ac = static_cast<char*>(a_buf);
  ulonglong2* table = reinterpret_cast<ulonglong2*>(ac);
  uint4* occ = reinterpret_cast<uint4*>(ac + table_b);
  long long* summary = reinterpret_cast<long long*>(ac + table_b + occ_b);
  void* sort_scratch = ac + table_b + occ_b + sum_b;
  e = spconv::launch_table_build(d_coords, n_in, table, slots, occ, summary, spconv::kSummaryHead + KV, stream);
  if (e == hipSuccess) e = spconv::launch_out_coords_count(op, d_coords, sort_scratch, summary + 1, stream);
  if (e == hipSuccess) {
    e = hipMemcpyAsync(m->slot->host, summary, 2 * sizeof(long long), hipMemcpyDeviceToHost, stream);
  }
  if (e == hipSuccess) e = hipEventRecord(m->slot->done, stream);
  if (e == hipSuccess) e = hipEventSynchronize(m->slot->done);
  if (e != hipSuccess) return discard(hip_fail(e, "strided map build"));
  const unsigned long long flags = static_cast<unsigned long long>(m->slot->host[0]);
  if (flags & spconv::kFlagRange) {
    return discard(fail(SPCONV_ERR_COORD_RANGE, "a coordinate is outside b in [0, 2^15), z, y, x in [0, 2^16)"));
  }
  if (flags & spconv::kFlagDuplicate) {
    return discard(fail(SPCONV_ERR_DUPLICATE_COORD, "two rows share one (b, z, y, x) coordinate"));
  }
  if (flags & spconv::kFlagTableFull) return discard(fail(SPCONV_ERR_DEVICE, "internal: hash table probe exceeded its bound"));
  const int64_t n_out = m->slot->host[1];
  if (n_out * KV >= (int64_t(1) << 31)) {
    return discard(fail(SPCONV_ERR_INVALID_ARG, "n_out x K^3 = %lld x %d must stay below 2^31", (long long)n_out, KV));
  }
  // Phase 2: the map over the n_out outputs.
  const int64_t cap = std::max<int64_t>(64, std::min<int64_t>(static_cast<int64_t>(KV) * n_out, op.m));
  m->n = n_out;
  m->tiles = (n_out + spconv::kTileRows - 1) / spconv::kTileRows;
  size_t block_bytes = 0;
  const GeneralLayout lay = general_layout(m->tiles, KV, cap, n_out, n_in, &block_bytes);
  e = hipMallocFromPoolAsync(&m->block, block_bytes, pool, stream);
  if (e != hipSuccess) return discard(hip_fail(e, "map allocation"));
  m->block_bytes = block_bytes;
  carve_general(lay, m);
  if (n_out > 0) {
    e = hipMallocFromPoolAsync(&b_buf, spconv::general_scratch_bytes(n_out, kernel_size), pool, stream);
    if (e != hipSuccess) return discard(hip_fail(e, "strided map workspace allocation"));
  }
  e = spconv::launch_out_coords_write(op, sort_scratch, m->out_coords, stream);
  if (e == hipSuccess) {
    e = hipMemcpyAsync(m->in_coords, d_coords, static_cast<size_t>(n_in) * 4 * sizeof(int32_t),
                       hipMemcpyDeviceToDevice, stream);
  }
  if (e == hipSuccess && n_out > 0) {
    spconv::GeneralMapArgs g;
    g.qcoords = m->out_coords;
    g.nq = n_out;
    g.table = table;
    g.table_slots = slots;
    g.K = kernel_size;
    g.lo = -((kernel_size - 1) / 2);
    g.stride = stride;
    g.mode = 0;
    spconv::carve_general_scratch(n_out, kernel_size, b_buf, &g);
    g.summary = summary;
    g.host_summary = m->slot->device;
    g.map = m->buf;
    e = spconv::launch_general_map(g, stream);
  }
  if (e != hipSuccess) return discard(hip_fail(e, "strided map launch"));
  if (n_out == 0) {
    mark_empty(m);
  } else {
    e = hipEventRecord(m->slot->done, stream);
    if (e != hipSuccess) return discard(hip_fail(e, "hipEventRecord"));
  }
  (void)hipFreeAsync(a_buf, stream);
  if (b_buf != nullptr) (void)hipFreeAsync(b_buf, stream);
  a_buf = b_buf = nullptr;
  st = finish_build(m);
  if (st != SPCONV_OK) {
    spconv_map_free(m);
    return st;
  }
  *out_map = m;
  return SPCONV_OK;
}

spconv_status spconv_map_transpose(spconv_map* map, void* hip_stream, spconv_map** out_map) {
  g_last_error.clear();
  if (out_map == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "out_map is NULL");
  *out_map = nullptr;
  if (map == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "map is NULL");
  if (map->kind != SPCONV_MAP_STRIDED) {
    return fail(SPCONV_ERR_UNSUPPORTED, "only a strided map has a transpose here (a submanifold map is its own, "
                                        "with mirrored weights)");
  }
  spconv_status st = finish_build(map);
  if (st != SPCONV_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  int device = 0;
  SPCONV_HIP(hipGetDevice(&device), "hipGetDevice");
  if (device != map->device) {
    return fail(SPCONV_ERR_INVALID_ARG, "the current device (%d) is not the map's (%d)", device, map->device);
  }
  st = order_after_build(map, stream);
  if (st != SPCONV_OK) return st;
  hipMemPool_t pool = nullptr;
  st = pool_for(device, &pool);
  if (st != SPCONV_OK) return st;
  spconv_map* t = new (std::nothrow) spconv_map;
  if (t == nullptr) return fail(SPCONV_ERR_OUT_OF_MEMORY, "host allocation");
  t->device = device;
  t->stream = stream;
  t->K = map->K;
  t->KV = map->KV;
  t->n = map->n_in;
  t->n_in = map->n;
  t->centre = -1;
  t->stride = map->stride;
  t->kind = SPCONV_MAP_TRANSPOSED;
  t->tiles = (t->n + spconv::kTileRows - 1) / spconv::kTileRows;
  void* a_buf = nullptr;
  auto discard = [&](spconv_status s2) {
    if (t->block != nullptr) (void)hipFreeAsync(t->block, stream);
    if (a_buf != nullptr) (void)hipFreeAsync(a_buf, stream);
    if (t->slot != nullptr) release_slot(device, t->slot);
    delete t;
    return s2;
  };
  st = acquire_slot(device, &t->slot);
  if (st != SPCONV_OK) {
    delete t;
    return st;
  }
  const int64_t cap = std::max<int64_t>(64, map->total);
  size_t block_bytes = 0;
  const GeneralLayout lay = general_layout(t->tiles, t->KV, cap, t->n, t->n_in, &block_bytes);
  hipError_t e = hipMallocFromPoolAsync(&t->block, block_bytes, pool, stream);
  if (e != hipSuccess) return discard(hip_fail(e, "map allocation"));
  t->block_bytes = block_bytes;
  carve_general(lay, t);
  e = hipMemcpyAsync(t->out_coords, map->in_coords, static_cast<size_t>(t->n) * 4 * sizeof(int32_t),
                     hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess && t->n_in > 0) {
    e = hipMemcpyAsync(t->in_coords, map->out_coords, static_cast<size_t>(t->n_in) * 4 * sizeof(int32_t),
                       hipMemcpyDeviceToDevice, stream);
  }
  if (e != hipSuccess) return discard(hip_fail(e, "hipMemcpyAsync"));
  if (map->total == 0) {
    mark_empty(t);
    *out_map = t;
    return SPCONV_OK;
  }
  // The strided map's outputs in a table; each of its inputs probes the
  // outputs q' with stride x q' + d = p.
  const int64_t slots = spconv::table_slots_for(t->n_in);
  const size_t table_b = align256(static_cast<size_t>(slots) * sizeof(ulonglong2));
  const size_t occ_b = align256(static_cast<size_t>(slots / 4) * sizeof(uint4));
  const size_t sum_b = align256(static_cast<size_t>(spconv::kSummaryHead + t->KV) * sizeof(long long));
  e = hipMallocFromPoolAsync(&a_buf, table_b + occ_b + sum_b + spconv::general_scratch_bytes(t->n, t->K), pool,
                             stream);
  if (e != hipSuccess) return discard(hip_fail(e, "transpose workspace allocation"));
  char* ac = static_cast<char*>(a_buf);
  ulonglong2* table = reinterpret_cast<ulonglong2*>(ac);
  uint4* occ = reinterpret_cast<uint4*>(ac + table_b);
  long long* summary = reinterpret_cast<long long*>(ac + table_b + occ_b);
  e = spconv::launch_table_build(map->out_coords, t->n_in, table, slots, occ, summary, spconv::kSummaryHead + t->KV,
                                 stream);
  if (e == hipSuccess) {
    spconv::GeneralMapArgs g;
    g.qcoords = t->out_coords;
    g.nq = t->n;
    g.table = table;
    g.table_slots = slots;
    g.K = t->K;
    g.lo = -((t->K - 1) / 2);
    g.stride = t->stride;
    g.mode = 1;
    spconv::carve_general_scratch(t->n, t->K, ac + table_b + occ_b + sum_b, &g);
    g.summary = summary;
    g.host_summary = t->slot->device;
    g.map = t->buf;
    e = spconv::launch_general_map(g, stream);
  }
  if (e == hipSuccess) e = hipEventRecord(t->slot->done, stream);
  if (e != hipSuccess) return discard(hip_fail(e, "transpose launch"));
  (void)hipFreeAsync(a_buf, stream);
  a_buf = nullptr;
  st = finish_build(t);
  if (st == SPCONV_OK && t->total != map->total) {
    st = fail(SPCONV_ERR_DEVICE, "internal: the transpose holds %lld entries, the map %lld", (long long)t->total,
              (long long)map->total);
  }
  if (st != SPCONV_OK) {
    spconv_map_free(t);
    return st;
  }
  *out_map = t;
  return SPCONV_OK;
}

spconv_status spconv_map_geometry(const spconv_map* map, int64_t* n_in, int64_t* n_out, int32_t* stride,
                                  int32_t* kind) {
  if (map == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "map is NULL");
  if (n_in) *n_in = map->n_in;
  if (n_out) *n_out = map->n;
  if (stride) *stride = map->stride;
  if (kind) *kind = map->kind;
  return SPCONV_OK;
}

spconv_status spconv_map_out_coords(const spconv_map* map, const int32_t** d_out_coords) {
  if (map == nullptr || d_out_coords == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "NULL argument");
  if (map->kind == SPCONV_MAP_SUBMANIFOLD) {
    return fail(SPCONV_ERR_UNSUPPORTED, "a submanifold map's outputs are its inputs (the caller's coordinates)");
  }
  *d_out_coords = map->out_coords;
  return SPCONV_OK;
}

spconv_status spconv_group_plan_counts(const int64_t* h_counts, int32_t kernel_volume, int32_t centre,
                                       double epsilon, double S, int32_t capacity, int32_t* h_offsets,
                                       int32_t* h_groups, int32_t* n_entries, int32_t* n_groups,
                                       int64_t* padded_rows) {
  g_last_error.clear();
  if (h_counts == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "h_counts is NULL");
  if (kernel_volume < 1 || kernel_volume > spconv::kMaxGroupEntries) {
    return fail(SPCONV_ERR_INVALID_ARG, "kernel_volume = %d not in [1, %d]", kernel_volume,
                spconv::kMaxGroupEntries);
  }
  if (centre < -1 || centre >= kernel_volume) {
    return fail(SPCONV_ERR_INVALID_ARG, "centre = %d not in [-1, %d)", centre, kernel_volume);
  }
  for (int32_t k = 0; k < kernel_volume; ++k) {
    if (h_counts[k] < 0 || h_counts[k] >= (int64_t(1) << 40)) {
      return fail(SPCONV_ERR_INVALID_ARG, "count %lld of offset %d not in [0, 2^40)", (long long)h_counts[k], k);
    }
  }
  spconv_status st = check_plan_args(epsilon, S);
  if (st != SPCONV_OK) return st;
  const spconv::GroupPlan plan = spconv::make_group_plan(h_counts, kernel_volume, centre, epsilon, S);
  const int32_t n = static_cast<int32_t>(plan.entries.size());
  if ((h_offsets != nullptr || h_groups != nullptr) && capacity < n) {
    return fail(SPCONV_ERR_INVALID_ARG, "capacity %d below the plan's %d entries", capacity, n);
  }
  for (int32_t i = 0; i < n; ++i) {
    if (h_offsets) h_offsets[i] = plan.entries[i];
    if (h_groups) h_groups[i] = plan.entry_group[i];
  }
  if (n_entries) *n_entries = n;
  if (n_groups) *n_groups = plan.groups;
  if (padded_rows) *padded_rows = plan.padded_rows;
  return SPCONV_OK;
}

spconv_status spconv_group_plan(spconv_map* map, double epsilon, double S, int32_t capacity, int32_t* h_offsets,
                                int32_t* h_groups, int32_t* n_entries, int32_t* n_groups, int64_t* padded_rows) {
  g_last_error.clear();
  if (map == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "map is NULL");
  spconv_status st = check_plan_args(epsilon, S);
  if (st != SPCONV_OK) return st;
  st = finish_build(map);
  if (st != SPCONV_OK) return st;
  return spconv_group_plan_counts(map->counts.data(), map->KV, map->centre, epsilon, S, capacity, h_offsets,
                                  h_groups, n_entries, n_groups, padded_rows);
}

spconv_status spconv_forward_grouped(const void* d_feats, const void* d_weights, spconv_map* map, int32_t c_in,
                                     int32_t c_out, spconv_dtype dtype, double epsilon, double S, void* d_out,
                                     void* hip_stream) {
  g_last_error.clear();
  spconv::ForwardArgs a;
  spconv_status st = forward_args(d_feats, d_weights, map, c_in, c_out, dtype, d_out, &a);
  if (st != SPCONV_OK) return st;
  st = check_plan_args(epsilon, S);
  if (st != SPCONV_OK) return st;
  if (!spconv::grouped_supported(a)) {
    return fail(SPCONV_ERR_UNSUPPORTED, "the grouped forward needs f16 or bf16, c_in %% 32 == 0 and c_out %% 16 == 0");
  }
  st = finish_build(map);
  if (st != SPCONV_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (map->total == 0) return zero_output(d_out, map->n, c_out, dtype, stream);
  const spconv::GroupPlan plan = spconv::make_group_plan(map->counts.data(), map->KV, map->centre, epsilon, S);
  return launch_grouped(map, a, plan, stream);
}

spconv_status spconv_select_dataflow(const void* d_feats, const void* d_weights, spconv_map* map, int32_t c_in,
                                     int32_t c_out, spconv_dtype dtype, const double* epsilons, int32_t n_epsilons,
                                     const double* thresholds, int32_t n_thresholds, int32_t reps, void* d_out,
                                     void* hip_stream, spconv_dataflow* best) {
  g_last_error.clear();
  if (best == nullptr) return fail(SPCONV_ERR_INVALID_ARG, "best is NULL");
  spconv::ForwardArgs a;
  spconv_status st = forward_args(d_feats, d_weights, map, c_in, c_out, dtype, d_out, &a);
  if (st != SPCONV_OK) return st;
  if (reps < 1 || reps > 1000) return fail(SPCONV_ERR_INVALID_ARG, "reps = %d not in [1, 1000]", reps);
  static const double kEps[] = {0.0, 0.1, 0.2, 0.3, 0.5, 1.0};
  static const double kS[] = {HUGE_VAL, 65536.0, 16384.0, 0.0};
  if (epsilons == nullptr) {
    epsilons = kEps;
    n_epsilons = static_cast<int32_t>(sizeof(kEps) / sizeof(kEps[0]));
  }
  if (thresholds == nullptr) {
    thresholds = kS;
    n_thresholds = static_cast<int32_t>(sizeof(kS) / sizeof(kS[0]));
  }
  if (n_epsilons < 0 || n_thresholds < 0 || n_epsilons > 64 || n_thresholds > 64) {
    return fail(SPCONV_ERR_INVALID_ARG, "grids of %d and %d values (at most 64 each)", n_epsilons, n_thresholds);
  }
  for (int32_t i = 0; i < n_epsilons; ++i) {
    st = check_plan_args(epsilons[i], 0.0);
    if (st != SPCONV_OK) return st;
  }
  for (int32_t i = 0; i < n_thresholds; ++i) {
    st = check_plan_args(0.0, thresholds[i]);
    if (st != SPCONV_OK) return st;
  }
  st = finish_build(map);
  if (st != SPCONV_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  std::memset(best, 0, sizeof(*best));
  best->kind = SPCONV_DATAFLOW_FUSED;
  if (map->total == 0) {
    best->candidates = 1;
    return zero_output(d_out, map->n, c_out, dtype, stream);
  }
  // Candidates: the fused forward, then each distinct plan of the grid.
  struct Candidate {
    bool grouped;
    double epsilon, S;
    spconv::GroupPlan plan;
  };
  std::vector<Candidate> cands;
  cands.push_back({false, 0.0, 0.0, {}});
  if (spconv::grouped_supported(a)) {
    for (int32_t j = 0; j < n_thresholds; ++j) {
      for (int32_t i = 0; i < n_epsilons; ++i) {
        spconv::GroupPlan p =
            spconv::make_group_plan(map->counts.data(), map->KV, map->centre, epsilons[i], thresholds[j]);
        bool seen = false;
        for (size_t c = 1; c < cands.size() && !seen; ++c) seen = same_plan(cands[c].plan, p);
        if (!seen) cands.push_back({true, epsilons[i], thresholds[j], std::move(p)});
      }
    }
  }
  auto run = [&](const Candidate& c) {
    return c.grouped ? launch_grouped(map, a, c.plan, stream) : launch_fused(map, a, stream);
  };
  hipEvent_t t0 = nullptr, t1 = nullptr;
  SPCONV_HIP(hipEventCreate(&t0), "hipEventCreate");
  hipError_t ec = hipEventCreate(&t1);
  if (ec != hipSuccess) {
    (void)hipEventDestroy(t0);
    return hip_fail(ec, "hipEventCreate");
  }
  size_t win = 0;
  float win_ms = 0.f;
  for (size_t c = 0; c < cands.size() && st == SPCONV_OK; ++c) {
    st = run(cands[c]);  // warm-up (workspace growth, first-touch)
    if (st != SPCONV_OK) break;
    ec = hipEventRecord(t0, stream);
    for (int32_t r = 0; r < reps && st == SPCONV_OK && ec == hipSuccess; ++r) st = run(cands[c]);
    if (st != SPCONV_OK) break;
    if (ec == hipSuccess) ec = hipEventRecord(t1, stream);
    if (ec == hipSuccess) ec = hipEventSynchronize(t1);
    float ms = 0.f;
    if (ec == hipSuccess) ec = hipEventElapsedTime(&ms, t0, t1);
    if (ec != hipSuccess) {
      st = hip_fail(ec, "dataflow timing");
      break;
    }
    ms /= static_cast<float>(reps);
    if (c == 0) best->fused_ms = ms;
    if (c == 0 || ms < win_ms) {
      win = c;
      win_ms = ms;
    }
  }
  (void)hipEventDestroy(t0);
  (void)hipEventDestroy(t1);
  if (st != SPCONV_OK) return st;
  // Leave the winner's result in d_out.
  st = run(cands[win]);
  if (st != SPCONV_OK) return st;
  best->kind = cands[win].grouped ? SPCONV_DATAFLOW_GROUPED : SPCONV_DATAFLOW_FUSED;
  best->groups = cands[win].grouped ? cands[win].plan.groups : 0;
  best->epsilon = cands[win].epsilon;
  best->S = cands[win].S;
  best->ms = win_ms;
  best->candidates = static_cast<int32_t>(cands.size());
  return SPCONV_OK;
}

void spconv_map_free(spconv_map* map) {
  if (map == nullptr) return;
  if (map->block != nullptr) release_block(map->device, map->stream, map->block, map->block_bytes);
  if (map->slot != nullptr) release_slot(map->device, map->slot);
  delete map;
}

}  // extern "C"
