// C ABI of the DeepSelect top-k library: argument validation, the launch planner, the
// workspace cache of ds_topk, and dispatch to the HIP kernels. Validation is pure host
// code and runs before any HIP call, so every error path works without a GPU.
#include <algorithm>
#include <cstring>
#include <cmath>
#include <map>
#include <mutex>
#include <unordered_map>
#include <utility>
#include <vector>

#include "ds_internal.h"

namespace {

using ds::kNumSelectShapes;
using ds::kSelectShapes;

constexpr int64_t kMaxLdsBytes = 160 * 1024;    // LDS per workgroup on gfx950
constexpr int64_t kMaxSliceBytes = 0x7FFFFF00;  // buffer offsets are 31-bit
constexpr int kChunkBf16 = 512, kChunkFp32 = 256;
constexpr int kMergeBlock = ds::kMergeShape.waves * ds::kMergeShape.cpw * 128;
// B2 when not forced: the largest of these (and at least k) that fits in LDS and is at most
// 1.5 sqrt(k (k + B)). The design note's expected-work bound (1 + k/B2)(k + B + B2) H_m is
// smallest at B2 = sqrt(k (k + B)); measured on MI355X, the power of two at or just above it
// is best (2048 at k = 512, B = 8192: long rows 56 -> 49 us per call, sampler 41 -> 40 us,
// indexer unchanged; 1024 at k = 32, B = 16384).
constexpr int kDefaultSlacks[] = {4096, 2048, 1024, 512, 256};
// default select shapes (indices into kSelectShapes), best first
// B = 16384 comes first but only takes its own bound-derived B2 (small k: fewer block
// barriers per element, measured 19 % faster at k = 32); larger k falls through to B = 8192
constexpr int kDefaultFp32[] = {9, 8, 7, 2, 1};  // 16x4 (B=16384), 16x2 (8192), 16x1 (4096), 4x2, 4x1
constexpr int kDefaultBf16[] = {8, 7, 3, 1, 0};  // 16x2 (B=16384), 16x1 (8192), 8x1 (4096), 4x1, 2x1
constexpr int kNumDefaults = 5;
constexpr int kMaxStepDownBlock = 8192;  // larger default blocks do not step their B2 down
constexpr int kMaxMergeLevels = 8;  // 16 slices per level at k <= 1024, 4 at k = 4096

int elem_bytes(int dtype) { return dtype == DS_BF16 ? 2 : 4; }
int chunk_elems(int dtype) { return dtype == DS_BF16 ? kChunkBf16 : kChunkFp32; }

int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

struct Plan {
  int dtype;
  int shape;        // index into kSelectShapes
  int block;        // B
  int slack;        // B2
  int slices;       // S
  int64_t slice_len;
  int sort_cap;
  size_t lds;
  bool presample;   // the first whole block sets a presampled threshold
  int order_group;  // G: the random order is over groups of G consecutive blocks
  bool lockstep;    // the design note's schedule: a barrier and the buffer check after every block
  bool unsorted;    // the outputs may hold the top k in any order (DS_OUTPUT_UNSORTED)
  bool idx64;       // int64 output indices (DS_OUTPUT_INDEX_INT64)
  int warmup;       // blocks of the warm-up window
  bool share;       // split rows share a threshold word per row (DS_SHARE_ON)
  size_t share_bytes;  // the row words at the start of the workspace (before the lists)
  // merge (slices > 1): DS_MERGE_LISTS (levels of the list-merge kernel over sorted slice
  // lists, group[l] lists merged together at level l) or DS_MERGE_SELECT (the merge kernel)
  int merge;
  int levels;
  int group[kMaxMergeLevels];
  int mslack;
  size_t mlds;
  int64_t ws_row_a;  // workspace row stride (entries) of the slice lists
  int64_t ws_row_b;  // and of the first list-merge level's output (after all rows of the former)
  size_t ws_bytes;
};

int device_cu_count() {
  static std::mutex mu;
  static std::unordered_map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> g(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return -1;
  cache[dev] = cus;
  return cus;
}

int check_basic(int64_t rows, int64_t n, int k, int dtype) {
  if (dtype != DS_BF16 && dtype != DS_FP32) return DS_ERR_INVALID_ARG;
  if (rows < 0 || n < 1 || n > INT32_MAX) return DS_ERR_INVALID_ARG;
  if (k < 1 || k > n) return DS_ERR_INVALID_ARG;
  if (k > DS_MAX_K) return DS_ERR_UNSUPPORTED;
  return DS_OK;
}

// Choose B, B2, slices and the kernel shape; cfg fields that are non-zero are forced.
// cus is the device's compute-unit count (only used when slices are automatic).
int make_plan(int64_t rows, int64_t n, int k, int dtype, const ds_config* cfg, int cus, Plan* out) {
  int st = check_basic(rows, n, k, dtype);
  if (st != DS_OK) return st;
  const ds_config c = cfg ? *cfg : ds_config{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  if (c.block < 0 || c.slack < 0 || c.slices < 0 || c.waves < 0) return DS_ERR_INVALID_ARG;
  if (c.presample != DS_PRESAMPLE_AUTO && c.presample != DS_PRESAMPLE_OFF && c.presample != DS_PRESAMPLE_ON)
    return DS_ERR_INVALID_ARG;
  if (c.order_group != 0 && c.order_group != 1 && c.order_group != 2 && c.order_group != 4)
    return DS_ERR_INVALID_ARG;
  if (c.merge != DS_MERGE_AUTO && c.merge != DS_MERGE_LISTS && c.merge != DS_MERGE_SELECT) return DS_ERR_INVALID_ARG;
  if (c.schedule != DS_SCHEDULE_AUTO && c.schedule != DS_SCHEDULE_FREE && c.schedule != DS_SCHEDULE_LOCKSTEP)
    return DS_ERR_INVALID_ARG;
  if (c.depth != 0) return DS_ERR_INVALID_ARG;  // reported by the plan, never forced
  if ((c.output & ~(DS_OUTPUT_UNSORTED | DS_OUTPUT_INDEX_INT64)) != 0) return DS_ERR_INVALID_ARG;
  if (c.warmup < 0) return DS_ERR_INVALID_ARG;
  if (c.share != DS_SHARE_AUTO && c.share != DS_SHARE_OFF && c.share != DS_SHARE_ON) return DS_ERR_INVALID_ARG;
  const int chunk = chunk_elems(dtype);
  const int eb = elem_bytes(dtype);

  // kernel shape: the forced block/waves, else the default per element type (16 waves and
  // B = 8192, measured best on MI355X for k = 512), stepping down to smaller blocks when the
  // candidate buffer would not fit in LDS
  const int sort_cap = pow2_at_least(k);
  int shape = -1, block = 0, slack = 0;
  size_t lds = 0;
  auto fit = [&](int s, bool strict = false) -> bool {
    const int b = kSelectShapes[s].waves * kSelectShapes[s].cpw * chunk;
    const double cap = 1.5 * std::sqrt(static_cast<double>(k) * (static_cast<double>(k) + b));
    bool tried = false;
    for (int want : kDefaultSlacks) {
      if (!c.slack && want > cap && want != kDefaultSlacks[sizeof(kDefaultSlacks) / sizeof(int) - 1]) continue;
      if (strict && tried) return false;  // only the bound-derived B2
      tried = true;
      int sl = c.slack ? c.slack : std::max(k, want);
      if (sl + b < sort_cap) {
        if (c.slack) return false;  // the final sort runs in the append region
        sl = sort_cap - b;
      }
      const size_t l = ds::select_lds_bytes(k, b, sl, kSelectShapes[s].waves);
      if (static_cast<int64_t>(l) > kMaxLdsBytes) {
        if (c.slack) return false;
        continue;
      }
      shape = s;
      block = b;
      slack = sl;
      lds = l;
      return true;
    }
    return false;
  };
  if (c.block || c.waves) {
    for (int s = 0; s < kNumSelectShapes && shape < 0; ++s) {
      const int b = kSelectShapes[s].waves * kSelectShapes[s].cpw * chunk;
      if (c.block && b != c.block) continue;
      if (c.waves && kSelectShapes[s].waves != c.waves) continue;
      if (!c.waves && kSelectShapes[s].waves != 4) continue;  // a forced block alone prefers 4 waves
      fit(s);
    }
    for (int s = 0; s < kNumSelectShapes && shape < 0; ++s) {
      const int b = kSelectShapes[s].waves * kSelectShapes[s].cpw * chunk;
      if (c.block && b != c.block) continue;
      if (c.waves && kSelectShapes[s].waves != c.waves) continue;
      fit(s);
    }
    if (shape < 0) return DS_ERR_UNSUPPORTED;
  } else {
    // the largest default block that is not longer than a slice (the whole row when the
    // slice count is automatic), else the smallest that fits
    const int* order = dtype == DS_BF16 ? kDefaultBf16 : kDefaultFp32;
    const int64_t cap = c.slices ? (n + c.slices - 1) / c.slices : n;
    for (int i = 0; i < kNumDefaults && shape < 0; ++i) {
      const int s = order[i];
      const int b = kSelectShapes[s].waves * kSelectShapes[s].cpw * chunk;
      if (b <= cap) fit(s, b > kMaxStepDownBlock);
    }
    for (int i = kNumDefaults - 1; i >= 0 && shape < 0; --i) fit(order[i]);
    if (shape < 0) return DS_ERR_UNSUPPORTED;
  }

  // slices: about one workgroup per compute unit, each slice at least 4 blocks and 16k (the
  // merge's work grows with slices * k: at k = 4096 on 2^20-element rows, 16 slices and two
  // list-merge levels took 157 us per call against 187 us for 32 slices and three levels)
  int64_t slices;
  if (c.slices) {
    slices = c.slices;
  } else {
    const int64_t r = rows > 0 ? rows : 1;
    const int64_t want = cus > 0 ? (static_cast<int64_t>(cus) + r - 1) / r : 1;
    const int64_t min_len = std::max<int64_t>(4 * static_cast<int64_t>(block), 16 * static_cast<int64_t>(k));
    const int64_t most = std::max<int64_t>(1, n / min_len);
    slices = std::max<int64_t>(1, std::min(want, most));
  }
  const int64_t min_slices = (n * eb + kMaxSliceBytes - 1) / kMaxSliceBytes;
  if (slices < min_slices) {
    if (c.slices) return DS_ERR_UNSUPPORTED;
    slices = min_slices;
  }
  int64_t per = (n + slices - 1) / slices;
  int64_t slice_len = (per + block - 1) / block * block;
  if (slice_len * eb > kMaxSliceBytes) slice_len = kMaxSliceBytes / eb / block * block;
  slices = (n + slice_len - 1) / slice_len;
  if (c.slices && slices != c.slices) return DS_ERR_UNSUPPORTED;  // forced count leaves an empty slice
  if (rows * slices > INT32_MAX) return DS_ERR_UNSUPPORTED;

  Plan p{};
  p.dtype = dtype;
  p.shape = shape;
  p.block = block;
  p.slack = slack;
  p.slices = static_cast<int>(slices);
  p.slice_len = slice_len;
  p.sort_cap = sort_cap;
  p.lds = lds;
  p.presample = c.presample != DS_PRESAMPLE_OFF && c.warmup == 0 && k <= 64 * kSelectShapes[shape].waves;
  p.warmup = c.warmup;
  // groups of two blocks pay off on long slices (consecutive loads in flight); short slices
  // keep single blocks, which randomise adversarial (sorted) slices better
  p.order_group = c.order_group ? c.order_group : ((slice_len + block - 1) / block >= 8 ? 2 : 1);
  // The free-running schedule wins while compactions are rare (the indexer: 25.2 against
  // 25.5 us per call); with a slack below half a block the buffer fills within a block and
  // free-running waves stop for compactions more often (the giant row, k = 32: 220 against
  // 197 us), so such plans keep the once-per-block check.
  p.lockstep = c.schedule == DS_SCHEDULE_LOCKSTEP || (c.schedule == DS_SCHEDULE_AUTO && 2 * slack < block);
  p.unsorted = (c.output & DS_OUTPUT_UNSORTED) != 0;
  p.idx64 = (c.output & DS_OUTPUT_INDEX_INT64) != 0;
  if (slices > 1) {
    const int64_t entries = slices * static_cast<int64_t>(k);
    if (entries * 8 > kMaxSliceBytes) return DS_ERR_UNSUPPORTED;
    p.ws_row_a = (entries + 1) & ~int64_t(1);
    // sharing pays where slices start without a presampled threshold (large k): their first
    // compactions come late, and a row threshold prunes them earlier (measured on MI355X:
    // long rows at k = 4096 in 32 slices, 10 % faster); with a presampled start the extra
    // zeroing launch costs more than it saves
    p.share = c.share == DS_SHARE_ON || (c.share == DS_SHARE_AUTO && !p.presample);
    p.share_bytes = p.share ? (static_cast<size_t>(rows) * 8 + 15) & ~size_t(15) : 0;
    p.ws_bytes = p.share_bytes + static_cast<size_t>(rows) * static_cast<size_t>(p.ws_row_a) * 8;
    p.merge = c.merge ? c.merge : DS_MERGE_LISTS;
    if (p.merge == DS_MERGE_LISTS) {
      // the fewest levels of at most gmax lists each, then the smallest group size per level
      // that still reaches one list in the levels left
      const int64_t gmax = std::min<int64_t>(ds::kMaxListGroup, ds::kListMergeLds / 8 / k);
      int levels = 0;
      for (int64_t reach = 1; reach < slices; reach *= gmax) ++levels;
      if (levels > kMaxMergeLevels) return DS_ERR_UNSUPPORTED;
      int64_t lists = slices;
      for (int l = 0; l < levels; ++l) {
        int64_t g = 2;
        for (;; ++g) {
          int64_t reach = 1;
          for (int e = l; e < levels; ++e) reach *= g;
          if (reach >= lists) break;
        }
        p.group[l] = static_cast<int>(g);
        lists = (lists + g - 1) / g;
        if (l == 0 && levels > 1) {
          p.ws_row_b = (lists * k + 1) & ~int64_t(1);
          p.ws_bytes += static_cast<size_t>(rows) * static_cast<size_t>(p.ws_row_b) * 8;
        }
      }
      p.levels = levels;
    } else {
      int ms = k > kMergeBlock ? k : kMergeBlock;
      if (ms + kMergeBlock < sort_cap) ms = sort_cap - kMergeBlock;
      p.mslack = ms;
      p.mlds = ds::select_lds_bytes(k, kMergeBlock, ms, ds::kMergeShape.waves);
      if (static_cast<int64_t>(p.mlds) > kMaxLdsBytes) return DS_ERR_UNSUPPORTED;
    }
  }
  *out = p;
  return DS_OK;
}

// make_plan behind a one-entry cache per thread: a caller that repeats the same call (the
// usual case in a serving or training loop) skips the planning.
struct PlanMemo {
  bool valid = false;
  int64_t rows = 0, n = 0;
  int k = 0, dtype = 0, cus = 0;
  bool has_cfg = false;
  ds_config cfg{};
  int status = DS_OK;
  Plan plan{};
};

int cached_plan(int64_t rows, int64_t n, int k, int dtype, const ds_config* cfg, int cus, Plan* out) {
  thread_local PlanMemo memo;
  const bool same = memo.valid && memo.rows == rows && memo.n == n && memo.k == k && memo.dtype == dtype &&
                    memo.cus == cus && memo.has_cfg == (cfg != nullptr) &&
                    (!cfg || std::memcmp(&memo.cfg, cfg, sizeof(ds_config)) == 0);
  if (!same) {
    memo.valid = true;
    memo.rows = rows;
    memo.n = n;
    memo.k = k;
    memo.dtype = dtype;
    memo.cus = cus;
    memo.has_cfg = cfg != nullptr;
    memo.cfg = cfg ? *cfg : ds_config{};
    memo.status = make_plan(rows, n, k, dtype, cfg, cus, &memo.plan);
  }
  if (memo.status == DS_OK) *out = memo.plan;
  return memo.status;
}

int check_call(const void* x, int64_t rows, int64_t n, int64_t row_stride, int k, int dtype, const void* out_vals,
               const void* out_idx) {
  int st = check_basic(rows, n, k, dtype);
  if (st != DS_OK) return st;
  if (row_stride < n) return DS_ERR_INVALID_ARG;
  if (rows == 0) return DS_OK;
  if (!x || (!out_vals && !out_idx)) return DS_ERR_INVALID_ARG;
  const int eb = elem_bytes(dtype);
  if (row_stride > (INT64_MAX / eb) / (rows > 0 ? rows : 1)) return DS_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(x) & 15) != 0 || ((row_stride * eb) & 15) != 0) return DS_ERR_ALIGNMENT;
  return DS_OK;
}

// The workspace is [shared row thresholds (sharing only)][slice lists][first list-merge level].
uint2* lists_of(const Plan& pl, void* ws) {
  return ws ? reinterpret_cast<uint2*>(static_cast<uint8_t*>(ws) + pl.share_bytes) : nullptr;
}

// The block order's mixed seed: the splitmix64 finaliser of the call's seed, computed once
// here (the kernels derive each workgroup's round keys from it).
uint64_t mix_seed(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int run_select(const Plan& pl, const void* x, const int32_t* lens, int64_t rows, int64_t n, int64_t row_stride, int k,
               uint64_t seed, void* out_vals, void* out_idx, void* ws, ds_stats* stats, hipStream_t stream) {
  (void)hipGetLastError();  // clear a stale error so a launch failure is reported as ours
  ds::SelectParams sp{};
  sp.x = static_cast<const uint8_t*>(x);
  sp.row_stride_bytes = row_stride * elem_bytes(pl.dtype);
  sp.n = n;
  sp.lens = lens;
  sp.slice_len = pl.slice_len;
  sp.slices = pl.slices;
  sp.k = k;
  sp.slack = pl.slack;
  sp.sort_cap = pl.sort_cap;
  sp.seed = mix_seed(seed);
  sp.ws = lists_of(pl, ws);
  sp.ws_row_entries = pl.ws_row_a;
  sp.out_vals = out_vals;
  sp.out_idx = ds::IdxOut{out_idx, pl.idx64 ? 1 : 0};
  sp.stats = stats;
  sp.sorted_lists = pl.merge == DS_MERGE_LISTS ? 1 : 0;
  sp.presample = pl.presample ? 1 : 0;
  sp.group_shift = pl.order_group == 4 ? 2 : (pl.order_group == 2 ? 1 : 0);
  sp.lockstep = pl.lockstep ? 1 : 0;
  sp.unsorted = pl.unsorted && pl.slices == 1 ? 1 : 0;
  sp.warmup = pl.warmup;
  if (pl.share) {  // the row words start at zero (below every element) in every call
    sp.share = static_cast<unsigned long long*>(ws);
    if (ds::launch_zero_words(sp.share, rows, stream) != hipSuccess) return DS_ERR_LAUNCH;
  }
  return ds::launch_select(pl.dtype, pl.shape, sp, rows, pl.lds, stream) == hipSuccess ? DS_OK : DS_ERR_LAUNCH;
}

int run_merge(const Plan& pl, const int32_t* lens, int64_t rows, int64_t n, int k, uint64_t seed, void* out_vals,
              void* out_idx, void* ws, hipStream_t stream) {
  if (pl.slices <= 1) return DS_OK;
  (void)hipGetLastError();
  ds::MergeParams mp{};
  mp.ws = lists_of(pl, ws);
  mp.entries = static_cast<int64_t>(pl.slices) * k;
  mp.row_entries = (mp.entries + 1) & ~int64_t(1);
  mp.n = n;
  mp.lens = lens;
  mp.slice_len = pl.slice_len;
  mp.k = k;
  mp.slack = pl.mslack;
  mp.sort_cap = pl.sort_cap;
  mp.seed = mix_seed(seed);
  mp.out_vals = out_vals;
  mp.out_idx = ds::IdxOut{out_idx, pl.idx64 ? 1 : 0};
  mp.unsorted = pl.unsorted ? 1 : 0;
  mp.presample = pl.presample && k <= 64 * ds::kMergeShape.waves ? 1 : 0;
  if (pl.merge == DS_MERGE_SELECT)
    return ds::launch_merge(pl.dtype, mp, rows, pl.mlds, stream) == hipSuccess ? DS_OK : DS_ERR_LAUNCH;
  // list merge: level l reads one workspace region and writes the other (or the outputs)
  uint2* const region[2] = {lists_of(pl, ws), lists_of(pl, ws) + rows * pl.ws_row_a};
  const int64_t row_of[2] = {pl.ws_row_a, pl.ws_row_b};
  int64_t lists = pl.slices;
  for (int l = 0; l < pl.levels; ++l) {
    const int g = pl.group[l];
    const bool last = l + 1 == pl.levels;
    mp.ws = region[l & 1];
    mp.row_entries = row_of[l & 1];
    mp.dst = last ? nullptr : region[(l + 1) & 1];
    mp.dst_row_entries = last ? 0 : row_of[(l + 1) & 1];
    mp.lists = static_cast<int32_t>(lists);
    mp.group = g;
    mp.per_wg = std::max(1, std::min(g, ds::kListMergeWaves * 64 / k));
    if (ds::launch_merge_lists(pl.dtype, mp, rows, stream) != hipSuccess) return DS_ERR_LAUNCH;
    lists = (lists + g - 1) / g;
  }
  return DS_OK;
}

int run(const Plan& pl, const void* x, const int32_t* lens, int64_t rows, int64_t n, int64_t row_stride, int k,
        uint64_t seed, void* out_vals, void* out_idx, void* ws, ds_stats* stats, hipStream_t stream) {
  int st = run_select(pl, x, lens, rows, n, row_stride, k, seed, out_vals, out_idx, ws, stats, stream);
  if (st != DS_OK) return st;
  return run_merge(pl, lens, rows, n, k, seed, out_vals, out_idx, ws, stream);
}

// Plan a call that brings its own workspace; validates the workspace against the plan.
int plan_with_workspace(int64_t rows, int64_t n, int k, int dtype, const ds_config* cfg, void* workspace,
                        size_t ws_bytes, Plan* p) {
  int cus = 0;
  if (!(cfg && cfg->slices)) {
    cus = device_cu_count();
    if (cus <= 0) return DS_ERR_DEVICE;
  }
  int st = cached_plan(rows, n, k, dtype, cfg, cus, p);
  if (st != DS_OK) return st;
  if (p->ws_bytes) {
    if (!workspace || ws_bytes < p->ws_bytes) return DS_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0) return DS_ERR_ALIGNMENT;
  }
  return DS_OK;
}

// Workspace cache of ds_topk, one buffer per (device, stream): calls on one stream are
// ordered by the stream, so they can share a buffer; calls on different streams never do.
// A buffer that was handed out is never freed before unload (a graph captured on its
// stream may still use it): when a stream needs more, the old buffer is retired and kept.
// Growing calls hipMalloc, which is refused while the stream is being captured.
struct WsBuf {
  void* ptr = nullptr;
  size_t bytes = 0;
};
struct WsCache {
  std::mutex mu;
  std::map<std::pair<int, uintptr_t>, WsBuf> bufs;
  std::vector<std::pair<int, void*>> retired;
  ~WsCache() {
    int old = 0;
    if (hipGetDevice(&old) != hipSuccess) return;
    auto release = [](int dev, void* p) {
      if (p && hipSetDevice(dev) == hipSuccess) (void)hipFree(p);
    };
    for (auto& kv : bufs) release(kv.first.first, kv.second.ptr);
    for (auto& r : retired) release(r.first, r.second);
    (void)hipSetDevice(old);
  }
};
WsCache& ws_cache() {
  static WsCache* c = new WsCache();  // never destroyed: the runtime may be gone at exit
  return *c;
}

// The cached workspace of at least `bytes` for (current device, stream), or an error.
int cached_workspace(size_t bytes, hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DS_ERR_DEVICE;
  WsCache& c = ws_cache();
  std::lock_guard<std::mutex> g(c.mu);
  WsBuf& slot = c.bufs[{dev, reinterpret_cast<uintptr_t>(stream)}];
  if (slot.bytes < bytes) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return DS_ERR_DEVICE;
    if (cs != hipStreamCaptureStatusNone) return DS_ERR_WORKSPACE;  // no allocation under capture
    void* ptr = nullptr;
    if (hipMalloc(&ptr, bytes) != hipSuccess) return DS_ERR_LAUNCH;
    if (slot.ptr) c.retired.emplace_back(dev, slot.ptr);
    slot.ptr = ptr;
    slot.bytes = bytes;
  }
  *out = slot.ptr;
  return DS_OK;
}

}  // namespace

namespace ds {

int topk_auto(const void* x, int64_t rows, int64_t n, int64_t row_stride, int k, int dtype, uint64_t seed,
              void* out_vals, int32_t* out_idx, void* stream, WorkspaceSource get_ws) {
  int st = check_call(x, rows, n, row_stride, k, dtype, out_vals, out_idx);
  if (st != DS_OK || rows == 0) return st;
  const int cus = device_cu_count();
  if (cus <= 0) return DS_ERR_DEVICE;
  Plan p;
  st = cached_plan(rows, n, k, dtype, nullptr, cus, &p);
  if (st != DS_OK) return st;
  void* ws = nullptr;
  if (p.ws_bytes) {
    st = get_ws(p.ws_bytes, stream, &ws);
    if (st != DS_OK) return st;
  }
  return run(p, x, nullptr, rows, n, row_stride, k, seed, out_vals, out_idx, ws, nullptr,
             static_cast<hipStream_t>(stream));
}

}  // namespace ds

extern "C" {

const char* ds_status_string(int status) {
  switch (status) {
    case DS_OK: return "DS_OK";
    case DS_ERR_INVALID_ARG: return "DS_ERR_INVALID_ARG";
    case DS_ERR_UNSUPPORTED: return "DS_ERR_UNSUPPORTED";
    case DS_ERR_ALIGNMENT: return "DS_ERR_ALIGNMENT";
    case DS_ERR_WORKSPACE: return "DS_ERR_WORKSPACE";
    case DS_ERR_LAUNCH: return "DS_ERR_LAUNCH";
    case DS_ERR_DEVICE: return "DS_ERR_DEVICE";
    default: return "DS_ERR_UNKNOWN";
  }
}

int ds_topk_plan(int64_t rows, int64_t n, int k, int dtype, const ds_config* cfg, ds_config* out) {
  if (!out) return DS_ERR_INVALID_ARG;
  int st = check_basic(rows, n, k, dtype);
  if (st != DS_OK) return st;
  int cus = 0;
  if (!(cfg && cfg->slices)) {
    cus = device_cu_count();
    if (cus <= 0) return DS_ERR_DEVICE;
  }
  Plan p;
  st = cached_plan(rows, n, k, dtype, cfg, cus, &p);
  if (st != DS_OK) return st;
  out->block = p.block;
  out->slack = p.slack;
  out->slices = p.slices;
  out->waves = kSelectShapes[p.shape].waves;
  out->presample = p.presample ? DS_PRESAMPLE_ON : DS_PRESAMPLE_OFF;
  out->order_group = p.order_group;
  out->merge = p.slices > 1 ? p.merge : DS_MERGE_AUTO;
  out->schedule = p.lockstep ? DS_SCHEDULE_LOCKSTEP : DS_SCHEDULE_FREE;
  out->depth = ds::depth_for(kSelectShapes[p.shape].waves, kSelectShapes[p.shape].cpw);
  out->output = (p.unsorted ? DS_OUTPUT_UNSORTED : 0) | (p.idx64 ? DS_OUTPUT_INDEX_INT64 : 0);
  out->warmup = p.warmup;
  out->share = p.share ? DS_SHARE_ON : (p.slices > 1 ? DS_SHARE_OFF : DS_SHARE_AUTO);
  return DS_OK;
}

int ds_topk_workspace_size(int64_t rows, int64_t n, int k, int dtype, const ds_config* cfg, size_t* bytes) {
  if (!bytes) return DS_ERR_INVALID_ARG;
  int st = check_basic(rows, n, k, dtype);
  if (st != DS_OK) return st;
  int cus = 0;
  if (!(cfg && cfg->slices)) {
    cus = device_cu_count();
    if (cus <= 0) return DS_ERR_DEVICE;
  }
  Plan p;
  st = cached_plan(rows, n, k, dtype, cfg, cus, &p);
  if (st != DS_OK) return st;
  *bytes = p.ws_bytes;
  return DS_OK;
}

int ds_topk_ex(const void* x, const int32_t* lens, int64_t rows, int64_t n, int64_t row_stride, int k, int dtype,
               uint64_t seed, void* out_vals, void* out_idx, void* workspace, size_t ws_bytes, const ds_config* cfg,
               ds_stats* stats, void* stream) {
  int st = check_call(x, rows, n, row_stride, k, dtype, out_vals, out_idx);
  if (st != DS_OK || rows == 0) return st;
  Plan p;
  st = plan_with_workspace(rows, n, k, dtype, cfg, workspace, ws_bytes, &p);
  if (st != DS_OK) return st;
  return run(p, x, lens, rows, n, row_stride, k, seed, out_vals, out_idx, workspace, stats,
             static_cast<hipStream_t>(stream));
}

int ds_topk_slices(const void* x, const int32_t* lens, int64_t rows, int64_t n, int64_t row_stride, int k,
                   int dtype, uint64_t seed, void* out_vals, void* out_idx, void* workspace, size_t ws_bytes,
                   const ds_config* cfg, ds_stats* stats, void* stream) {
  int st = check_call(x, rows, n, row_stride, k, dtype, out_vals, out_idx);
  if (st != DS_OK || rows == 0) return st;
  Plan p;
  st = plan_with_workspace(rows, n, k, dtype, cfg, workspace, ws_bytes, &p);
  if (st != DS_OK) return st;
  return run_select(p, x, lens, rows, n, row_stride, k, seed, out_vals, out_idx, workspace, stats,
                    static_cast<hipStream_t>(stream));
}

int ds_topk_merge(const int32_t* lens, int64_t rows, int64_t n, int k, int dtype, uint64_t seed, void* out_vals,
                  void* out_idx, void* workspace, size_t ws_bytes, const ds_config* cfg, void* stream) {
  int st = check_basic(rows, n, k, dtype);
  if (st != DS_OK || rows == 0) return st;
  if (!out_vals && !out_idx) return DS_ERR_INVALID_ARG;
  Plan p;
  st = plan_with_workspace(rows, n, k, dtype, cfg, workspace, ws_bytes, &p);
  if (st != DS_OK) return st;
  return run_merge(p, lens, rows, n, k, seed, out_vals, out_idx, workspace, static_cast<hipStream_t>(stream));
}

int ds_topk(const void* x, int64_t rows, int64_t n, int64_t row_stride, int k, int dtype, uint64_t seed,
            void* out_vals, int32_t* out_idx, void* stream) {
  return ds::topk_auto(x, rows, n, row_stride, k, dtype, seed, out_vals, out_idx, stream,
                       [](size_t bytes, void* s, void** out) {
                         return cached_workspace(bytes, static_cast<hipStream_t>(s), out);
                       });
}

int64_t ds_probe_sink_words(int64_t bytes) { return bytes <= 0 ? 0 : ds::probe_read_groups(bytes); }

int ds_probe_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes <= 0 || (bytes & 15) != 0) return DS_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(src) & 15) != 0) return DS_ERR_ALIGNMENT;
  (void)hipGetLastError();
  return ds::launch_probe_read(src, bytes, sink, static_cast<hipStream_t>(stream)) == hipSuccess ? DS_OK
                                                                                                  : DS_ERR_LAUNCH;
}

int ds_probe_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  if (!src || !dst || bytes <= 0 || (bytes & 15) != 0) return DS_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(dst) & 15) != 0)
    return DS_ERR_ALIGNMENT;
  (void)hipGetLastError();
  return ds::launch_probe_copy(dst, src, bytes, static_cast<hipStream_t>(stream)) == hipSuccess ? DS_OK
                                                                                                  : DS_ERR_LAUNCH;
}

}  // extern "C"
