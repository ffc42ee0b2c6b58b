// Internal interface between the C-ABI layer (ds_api.cpp) and the HIP kernels (ds_device.h,
// ds_select.hip, ds_merge.hip, ds_noalloc.hip). Not installed; the public interface is
// include/dstopk.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dstopk.h"

namespace ds {

// An index output, [rows][k] int32, or int64 when `wide` (NULL: no index output).
struct IdxOut {
  void* p;
  int32_t wide;
};

// One workgroup runs DeepSelect over one slice [slice*slice_len, min(n, (slice+1)*slice_len))
// of one row. Candidates live in LDS as (key, index) pairs.
struct SelectParams {
  const uint8_t* x;          // row 0, slice 0
  int64_t row_stride_bytes;  // bytes between rows
  int64_t n;                 // elements per row (the longest row when lens is set)
  const int32_t* lens;       // NULL, or row r holds min(max(lens[r], 0), n) elements
  int64_t slice_len;         // elements per slice, a multiple of the block size
  int32_t slices;            // workgroups per row
  int32_t k;
  int32_t slack;             // B2
  int32_t sort_cap;          // power of two >= k (final sort width)
  uint64_t seed;
  uint2* ws;                 // slices > 1: survivors, row r at ws + r*ws_row_entries, slice s at +s*k
  int64_t ws_row_entries;    // slices*k rounded up to even (16-byte rows)
  void* out_vals;            // slices == 1: output values [rows][k]
  IdxOut out_idx;            // slices == 1: output indices [rows][k]
  ds_stats* stats;           // NULL or [rows][slices]
  int32_t sorted_lists;      // slices > 1: store each slice's survivors sorted (for the list merge)
  int32_t presample;         // nonzero: the first whole block sets a presampled threshold
  int32_t group_shift;       // log2 of G: the block order is random over groups of G blocks
  int32_t lockstep;          // nonzero: a barrier and the buffer check after every block
  int32_t unsorted;          // slices == 1: the k survivors may be written in any order
  int32_t warmup;            // blocks of the warm-up window (0: none)
  unsigned long long* share; // NULL, or one shared threshold word per row (zero on entry)
};

// The merge of split rows. The merge kernel: one workgroup per row runs DeepSelect over the
// row's slices*k survivors (ws, entries, row_entries, slack, seed, presample). One level of
// the list merge: the row's `lists` sorted lists of k entries at ws are merged in groups of
// `group` consecutive lists; group g's k best go to dst (row r at dst + r*dst_row_entries,
// group g at +g*k) as sorted pairs, or to the outputs when dst is NULL (the level has one
// group). Each list-merge workgroup places per_wg lists of one group.
struct MergeParams {
  const uint2* ws;     // row r's entries at ws + r*row_entries
  int64_t entries;     // slices * k
  int64_t row_entries; // entries rounded up to even (16-byte rows)
  int64_t n;           // row length (indices lie in [0, n))
  const int32_t* lens; // NULL, or ragged rows as in SelectParams
  int64_t slice_len;   // elements per slice
  int32_t k;
  int32_t slack;
  int32_t sort_cap;
  uint64_t seed;
  void* out_vals;
  IdxOut out_idx;
  int32_t presample;   // nonzero: the first whole block sets a presampled threshold
  int32_t unsorted;    // merge kernel: the k survivors may be written in any order
  uint2* dst;
  int64_t dst_row_entries;
  int32_t lists;
  int32_t group;
  int32_t per_wg;
  int32_t pk;    // ceil(k / group), set by the launcher
  int64_t row0;  // first row of a launch, set by the launcher
};

// A compiled kernel shape: waves per workgroup and 16-byte chunks per wave per block.
struct Shape {
  int waves;
  int cpw;
};

// Select-kernel shapes built for each element type. The block size is
// waves * cpw * 64 lanes * (16 / elem_bytes) elements.
constexpr Shape kSelectShapes[] = {{2, 1}, {4, 1}, {4, 2}, {8, 1}, {8, 2}, {4, 4}, {8, 4}, {16, 1}, {16, 2}, {16, 4}};
constexpr int kNumSelectShapes = sizeof(kSelectShapes) / sizeof(kSelectShapes[0]);
constexpr Shape kMergeShape = {16, 2};  // 16 waves x 2 chunks x 128 entries = 4096 entries per block

// Blocks in flight per wave in a select workgroup of `waves` waves with `cpw` 16-byte chunks
// per wave per block: four (at most 16 VGPRs of loads), or two for four chunks. The presampled
// start covers the whole blocks among the first depth_for blocks of the order.
constexpr int depth_for(int waves, int cpw) { return (void)waves, cpw >= 4 ? 2 : 4; }

// LDS bytes a select/merge workgroup needs, and the part of them that is not the dynamic
// array (the per-workgroup scalars).
size_t select_lds_bytes(int k, int block, int slack, int waves);
size_t select_scalars_bytes();

// The list merge merges at most this many sorted lists together (one level), whose entries
// take at most kListMergeLds bytes of LDS, with kListMergeWaves waves per workgroup.
constexpr uint32_t kMaxListGroup = 16;
constexpr int64_t kListMergeLds = 128 * 1024;
constexpr int kListMergeWaves = 8;

// ds_topk's body (argument checks, the automatic plan, the launches) with the split rows'
// workspace taken from `get_ws(bytes, stream, &ptr)` (a status code; called only when the
// plan needs a workspace, before anything is enqueued).
using WorkspaceSource = int (*)(size_t bytes, void* stream, void** out);
int topk_auto(const void* x, int64_t rows, int64_t n, int64_t row_stride, int k, int dtype, uint64_t seed,
              void* out_vals, int32_t* out_idx, void* stream, WorkspaceSource get_ws);

// The select-kernel launcher of one element type and counter mode (one object each).
#define DS_SELECT_PART_NAME(dt, st, ex) launch_select_part_##dt##_##st##_##ex
#define DS_DECLARE_SELECT_PART(dt, st, ex) \
  hipError_t DS_SELECT_PART_NAME(dt, st, ex)(int shape, const SelectParams& p, int64_t rows, size_t lds, hipStream_t stream)
DS_DECLARE_SELECT_PART(0, 0, 0);
DS_DECLARE_SELECT_PART(0, 0, 1);
DS_DECLARE_SELECT_PART(0, 1, 0);
DS_DECLARE_SELECT_PART(0, 1, 1);
DS_DECLARE_SELECT_PART(1, 0, 0);
DS_DECLARE_SELECT_PART(1, 0, 1);
DS_DECLARE_SELECT_PART(1, 1, 0);
DS_DECLARE_SELECT_PART(1, 1, 1);

// Launchers; return hipSuccess or the launch error.
hipError_t launch_select(int dtype, int shape_index, const SelectParams& p, int64_t rows, size_t lds_bytes,
                         hipStream_t stream);
hipError_t launch_merge(int dtype, const MergeParams& p, int64_t rows, size_t lds_bytes, hipStream_t stream);
// One level of the list merge (p.lists, p.group, p.per_wg, p.dst).
hipError_t launch_merge_lists(int dtype, const MergeParams& p, int64_t rows, hipStream_t stream);
hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);
int64_t probe_read_groups(int64_t bytes);
hipError_t launch_probe_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);
hipError_t launch_zero_words(unsigned long long* p, int64_t n, hipStream_t stream);

}  // namespace ds
