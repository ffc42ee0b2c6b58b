// Merge-kernel and list-merge instantiations, the probes, and the launch entry points the
// C-ABI layer calls (the select kernels live in the ds_select.hip objects).
#include "ds_device.h"

namespace ds {
namespace {

// --------------------------------------------------------------------------- probes
constexpr uint32_t kProbeThreads = 256;
constexpr uint32_t kProbeUnroll = 4;
constexpr uint32_t kProbeTile = kProbeThreads * 16 * kProbeUnroll;  // bytes per workgroup step

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* src, int64_t vecs, uint32_t* sink) {
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads * kProbeUnroll;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads * kProbeUnroll + threadIdx.x; i < vecs;
       i += stride) {
    u32x4 r[kProbeUnroll];
#pragma unroll
    for (uint32_t u = 0; u < kProbeUnroll; ++u) {
      const int64_t j = i + u * kProbeThreads;
      r[u] = j < vecs ? src[j] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (uint32_t u = 0; u < kProbeUnroll; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
  for (uint32_t o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  __shared__ uint32_t part[kProbeThreads / 64];
  if ((threadIdx.x & 63u) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (uint32_t w = 0; w < kProbeThreads / 64; ++w) a ^= part[w];
    sink[blockIdx.x] = a;
  }
}

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(u32x4* dst, const u32x4* src, int64_t vecs) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads * kProbeUnroll;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads * kProbeUnroll + threadIdx.x; i < vecs;
       i += stride) {
    u32x4 r[kProbeUnroll];
#pragma unroll
    for (uint32_t u = 0; u < kProbeUnroll; ++u) {
      const int64_t j = i + u * kProbeThreads;
      if (j < vecs) r[u] = src[j];
    }
#pragma unroll
    for (uint32_t u = 0; u < kProbeUnroll; ++u) {
      const int64_t j = i + u * kProbeThreads;
      if (j < vecs) dst[j] = r[u];
    }
  }
}

// Rows per list-merge launch (the grid's z dimension; a multiple of 8, see xcd_unit).
constexpr int64_t kMaxGridRows = 65528;

// One instantiation per bound on the lists merged together, and per number of entries a
// thread searches at once.
template <int DT, uint32_t MAXS, uint32_t EB, int W = kListMergeWaves>
hipError_t launch_merge_lists_t(const MergeParams& p, int64_t rows, size_t lds, hipStream_t stream) {
  auto kern = merge_lists_kernel<DT, W, MAXS, EB>;
  {
    const hipError_t e = allow_lds<merge_lists_kernel<DT, W, MAXS, EB>>(lds);
    if (e != hipSuccess) return e;
  }
  const int64_t G = p.group, wpg = (G + p.per_wg - 1) / p.per_wg, groups = (p.lists + G - 1) / G;
  MergeParams q = p;
  q.pk = (p.k + p.group - 1) / p.group;
  for (int64_t r0 = 0; r0 < rows; r0 += kMaxGridRows) {
    q.row0 = r0;
    const int64_t nr = rows - r0 < kMaxGridRows ? rows - r0 : kMaxGridRows;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(wpg), static_cast<uint32_t>(groups), static_cast<uint32_t>(nr)),
                       dim3(W * 64), lds, stream, q.ws, q.row_entries, q.row0, q.lists, q.group, q.per_wg,
                       q.k, q.pk, static_cast<int32_t>(wpg), static_cast<int32_t>(groups), static_cast<int32_t>(nr), q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int DT>
hipError_t launch_merge_lists_dt(const MergeParams& p, int64_t rows, size_t lds, hipStream_t stream) {
  const int32_t g = p.group < p.lists ? p.group : p.lists;
  // long lists: every thread searches several entries at once (small groups keep the
  // registers of the interleaved searches in bounds), on 16 waves (a workgroup places one
  // list either way; k = 4096: two levels 137 -> 134 us, where 16 waves for short lists
  // were slower)
  const bool longl = p.k >= 1024;
  if (g <= 2) return longl ? launch_merge_lists_t<DT, 2, 4, 16>(p, rows, lds, stream)
                           : launch_merge_lists_t<DT, 2, 1>(p, rows, lds, stream);
  if (g <= 4) return longl ? launch_merge_lists_t<DT, 4, 4, 16>(p, rows, lds, stream)
                           : launch_merge_lists_t<DT, 4, 1>(p, rows, lds, stream);
  if (g <= 8) return longl ? launch_merge_lists_t<DT, 8, 2, 16>(p, rows, lds, stream)
                           : launch_merge_lists_t<DT, 8, 1>(p, rows, lds, stream);
  static_assert(kMaxListGroup == 16, "instantiations cover groups up to kMaxListGroup");
  return launch_merge_lists_t<DT, kMaxListGroup, 1>(p, rows, lds, stream);
}

template <int DT>
hipError_t launch_merge_dt(const MergeParams& p, int64_t rows, size_t lds, hipStream_t stream) {
  constexpr int W = kMergeShape.waves, C = kMergeShape.cpw;
  auto kern = merge_kernel<DT, W, C>;
  {
    const hipError_t e = allow_lds<merge_kernel<DT, W, C>>(lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(rows)), dim3(W * 64), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t select_scalars_bytes() { return sizeof(Scalars); }

size_t select_lds_bytes(int k, int block, int slack, int waves) {
  (void)waves;
  const size_t k4 = round4(static_cast<uint32_t>(k)), pc = round4(static_cast<uint32_t>(slack + block));
  return (2 * (k4 + pc + kDummySlots) + 2 * k4 + 2 * kBins + kOrdCap) * 4 + sizeof(Scalars);
}

// The counters and the extended features (ragged rows, the warm-up window, the shared row
// threshold) are separate instantiations (objects of their own), so the kernel of a plain
// call carries none of their code.
hipError_t launch_select(int dtype, int shape_index, const SelectParams& p, int64_t rows, size_t lds_bytes,
                         hipStream_t stream) {
  const size_t dyn = lds_bytes - sizeof(Scalars);
  const bool ext = p.lens || p.warmup || p.share;
  const int part = (dtype == DS_BF16 ? 0 : 4) + (p.stats ? 2 : 0) + (ext ? 1 : 0);
  switch (part) {
    case 0: return DS_SELECT_PART_NAME(0, 0, 0)(shape_index, p, rows, dyn, stream);
    case 1: return DS_SELECT_PART_NAME(0, 0, 1)(shape_index, p, rows, dyn, stream);
    case 2: return DS_SELECT_PART_NAME(0, 1, 0)(shape_index, p, rows, dyn, stream);
    case 3: return DS_SELECT_PART_NAME(0, 1, 1)(shape_index, p, rows, dyn, stream);
    case 4: return DS_SELECT_PART_NAME(1, 0, 0)(shape_index, p, rows, dyn, stream);
    case 5: return DS_SELECT_PART_NAME(1, 0, 1)(shape_index, p, rows, dyn, stream);
    case 6: return DS_SELECT_PART_NAME(1, 1, 0)(shape_index, p, rows, dyn, stream);
    default: return DS_SELECT_PART_NAME(1, 1, 1)(shape_index, p, rows, dyn, stream);
  }
}

hipError_t launch_merge_lists(int dtype, const MergeParams& p, int64_t rows, hipStream_t stream) {
  const size_t lds =
      static_cast<size_t>(p.group < p.lists ? p.group : p.lists) * static_cast<size_t>(p.k) * 8 + kMaxListGroup * 4;
  return dtype == DS_BF16 ? launch_merge_lists_dt<DS_BF16>(p, rows, lds, stream)
                          : launch_merge_lists_dt<DS_FP32>(p, rows, lds, stream);
}

hipError_t launch_merge(int dtype, const MergeParams& p, int64_t rows, size_t lds_bytes, hipStream_t stream) {
  const size_t dyn = lds_bytes - sizeof(Scalars);
  return dtype == DS_BF16 ? launch_merge_dt<DS_BF16>(p, rows, dyn, stream)
                          : launch_merge_dt<DS_FP32>(p, rows, dyn, stream);
}

int64_t probe_read_groups(int64_t bytes) {
  int64_t g = (bytes + kProbeTile - 1) / kProbeTile;
  return g < 1 ? 1 : (g > 4096 ? 4096 : g);
}

hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t g = probe_read_groups(bytes);
  hipLaunchKernelGGL(probe_read_kernel, dim3(static_cast<uint32_t>(g)), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

// Zeroes n 64-bit words (the shared row thresholds before a call's select launch): a kernel,
// not a memset, so that a captured graph replays it like any other launch.
__global__ __launch_bounds__(256) void zero_words_kernel(unsigned long long* p, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0ull;
}

hipError_t launch_zero_words(unsigned long long* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t g = (n + 255) / 256;
  hipLaunchKernelGGL(zero_words_kernel, dim3(static_cast<uint32_t>(g > 1024 ? 1024 : g)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  const int64_t g = probe_read_groups(bytes);
  hipLaunchKernelGGL(probe_copy_kernel, dim3(static_cast<uint32_t>(g)), dim3(kProbeThreads), 0, stream,
                     static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), bytes / 16);
  return hipGetLastError();
}

}  // namespace ds
