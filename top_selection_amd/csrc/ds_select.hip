// Select-kernel instantiations of one element type, counter mode and feature set, chosen by
// DS_PART_DT (DS_BF16 / DS_FP32), DS_PART_STATS (0 / 1) and DS_PART_EXT (0 / 1: ragged rows,
// warm-up window, shared row threshold) at compile time: the build compiles this file once
// per combination, in parallel, and links the objects into one library.
#include "ds_device.h"

#ifndef DS_PART_DT
#error "DS_PART_DT must be defined"
#endif
#ifndef DS_PART_STATS
#error "DS_PART_STATS must be defined"
#endif
#ifndef DS_PART_EXT
#error "DS_PART_EXT must be defined"
#endif

namespace ds {
namespace {

template <int DT, int W, int C, bool STATS, bool EXT>
hipError_t launch_select_shape(const SelectParams& p, int64_t rows, size_t lds, hipStream_t stream) {
  const hipError_t e = allow_lds<select_kernel<DT, W, C, STATS, EXT>>(lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((select_kernel<DT, W, C, STATS, EXT>), dim3(static_cast<uint32_t>(rows * p.slices)), dim3(W * 64),
                     lds, stream, p.x, p.row_stride_bytes, p.n, p.slice_len, p.seed, p.slices, p.group_shift,
                     static_cast<int32_t>(rows), p.lens, p);
  return hipGetLastError();
}

template <int DT, bool STATS, bool EXT>
hipError_t launch_select_st(int shape, const SelectParams& p, int64_t rows, size_t lds, hipStream_t s) {
  switch (shape) {
    case 0: return launch_select_shape<DT, 2, 1, STATS, EXT>(p, rows, lds, s);
    case 1: return launch_select_shape<DT, 4, 1, STATS, EXT>(p, rows, lds, s);
    case 2: return launch_select_shape<DT, 4, 2, STATS, EXT>(p, rows, lds, s);
    case 3: return launch_select_shape<DT, 8, 1, STATS, EXT>(p, rows, lds, s);
    case 4: return launch_select_shape<DT, 8, 2, STATS, EXT>(p, rows, lds, s);
    case 5: return launch_select_shape<DT, 4, 4, STATS, EXT>(p, rows, lds, s);
    case 6: return launch_select_shape<DT, 8, 4, STATS, EXT>(p, rows, lds, s);
    case 7: return launch_select_shape<DT, 16, 1, STATS, EXT>(p, rows, lds, s);
    case 8: return launch_select_shape<DT, 16, 2, STATS, EXT>(p, rows, lds, s);
    case 9: return launch_select_shape<DT, 16, 4, STATS, EXT>(p, rows, lds, s);
    default: return hipErrorInvalidValue;
  }
}


}  // namespace

#define DS_PART_NAME(dt, st, ex) DS_SELECT_PART_NAME(dt, st, ex)  // expands the part macros first
hipError_t DS_PART_NAME(DS_PART_DT, DS_PART_STATS, DS_PART_EXT)(int shape, const SelectParams& p, int64_t rows,
                                                                size_t lds, hipStream_t stream) {
  return launch_select_st<DS_PART_DT, DS_PART_STATS != 0, DS_PART_EXT != 0>(shape, p, rows, lds, stream);
}

}  // namespace ds
