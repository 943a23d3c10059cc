// ar_internal.h -- interface between the host runtime (ar_api.cpp) and the
// gfx950 kernels (ar_kernels.hip).  Not installed; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "ar.h"

namespace mpp {

// One wave handles a "wave tile" of 512 consecutive elements per step: 64
// lanes x 8 elements.  Every vector path works in whole wave tiles; the
// remainder of a range (< 512 elements) is done element by element.
constexpr unsigned kWaveTile = 512;

// Kernel arguments, passed by value (kernarg segment, ~470 B).  The launch
// covers R sources and n_dst destinations over gridDim.y ranges, each walked
// by gridDim.x workgroups:
//   chunk_elems > 0: range y is the plan chunk [y * chunk_elems,
//                    min((y + 1) * chunk_elems, n));
//   chunk_elems == 0: range y is the slice [slice_start[y], slice_start[y] +
//                    slice_len[y]) (per-rank slices; gridDim.y <= AR_MAX_RANKS).
struct KernelArgs {
    const void *src[AR_MAX_RANKS];
    float      *dst[AR_MAX_RANKS];
    uint64_t    slice_start[AR_MAX_RANKS];
    unsigned    slice_len[AR_MAX_RANKS];
    unsigned    n;
    unsigned    chunk_elems;
    int         R;
    int         n_dst;
};

// Largest element count one launch covers (32-bit element indices inside the
// kernels; byte offsets are formed in 64 bits).
constexpr size_t kMaxLaunchElems = size_t(1) << 30;

enum class Family : int {
    SingleShot = 0,   // one wave tile per wave, no loop: decode-sized vectors
    StreamReg  = 1,   // persistent waves, register-staged batches of tiles
    StreamLds  = 2,   // persistent waves, double-buffered LDS staging
};

struct LaunchShape {
    unsigned grid_x;      // workgroups per slice
    unsigned grid_y;      // slices
    unsigned block;       // threads per workgroup
    unsigned lds_bytes;   // dynamic LDS per workgroup
};

// Launch one kernel of `family` for the given element types on `stream`.
// `wire` is an ar_dtype; `src_is_wire` selects 16-bit sources.  The caller
// has validated every argument and sized the shape with plan_shape().
hipError_t launch(Family family, int wire, bool src_is_wire, const KernelArgs &args,
                  const LaunchShape &shape, hipStream_t stream);

// Pick a launch shape for `family` covering `max_slice_len` elements per
// slice.  `cu_count` is the device's compute-unit count; `grid_override`
// (> 0) fixes the workgroups per slice.
LaunchShape plan_shape(Family family, int wire, bool src_is_wire, int R, unsigned max_slice_len,
                       unsigned n_slices, int cu_count, int grid_override);

// Elements processed per wave per loop iteration (a multiple of kWaveTile).
unsigned stream_tile_elems(Family family, bool src_is_wire, int R);

}  // namespace mpp
