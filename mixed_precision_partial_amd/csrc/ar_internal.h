// ar_internal.h -- interface between the host runtime (ar_api.cpp) and the
// gfx950 kernels (ar_device.h, ar_k_*.hip, ar_launch.hip).  Not installed; not
// part of the C ABI.
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

// Kernel arguments for a kernel whose rank bucket is NR, passed by value: the
// kernarg segment of a launch holds exactly this struct, so the small buckets
// launch with small argument blocks (the runtime's per-launch host cost grows
// with the argument size on MI355X: about 0.8 us more for ~500 B than for a
// few bytes, a quarter of a decode-sized call).  The launch covers R sources
// and n_dst destinations over gridDim.y ranges, each walked by the `waves`
// waves of gridDim.x workgroups:
//   strided ranges (every schedule but the broadcast one): range y has
//       min(cols, n - y * cols) elements and starts at element
//       y * src_stride / y * dst_stride / y * res_stride of the sources /
//       destinations / element-wise residual -- consecutive 1-D chunks
//       (strides = cols) or the rows of row-strided tensors;
//   slice ranges (RS_BCAST, a separate kernel instance): range y is
//       [slice_start[y], slice_start[y] + slice_len[y]) of every tensor,
//       gridDim.y <= R.
// The scalars a wave needs first sit at the front so that one batch of
// scalar loads fetches them together with the pointers.
template <int NR>
struct LaunchArgs {
    uint64_t    n;          // elements of the launch (strided ranges)
    unsigned    cols;       // elements per strided range
    unsigned    waves;      // waves per range: gridDim.x * (block / 64)
    int         R;
    int         n_dst;
    unsigned    active;     // bit r: rank r has a partial; an inactive rank is +0.0
    unsigned    res_len;    // residual: 0 = element-wise (range offset + element),
                            // else a 1-D broadcast row of res_len elements (a
                            // multiple of 8) indexed by call position
    unsigned    res_phase;  // 1-D row: column of launch element 0 in the row
    unsigned    res_reuse;  // 1: residual elements are re-read (a broadcast row)
    uint64_t    src_stride; // strided ranges: elements between range starts
    uint64_t    dst_stride;
    uint64_t    res_stride; // 0 with res_len 0: one row added to every range
    const void *res;        // residual in the destination type, or nullptr
    const void *src[NR];
    void       *dst[NR];    // binary32, or 16-bit for a narrow destination
    uint64_t    slice_start[NR];
    unsigned    slice_len[NR];
    unsigned    map_lc;     // workgroup placement over the XCDs: log2 of the
                            // run of consecutive workgroups' tiles an XCD takes
                            // per round (see xcd_virtual_block); 0 = the
                            // hardware's own one-by-one round robin
};

// Workgroup placement over the 8 XCDs.  The dispatcher hands workgroup b of
// a launch to XCD b mod 8.  With runs of C = 2^lc workgroups, the grid's
// first 8C x floor(G / 8C) workgroups are renumbered so that XCD x processes,
// in each round, the tiles of C consecutive virtual workgroups (its run of
// the round), and the runs of successive rounds follow each other through
// the tensor:  b = 8 j + x  ->  v = (8 floor(j / C) + x) C + (j mod C).
// The remaining workgroups keep their index, so the map is a permutation of
// [0, G): every tile is still processed exactly once (which workgroup does it
// has no effect on any value).  lc = 0 is the identity.
__host__ __device__ inline unsigned xcd_virtual_block(unsigned b, unsigned G, unsigned lc) {
    const unsigned full = G & ~((8u << lc) - 1u);
    if (b >= full) return b;
    const unsigned x = b & 7u;
    const unsigned j = b >> 3;
    return ((((j >> lc) << 3) + x) << lc) + (j & ((1u << lc) - 1u));
}

// What the host fills in for any rank count; launch() copies it into the
// LaunchArgs of the chosen kernel's bucket.
struct KernelArgs : LaunchArgs<AR_MAX_RANKS> {
    int store_nt;   // 1: non-temporal stores, 0: ordinary (cached) stores;
                    // selects the kernel instance, not passed to the GPU
    size_t xcd_run_elems; // placement: elements of each source an XCD
                          // streams per run (launch() derives map_lc from
                          // it); below one workgroup's share keeps the
                          // identity placement
};

// Largest element count one launch covers (32-bit element indices inside the
// kernels; byte offsets are formed in 64 bits).
constexpr size_t kMaxLaunchElems = size_t(1) << 30;

enum class Family : int {
    SingleShot = 0,   // one wave tile per wave, no loop: decode-sized vectors
    StreamReg  = 1,   // persistent waves, register-staged batches of tiles
    StreamLds  = 2,   // persistent waves, double-buffered LDS staging
};

// A device's CU count and LDS bytes per CU, for launches that hold a CU below
// its full wave occupancy.
struct CuLimits {
    unsigned cu_count;
    unsigned lds_bytes;   // 0: unknown (no hold)
};

struct LaunchShape {
    unsigned grid_x;      // workgroups per slice
    unsigned grid_y;      // slices
    unsigned block;       // threads per workgroup
    unsigned lds_bytes;   // dynamic LDS per workgroup
    unsigned hold_waves;  // 0, or resident waves per CU to hold the launch to
    CuLimits cu;          // the device, for the hold
};

// Element types of a launch: wire type (ar_dtype), 16-bit sources, and a
// narrow destination (destination type == wire type; implies 16-bit sources).
struct Types {
    int wire;
    bool src_is_wire;
    bool dst_narrow;
};

// Launch one kernel of `family` for the given element types on `stream`.
// `sliced` selects the slice-range instance; a non-null args.res selects the
// residual instance (register-staged or single-shot families only).  The
// caller has validated every argument and sized the shape with plan_shape();
// launch() fills args.waves.
hipError_t launch(Family family, const Types &types, bool sliced, KernelArgs args, const LaunchShape &shape,
                  hipStream_t stream);

// Pick a launch shape for `family` covering `max_slice_len` elements per
// slice (`res`: the call adds a residual, which selects other kernel
// instances).  `cu_count` is the device's compute-unit count;
// `grid_override` (> 0) fixes the workgroups per slice.
LaunchShape plan_shape(Family family, bool src_is_wire, int R, bool res, unsigned max_slice_len, unsigned n_slices,
                       int cu_count, int grid_override);

// Placement exponent for a streaming launch whose workgroups each process
// `wg_elems` elements, grid_x workgroups per range: the largest lc < 16 with
// 2^lc workgroups' share <= run_elems and 8 runs <= grid_x (one whole round
// inside a range); 0 (identity) otherwise.
inline unsigned xcd_map_lc(unsigned grid_x, size_t wg_elems, size_t run_elems) {
    if (wg_elems == 0) return 0;
    unsigned lc = 0;
    while (lc < 15 && (wg_elems << (lc + 1)) <= run_elems && (uint64_t(8) << (lc + 1)) <= grid_x) ++lc;
    return lc;
}

// Dynamic LDS per one-wave workgroup that lets at most `waves` of them reside
// on a CU; the kernel never touches it.  0 (no hold) when the CU's LDS is
// unknown or the grid's `wgs` workgroups would not fill every CU to `waves`
// anyway.  The bytes are the smallest multiple of 512 with
// floor(lds_bytes / bytes) == waves.
inline unsigned hold_lds_bytes(const CuLimits &cu, uint64_t wgs, unsigned waves) {
    if (waves == 0 || cu.lds_bytes == 0 || cu.cu_count == 0) return 0;
    if (wgs < uint64_t(cu.cu_count) * waves) return 0;
    const unsigned bytes = (cu.lds_bytes / (waves + 1) / 512u + 1u) * 512u;
    return bytes <= 65536u && cu.lds_bytes / bytes == waves ? bytes : 0u;
}

// Resident waves per CU the two-rank kernels are held to by default, without
// and with a residual.  One-wave workgroups would otherwise fill a CU to 32
// waves; fewer loads in flight per CU stream faster on MI355X (bench.py
// --hold-study, one box, bit-identical outputs: the prefill call 15.42 us
// unheld, 15.21 held at 18-20 waves, 15.42 at 14; with an element-wise
// residual 20.21 unheld, 19.62 at 14, 19.91 at 18; with a 4096-element row
// 15.63 unheld, 15.38 at 14, 15.52 at 18; the row-strided forms alike).
constexpr unsigned kPairWaves = 18;
constexpr unsigned kPairResWaves = 14;
// Resident waves per CU the kernels for two to four active partials are held to
// by default, by active partials (2, 3, 4): fewer streams in flight per wave
// leave room for more waves (bench.py --hold-study, the prefill shape on one
// box, bit-identical outputs: two active of four ranks 15.53 us unheld, 15.33
// at 18 waves, 15.68 at 14; three ranks 20.16 unheld, 19.68 at 14, 19.94 at
// 18; four ranks with one inactive 20.13 unheld, 19.64 at 14; four ranks
// 25.42 unheld, 24.83 at 10, 25.28 at 14).
constexpr unsigned kFewWaves[3] = {18, 14, 10};
// and with an element-wise residual, one more read stream (the same study:
// two active of four 20.32 us unheld, 19.99 at 14; three ranks 25.80 unheld,
// 25.12 at 10; four ranks 31.47 unheld, 30.48 at 8, 30.70 at 10)
constexpr unsigned kFewResWaves[3] = {14, 10, 8};

// The two-rank contiguous kernels (k_pair, k_pair_res): dst[i] = wire(src0[i])
// + wire(src1[i]) in binary32, then + res[i] (res_kind 1, element-wise) or
// + res[(i + res_phase) mod res_len] (res_kind 2, a broadcast row of res_len
// elements, a multiple of 8, res_phase < res_len), for i < n (n <=
// kMaxLaunchElems); one 1-D launch on `stream`, XCD runs of about run_elems
// elements, every CU held to `hold_waves` resident waves (0: no hold).
// Every pointer is a binary32 device array, 16-byte aligned.
hipError_t launch_pair(int wire, int res_kind, size_t n, void *dst, const void *src0, const void *src1,
                       const void *res, size_t res_len, size_t res_phase, size_t run_elems, unsigned hold_waves,
                       const CuLimits &cu, hipStream_t stream);

// The two-rank kernel for 16-bit partials into the same 16-bit type
// (k_pair16): dst[i] = RN_W(widen(src0[i]) + widen(src1[i])) for i < n (n <=
// kMaxLaunchElems), wire = destination type W (AR_F16 or AR_BF16), no
// residual; one 1-D launch on `stream`, XCD runs of about run_elems elements,
// every CU held to `hold_waves` resident waves (0: no hold).  Every pointer is
// a 16-bit device array, 16-byte aligned.
hipError_t launch_pair16(int wire, size_t n, void *dst, const void *src0, const void *src1, size_t run_elems,
                         unsigned hold_waves, const CuLimits &cu, hipStream_t stream);

// The active partials of a call with R ranks (srcs[r] == nullptr: inactive),
// compacted in rank order into act[0 .. min(A, 4)), and the gaps that hold
// inactive ranks: bit g of *zmask is set when an inactive rank lies before
// active partial g (g = A: after the last).  Returns A, the active count.
inline int few_compact(const void *const *srcs, int R, const void *act[4], unsigned *zmask) {
    int A = 0;
    unsigned z = 0;
    for (int r = 0; r < R; ++r) {
        if (srcs[r] == nullptr) {
            z |= 1u << A;
        } else {
            if (A < 4) act[A] = srcs[r];
            ++A;
        }
    }
    *zmask = z;
    return A;
}

// The kernels for two to four active binary32 partials (k_few): dst[i] = the
// fold in rank order of wire(srcs[a][i]) over the `active` compacted active
// partials, with +0.0 added at every gap g (before active partial g; g =
// active after the last) whose bit g is set in zmask, where the fold over all
// ranks meets inactive ones, then + res[i] when res is not NULL (an
// element-wise residual), for i < n (n <= kMaxLaunchElems), wire AR_F32,
// AR_F16 or AR_BF16; one 1-D launch on `stream`, XCD runs of about run_elems
// elements, every CU held to `hold_waves` resident waves (0: no hold).  Every
// pointer is a binary32 device array, 16-byte aligned.
hipError_t launch_few(int wire, int active, size_t n, void *dst, const void *const *srcs, unsigned zmask,
                      const void *res, size_t run_elems, unsigned hold_waves, const CuLimits &cu,
                      hipStream_t stream);

// The two-rank kernels over row-strided tensors (k_pair_rows): row i, column
// j of the destination = wire(src0) + wire(src1) (+ the residual: res_kind 1
// element-wise with its own row stride, 2 one bias row of cols elements) at
// row i·stride + j of each tensor, for rows x cols elements (cols a multiple
// of 512, rows·cols <= kMaxLaunchElems, strides in elements, below 2^32);
// one 1-D launch on `stream`, XCD runs of about run_elems elements, every
// CU held to `hold_waves` resident waves (0: no hold).
hipError_t launch_pair_rows(int wire, int res_kind, size_t rows, size_t cols, size_t src_stride, size_t dst_stride,
                            void *dst, const void *src0, const void *src1, const void *res, size_t res_stride,
                            size_t run_elems, unsigned hold_waves, const CuLimits &cu, hipStream_t stream);

// Size of the library's static staging array (one per device), the only
// device memory ar_reduce_staged_static uses beyond the caller's buffers.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
constexpr int kMaxStaticScratchDevices = 64;

// Device address of the static staging array on `device`, which the caller
// has made current.  Looked up with hipGetSymbolAddress the first time per
// device and kept; returns the runtime's error when the lookup fails.
hipError_t static_scratch(int device, void **out);

// Elements processed per wave per loop iteration (a multiple of kWaveTile).
unsigned stream_tile_elems(Family family, bool src_is_wire, int R);

}  // namespace mpp
