// bench_ceiling.hip -- reference streaming kernels for the benchmark's
// achievable-bandwidth ceilings.  Not part of the reduce library: built into
// its own libmpp_ceiling.so, loaded by bench.py only.
//
// k_pattern<R, D, SP> reads R streams and writes D streams of `bytes` each
// and does nothing else worth the name: the only arithmetic is a 32-bit
// integer add across the R loaded words, which keeps every loaded byte live.
// The layout and launch shape are the reduce's binary32 wave tile: one wave
// covers 2 KiB of every stream as two 1 KiB instructions (lane l at byte
// 16 l and 1024 + 16 l), one tile per wave, 256- or 64-thread workgroups
// (the reduce's register- and LDS-staged families use both), a grid sized to
// the work.  Loads are non-temporal; stores follow SP (0 write-back,
// 1 non-temporal, 2 device-scope write-through).  R = 1, D = 1 is the plain
// 16-byte copy kernel; R = 2, D = 1 the two-read / one-write stream of the
// prefill reduce; R = 3, D = 1 the same with an element-wise residual, or
// three active ranks; R = 4, D = 4 the slice + broadcast pattern; R = 8, D = 1
// the eight-rank reduce.  A narrow-destination pattern is the same kernel at the
// 16-bit byte counts (the data are bits either way).
//
// The tile count, the placement exponent and the stream pointers are scalar
// parameters in that order, so the dispatcher preloads everything a wave of
// the one- and two-source patterns needs into SGPRs (eight dwords), as it
// does for the reduce's own streaming kernels: no wave waits on an argument
// load before its first address.  Workgroups can be renumbered with the
// reduce's XCD placement map (runs of 2^lc workgroups per XCD), so that the
// ceiling is taken with the same placement as the kernel it is compared with.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "ar_internal.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr unsigned kTileBytes = 2048;   // per stream per wave
constexpr int kMaxR = 8;
constexpr int kMaxD = 4;

__device__ __forceinline__ u32x4 load_nt(const char *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

template <int SP>
__device__ __forceinline__ void store(char *base, unsigned off, u32x4 v) {
    if constexpr (SP == 2) {
        // raw buffer resource over the wave's 2 KiB, sc1 (device-scope write-through)
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, kTileBytes, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, static_cast<int>(off), 0, 16);
    } else if constexpr (SP == 1) {
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(base + off));
    } else {
        *reinterpret_cast<u32x4 *>(base + off) = v;
    }
}

template <int R, int D, int SP, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_pattern(unsigned tiles, unsigned lc, char *d0, const char *s0,
                                                   const char *s1, const char *s2, const char *s3, const char *s4,
                                                   const char *s5, const char *s6, const char *s7, char *d1,
                                                   char *d2, char *d3) {
    const unsigned lane = threadIdx.x & 63u;
    // the grid size from the tile count (a shift), not from the dispatch's
    // hidden arguments, which lie beyond the preloaded dwords
    const unsigned G = (tiles + BLOCK / 64 - 1) / (BLOCK / 64);
    const unsigned w = mpp::xcd_virtual_block(blockIdx.x, G, lc) * (BLOCK / 64) +
                       __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    if (w >= tiles) return;
    const size_t t = static_cast<size_t>(w) * kTileBytes;
    const char *s[kMaxR] = {s0, s1, s2, s3, s4, s5, s6, s7};
    char *d[kMaxD] = {d0, d1, d2, d3};
    u32x4 v[R][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < R; ++r) v[r][j] = load_nt(s[r] + t + 1024 * j + 16 * lane);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        u32x4 acc = v[0][j];
#pragma unroll
        for (int r = 1; r < R; ++r) acc += v[r][j];
#pragma unroll
        for (int q = 0; q < D; ++q) store<SP>(d[q] + t, 1024 * j + 16 * lane, acc);
    }
}

// Instances: [workgroup size: 256, 64][pattern][store policy]; patterns (R, D) =
// (1,1), (2,1), (4,4), (8,1), (3,1).
#define MPP_CEIL_ROW(R, D, B) \
    {reinterpret_cast<const void *>(&k_pattern<R, D, 0, B>), reinterpret_cast<const void *>(&k_pattern<R, D, 1, B>), \
     reinterpret_cast<const void *>(&k_pattern<R, D, 2, B>)}
#define MPP_CEIL_TABLE(B) \
    {MPP_CEIL_ROW(1, 1, B), MPP_CEIL_ROW(2, 1, B), MPP_CEIL_ROW(4, 4, B), MPP_CEIL_ROW(8, 1, B), MPP_CEIL_ROW(3, 1, B)}
const void *const kPatterns[2][5][3] = {MPP_CEIL_TABLE(256), MPP_CEIL_TABLE(64)};
#undef MPP_CEIL_TABLE
#undef MPP_CEIL_ROW

int pattern_index(int R, int D) {
    if (R == 1 && D == 1) return 0;
    if (R == 2 && D == 1) return 1;
    if (R == 4 && D == 4) return 2;
    if (R == 8 && D == 1) return 3;
    if (R == 3 && D == 1) return 4;
    return -1;
}

}  // namespace

// Enqueue one pass of the (R, D) pattern over `bytes` of every stream on
// `stream` (a hipStream_t; NULL = the null stream).  Every pointer is device
// memory, 16-byte aligned, `bytes` long; `bytes` is a multiple of 2048 and at
// most 2^31 tiles.  `block`: 256 or 64 threads per workgroup.  `run_bytes`:
// XCD placement runs of about this many bytes of every stream (0 = the
// hardware's own placement).  `waves_per_cu`: 0, or hold every CU to that
// many resident waves (rounded down to whole workgroups) with dynamic LDS the
// kernel does not use, as the reduce's two-rank kernels are held.  Returns 0
// when enqueued, 1 for an unsupported or invalid request (nothing enqueued),
// 4 for a HIP error.
extern "C" __attribute__((visibility("default"))) int mpp_ceiling_launch(int R, int D, int store_policy, int block,
                                                                         const void *const *srcs,
                                                                         void *const *dsts, size_t bytes,
                                                                         size_t run_bytes, int waves_per_cu,
                                                                         void *stream) {
    const int p = pattern_index(R, D);
    if (p < 0 || store_policy < 0 || store_policy > 2 || srcs == nullptr || dsts == nullptr) return 1;
    if (block != 256 && block != 64) return 1;
    if (waves_per_cu < 0 || waves_per_cu > 64) return 1;
    if (bytes == 0 || bytes % kTileBytes != 0 || bytes / kTileBytes >= (size_t(1) << 31)) return 1;
    const char *s[kMaxR] = {};
    char *d[kMaxD] = {};
    for (int r = 0; r < R; ++r) {
        if (srcs[r] == nullptr || reinterpret_cast<uintptr_t>(srcs[r]) % 16 != 0) return 1;
        s[r] = static_cast<const char *>(srcs[r]);
    }
    for (int q = 0; q < D; ++q) {
        if (dsts[q] == nullptr || reinterpret_cast<uintptr_t>(dsts[q]) % 16 != 0) return 1;
        d[q] = static_cast<char *>(dsts[q]);
    }
    unsigned tiles = static_cast<unsigned>(bytes / kTileBytes);
    const unsigned wpb = static_cast<unsigned>(block) / 64;
    const unsigned grid = (tiles + wpb - 1) / wpb;
    unsigned lc = mpp::xcd_map_lc(grid, size_t(wpb) * kTileBytes, run_bytes);
    unsigned hold = 0;
    if (waves_per_cu > 0) {
        int dev = 0, cus = 0, lds = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess) {
            return 4;
        }
        const mpp::CuLimits cu{static_cast<unsigned>(cus), static_cast<unsigned>(lds)};
        hold = mpp::hold_lds_bytes(cu, grid, static_cast<unsigned>(waves_per_cu) / wpb);
    }
    void *args[] = {&tiles, &lc, &d[0], &s[0], &s[1], &s[2], &s[3], &s[4], &s[5], &s[6], &s[7], &d[1], &d[2], &d[3]};
    const hipError_t e = hipLaunchKernel(kPatterns[block == 64 ? 1 : 0][p][store_policy], dim3(grid), dim3(block),
                                         args, hold, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? 0 : 4;
}
