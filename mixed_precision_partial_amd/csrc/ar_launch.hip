// ar_launch.hip -- launch shapes and kernel selection for the tables that
// the ar_k_*.hip files define, and the library's static staging array.
#include "ar_device.h"

#include <algorithm>
#include <mutex>
#include <unordered_map>

namespace mpp {
namespace {

int combo_index(const Types &t) {
    if (t.dst_narrow) return t.wire == AR_BF16 ? 5 : 6;
    if (t.wire == AR_F32) return 0;
    if (!t.src_is_wire) return t.wire == AR_BF16 ? 1 : 2;
    return t.wire == AR_BF16 ? 3 : 4;
}

int bucket_index(int R) {
    if (R <= 2) return 0;
    if (R <= 4) return 1;
    if (R <= 8) return 2;
    return 3;
}

int bucket_ranks(int R) {
    static const int kB[4] = {2, 4, 8, 16};
    return kB[bucket_index(R)];
}

unsigned batch_tiles(Family family, bool src_is_wire, int R) {
    if (family == Family::SingleShot) return 1;
    if (family == Family::StreamLds) return static_cast<unsigned>(lds_batch(src_is_wire, bucket_ranks(R)));
    return static_cast<unsigned>(stream_batch(src_is_wire, bucket_ranks(R)));
}

// `hot`: the kernel takes the preloaded leading fields before the argument
// block (the plain streaming instances); the residual and single-shot
// instances take the block alone.
template <int NR>
hipError_t launch_as(const void *fn, const KernelArgs &a, const LaunchShape &shape, bool hot, hipStream_t stream) {
    LaunchArgs<NR> b;
    b.n = a.n;
    b.cols = a.cols;
    b.waves = a.waves;
    b.R = a.R;
    b.n_dst = a.n_dst;
    b.active = a.active;
    b.res_len = a.res_len;
    b.res_phase = a.res_phase;
    b.res_reuse = a.res_reuse;
    b.src_stride = a.src_stride;
    b.dst_stride = a.dst_stride;
    b.res_stride = a.res_stride;
    b.res = a.res;
    b.map_lc = a.map_lc;
    for (int r = 0; r < NR; ++r) {
        b.src[r] = a.src[r];
        b.dst[r] = a.dst[r];
        b.slice_start[r] = a.slice_start[r];
        b.slice_len[r] = a.slice_len[r];
    }
    // the leading scalar parameters (preloaded into SGPRs), then the block;
    // the shape dword packs the wave count (below 2^24), the destination
    // count minus one (1 .. 16) and the placement exponent (below 16)
    uint64_t hot_n = b.n, hot_src_stride = b.src_stride, hot_dst_stride = b.dst_stride;
    unsigned hot_cols = b.cols;
    unsigned hot_shape = b.waves | (static_cast<unsigned>(b.n_dst - 1) << 24) | (b.map_lc << 28);
    const void *hot_src0 = b.src[0], *hot_src1 = b.src[1];
    void *hot_dst0 = b.dst[0];
    void *hot_kargs[] = {&hot_n, &hot_cols, &hot_shape, &hot_src_stride, &hot_dst_stride,
                         &hot_src0, &hot_src1, &hot_dst0, &b};
    void *block_kargs[] = {&b};
    return hipLaunchKernel(fn, dim3(shape.grid_x, shape.grid_y, 1), dim3(shape.block, 1, 1),
                           hot ? hot_kargs : block_kargs, shape.lds_bytes, stream);
}

// Static LDS bytes of a kernel (its own __shared__ arrays), looked up once per
// kernel: the occupancy hold adds dynamic LDS on top of it.
hipError_t static_lds_bytes(const void *fn, unsigned *out) {
    static std::mutex mu;
    static std::unordered_map<const void *, unsigned> seen;
    std::lock_guard<std::mutex> lock(mu);
    auto it = seen.find(fn);
    if (it == seen.end()) {
        hipFuncAttributes fa{};
        const hipError_t e = hipFuncGetAttributes(&fa, fn);
        if (e != hipSuccess) return e;
        it = seen.emplace(fn, static_cast<unsigned>(fa.sharedSizeBytes)).first;
    }
    *out = it->second;
    return hipSuccess;
}

// Staging memory of ar_reduce_staged_static: one array per device, part of
// the code object (the loader places it on every device the library runs
// on, where it stays until the process ends).  Host code never passes the
// name `scratch` itself to a kernel or a copy -- on the host it is only a
// stand-in for the symbol -- but the device address static_scratch() looks up.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

}  // namespace

hipError_t launch_pair(int wire, int res_kind, size_t n, void *dst, const void *src0, const void *src1,
                       const void *res, size_t res_len, size_t res_phase, size_t run_elems, unsigned hold_waves,
                       const CuLimits &cu, hipStream_t stream) {
    if (wire < AR_F32 || wire > AR_BF16 || res_kind < 0 || res_kind > 2 || n == 0 || n > kMaxLaunchElems) {
        return hipErrorInvalidValue;
    }
    if (res_kind == 2 && (res_len == 0 || res_len % 8 != 0 || res_len > kMaxLaunchElems || res_phase >= res_len)) {
        return hipErrorInvalidValue;
    }
    if (res_kind != 0 && res == nullptr) return hipErrorInvalidValue;
    unsigned tiles = static_cast<unsigned>(n / kWaveTile);
    unsigned rem = static_cast<unsigned>(n % kWaveTile);
    const unsigned waves = tiles + (rem != 0 ? 1u : 0u);
    const unsigned wpb = kPairBlock / kWave;
    const unsigned grid = (waves + wpb - 1) / wpb;
    unsigned lc = xcd_map_lc(grid, static_cast<size_t>(wpb) * kWaveTile, run_elems);
    float *d = static_cast<float *>(dst);
    const float *a = static_cast<const float *>(src0);
    const float *b = static_cast<const float *>(src1);
    const float *r = static_cast<const float *>(res);
    unsigned rl = static_cast<unsigned>(res_kind == 2 ? res_len : 0);
    unsigned ph = static_cast<unsigned>(res_kind == 2 ? res_phase : 0);
    // row kinds: 4 a power of two, 2 at least one wave tile, 3 shorter
    const int kind = res_kind < 2 ? res_kind : ((res_len & (res_len - 1)) == 0 ? 4 : (res_len >= kWaveTile ? 2 : 3));
    void *args[] = {&tiles, &rem, &d, &a, &b, &lc, &r, &rl, &ph};
    const unsigned hold = hold_lds_bytes(cu, grid, hold_waves);
    return hipLaunchKernel(kPair[kind][wire], dim3(grid), dim3(kPairBlock), args, hold, stream);
}

hipError_t launch_pair16(int wire, size_t n, void *dst, const void *src0, const void *src1, size_t run_elems,
                         unsigned hold_waves, const CuLimits &cu, hipStream_t stream) {
    if ((wire != AR_F16 && wire != AR_BF16) || n == 0 || n > kMaxLaunchElems) return hipErrorInvalidValue;
    unsigned tiles = static_cast<unsigned>(n / kWaveTile);
    unsigned rem = static_cast<unsigned>(n % kWaveTile);
    const unsigned grid = tiles + (rem != 0 ? 1u : 0u);
    unsigned lc = xcd_map_lc(grid, kWaveTile, run_elems);
    uint16_t *d = static_cast<uint16_t *>(dst);
    const uint16_t *a = static_cast<const uint16_t *>(src0);
    const uint16_t *b = static_cast<const uint16_t *>(src1);
    void *args[] = {&tiles, &rem, &d, &a, &b, &lc};
    return hipLaunchKernel(kPair16[wire == AR_BF16 ? 1 : 0], dim3(grid), dim3(kPairBlock), args,
                           hold_lds_bytes(cu, grid, hold_waves), stream);
}

hipError_t launch_few(int wire, int active, size_t n, void *dst, const void *const *srcs, unsigned zmask,
                      const void *res, size_t run_elems, unsigned hold_waves, const CuLimits &cu,
                      hipStream_t stream) {
    if (wire < AR_F32 || wire > AR_BF16 || active < 2 || active > 4 || n == 0 || n > kMaxLaunchElems ||
        srcs == nullptr || zmask >= (1u << (active + 1))) {
        return hipErrorInvalidValue;
    }
    const float *s[4] = {};
    for (int a = 0; a < active; ++a) {
        if (srcs[a] == nullptr) return hipErrorInvalidValue;
        s[a] = static_cast<const float *>(srcs[a]);
    }
    unsigned tiles = static_cast<unsigned>(n / kWaveTile);
    unsigned rem = static_cast<unsigned>(n % kWaveTile);
    const unsigned grid = tiles + (rem != 0 ? 1u : 0u);
    unsigned lc = xcd_map_lc(grid, kWaveTile, run_elems);
    float *d = static_cast<float *>(dst);
    const float *r = static_cast<const float *>(res);
    void *args[] = {&tiles, &rem, &d, &s[0], &s[1], &lc, &s[2], &s[3], &zmask, &r};
    return hipLaunchKernel(kFew[res != nullptr ? 1 : 0][active - 2][wire], dim3(grid), dim3(kPairBlock), args,
                           hold_lds_bytes(cu, grid, hold_waves), stream);
}

hipError_t launch_pair_rows(int wire, int res_kind, size_t rows, size_t cols, size_t src_stride, size_t dst_stride,
                            void *dst, const void *src0, const void *src1, const void *res, size_t res_stride,
                            size_t run_elems, unsigned hold_waves, const CuLimits &cu, hipStream_t stream) {
    if (wire < AR_F32 || wire > AR_BF16 || res_kind < 0 || res_kind > 2 || rows == 0 || cols == 0 ||
        cols % kWaveTile != 0 || rows * cols > kMaxLaunchElems || src_stride < cols || dst_stride < cols ||
        src_stride >= (size_t(1) << 32) || dst_stride >= (size_t(1) << 32) || res_stride >= (size_t(1) << 32)) {
        return hipErrorInvalidValue;
    }
    if (res_kind != 0 && res == nullptr) return hipErrorInvalidValue;
    if (res_kind == 1 && res_stride < cols) return hipErrorInvalidValue;
    const size_t tpr = cols / kWaveTile;
    unsigned tiles = static_cast<unsigned>(rows * tpr);
    const bool p2 = (tpr & (tpr - 1)) == 0;
    unsigned tpr_arg = static_cast<unsigned>(p2 ? __builtin_ctzll(tpr) : tpr);
    unsigned ss = static_cast<unsigned>(src_stride), ds = static_cast<unsigned>(dst_stride);
    unsigned rs = static_cast<unsigned>(res_kind == 1 ? res_stride : 0);
    // one wave per workgroup: the grid is the tile count
    unsigned lc = xcd_map_lc(tiles, kWaveTile, run_elems);
    float *d = static_cast<float *>(dst);
    const float *a = static_cast<const float *>(src0);
    const float *b = static_cast<const float *>(src1);
    const float *r = static_cast<const float *>(res);
    void *args[] = {&tiles, &tpr_arg, &ss, &ds, &d, &a, &b, &lc, &r, &rs};
    const unsigned hold = hold_lds_bytes(cu, tiles, hold_waves);
    return hipLaunchKernel(kPairRows[res_kind][p2 ? 1 : 0][wire], dim3(tiles), dim3(kPairBlock), args, hold, stream);
}

hipError_t static_scratch(int device, void **out) {
    static std::mutex mu;
    static void *addr[kMaxStaticScratchDevices] = {};
    if (out == nullptr || device < 0 || device >= kMaxStaticScratchDevices) return hipErrorInvalidValue;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[device] == nullptr) {
        // the caller has made `device` current: each device has its own copy
        // of the array at its own address
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[device] = p;
    }
    *out = addr[device];
    return hipSuccess;
}

unsigned stream_tile_elems(Family family, bool src_is_wire, int R) {
    return kWaveTile * batch_tiles(family, src_is_wire, R);
}

LaunchShape plan_shape(Family family, bool src_is_wire, int R, bool res, unsigned max_slice_len, unsigned n_slices,
                       int cu_count, int grid_override) {
    LaunchShape s{};
    s.grid_y = n_slices;
    s.lds_bytes = 0;
    if (family == Family::SingleShot) {
        // One wave per tile, 64-thread workgroups: a decode vector spreads over
        // as many CUs as it has tiles, and no workgroup waits on a sibling.
        s.block = kSingleShotBlock;
        const unsigned tiles = (max_slice_len + kWaveTile - 1) / kWaveTile;
        unsigned g = tiles == 0 ? 1 : tiles;
        const unsigned cap = static_cast<unsigned>(cu_count) * 16u;
        if (g > cap) g = cap;
        s.grid_x = grid_override > 0 ? static_cast<unsigned>(grid_override) : g;
        return s;
    }
    s.block = family == Family::StreamLds ? kLdsBlock
                                          : static_cast<unsigned>(stream_block(bucket_ranks(R), res, src_is_wire));
    const unsigned wpb = s.block / kWave;
    const unsigned per_wave = stream_tile_elems(family, src_is_wire, R);
    const unsigned batches = (max_slice_len + per_wave - 1) / per_wave;
    unsigned g = (batches + wpb - 1) / wpb;
    if (g == 0) g = 1;
    // optional persistent-grid cap (k workgroups per CU, shared by the ranges
    // of the launch); 0 keeps the one-shot grid
    const unsigned per_cu = family == Family::StreamLds ? MPP_LDS_WG_PER_CU : MPP_STREAM_WG_PER_CU;
    unsigned cap = per_cu == 0 ? 65535u : static_cast<unsigned>(cu_count) * per_cu / (n_slices ? n_slices : 1u);
    if (cap < 1) cap = 1;
    if (cap > 65535u) cap = 65535u;
    if (g > cap) g = cap;
    s.grid_x = grid_override > 0 ? static_cast<unsigned>(grid_override) : g;
    return s;
}

hipError_t launch(Family family, const Types &types, bool sliced, KernelArgs a, const LaunchShape &shape,
                  hipStream_t stream) {
    if (types.dst_narrow && (!types.src_is_wire || types.wire == AR_F32)) return hipErrorInvalidValue;
    const int c = combo_index(types);
    const int b = bucket_index(a.R);
    const int nt = a.store_nt ? 1 : 0;
    const int sl = sliced ? 1 : 0;
    const int res = a.res != nullptr ? 1 : 0;
    const unsigned full = a.R >= 32 ? ~0u : ((1u << a.R) - 1u);
    const int m = (a.active & full) == full ? 0 : 1;   // some rank inactive
    const void *fn = nullptr;
    switch (family) {
    case Family::SingleShot:
        if (sliced) return hipErrorNotSupported;
        fn = kSingleShot[res][m][c][b];
        break;
    case Family::StreamReg:
        fn = res ? (m ? kStreamRegResM : kStreamRegRes)[nt][sl][c][b] : (m ? kStreamRegM : kStreamReg)[nt][sl][c][b];
        break;
    case Family::StreamLds:
        fn = res ? (m ? kStreamLdsResM : kStreamLdsRes)[nt][sl][c][b] : (m ? kStreamLdsM : kStreamLds)[nt][sl][c][b];
        break;
    default: return hipErrorNotSupported;
    }
    // the kernels index their waves with the workgroup size they were built for
    const unsigned want_block =
        family == Family::SingleShot ? kSingleShotBlock
        : family == Family::StreamLds
            ? kLdsBlock
            : static_cast<unsigned>(stream_block(bucket_ranks(a.R), res != 0, types.src_is_wire));
    if (shape.block != want_block) return hipErrorInvalidValue;
    a.waves = shape.grid_x * (shape.block / kWave);
    // the kernels write destination 0 unconditionally; the shape dword carries
    // the wave count, the destination count and the placement exponent
    if (a.waves >= (1u << 24) || a.n_dst < 1 || a.n_dst > AR_MAX_RANKS) return hipErrorInvalidValue;
    // elements one workgroup processes (its waves' batches)
    const size_t wg_elems = static_cast<size_t>(shape.block / kWave) * batch_tiles(family, types.src_is_wire, a.R) *
                            kWaveTile;
    a.map_lc = family == Family::SingleShot ? 0u : xcd_map_lc(shape.grid_x, wg_elems, a.xcd_run_elems);
    const bool hot = family != Family::SingleShot && !res;
    // occupancy hold: dynamic LDS on top of the kernel's own, so that at most
    // hold_waves (rounded down to whole workgroups) share a CU
    LaunchShape held = shape;
    if (shape.hold_waves > 0 && family != Family::SingleShot) {
        const unsigned wgs = std::max(1u, shape.hold_waves / (shape.block / kWave));
        const unsigned want = hold_lds_bytes(shape.cu, uint64_t(shape.grid_x) * shape.grid_y, wgs);
        unsigned own = 0;
        if (want > 0) {
            const hipError_t e = static_lds_bytes(fn, &own);
            if (e != hipSuccess) return e;
        }
        if (want > own) held.lds_bytes = std::max(held.lds_bytes, want - own);
    }
    switch (b) {
    case 0: return launch_as<2>(fn, a, held, hot, stream);
    case 1: return launch_as<4>(fn, a, held, hot, stream);
    case 2: return launch_as<8>(fn, a, held, hot, stream);
    default: return launch_as<16>(fn, a, held, hot, stream);
    }
}

}  // namespace mpp
