// ar_api.cpp -- host runtime behind the C ABI in ar.h: argument validation,
// the mode / chunk / slice plan, launches on the caller's stream and the
// host-staged copy pipeline.
//
// Passages this follows:
//   - "CUDA allreduce.cu" page: the size-based choice between a low-overhead
//     single-kernel path for small reductions and a chunked copy-engine path
//     for large ones (file header comment, size constants); launches stay on
//     the caller's stream because same-stream order already provides the
//     hand-off (chunked-kernel launch loop); the copy-engine path records an
//     event on the compute stream, has the copy stream wait for it, copies in
//     chunks with one event each, then runs the add kernel (copy_impl, stage
//     2) -- re-shaped here for one GPU, where the peers' sends are pinned host
//     buffers that already hold the partials; init returns a failure instead
//     of crashing, and free drains before releasing.
//   - "Hexagon allreduce-ops.c" page: rank-count checks and status codes in
//     op_allreduce / validate_allreduce; each rank owns an element range and
//     writes it to every destination.
//   - "llama.cpp commit log" page, SYCL tensor-parallel commit: no per-call
//     host synchronisation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "ar.h"
#include "ar_internal.h"

#define AR_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kMiB = size_t(1) << 20;
constexpr size_t kDefaultSingleShotMax = 1 * kMiB;
constexpr size_t kDefaultChunkBytes = 4 * kMiB;
// Host-staged copy chunk: clamp(bytes per rank / 2, 512 KiB, 64 MiB) of source
// bytes per rank -- two chunks or more, each large: measured on MI355X the
// fixed cost per copy outweighs the overlap that many small chunks would buy
// (the add kernel of a chunk is ~100x shorter than its copy over PCIe).
constexpr size_t kHostChunkMin = 512 * 1024;
constexpr size_t kHostChunkMax = 64 * kMiB;
constexpr int kDefaultHostSlots = 3;

constexpr int kMaxHostSlots = 64;
// Workgroup placement over the XCDs (see xcd_virtual_block): each XCD
// streams runs of this many elements of every source (512 KiB of a binary32
// source, 256 KiB of a 16-bit one); twice that in the broadcast schedule.
constexpr size_t kDefaultXcdRunElems = size_t(1) << 17;
constexpr size_t kDefaultXcdRunElemsBcast = size_t(1) << 18;

int elem_bytes(int t) { return t == AR_F32 ? 4 : 2; }
bool valid_type(int t) { return t == AR_F32 || t == AR_F16 || t == AR_BF16; }

size_t env_size(const char *name, size_t fallback) {
    const char *v = std::getenv(name);
    if (v == nullptr || *v == '\0') return fallback;
    char *end = nullptr;
    const unsigned long long x = std::strtoull(v, &end, 10);
    return end != v ? static_cast<size_t>(x) : fallback;
}

// A signed integer variable (out of int's range: an invalid value)
long env_long(const char *name, long fallback) {
    const char *v = std::getenv(name);
    if (v == nullptr || *v == '\0') return fallback;
    char *end = nullptr;
    const long x = std::strtol(v, &end, 10);
    return end != v ? x : fallback;
}

// Resolved configuration: explicit fields first, then AR_* environment
// variables, then the defaults.
struct Config {
    size_t single_shot_max_bytes = kDefaultSingleShotMax;
    size_t chunk_bytes = kDefaultChunkBytes;
    size_t host_chunk_bytes = 0;   // 0: per-call heuristic
    int host_slots = kDefaultHostSlots;
    int grid_wgs = 0;
    int stream_kernel = 0;
    int store_policy = 0;
    int host_path = 0;
    size_t xcd_run_elems = 0;   // 0: automatic per call (xcd_run_for)
    long occupancy_hold = 0;    // 0 automatic, -1 none, 1..32 every streaming launch
};

int resolve_config(const ar_config *cfg, Config *out) {
    Config c;
    c.single_shot_max_bytes = env_size("AR_SINGLE_SHOT_MAX_BYTES", kDefaultSingleShotMax);
    c.chunk_bytes = env_size("AR_CHUNK_BYTES", kDefaultChunkBytes);
    c.host_chunk_bytes = env_size("AR_HOST_CHUNK_BYTES", 0);
    c.host_slots = static_cast<int>(env_size("AR_HOST_SLOTS", kDefaultHostSlots));
    c.grid_wgs = static_cast<int>(env_size("AR_GRID_WGS", 0));
    c.stream_kernel = static_cast<int>(env_size("AR_STREAM_KERNEL", 0));
    c.store_policy = static_cast<int>(env_size("AR_STORE_POLICY", 0));
    c.host_path = static_cast<int>(env_size("AR_HOST_PATH", 0));
    c.xcd_run_elems = env_size("AR_XCD_RUN_ELEMS", 0);
    c.occupancy_hold = env_long("AR_OCCUPANCY_HOLD", 0);
    if (cfg != nullptr) {
        if (cfg->host_slots < 0 || cfg->grid_wgs < 0 || cfg->stream_kernel < 0 || cfg->stream_kernel > 2 ||
            cfg->store_policy < 0 || cfg->store_policy > 2 || cfg->host_path < 0 || cfg->host_path > 2) {
            return AR_ERR_INVALID;
        }
        if (cfg->xcd_run_elems) c.xcd_run_elems = cfg->xcd_run_elems;
        if (cfg->single_shot_max_bytes) c.single_shot_max_bytes = cfg->single_shot_max_bytes;
        if (cfg->chunk_bytes) c.chunk_bytes = cfg->chunk_bytes;
        if (cfg->host_chunk_bytes) c.host_chunk_bytes = cfg->host_chunk_bytes;
        if (cfg->host_slots) c.host_slots = cfg->host_slots;
        if (cfg->grid_wgs) c.grid_wgs = cfg->grid_wgs;
        if (cfg->stream_kernel) c.stream_kernel = cfg->stream_kernel;
        if (cfg->store_policy) c.store_policy = cfg->store_policy;
        if (cfg->host_path) c.host_path = cfg->host_path;
        if (cfg->occupancy_hold) c.occupancy_hold = cfg->occupancy_hold;
    }
    if (c.host_slots < 1 || c.host_slots > kMaxHostSlots) return AR_ERR_INVALID;
    if (c.stream_kernel < 0 || c.stream_kernel > 2) return AR_ERR_INVALID;
    if (c.grid_wgs < 0 || c.grid_wgs > 65535) return AR_ERR_INVALID;
    if (c.store_policy < 0 || c.store_policy > 2) return AR_ERR_INVALID;
    if (c.host_path < 0 || c.host_path > 2) return AR_ERR_INVALID;
    if (c.occupancy_hold < -1 || c.occupancy_hold > 32) return AR_ERR_INVALID;
    *out = c;
    return AR_OK;
}

// [a, a + na) and [b, b + nb) share a byte; exact for any addresses and
// lengths (no sum that could wrap).
bool ranges_overlap(uintptr_t a, size_t na, uintptr_t b, size_t nb) {
    if (na == 0 || nb == 0) return false;
    return a >= b ? a - b < nb : b - a < na;
}

size_t round_down(size_t x, size_t m) { return x / m * m; }

// Placement run of a streaming launch: the configured value, else, for up to
// four ranks, 2^17 elements of each source (2^18 in the broadcast schedule),
// and the hardware's own placement beyond.  Measured on MI355X against the
// identity placement, same machine each time, bit-identical outputs: prefill
// reduce 15.69 against 15.90 us, prefill + element-wise residual 19.80
// against 20.25 us, bf16 partials into a bf16 destination 8.68 against
// 8.78 us (8.85 with 2^18), 4-rank broadcast into fp16 destinations 43.55
// against 46.33 us (44.78 with 2^17; on another machine 43.61 against 44.82),
// fp32 partials 86.3 against 87.2 us with 2^17; but R = 8 fp32 partials
// [8192 x 8192] 373-387 against 360 us at every run length tried.
size_t xcd_run_for(const Config &cfg, int R, bool bcast) {
    if (cfg.xcd_run_elems) return cfg.xcd_run_elems;
    if (R > 4) return 0;
    return bcast ? kDefaultXcdRunElemsBcast : kDefaultXcdRunElems;
}

// The optional residual of ar_reduce_add: `len` elements of the destination
// type, added element-wise (len == n) or as one row broadcast to every row.
struct Residual {
    const void *ptr = nullptr;
    size_t len = 0;
};

// Row-strided tensors of ar_reduce_rows: `rows` rows of `cols` elements, row i
// of the sources / destinations / element-wise residual at element
// i * src_stride / i * dst_stride / i * res_stride (res_stride 0: one residual
// row for every row).
struct Rows {
    size_t rows = 0;
    size_t cols = 0;
    size_t src_stride = 0;
    size_t dst_stride = 0;
    size_t res_stride = 0;
};

// Elements from the first to the last element of `rows` rows of `cols`.
size_t extent(size_t rows, size_t cols, size_t stride) {
    return rows == 0 || cols == 0 ? 0 : (rows - 1) * stride + cols;
}

// Everything ar_reduce checks without the HIP runtime, plus the plan.  With
// `rows` the call is row-strided (n = rows x cols); otherwise every tensor is
// contiguous.
int validate_and_plan(const Config &cfg, void *const *dst, const void *const *srcs, int R, size_t n,
                      int dst_type, int wire_type, unsigned mode, const Residual &res, bool srcs_on_host,
                      ar_plan *plan, const Rows *rows = nullptr) {
    if (R < 2 || R > AR_MAX_RANKS) return AR_ERR_INVALID;
    if (!valid_type(dst_type) || !valid_type(wire_type)) return AR_ERR_INVALID;
    if ((mode & ~(AR_MODE_MASK | AR_SRC_WIRE | AR_SRC_INACTIVE_NULL)) != 0) return AR_ERR_INVALID;
    const bool allow_inactive = (mode & AR_SRC_INACTIVE_NULL) != 0;
    const int base = static_cast<int>(mode & AR_MODE_MASK);
    if (base < AR_MODE_AUTO || base > AR_MODE_HOST_STAGED) return AR_ERR_INVALID;
    if (elem_bytes(wire_type) > elem_bytes(dst_type)) return AR_ERR_INVALID;
    // a narrow destination is built for its own wire type only (the narrow
    // combinations the CUDA page launches: half/half and bf16/bf16)
    if (dst_type != AR_F32 && wire_type != dst_type) return AR_ERR_UNSUPPORTED;
    if (dst == nullptr || srcs == nullptr) return AR_ERR_INVALID;

    const bool dst_narrow = dst_type != AR_F32;
    // a narrow destination's sources hold its type (AR_SRC_WIRE or not)
    const bool src_wire = (mode & AR_SRC_WIRE) != 0 || dst_narrow;
    const int src_bytes = src_wire ? elem_bytes(wire_type) : elem_bytes(dst_type);
    const int wire_bytes = elem_bytes(wire_type);
    const int dst_bytes = elem_bytes(dst_type);
    int res_kind = 0;
    if (rows != nullptr) {
        // every row start 16-byte aligned: the kernels move 16 B per lane
        if (rows->src_stride < rows->cols || rows->dst_stride < rows->cols) return AR_ERR_INVALID;
        if ((rows->src_stride * static_cast<size_t>(src_bytes)) % 16 != 0 ||
            (rows->dst_stride * static_cast<size_t>(dst_bytes)) % 16 != 0) {
            return AR_ERR_INVALID;
        }
        if (rows->cols > mpp::kMaxLaunchElems) return AR_ERR_UNSUPPORTED;
        if (res.ptr != nullptr && n > 0) {
            if (rows->res_stride != 0 && rows->res_stride < rows->cols) return AR_ERR_INVALID;
            if ((rows->res_stride * static_cast<size_t>(dst_bytes)) % 16 != 0) return AR_ERR_INVALID;
            if (reinterpret_cast<uintptr_t>(res.ptr) % 16 != 0) return AR_ERR_INVALID;
            res_kind = rows->res_stride == 0 ? 2 : 1;
        }
    } else if (res.ptr != nullptr && n > 0) {
        if (res.len == 0 || res.len > n || n % res.len != 0) return AR_ERR_INVALID;
        if (reinterpret_cast<uintptr_t>(res.ptr) % 16 != 0) return AR_ERR_INVALID;
        res_kind = res.len == n ? 1 : 2;
        // a broadcast row is read 16 bytes at a time by lanes whose 4 or 8
        // consecutive elements must stay inside one row
        if (res_kind == 2 && (res.len % 8 != 0 || res.len > mpp::kMaxLaunchElems)) return AR_ERR_UNSUPPORTED;
    }

    int resolved = base;
    if (base == AR_MODE_AUTO) {
        if (srcs_on_host) {
            resolved = AR_MODE_HOST_STAGED;
        } else if (n <= SIZE_MAX / (4 * AR_MAX_RANKS) &&
                   n * static_cast<size_t>(wire_bytes) * static_cast<size_t>(R) <
                       (cfg.single_shot_max_bytes > SIZE_MAX / 2 ? SIZE_MAX : 2 * cfg.single_shot_max_bytes)) {
            // the limit is per rank at R = 2 and scales with the total wire bytes
            // of all ranks: measured on MI355X (graph-replayed kernel time), the
            // single-shot launch wins below ~2 MiB of wire bytes in total, at
            // R = 2 (ahead at 512 KiB per rank, behind at 1 MiB) as at R = 8
            // (ahead at 128 KiB per rank, behind at 256 KiB)
            resolved = AR_MODE_SINGLE_SHOT;
        } else {
            resolved = AR_MODE_CHUNKED;
        }
    }
    const int n_dst = resolved == AR_MODE_RS_BCAST ? R : 1;

    for (int d = 0; d < n_dst; ++d) {
        if (dst[d] == nullptr) return AR_ERR_INVALID;
        if (reinterpret_cast<uintptr_t>(dst[d]) % 16 != 0) return AR_ERR_INVALID;
    }
    unsigned active = 0;
    for (int r = 0; r < R; ++r) {
        if (srcs[r] == nullptr) {
            if (!allow_inactive) return AR_ERR_INVALID;
            continue;
        }
        active |= 1u << r;
        if (reinterpret_cast<uintptr_t>(srcs[r]) % 16 != 0) return AR_ERR_INVALID;
    }
    if (n > (SIZE_MAX / 8) / AR_MAX_RANKS) return AR_ERR_INVALID;

    // bytes each tensor spans (row-strided tensors: first to last element)
    const size_t dst_len = (rows ? extent(rows->rows, rows->cols, rows->dst_stride) : n) * static_cast<size_t>(dst_bytes);
    const size_t src_len = (rows ? extent(rows->rows, rows->cols, rows->src_stride) : n) * static_cast<size_t>(src_bytes);
    size_t res_bytes = 0;
    if (res_kind != 0) {
        const size_t res_elems = rows ? (res_kind == 2 ? rows->cols : extent(rows->rows, rows->cols, rows->res_stride))
                                      : res.len;
        res_bytes = res_elems * static_cast<size_t>(dst_bytes);
    }
    // the same layout on both sides of an exact in-place use
    const bool same_src_layout = rows == nullptr || rows->src_stride == rows->dst_stride;
    const bool same_res_layout = rows == nullptr || rows->res_stride == rows->dst_stride;
    if (n > 0) {
        for (int d = 0; d < n_dst; ++d) {
            const uintptr_t pd = reinterpret_cast<uintptr_t>(dst[d]);
            for (int e = d + 1; e < n_dst; ++e) {
                if (ranges_overlap(pd, dst_len, reinterpret_cast<uintptr_t>(dst[e]), dst_len)) {
                    return AR_ERR_INVALID;
                }
            }
            for (int r = 0; r < R; ++r) {
                if (srcs[r] == nullptr) continue;
                const uintptr_t ps = reinterpret_cast<uintptr_t>(srcs[r]);
                if (!ranges_overlap(pd, dst_len, ps, src_len)) continue;
                // exactly in place with equal element width is the one allowed overlap:
                // every element is read from all sources before the same thread writes it
                if (!(ps == pd && src_bytes == dst_bytes && same_src_layout)) return AR_ERR_INVALID;
            }
            if (res_kind != 0) {
                // an element-wise residual may be a destination itself (x += reduce):
                // each element's residual is read by the thread that writes it; a
                // broadcast row is read by every row, so it must not be written
                const uintptr_t pr = reinterpret_cast<uintptr_t>(res.ptr);
                if (ranges_overlap(pd, dst_len, pr, res_bytes) && !(res_kind == 1 && pr == pd && same_res_layout)) {
                    return AR_ERR_INVALID;
                }
            }
        }
    }

    if (plan != nullptr) {
        std::memset(plan, 0, sizeof(*plan));
        plan->mode = resolved;
        plan->n_dst = n_dst;
        plan->active_mask = active;
        plan->src_bytes = src_bytes;
        plan->wire_bytes = wire_bytes;
        const size_t algo_src = n * static_cast<size_t>(src_bytes);
        const size_t algo_dst = n * static_cast<size_t>(dst_bytes);
        size_t algo_res = 0;
        if (res_kind == 1) algo_res = n * static_cast<size_t>(dst_bytes);
        if (res_kind == 2) algo_res = (rows ? rows->cols : res.len) * static_cast<size_t>(dst_bytes);
        if (rows != nullptr) {
            // one range per row on the device; host-staged copies move whole rows
            size_t chunk_rows = 1;
            if (resolved == AR_MODE_HOST_STAGED && rows->cols > 0) {
                size_t hb = cfg.host_chunk_bytes;
                if (hb == 0) hb = std::min(kHostChunkMax, std::max(kHostChunkMin, algo_src / 2));
                chunk_rows = std::max<size_t>(1, hb / (rows->cols * static_cast<size_t>(src_bytes)));
                chunk_rows = std::min(chunk_rows, std::max<size_t>(1, mpp::kMaxLaunchElems / rows->cols));
            }
            plan->chunk_elems = chunk_rows * rows->cols;
            plan->n_chunks = n == 0 ? 0 : (rows->rows + chunk_rows - 1) / chunk_rows;
        } else {
            size_t chunk;
            if (resolved == AR_MODE_HOST_STAGED) {
                size_t hb = cfg.host_chunk_bytes;
                if (hb == 0) hb = std::min(kHostChunkMax, std::max(kHostChunkMin, src_len / 2));
                chunk = hb / static_cast<size_t>(src_bytes);
            } else {
                chunk = cfg.chunk_bytes / static_cast<size_t>(wire_bytes);
            }
            chunk = round_down(chunk, mpp::kWaveTile);
            if (chunk < mpp::kWaveTile) chunk = mpp::kWaveTile;
            if (chunk > mpp::kMaxLaunchElems) chunk = mpp::kMaxLaunchElems;
            if (resolved == AR_MODE_SINGLE_SHOT) chunk = n > 0 ? n : 1;
            plan->chunk_elems = chunk;
            plan->n_chunks = n == 0 ? 0 : (n + chunk - 1) / chunk;
        }
        if (resolved == AR_MODE_RS_BCAST && rows == nullptr) {
            // rank r owns [floor(r n / R), floor((r+1) n / R)), boundaries on wave tiles
            for (int r = 0; r < R; ++r) {
                const size_t s = round_down(static_cast<size_t>(r) * (n / R) + (static_cast<size_t>(r) * (n % R)) / R,
                                            mpp::kWaveTile);
                const size_t e = r + 1 == R ? n
                                            : round_down(static_cast<size_t>(r + 1) * (n / R) +
                                                             (static_cast<size_t>(r + 1) * (n % R)) / R,
                                                         mpp::kWaveTile);
                plan->slice_start[r] = s;
                plan->slice_len[r] = e - s;
            }
        }
        // an inactive rank is never read
        const size_t n_active = static_cast<size_t>(__builtin_popcount(active));
        plan->algo_bytes = n_active * algo_src + static_cast<size_t>(n_dst) * algo_dst + algo_res;
        plan->dst_bytes = dst_bytes;
        plan->residual_kind = res_kind;
        // Automatic store policy, measured on MI355X: when the call writes at
        // least as many bytes as it reads (broadcast to R destinations, 16-bit
        // sources at R = 2) non-temporal stores are faster; when reads dominate,
        // stores kept in the cache hierarchy are (write-through for fp32
        // sources, so the writes overlap the reads instead of waiting in L2
        // for the end of the kernel; write-back for the 16-bit layouts).  The
        // rule weighs the call's shape, all R sources whether active or not:
        // with inactive ranks kept stores stay the faster ones for one fp32
        // destination (1 of 2 ranks active at the prefill size: 11.8 against
        // 12.3 us streaming).
        const size_t written = static_cast<size_t>(n_dst) * algo_dst;
        const size_t read = static_cast<size_t>(R) * algo_src + (res_kind == 1 ? algo_res : 0);
        plan->store_nt = cfg.store_policy == 2 || (cfg.store_policy == 0 && written >= read);
        // host-staged sources: copy-engine pipeline (1) or the kernel reading
        // the pinned buffers over PCIe directly (2)
        // (automatic: direct reads -- measured on MI355X they match the best
        // copy-engine pipeline for large calls and are 7x faster for
        // decode-sized ones, 5.4 against 37 us; the copy engine leaves the CUs
        // free for other streams while the bytes cross PCIe)
        plan->host_direct = resolved == AR_MODE_HOST_STAGED && cfg.host_path != 1;
        // streaming kernel family: explicit choice, else the family measured
        // faster on MI355X for the call's kind and rank count (same machine,
        // inputs not in any cache, bit-identical outputs):
        //   - with a residual: LDS-staged for the broadcast schedule (R = 4:
        //     98-102 against 105-108 us element-wise, 88.5 against 90.7 us with
        //     a row), register-staged otherwise (a broadcast row on the prefill
        //     shape: 17.4 against 18.3 us; 8 ranks: 374 against 411 us);
        //   - broadcast schedule: LDS-staged (R = 4, fp32 sources: 88 against
        //     95 us; 16-bit sources at every R; R = 2 on the prefill shape with
        //     one-wave register workgroups: fp32 sources 22.54-22.68 against
        //     22.91-23.04 us, bf16 into bf16 11.52 against 12.94 us);
        //   - CHUNKED: register-staged for fp32 sources (prefill 15.7 against
        //     16.4 us, R = 8 363 against 416 us); for 16-bit sources the rank
        //     masks below, from a sweep of R on the prefill shape with one-wave
        //     register workgroups (into fp32, register against LDS-staged:
        //     R = 2 13.44 / 12.73 us, 3 15.55 / 16.64, 4 17.71 / 17.89, 5 22.67
        //     / 22.38, 6-8 0.6-1.4 us slower, 12 and 16 faster; narrow: R = 2
        //     9.08 / 8.54, 3 11.50 / 12.37, 4 14.12 / 14.59, 5 20.03 / 20.51,
        //     6-8 0.7-2.0 us slower, 12 and 16 faster);
        //   - host-staged calls: LDS-staged for two 16-bit sources only.
        constexpr unsigned kLds16ToF32 = (1u << 2) | (1u << 5) | (1u << 6) | (1u << 7) | (1u << 8);
        constexpr unsigned kLds16Narrow = (1u << 2) | (1u << 6) | (1u << 7) | (1u << 8);
        if (resolved == AR_MODE_SINGLE_SHOT) {
            plan->stream_kernel = 0;
        } else if (cfg.stream_kernel != 0) {
            plan->stream_kernel = cfg.stream_kernel;
        } else {
            bool lds;
            if (res_kind != 0) {
                lds = resolved == AR_MODE_RS_BCAST;
            } else if (resolved == AR_MODE_RS_BCAST) {
                lds = true;
            } else if (resolved == AR_MODE_HOST_STAGED) {
                lds = src_wire && R == 2;
            } else {
                lds = src_wire && (((dst_narrow ? kLds16Narrow : kLds16ToF32) >> R) & 1u) != 0;
            }
            plan->stream_kernel = lds ? 2 : 1;
        }
        // the two-rank contiguous kernels for the commonest call: two active
        // binary32 partials into one binary32 destination (with or without a
        // residual), kept stores, the launch shape left to the library, chunked
        // or single-shot (measured before the occupancy hold below, which
        // widened the lead: prefill call 15.45 against 15.82 us with the
        // register-staged kernel, 20.2 against 21.2-22.8 us with an
        // element-wise residual, 15.6 against 16.4-17.3 us with a row; a decode
        // vector of 4096, replayed from a HIP graph, 1.68 against 1.74-1.78 us
        // with the single-shot kernel; same machine, bit-identical outputs)
        // Row-strided tensors take them when every row is whole wave tiles and
        // the strides fit 32 bits (a 2048 x 4096 block in rows of 4608 / 4352,
        // same machine: 15.40 against 15.82 us on the register-staged kernel,
        // 15.57 against 16.17 us with a bias row, 20.13 against 21.48-23.20 us
        // with a strided element-wise residual; the general kernels' few
        // workgroups per row keep the hardware's XCD order).
        const bool pair_rows = rows != nullptr && rows->cols > 0 && rows->cols % mpp::kWaveTile == 0 &&
                               rows->src_stride < (size_t(1) << 32) && rows->dst_stride < (size_t(1) << 32) &&
                               rows->res_stride < (size_t(1) << 32);
        if ((resolved == AR_MODE_CHUNKED || resolved == AR_MODE_SINGLE_SHOT) && cfg.stream_kernel == 0 &&
            (rows == nullptr || pair_rows) && R == 2 && active == 0x3u && !src_wire && dst_bytes == 4 &&
            !plan->store_nt && cfg.grid_wgs == 0) {
            plan->stream_kernel = 3;
        }
        // and the two-rank 16-bit kernel: two active 16-bit partials into a
        // contiguous destination of their type, no residual, same conditions
        // otherwise (bf16 prefill shape, 2 x [2048 x 4096] into bf16:
        // bench.py --family-study measures it against the LDS-staged kernel)
        if ((resolved == AR_MODE_CHUNKED || resolved == AR_MODE_SINGLE_SHOT) && cfg.stream_kernel == 0 &&
            rows == nullptr && R == 2 && active == 0x3u && dst_narrow && res_kind == 0 && !plan->store_nt &&
            cfg.grid_wgs == 0) {
            plan->stream_kernel = 3;
        }
        // the kernels for two to four active binary32 partials: three or four
        // ranks, or two to four active ones among more, no residual or an
        // element-wise one, contiguous, the two-rank kernels' conditions
        // otherwise
        if ((resolved == AR_MODE_CHUNKED || resolved == AR_MODE_SINGLE_SHOT) && cfg.stream_kernel == 0 &&
            rows == nullptr && res_kind <= 1 && !src_wire && dst_bytes == 4 && !plan->store_nt &&
            cfg.grid_wgs == 0 && n_active >= 2 && n_active <= 4 && !(R == 2 && active == 0x3u)) {
            plan->stream_kernel = 4;
        }
        // occupancy hold: an explicit one holds every streaming launch; the
        // automatic one holds the binary32 two-rank kernels (18 waves, 14 with
        // a residual: the figures are at kPairWaves) and the kernels for two to
        // four active partials (kFewWaves); the general kernels and the 16-bit
        // two-rank kernel gained nothing from one (bench.py --hold-study)
        plan->hold_waves = 0;
        if (cfg.occupancy_hold > 0) {
            plan->hold_waves = plan->stream_kernel == 0 ? 0 : static_cast<int>(cfg.occupancy_hold);
        } else if (cfg.occupancy_hold == 0 && plan->stream_kernel == 3 && dst_bytes == 4) {
            plan->hold_waves = static_cast<int>(res_kind != 0 ? mpp::kPairResWaves : mpp::kPairWaves);
        } else if (cfg.occupancy_hold == 0 && plan->stream_kernel == 4) {
            plan->hold_waves = static_cast<int>(res_kind != 0 ? mpp::kFewResWaves[n_active - 2]
                                                              : mpp::kFewWaves[n_active - 2]);
        }
    }
    return AR_OK;
}

}  // namespace

struct ar_ctx {
    int device = -1;
    int cu_count = 0;
    unsigned lds_per_cu = 0;   // LDS bytes per CU (0: unknown)
    Config cfg;
    hipStream_t copy_stream = nullptr;
    // host-staged scratch ring: slots x R x chunk source elements
    void *scratch = nullptr;
    size_t scratch_bytes = 0;
    std::vector<hipEvent_t> ev_h2d;    // per slot: its H2D copies landed
    std::vector<hipEvent_t> ev_free;   // per slot: the add kernel reading it finished
    std::vector<char> slot_used;
    hipEvent_t ev_start = nullptr;     // caller-stream order point before the copies
    unsigned next_slot = 0;
    // device address of the library's static staging array on this device
    // (ar_reduce_staged_static); shared by every context on the device.  The
    // array is one slot of this context's own bookkeeping, apart from the ring
    // above: its copies landed / the add kernel reading it finished.
    void *static_scratch = nullptr;
    hipEvent_t ev_static_h2d = nullptr;
    hipEvent_t ev_static_free = nullptr;
    char static_used = 0;
    unsigned static_next = 0;
};

namespace {

mpp::CuLimits cu_limits(const ar_ctx *c) {
    return mpp::CuLimits{static_cast<unsigned>(c->cu_count), c->lds_per_cu};
}

// A general launch shape with the plan's occupancy hold and the device's limits.
mpp::LaunchShape held(const ar_ctx *c, const ar_plan &plan, mpp::LaunchShape s) {
    s.hold_waves = static_cast<unsigned>(plan.hold_waves);
    s.cu = cu_limits(c);
    return s;
}

// Makes `dev` current for the scope and restores the caller's device; no
// runtime call beyond the query when `dev` is already current (the common
// case, and the cheap one on a latency-bound decode call).
struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    bool switched = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) return;
        if (prev == dev) {
            ok = true;
        } else if (hipSetDevice(dev) == hipSuccess) {
            ok = true;
            switched = true;
        }
    }
    ~DeviceGuard() {
        if (switched) (void)hipSetDevice(prev);
    }
};

void destroy(ar_ctx *c) {
    if (c->copy_stream) (void)hipStreamSynchronize(c->copy_stream);
    for (hipEvent_t e : c->ev_free) {
        if (e) (void)hipEventSynchronize(e);
    }
    if (c->ev_static_free) (void)hipEventSynchronize(c->ev_static_free);
    if (c->scratch) (void)hipFree(c->scratch);
    for (hipEvent_t e : c->ev_h2d) if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : c->ev_free) if (e) (void)hipEventDestroy(e);
    if (c->ev_static_h2d) (void)hipEventDestroy(c->ev_static_h2d);
    if (c->ev_static_free) (void)hipEventDestroy(c->ev_static_free);
    if (c->ev_start) (void)hipEventDestroy(c->ev_start);
    if (c->copy_stream) (void)hipStreamDestroy(c->copy_stream);
    delete c;
}

enum class Kind { Device, PinnedHost, Other };

// Memory kind of [p, p + bytes) and whether the whole range lies inside one
// allocation of the runtime.  Clears the runtime's sticky last-error on a
// failed lookup so the caller's next HIP call does not see it.
Kind memory_kind(const void *p, size_t bytes, int device, const void **device_view = nullptr) {
    hipPointerAttribute_t at;
    std::memset(&at, 0, sizeof(at));
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();
        return Kind::Other;
    }
    Kind k;
    if (at.type == hipMemoryTypeDevice && at.device == device) {
        k = Kind::Device;
    } else if (at.type == hipMemoryTypeHost) {
        k = Kind::PinnedHost;
    } else {
        return Kind::Other;
    }
    void *base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void *>(p)) != hipSuccess) {
        (void)hipGetLastError();
        return Kind::Other;
    }
    const uintptr_t b = reinterpret_cast<uintptr_t>(base);
    const uintptr_t q = reinterpret_cast<uintptr_t>(p);
    if (q < b || q - b > size || bytes > size - (q - b)) return Kind::Other;
    if (device_view != nullptr) {
        // the address kernels use for this memory (pinned host memory is mapped
        // into the device's address space; the runtime reports where)
        *device_view = k == Kind::PinnedHost ? at.devicePointer : p;
        if (*device_view == nullptr) return Kind::Other;
    }
    return k;
}

mpp::Family stream_family(const ar_plan &plan) {
    return plan.stream_kernel == 2 ? mpp::Family::StreamLds : mpp::Family::StreamReg;
}

int hip_status(hipError_t e) { return e == hipSuccess ? AR_OK : AR_ERR_RUNTIME; }

mpp::Types launch_types(const ar_plan &plan, int wire_type) {
    return mpp::Types{wire_type, plan.src_bytes == 2, plan.dst_bytes == 2};
}

// Residual fields of a 1-D launch whose element 0 is element `first` of the
// call; consecutive ranges of `cols` elements (strides = cols).
void set_ranges_1d(mpp::KernelArgs &a, const Residual &res, size_t n, size_t first, size_t cols, int dst_bytes) {
    a.cols = static_cast<unsigned>(cols);
    a.src_stride = cols;
    a.dst_stride = cols;
    a.res_stride = cols;
    if (res.ptr == nullptr) return;
    if (res.len == n) {
        a.res = static_cast<const char *>(res.ptr) + first * static_cast<size_t>(dst_bytes);
        a.res_len = 0;
        a.res_phase = 0;
        a.res_reuse = 0;
    } else {
        a.res = res.ptr;
        a.res_len = static_cast<unsigned>(res.len);
        a.res_phase = static_cast<unsigned>(first % res.len);
        a.res_reuse = 1;
    }
}

// SINGLE_SHOT / CHUNKED / RS_BCAST: launches on the caller's stream, at most
// kMaxLaunchElems elements per launch.
int run_device(ar_ctx *c, const ar_plan &plan, void *const *dst, const void *const *srcs, int R, size_t n,
               int wire_type, const Residual &res, hipStream_t stream) {
    const mpp::Family family = plan.mode == AR_MODE_SINGLE_SHOT ? mpp::Family::SingleShot : stream_family(plan);
    const mpp::Types types = launch_types(plan, wire_type);
    const size_t sb = static_cast<size_t>(plan.src_bytes);
    const size_t db = static_cast<size_t>(plan.dst_bytes);

    if (plan.mode == AR_MODE_RS_BCAST) {
        // gridDim.y = the ranks' slices; a slice longer than one launch covers
        // is cut into pieces at the same relative offset in every slice.  The
        // slice ranges are element indices of the whole call, so the residual
        // is indexed from element 0.
        size_t longest = 0;
        for (int r = 0; r < R; ++r) longest = std::max(longest, static_cast<size_t>(plan.slice_len[r]));
        for (size_t p0 = 0; p0 < longest; p0 += mpp::kMaxLaunchElems) {
            mpp::KernelArgs a{};
            a.xcd_run_elems = xcd_run_for(c->cfg, R, true);
            a.R = R;
            a.n_dst = R;
            a.store_nt = plan.store_nt;
            a.active = plan.active_mask;
            set_ranges_1d(a, res, n, 0, 0, plan.dst_bytes);
            unsigned max_len = 0;
            for (int r = 0; r < R; ++r) {
                const size_t len = plan.slice_len[r] > p0 ? std::min(mpp::kMaxLaunchElems, plan.slice_len[r] - p0) : 0;
                a.slice_start[r] = plan.slice_start[r] + p0;
                a.slice_len[r] = static_cast<unsigned>(len);
                max_len = std::max<unsigned>(max_len, static_cast<unsigned>(len));
                a.src[r] = srcs[r];
                a.dst[r] = dst[r];
            }
            const mpp::LaunchShape shape = held(c, plan, mpp::plan_shape(family, types.src_is_wire, R, res.ptr != nullptr, max_len,
                                                           static_cast<unsigned>(R), c->cu_count, c->cfg.grid_wgs));
            if (int rc = hip_status(mpp::launch(family, types, true, a, shape, stream))) return rc;
        }
        return AR_OK;
    }

    if (plan.stream_kernel == 3 && plan.dst_bytes == 2) {
        // the two-rank 16-bit kernel: one 1-D launch per launch piece
        for (size_t p0 = 0; p0 < n; p0 += mpp::kMaxLaunchElems) {
            const size_t len = std::min(mpp::kMaxLaunchElems, n - p0);
            if (int rc = hip_status(mpp::launch_pair16(wire_type, len, static_cast<char *>(dst[0]) + p0 * db,
                                                       static_cast<const char *>(srcs[0]) + p0 * sb,
                                                       static_cast<const char *>(srcs[1]) + p0 * sb,
                                                       xcd_run_for(c->cfg, R, false),
                                                       static_cast<unsigned>(plan.hold_waves), cu_limits(c),
                                                       stream))) {
                return rc;
            }
        }
        return AR_OK;
    }
    if (plan.stream_kernel == 4) {
        // two to four active binary32 partials: compacted in rank order, with
        // the gaps where inactive ranks add +0.0; one 1-D launch per piece
        const void *act[4] = {};
        unsigned zmask = 0;
        const int A = mpp::few_compact(srcs, R, act, &zmask);
        if (A < 2 || A > 4) return AR_ERR_INVALID;
        for (size_t p0 = 0; p0 < n; p0 += mpp::kMaxLaunchElems) {
            const size_t len = std::min(mpp::kMaxLaunchElems, n - p0);
            const void *piece[4] = {};
            for (int a = 0; a < A; ++a) piece[a] = static_cast<const char *>(act[a]) + p0 * sb;
            const void *rp = res.ptr == nullptr ? nullptr : static_cast<const char *>(res.ptr) + p0 * db;
            if (int rc = hip_status(mpp::launch_few(wire_type, A, len, static_cast<char *>(dst[0]) + p0 * db, piece,
                                                    zmask, rp, xcd_run_for(c->cfg, A, false),
                                                    static_cast<unsigned>(plan.hold_waves), cu_limits(c), stream))) {
                return rc;
            }
        }
        return AR_OK;
    }
    if (plan.stream_kernel == 3) {
        // two-rank contiguous kernels: one 1-D launch per launch piece; an
        // element-wise residual moves with the piece, a broadcast row keeps
        // its base and takes the piece's phase in it
        const int rk = res.ptr == nullptr ? 0 : (res.len == n ? 1 : 2);
        for (size_t p0 = 0; p0 < n; p0 += mpp::kMaxLaunchElems) {
            const size_t len = std::min(mpp::kMaxLaunchElems, n - p0);
            const void *rp = rk == 1 ? static_cast<const char *>(res.ptr) + p0 * db : res.ptr;
            if (int rc = hip_status(mpp::launch_pair(wire_type, rk, len, static_cast<char *>(dst[0]) + p0 * db,
                                                     static_cast<const char *>(srcs[0]) + p0 * sb,
                                                     static_cast<const char *>(srcs[1]) + p0 * sb, rp,
                                                     rk == 2 ? res.len : 0, rk == 2 ? p0 % res.len : 0,
                                                     xcd_run_for(c->cfg, R, false),
                                                     static_cast<unsigned>(plan.hold_waves), cu_limits(c),
                                                     stream))) {
                return rc;
            }
        }
        return AR_OK;
    }
    for (size_t p0 = 0; p0 < n; p0 += mpp::kMaxLaunchElems) {
        const size_t len = std::min(mpp::kMaxLaunchElems, n - p0);
        mpp::KernelArgs a{};
        a.xcd_run_elems = xcd_run_for(c->cfg, R, false);
        a.R = R;
        a.n_dst = 1;
        a.n = len;
        a.store_nt = plan.mode == AR_MODE_SINGLE_SHOT ? 0 : plan.store_nt;
        a.active = plan.active_mask;
        for (int r = 0; r < R; ++r) {
            a.src[r] = srcs[r] == nullptr ? nullptr : static_cast<const char *>(srcs[r]) + p0 * sb;
        }
        a.dst[0] = static_cast<char *>(dst[0]) + p0 * db;
        // CHUNKED: gridDim.y walks the plan's chunks; SINGLE_SHOT: one range
        size_t cols = len;
        if (plan.mode == AR_MODE_CHUNKED) {
            cols = std::min(plan.chunk_elems, len);
            if ((len + cols - 1) / cols > 65535) cols = round_down((len + 65534) / 65535 + mpp::kWaveTile - 1,
                                                                   mpp::kWaveTile);
        }
        set_ranges_1d(a, res, n, p0, cols, plan.dst_bytes);
        const unsigned n_ranges = static_cast<unsigned>((len + cols - 1) / cols);
        const mpp::LaunchShape shape = held(c, plan, mpp::plan_shape(family, types.src_is_wire, R, res.ptr != nullptr,
                                                       static_cast<unsigned>(cols), n_ranges, c->cu_count,
                                                       c->cfg.grid_wgs));
        if (int rc = hip_status(mpp::launch(family, types, false, a, shape, stream))) return rc;
    }
    return AR_OK;
}

// Row-strided calls on the device (SINGLE_SHOT / CHUNKED / RS_BCAST, and
// host-staged calls that read the pinned rows directly): gridDim.y = rows,
// at most 65535 per launch, each row walked like a 1-D range.  The broadcast
// schedule writes every row to all R destinations (its rows are spread over
// the grid instead of per-rank slices; the bytes are the same).
int run_rows(ar_ctx *c, const ar_plan &plan, void *const *dst, const void *const *srcs, int R, const Rows &rw,
             int wire_type, const Residual &res, hipStream_t stream) {
    const mpp::Family family = plan.mode == AR_MODE_SINGLE_SHOT ? mpp::Family::SingleShot : stream_family(plan);
    const mpp::Types types = launch_types(plan, wire_type);
    const size_t sb = static_cast<size_t>(plan.src_bytes);
    const size_t db = static_cast<size_t>(plan.dst_bytes);
    if (plan.stream_kernel == 3) {
        // two-rank row-strided kernel: one 1-D launch per piece of whole rows
        const int rk = res.ptr == nullptr ? 0 : (rw.res_stride == 0 ? 2 : 1);
        const size_t piece = std::max<size_t>(1, mpp::kMaxLaunchElems / rw.cols);
        for (size_t r0 = 0; r0 < rw.rows; r0 += piece) {
            const size_t nr = std::min(piece, rw.rows - r0);
            const void *rp = rk == 1 ? static_cast<const char *>(res.ptr) + r0 * rw.res_stride * db : res.ptr;
            if (int rc = hip_status(mpp::launch_pair_rows(
                    wire_type, rk, nr, rw.cols, rw.src_stride, rw.dst_stride,
                    static_cast<char *>(dst[0]) + r0 * rw.dst_stride * db,
                    static_cast<const char *>(srcs[0]) + r0 * rw.src_stride * sb,
                    static_cast<const char *>(srcs[1]) + r0 * rw.src_stride * sb, rp, rw.res_stride,
                    xcd_run_for(c->cfg, R, false), static_cast<unsigned>(plan.hold_waves), cu_limits(c),
                    stream))) {
                return rc;
            }
        }
        return AR_OK;
    }
    constexpr size_t kMaxRows = 65535;
    for (size_t r0 = 0; r0 < rw.rows; r0 += kMaxRows) {
        const size_t nr = std::min(kMaxRows, rw.rows - r0);
        mpp::KernelArgs a{};
        a.xcd_run_elems = xcd_run_for(c->cfg, R, plan.mode == AR_MODE_RS_BCAST);
        a.R = R;
        a.n_dst = plan.n_dst;
        a.n = nr * rw.cols;
        a.cols = static_cast<unsigned>(rw.cols);
        a.src_stride = rw.src_stride;
        a.dst_stride = rw.dst_stride;
        a.store_nt = plan.mode == AR_MODE_SINGLE_SHOT ? 0 : plan.store_nt;
        a.active = plan.active_mask;
        for (int r = 0; r < R; ++r) {
            a.src[r] = srcs[r] == nullptr ? nullptr : static_cast<const char *>(srcs[r]) + r0 * rw.src_stride * sb;
        }
        for (int d = 0; d < plan.n_dst; ++d) a.dst[d] = static_cast<char *>(dst[d]) + r0 * rw.dst_stride * db;
        if (res.ptr != nullptr) {
            a.res = static_cast<const char *>(res.ptr) + r0 * rw.res_stride * db;
            a.res_stride = rw.res_stride;
            a.res_reuse = rw.res_stride == 0 ? 1 : 0;
        }
        const mpp::LaunchShape shape = held(c, plan, mpp::plan_shape(family, types.src_is_wire, R, res.ptr != nullptr,
                                                       static_cast<unsigned>(rw.cols), static_cast<unsigned>(nr),
                                                       c->cu_count, c->cfg.grid_wgs));
        if (int rc = hip_status(mpp::launch(family, types, false, a, shape, stream))) return rc;
    }
    return AR_OK;
}

int ensure_scratch(ar_ctx *c, size_t bytes) {
    if (c->scratch_bytes >= bytes) return AR_OK;
    // the old ring may still be read by enqueued kernels or written by copies
    if (hipStreamSynchronize(c->copy_stream) != hipSuccess) return AR_ERR_RUNTIME;
    for (size_t s = 0; s < c->ev_free.size(); ++s) {
        if (c->slot_used[s] && hipEventSynchronize(c->ev_free[s]) != hipSuccess) return AR_ERR_RUNTIME;
    }
    if (c->scratch) {
        if (hipFree(c->scratch) != hipSuccess) return AR_ERR_RUNTIME;
        c->scratch = nullptr;
        c->scratch_bytes = 0;
    }
    void *p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return AR_ERR_NOMEM;
    }
    c->scratch = p;
    c->scratch_bytes = bytes;
    std::fill(c->slot_used.begin(), c->slot_used.end(), 0);
    return AR_OK;
}

// HOST_STAGED: chunk c of every rank is copied host -> HBM slot (c mod K) on
// the internal copy stream; the caller's stream waits for that slot's copies,
// runs the add kernel over the slot and marks the slot free again.  The copy
// of a later chunk into the same slot waits for that mark, so copies run ahead
// of the adds by up to K chunks.  The ring is the context's (K = host_slots,
// grown with hipMalloc when too small), or, with `fixed`, the `fixed_bytes`
// at `fixed` as one slot with its own events: the chunk is then what R ranks
// fit there, and nothing is allocated; a configured copy chunk that does not
// fit is AR_ERR_NOMEM.  One slot for the fixed array, because the chunk size
// decides the copy engine's rate: measured on MI355X, R = 8 bf16 partials
// [8192 x 8192] (1 GiB over PCIe) took 20.7 ms with one 8 MiB-per-rank slot,
// 25.5 ms with two 4 MiB slots and 28.4 ms with three 2.7 MiB slots in the
// same 64 MiB, against 18.7 ms for one plain 1 GiB copy; the context's ring
// at 8 MiB chunks takes 20.5 ms with three slots and 20.7 with one.
struct SlotRing {
    unsigned K;
    unsigned *next;
    char *used;
    hipEvent_t *h2d;
    hipEvent_t *free;
};

int run_host_staged(ar_ctx *c, const ar_plan &plan, void *const *dst, const void *const *srcs, int R, size_t n,
                    int wire_type, const Residual &res, hipStream_t stream, void *fixed = nullptr,
                    size_t fixed_bytes = 0) {
    const mpp::Types types = launch_types(plan, wire_type);
    const size_t sb = static_cast<size_t>(plan.src_bytes);
    const size_t db = static_cast<size_t>(plan.dst_bytes);
    const SlotRing slots = fixed != nullptr
                               ? SlotRing{1u, &c->static_next, &c->static_used, &c->ev_static_h2d, &c->ev_static_free}
                               : SlotRing{static_cast<unsigned>(c->cfg.host_slots), &c->next_slot,
                                          c->slot_used.data(), c->ev_h2d.data(), c->ev_free.data()};
    const size_t K = slots.K;
    size_t chunk = plan.chunk_elems;
    if (fixed != nullptr) {
        const size_t fit = round_down(fixed_bytes / (K * static_cast<size_t>(R) * sb), mpp::kWaveTile);
        if (fit < mpp::kWaveTile) return AR_ERR_NOMEM;
        if (c->cfg.host_chunk_bytes != 0 && chunk > fit) return AR_ERR_NOMEM;
        chunk = c->cfg.host_chunk_bytes != 0 ? chunk : fit;
    }
    const size_t n_chunks = (n + chunk - 1) / chunk;
    const size_t rank_stride = chunk * sb;
    const size_t slot_stride = rank_stride * static_cast<size_t>(R);
    char *ring = static_cast<char *>(fixed);
    if (ring == nullptr) {
        if (int rc = ensure_scratch(c, slot_stride * K)) return rc;
        ring = static_cast<char *>(c->scratch);
    }

    if (hipEventRecord(c->ev_start, stream) != hipSuccess) return AR_ERR_RUNTIME;
    if (hipStreamWaitEvent(c->copy_stream, c->ev_start, 0) != hipSuccess) return AR_ERR_RUNTIME;

    const mpp::Family family = stream_family(plan);
    for (size_t ch = 0; ch < n_chunks; ++ch) {
        const size_t e0 = ch * chunk;
        const size_t len = std::min(chunk, n - e0);
        const unsigned slot = *slots.next % static_cast<unsigned>(K);
        *slots.next = (slot + 1) % static_cast<unsigned>(K);
        char *slot_base = ring + slot * slot_stride;

        if (slots.used[slot] && hipStreamWaitEvent(c->copy_stream, slots.free[slot], 0) != hipSuccess) {
            return AR_ERR_RUNTIME;
        }
        for (int r = 0; r < R; ++r) {
            if (srcs[r] == nullptr) continue;   // inactive rank: nothing crosses PCIe
            if (hipMemcpyAsync(slot_base + r * rank_stride, static_cast<const char *>(srcs[r]) + e0 * sb, len * sb,
                               hipMemcpyHostToDevice, c->copy_stream) != hipSuccess) {
                return AR_ERR_RUNTIME;
            }
        }
        if (hipEventRecord(slots.h2d[slot], c->copy_stream) != hipSuccess) return AR_ERR_RUNTIME;
        if (hipStreamWaitEvent(stream, slots.h2d[slot], 0) != hipSuccess) return AR_ERR_RUNTIME;

        mpp::KernelArgs a{};
        a.xcd_run_elems = xcd_run_for(c->cfg, R, false);
        a.R = R;
        a.n_dst = 1;
        a.n = len;
        a.store_nt = plan.store_nt;
        a.active = plan.active_mask;
        for (int r = 0; r < R; ++r) a.src[r] = srcs[r] == nullptr ? nullptr : slot_base + r * rank_stride;
        a.dst[0] = static_cast<char *>(dst[0]) + e0 * db;
        set_ranges_1d(a, res, n, e0, len, plan.dst_bytes);
        const mpp::LaunchShape shape = held(c, plan, mpp::plan_shape(family, types.src_is_wire, R, res.ptr != nullptr,
                                                       static_cast<unsigned>(len), 1, c->cu_count, c->cfg.grid_wgs));
        if (int rc = hip_status(mpp::launch(family, types, false, a, shape, stream))) return rc;
        if (hipEventRecord(slots.free[slot], stream) != hipSuccess) return AR_ERR_RUNTIME;
        slots.used[slot] = 1;
    }
    return AR_OK;
}

// HOST_STAGED for row-strided sources: the copy engine moves chunks of rows
// with 2-D copies (row pitch = the source stride), packing them into HBM
// scratch at a pitch of cols elements rounded up to 16 bytes (the kernels
// read every row start with 16-byte loads), then the add kernel reads the
// packed rows and writes the strided destination rows -- the same slot /
// event ring as the 1-D form.
int run_host_staged_rows(ar_ctx *c, const ar_plan &plan, void *const *dst, const void *const *srcs, int R,
                         const Rows &rw, int wire_type, const Residual &res, hipStream_t stream) {
    const size_t sb = static_cast<size_t>(plan.src_bytes);
    const size_t chunk_rows = plan.chunk_elems / rw.cols;
    const size_t K = static_cast<size_t>(c->cfg.host_slots);
    const size_t pitch_bytes = (rw.cols * sb + 15) / 16 * 16;   // packed row pitch
    const size_t rank_stride = chunk_rows * pitch_bytes;
    const size_t slot_stride = rank_stride * static_cast<size_t>(R);
    if (int rc = ensure_scratch(c, slot_stride * K)) return rc;

    if (hipEventRecord(c->ev_start, stream) != hipSuccess) return AR_ERR_RUNTIME;
    if (hipStreamWaitEvent(c->copy_stream, c->ev_start, 0) != hipSuccess) return AR_ERR_RUNTIME;

    for (size_t r0 = 0; r0 < rw.rows; r0 += chunk_rows) {
        const size_t nr = std::min(chunk_rows, rw.rows - r0);
        const unsigned slot = c->next_slot;
        c->next_slot = (c->next_slot + 1) % static_cast<unsigned>(K);
        char *slot_base = static_cast<char *>(c->scratch) + slot * slot_stride;
        if (c->slot_used[slot] && hipStreamWaitEvent(c->copy_stream, c->ev_free[slot], 0) != hipSuccess) {
            return AR_ERR_RUNTIME;
        }
        const void *packed[AR_MAX_RANKS];
        for (int r = 0; r < R; ++r) {
            packed[r] = nullptr;
            if (srcs[r] == nullptr) continue;   // inactive rank: nothing crosses PCIe
            if (hipMemcpy2DAsync(slot_base + r * rank_stride, pitch_bytes,
                                 static_cast<const char *>(srcs[r]) + r0 * rw.src_stride * sb, rw.src_stride * sb,
                                 rw.cols * sb, nr, hipMemcpyHostToDevice, c->copy_stream) != hipSuccess) {
                return AR_ERR_RUNTIME;
            }
            packed[r] = slot_base + r * rank_stride;
        }
        if (hipEventRecord(c->ev_h2d[slot], c->copy_stream) != hipSuccess) return AR_ERR_RUNTIME;
        if (hipStreamWaitEvent(stream, c->ev_h2d[slot], 0) != hipSuccess) return AR_ERR_RUNTIME;

        Rows part = rw;
        part.rows = nr;
        part.src_stride = pitch_bytes / sb;
        void *dst_part[AR_MAX_RANKS];
        for (int d = 0; d < plan.n_dst; ++d) {
            dst_part[d] = static_cast<char *>(dst[d]) + r0 * rw.dst_stride * static_cast<size_t>(plan.dst_bytes);
        }
        Residual res_part = res;
        if (res.ptr != nullptr) {
            res_part.ptr = static_cast<const char *>(res.ptr) + r0 * rw.res_stride * static_cast<size_t>(plan.dst_bytes);
        }
        ar_plan kernel_plan = plan;
        kernel_plan.mode = AR_MODE_CHUNKED;
        if (int rc = run_rows(c, kernel_plan, dst_part, packed, R, part, wire_type, res_part, stream)) return rc;
        if (hipEventRecord(c->ev_free[slot], stream) != hipSuccess) return AR_ERR_RUNTIME;
        c->slot_used[slot] = 1;
    }
    return AR_OK;
}

}  // namespace

AR_API const char *ar_status_str(int status) {
    switch (status) {
    case AR_OK: return "AR_OK";
    case AR_ERR_INVALID: return "AR_ERR_INVALID";
    case AR_ERR_UNSUPPORTED: return "AR_ERR_UNSUPPORTED";
    case AR_ERR_NOMEM: return "AR_ERR_NOMEM";
    case AR_ERR_RUNTIME: return "AR_ERR_RUNTIME";
    default: return "AR_ERR_UNKNOWN";
    }
}

AR_API int ar_plan_query(const ar_config *cfg, void *const *dst, const void *const *srcs, int R, size_t n,
                         ar_dtype dst_type, ar_dtype wire_type, unsigned mode, int srcs_on_host, ar_plan *plan) {
    Config c;
    if (int rc = resolve_config(cfg, &c)) return rc;
    return validate_and_plan(c, dst, srcs, R, n, dst_type, wire_type, mode, Residual{}, srcs_on_host != 0, plan);
}

AR_API int ar_plan_query_add(const ar_config *cfg, void *const *dst, const void *const *srcs, int R, size_t n,
                             ar_dtype dst_type, ar_dtype wire_type, unsigned mode, const void *residual, size_t residual_len,
                             int srcs_on_host, ar_plan *plan) {
    Config c;
    if (int rc = resolve_config(cfg, &c)) return rc;
    if (residual == nullptr) return AR_ERR_INVALID;
    Residual res;
    res.ptr = residual;
    res.len = residual_len;
    return validate_and_plan(c, dst, srcs, R, n, dst_type, wire_type, mode, res, srcs_on_host != 0, plan);
}

AR_API int ar_init(ar_ctx **out, int hip_device, const ar_config *cfg) {
    if (out == nullptr) return AR_ERR_INVALID;
    *out = nullptr;
    Config conf;
    if (int rc = resolve_config(cfg, &conf)) return rc;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess) {
        (void)hipGetLastError();
        return AR_ERR_RUNTIME;
    }
    if (hip_device < 0 || hip_device >= count) return AR_ERR_INVALID;

    // the kernels are built for gfx950 only: refuse another part up front
    // instead of failing at the first launch
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, hip_device) != hipSuccess) {
        (void)hipGetLastError();
        return AR_ERR_RUNTIME;
    }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return AR_ERR_UNSUPPORTED;

    DeviceGuard guard(hip_device);
    if (!guard.ok) return AR_ERR_RUNTIME;

    ar_ctx *c = new (std::nothrow) ar_ctx();
    if (c == nullptr) return AR_ERR_NOMEM;
    c->device = hip_device;
    c->cfg = conf;
    int rc = AR_OK;
    if (hipDeviceGetAttribute(&c->cu_count, hipDeviceAttributeMultiprocessorCount, hip_device) != hipSuccess ||
        c->cu_count <= 0) {
        rc = AR_ERR_RUNTIME;
    }
    // LDS per CU, for the two-rank kernels' occupancy hold (left at 0, no
    // hold, when the runtime does not report it)
    int lds_cu = 0;
    if (rc == AR_OK &&
        hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, hip_device) == hipSuccess &&
        lds_cu > 0) {
        c->lds_per_cu = static_cast<unsigned>(lds_cu);
    }
    if (rc == AR_OK && hipStreamCreateWithFlags(&c->copy_stream, hipStreamNonBlocking) != hipSuccess) {
        c->copy_stream = nullptr;
        rc = AR_ERR_RUNTIME;
    }
    if (rc == AR_OK && hipEventCreateWithFlags(&c->ev_start, hipEventDisableTiming) != hipSuccess) {
        c->ev_start = nullptr;
        rc = AR_ERR_RUNTIME;
    }
    // the static staging array's address on this device (the guard above made
    // it current); looked up once per device and shared by its contexts
    if (rc == AR_OK && mpp::static_scratch(hip_device, &c->static_scratch) != hipSuccess) {
        c->static_scratch = nullptr;
        rc = AR_ERR_RUNTIME;
    }
    if (rc == AR_OK && hipEventCreateWithFlags(&c->ev_static_h2d, hipEventDisableTiming) != hipSuccess) {
        c->ev_static_h2d = nullptr;
        rc = AR_ERR_RUNTIME;
    }
    if (rc == AR_OK && hipEventCreateWithFlags(&c->ev_static_free, hipEventDisableTiming) != hipSuccess) {
        c->ev_static_free = nullptr;
        rc = AR_ERR_RUNTIME;
    }
    if (rc == AR_OK) {
        const size_t K = static_cast<size_t>(conf.host_slots);
        c->ev_h2d.assign(K, nullptr);
        c->ev_free.assign(K, nullptr);
        c->slot_used.assign(K, 0);
        for (size_t s = 0; s < K && rc == AR_OK; ++s) {
            if (hipEventCreateWithFlags(&c->ev_h2d[s], hipEventDisableTiming) != hipSuccess) {
                c->ev_h2d[s] = nullptr;
                rc = AR_ERR_RUNTIME;
            } else if (hipEventCreateWithFlags(&c->ev_free[s], hipEventDisableTiming) != hipSuccess) {
                c->ev_free[s] = nullptr;
                rc = AR_ERR_RUNTIME;
            }
        }
    }
    if (rc != AR_OK) {
        (void)hipGetLastError();
        destroy(c);
        return rc;
    }
    *out = c;
    return AR_OK;
}

namespace {

// `static_staging`: ar_reduce_staged_static -- a host-staged call only, always
// through the copy engine, its ring in the static staging array.
int reduce_impl(ar_ctx *ctx, void *const *dst, const void *const *srcs, int R, size_t n, int dst_type,
                int wire_type, unsigned mode, const Residual &res, const Rows *rows, void *hip_stream,
                bool static_staging = false) {
    if (ctx == nullptr) return AR_ERR_INVALID;
    // cheap checks first, without touching the runtime
    ar_plan plan;
    const bool auto_mode = (mode & AR_MODE_MASK) == AR_MODE_AUTO;
    int rc = validate_and_plan(ctx->cfg, dst, srcs, R, n, dst_type, wire_type, mode, res, false, &plan, rows);
    if (rc != AR_OK) return rc;

    // bytes each tensor spans, for the memory-kind and range checks
    const size_t src_len = (rows ? extent(rows->rows, rows->cols, rows->src_stride) : n) *
                           static_cast<size_t>(plan.src_bytes);
    const size_t dst_len = (rows ? extent(rows->rows, rows->cols, rows->dst_stride) : n) *
                           static_cast<size_t>(plan.dst_bytes);
    size_t res_len = res.len;
    if (rows != nullptr) {
        res_len = rows->res_stride == 0 ? rows->cols : extent(rows->rows, rows->cols, rows->res_stride);
    }

    DeviceGuard guard(ctx->device);
    if (!guard.ok) return AR_ERR_RUNTIME;

    int first_active = -1;
    for (int r = 0; r < R && first_active < 0; ++r) {
        if (srcs[r] != nullptr) first_active = r;
    }
    if (n > 0 && first_active >= 0 && (auto_mode || plan.mode == AR_MODE_HOST_STAGED)) {
        // memory kinds decide AUTO between host-staged and device modes
        const Kind k0 = memory_kind(srcs[first_active], src_len, ctx->device);
        if (k0 == Kind::Other) return AR_ERR_INVALID;
        if (auto_mode && k0 == Kind::PinnedHost) {
            rc = validate_and_plan(ctx->cfg, dst, srcs, R, n, dst_type, wire_type, mode, res, true, &plan, rows);
            if (rc != AR_OK) return rc;
        }
    }
    if (n == 0) return AR_OK;
    if (static_staging) {
        if (plan.mode != AR_MODE_HOST_STAGED) return AR_ERR_INVALID;
        plan.host_direct = 0;
    }

    const Kind want_src = plan.mode == AR_MODE_HOST_STAGED ? Kind::PinnedHost : Kind::Device;
    const void *src_view[AR_MAX_RANKS];
    for (int r = 0; r < R; ++r) {
        src_view[r] = nullptr;
        if (srcs[r] == nullptr) continue;   // inactive rank (validated above)
        if (memory_kind(srcs[r], src_len, ctx->device, &src_view[r]) != want_src) return AR_ERR_INVALID;
    }
    for (int d = 0; d < plan.n_dst; ++d) {
        if (memory_kind(dst[d], dst_len, ctx->device) != Kind::Device) return AR_ERR_INVALID;
    }
    if (res.ptr != nullptr &&
        memory_kind(res.ptr, res_len * static_cast<size_t>(plan.dst_bytes), ctx->device) != Kind::Device) {
        return AR_ERR_INVALID;
    }

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (plan.mode == AR_MODE_HOST_STAGED && !plan.host_direct) {
        // the copy-engine pipeline synchronises when it grows its scratch ring and
        // chains events across its own stream and calls: it cannot be recorded
        // into a graph, so a call under stream capture is refused before anything
        // is enqueued (the direct path and every device schedule are capturable)
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
            (void)hipGetLastError();
            return AR_ERR_RUNTIME;
        }
        if (cs != hipStreamCaptureStatusNone) return AR_ERR_UNSUPPORTED;
    }
    if (rows != nullptr) {
        if (plan.mode != AR_MODE_HOST_STAGED) return run_rows(ctx, plan, dst, srcs, R, *rows, wire_type, res, stream);
        if (plan.host_direct) {
            ar_plan direct = plan;
            direct.mode = AR_MODE_CHUNKED;
            return run_rows(ctx, direct, dst, src_view, R, *rows, wire_type, res, stream);
        }
        return run_host_staged_rows(ctx, plan, dst, srcs, R, *rows, wire_type, res, stream);
    }
    if (plan.mode == AR_MODE_HOST_STAGED) {
        if (plan.host_direct) {
            // one streaming launch whose loads cross PCIe: the kernel reads the
            // pinned partials through their device mapping, no HBM staging
            ar_plan direct = plan;
            direct.mode = AR_MODE_CHUNKED;
            return run_device(ctx, direct, dst, src_view, R, n, wire_type, res, stream);
        }
        if (static_staging) {
            return run_host_staged(ctx, plan, dst, srcs, R, n, wire_type, res, stream, ctx->static_scratch,
                                   mpp::kStaticScratchBytes);
        }
        return run_host_staged(ctx, plan, dst, srcs, R, n, wire_type, res, stream);
    }
    return run_device(ctx, plan, dst, srcs, R, n, wire_type, res, stream);
}

}  // namespace

AR_API int ar_reduce(ar_ctx *ctx, void *const *dst, const void *const *srcs, int R, size_t n, ar_dtype dst_type,
                     ar_dtype wire_type, unsigned mode, void *hip_stream) {
    return reduce_impl(ctx, dst, srcs, R, n, dst_type, wire_type, mode, Residual{}, nullptr, hip_stream);
}

AR_API int ar_reduce_staged_static(ar_ctx *ctx, void *const *dst, const void *const *srcs, int R, size_t n,
                                   ar_dtype dst_type, ar_dtype wire_type, unsigned mode, void *hip_stream) {
    return reduce_impl(ctx, dst, srcs, R, n, dst_type, wire_type, mode, Residual{}, nullptr, hip_stream, true);
}

AR_API int ar_reduce_add(ar_ctx *ctx, void *const *dst, const void *const *srcs, int R, size_t n, ar_dtype dst_type,
                         ar_dtype wire_type, unsigned mode, const void *residual, size_t residual_len, void *hip_stream) {
    if (residual == nullptr) return AR_ERR_INVALID;
    Residual res;
    res.ptr = residual;
    res.len = residual_len;
    return reduce_impl(ctx, dst, srcs, R, n, dst_type, wire_type, mode, res, nullptr, hip_stream);
}

namespace {

// An ar_rows shape as the internal form, with n = rows x cols; false if the
// element count overflows.
bool rows_of(const ar_rows *shape, Rows *rw, size_t *n) {
    rw->rows = shape->rows;
    rw->cols = shape->cols;
    rw->src_stride = shape->src_stride;
    rw->dst_stride = shape->dst_stride;
    rw->res_stride = shape->res_stride;
    if (rw->cols != 0 && rw->rows > SIZE_MAX / rw->cols) return false;
    *n = rw->rows * rw->cols;
    // the furthest element any tensor reaches must stay addressable
    const size_t strides[3] = {rw->src_stride, rw->dst_stride, rw->res_stride};
    for (size_t st : strides) {
        if (rw->rows > 1 && st > (SIZE_MAX / 16) / rw->rows) return false;
    }
    return true;
}

}  // namespace

AR_API int ar_reduce_rows(ar_ctx *ctx, void *const *dst, const void *const *srcs, int R, const ar_rows *shape,
                          ar_dtype dst_type, ar_dtype wire_type, unsigned mode, const void *residual, void *hip_stream) {
    if (ctx == nullptr || shape == nullptr) return AR_ERR_INVALID;
    Rows rw;
    size_t n = 0;
    if (!rows_of(shape, &rw, &n)) return AR_ERR_INVALID;
    Residual res;
    res.ptr = residual;
    res.len = 0;
    return reduce_impl(ctx, dst, srcs, R, n, dst_type, wire_type, mode, res, &rw, hip_stream);
}

AR_API int ar_plan_query_rows(const ar_config *cfg, void *const *dst, const void *const *srcs, int R,
                              const ar_rows *shape, ar_dtype dst_type, ar_dtype wire_type, unsigned mode, const void *residual,
                              int srcs_on_host, ar_plan *plan) {
    Config c;
    if (int rc = resolve_config(cfg, &c)) return rc;
    if (shape == nullptr) return AR_ERR_INVALID;
    Rows rw;
    size_t n = 0;
    if (!rows_of(shape, &rw, &n)) return AR_ERR_INVALID;
    Residual res;
    res.ptr = residual;
    return validate_and_plan(c, dst, srcs, R, n, dst_type, wire_type, mode, res, srcs_on_host != 0, plan, &rw);
}

AR_API int ar_free(ar_ctx *ctx) {
    if (ctx == nullptr) return AR_OK;
    DeviceGuard guard(ctx->device);
    destroy(ctx);
    return AR_OK;
}
