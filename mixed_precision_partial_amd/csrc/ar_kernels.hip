// ar_kernels.hip -- gfx950 kernels of the mixed-precision partial-sum reduce.
//
// Every kernel computes, for each element i of its range and every
// destination d:
//     acc = wire(src_0[i]); acc = acc + wire(src_r[i]) for r = 1 .. R-1
//     dst_d[i] = acc
// where wire(x) rounds a binary32 partial to the wire type (RNE) and widens it
// back exactly, or just widens when the source already holds the wire type.
// The fold runs in rank order with one binary32 rounding per add ("Hexagon
// allreduce-ops.c" page, allreduce_thread_dma_1d: s0 + s1, then + s2 ...), and
// the local partial is rounded like the peers' ("CUDA allreduce.cu" page,
// "Chunked kernel AllReduce" comment block, phase 3).
//
// The path is a stream over HBM with at most 0.1 flop per byte, so nothing
// here is a contraction and nothing uses MFMA.  What matters is keeping
// enough 16-byte loads in flight per CU and writing whole cache lines:
//   * A wave owns a "wave tile" of 512 elements: 64 lanes x 8 elements.
//     binary32 sources are read as two dwordx4 loads per lane, each covering
//     1 KiB contiguous per wave instruction; 16-bit sources are one dwordx4 per
//     lane (8 consecutive elements).
//   * The single-shot kernel gives each wave one tile and exits: the decode
//     case is bound by launch latency, so it issues every load of the tile at
//     once and keeps the grid just large enough.
//   * The streaming kernel keeps waves resident and walks batches of U tiles,
//     issuing all R x U x 16 B loads of a batch before the first add so that
//     many independent loads are in flight per lane.
//   * The rank count is a template bucket (2, 4, 8, 16) with the real R tested
//     against compile-time rank indices, so every kernarg access uses a
//     constant offset (no private-memory copies) and all loads of a batch can
//     issue back to back.
#include "ar_internal.h"

namespace mpp {
namespace {

constexpr int kWave = 64;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float f32_from_bits(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t bits_from_f32(float f) { return __builtin_bit_cast(uint32_t, f); }

template <bool NT>
__device__ __forceinline__ u32x4 load16(const void *p) {
    if constexpr (NT) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    } else {
        return *reinterpret_cast<const u32x4 *>(p);
    }
}

template <bool NT>
__device__ __forceinline__ void store16(float *p, float a, float b, float c, float d) {
    const u32x4 v = {bits_from_f32(a), bits_from_f32(b), bits_from_f32(c), bits_from_f32(d)};
    if constexpr (NT) {
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
    } else {
        *reinterpret_cast<u32x4 *>(p) = v;
    }
}

// round_W then widen, two binary32 values at a time (the conversions on
// gfx950 are packed: v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 round to nearest
// even under the default mode, keep subnormals and map NaN to NaN).
template <int W>
__device__ __forceinline__ void wire_pair(float &x, float &y) {
    if constexpr (W == AR_BF16) {
        const bf16x2 p = __builtin_convertvector((f32x2){x, y}, bf16x2);
        const uint32_t w = __builtin_bit_cast(uint32_t, p);
        x = f32_from_bits(w << 16);
        y = f32_from_bits(w & 0xFFFF0000u);
    } else if constexpr (W == AR_F16) {
        const f16x2 p = __builtin_convertvector((f32x2){x, y}, f16x2);
        x = static_cast<float>(p.x);
        y = static_cast<float>(p.y);
    }
}

// Widen a pair of 16-bit wire values packed in one dword (element 2k in the
// low half, 2k+1 in the high half).
template <int W>
__device__ __forceinline__ void widen_pair(uint32_t w, float &x, float &y) {
    if constexpr (W == AR_BF16) {
        x = f32_from_bits(w << 16);
        y = f32_from_bits(w & 0xFFFF0000u);
    } else {
        const f16x2 p = __builtin_bit_cast(f16x2, w);
        x = static_cast<float>(p.x);
        y = static_cast<float>(p.y);
    }
}

// One element, scalar path (range remainders).
template <int W, bool SW>
__device__ __forceinline__ float wire_one(const void *src, size_t i) {
    if constexpr (SW) {
        const uint32_t h = reinterpret_cast<const uint16_t *>(src)[i];
        float x, y;
        widen_pair<W>(h, x, y);
        return x;
    } else {
        float x = reinterpret_cast<const float *>(src)[i];
        float y = 0.0f;
        wire_pair<W>(x, y);
        return x;
    }
}

// ---------------------------------------------------------------------------
// Lane layout of one wave tile (512 elements starting at element `t`):
//   binary32 sources / all destinations of binary32 sources:
//       part j in {0,1}: elements t + 256 j + 4 lane + {0..3}
//   16-bit sources: elements t + 8 lane + {0..7} (one dwordx4)
//       destinations: t + 8 lane + 4 j + {0..3}
// ---------------------------------------------------------------------------
template <bool SW>
struct Tile {
    static constexpr int kRaw = SW ? 1 : 2;   // dwordx4 loads per lane per source
};

template <int W, bool SW, bool NT>
__device__ __forceinline__ void tile_load(const void *src, size_t t, int lane, u32x4 (&raw)[Tile<SW>::kRaw]) {
    if constexpr (SW) {
        raw[0] = load16<NT>(reinterpret_cast<const uint16_t *>(src) + t + 8 * lane);
    } else {
        const float *s = reinterpret_cast<const float *>(src) + t + 4 * lane;
        raw[0] = load16<NT>(s);
        raw[1] = load16<NT>(s + 256);
    }
}

template <int W, bool SW>
__device__ __forceinline__ void tile_values(const u32x4 (&raw)[Tile<SW>::kRaw], float (&v)[8]) {
    if constexpr (SW) {
#pragma unroll
        for (int k = 0; k < 4; ++k) widen_pair<W>(raw[0][k], v[2 * k], v[2 * k + 1]);
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int k = 0; k < 4; k += 2) {
                float x = f32_from_bits(raw[j][k]);
                float y = f32_from_bits(raw[j][k + 1]);
                wire_pair<W>(x, y);
                v[4 * j + k] = x;
                v[4 * j + k + 1] = y;
            }
        }
    }
}

template <bool SW, bool NT>
__device__ __forceinline__ void tile_store_as(float *dst, size_t t, int lane, const float (&acc)[8]) {
    if constexpr (SW) {
        float *p = dst + t + 8 * lane;
        store16<NT>(p, acc[0], acc[1], acc[2], acc[3]);
        store16<NT>(p + 4, acc[4], acc[5], acc[6], acc[7]);
    } else {
        float *p = dst + t + 4 * lane;
        store16<NT>(p, acc[0], acc[1], acc[2], acc[3]);
        store16<NT>(p + 256, acc[4], acc[5], acc[6], acc[7]);
    }
}



// Rank r takes part with a partial (bit r of the launch's mask); an inactive
// rank's partial is +0.0 everywhere: nothing is loaded and +0.0 is added in
// its place, which keeps -0 + inactive == +0 like a zeroed shard.
// MASKED = false is the common case (every rank active): the test folds away
// and the loads of a batch stay one straight-line sequence.  The host picks
// the masked kernel instance only when some rank is inactive: per-rank
// branches around loads make the compiler drain each rank's loads before
// issuing the next, so the common case must not carry them.
template <bool MASKED>
__device__ __forceinline__ bool rank_active(const KernelArgs &a, int r) {
    if constexpr (MASKED) {
        return (a.active >> r) & 1u;
    } else {
        return true;
    }
}


// Issue every load of a batch of U consecutive wave tiles starting at
// element `t` (slice offset included) for the first R of RB sources, tile by
// tile: the loads of tile 0 are the oldest in flight, so tile 0 can be folded
// and stored while the later tiles' loads are still arriving.
template <int W, bool SW, int RB, int U, bool NT, bool MASKED>
__device__ __forceinline__ void load_batch(const KernelArgs &a, size_t t, int lane,
                                           u32x4 (&raw)[RB][U][Tile<SW>::kRaw]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if ((r < 2 || r < a.R) && rank_active<MASKED>(a, r)) {
                tile_load<W, SW, NT>(a.src[r], t + u * kWaveTile, lane, raw[r][u]);
            }
        }
        // keep tile order: the scheduler must not hoist a later tile's loads
        // above this one's
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Fold each tile of the batch in rank order and store it to every
// destination before the next tile is folded.  Loads use NT; stores use ST
// (non-temporal for calls that write at least as much as they read,
// ordinary write-back stores otherwise, which drain from L2 / Infinity Cache
// while the next kernel reads).  The store policy is a template parameter:
// two stores that differ only in their cache hint would be merged into one
// by the compiler.
template <int W, bool SW, int RB, int U, bool NT, bool ST, bool MASKED>
__device__ __forceinline__ void fold_store(const KernelArgs &a, size_t t, int lane,
                                           const u32x4 (&raw)[RB][U][Tile<SW>::kRaw]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float acc[8];
        if (rank_active<MASKED>(a, 0)) {
            tile_values<W, SW>(raw[0][u], acc);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
        }
#pragma unroll
        for (int r = 1; r < RB; ++r) {
            if (r < 2 || r < a.R) {
                float w[8];
                if (rank_active<MASKED>(a, r)) {
                    tile_values<W, SW>(raw[r][u], w);
                } else {
#pragma unroll
                    for (int k = 0; k < 8; ++k) w[k] = 0.0f;
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] = acc[k] + w[k];
            }
        }
#pragma unroll
        for (int d = 0; d < RB; ++d) {
            if (d < a.n_dst) tile_store_as<SW, ST>(a.dst[d], t + u * kWaveTile, lane, acc);
        }
    }
}

template <int W, bool SW, int RB, int U, bool NT, bool ST, bool MASKED>
__device__ __forceinline__ void reduce_tiles(const KernelArgs &a, size_t t, int lane) {
    u32x4 raw[RB][U][Tile<SW>::kRaw];
    load_batch<W, SW, RB, U, NT, MASKED>(a, t, lane, raw);
    fold_store<W, SW, RB, U, NT, ST, MASKED>(a, t, lane, raw);
}

// Elements [begin, end) of the launch, one per lane per step (end - begin is
// below one wave tile, so this is at most 8 steps).
template <int W, bool SW, int RB>
__device__ __forceinline__ void reduce_scalar(const KernelArgs &a, size_t begin, size_t end, int lane) {
    for (size_t e = begin + lane; e < end; e += kWave) {
        float acc = rank_active<true>(a, 0) ? wire_one<W, SW>(a.src[0], e) : 0.0f;
#pragma unroll
        for (int r = 1; r < RB; ++r) {
            if (r < 2 || r < a.R) acc = acc + (rank_active<true>(a, r) ? wire_one<W, SW>(a.src[r], e) : 0.0f);
        }
#pragma unroll
        for (int d = 0; d < RB; ++d) {
            if (d < a.n_dst) a.dst[d][e] = acc;
        }
    }
}

// The element range [off, off + len) of this workgroup's gridDim.y index.
// Both forms only read launch arguments at fixed offsets (the slice form
// indexes with blockIdx.y, which is known at wave start), so a wave fetches
// everything it needs in one batch of scalar loads.
template <bool SLICED>
__device__ __forceinline__ void range_of(const KernelArgs &a, size_t &off, unsigned &len) {
    const unsigned y = blockIdx.y;
    if constexpr (SLICED) {
        off = a.slice_start[y];
        len = a.slice_len[y];
    } else {
        const unsigned start = y * a.chunk_elems;
        const unsigned left = a.n - start;
        off = start;
        len = left < a.chunk_elems ? left : a.chunk_elems;
    }
}

// Whole wave tiles after the batched part, then the element remainder on
// wave 0 of workgroup 0 of the range.
template <int W, bool SW, int RB, int U, bool NT, bool ST, bool MASKED>
__device__ __forceinline__ void reduce_rest(const KernelArgs &a, size_t off, unsigned len, unsigned done,
                                            unsigned gw, unsigned nw, int lane) {
    if constexpr (U > 1) {
        const unsigned n_one = (len - done) / kWaveTile;
        for (unsigned t = gw; t < n_one; t += nw) {
            reduce_tiles<W, SW, RB, 1, NT, ST, MASKED>(a, off + done + (size_t)t * kWaveTile, lane);
        }
    }
    const unsigned vec_end = (len / kWaveTile) * kWaveTile;
    if (vec_end < len && gw == 0) {
        reduce_scalar<W, SW, RB>(a, off + vec_end, off + len, lane);
    }
}

// Walk the wave tiles of this workgroup's range: batches of U tiles strided
// over the `a.waves` waves of the range, then the remainder.  BLOCK is the
// workgroup size the kernel is always launched with (no read of blockDim).
template <int W, bool SW, int RB, int U, bool NT, bool ST, int BLOCK, bool SLICED, bool MASKED>
__device__ __forceinline__ void reduce_range(const KernelArgs &a) {
    constexpr unsigned wpb = BLOCK / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const unsigned gw = blockIdx.x * wpb + threadIdx.x / kWave;
    const unsigned nw = a.waves;
    size_t off;
    unsigned len;
    range_of<SLICED>(a, off, len);

    constexpr unsigned big = kWaveTile * U;
    const unsigned n_big = len / big;
    for (unsigned t = gw; t < n_big; t += nw) {
        reduce_tiles<W, SW, RB, U, NT, ST, MASKED>(a, off + (size_t)t * big, lane);
    }
    reduce_rest<W, SW, RB, U, NT, ST, MASKED>(a, off, len, n_big * big, gw, nw, lane);
}



constexpr int kSingleShotBlock = 64;
constexpr int kStreamBlock = 256;
constexpr int kLdsBlock = 64;

template <int W, bool SW, int RB>
__global__ __launch_bounds__(kSingleShotBlock) void k_single_shot(KernelArgs a) {
    reduce_range<W, SW, RB, 1, false, false, kSingleShotBlock, false, false>(a);
}

template <int W, bool SW, int RB>
__global__ __launch_bounds__(kSingleShotBlock) void k_single_shot_m(KernelArgs a) {
    reduce_range<W, SW, RB, 1, false, false, kSingleShotBlock, false, true>(a);
}

// Streaming-kernel tuning (compile-time; measured on MI355X):
//   MPP_STREAM_LOADS  target dwordx4 loads per lane per batch (R x U x K)
//   MPP_STREAM_MAXU   cap on tiles per batch
//   MPP_STREAM_NT     1: non-temporal loads (streaming, no reuse); the store
//                     policy is a launch argument
//   MPP_STREAM_WG_PER_CU  0: one-shot grid (one batch per wave, the hardware
//                     back-fills CUs as waves retire); k > 0: persistent grid
//                     of k workgroups per CU
#ifndef MPP_STREAM_LOADS
#define MPP_STREAM_LOADS 8
#endif
#ifndef MPP_STREAM_MAXU
#define MPP_STREAM_MAXU 4
#endif
#ifndef MPP_STREAM_NT
#define MPP_STREAM_NT 1
#endif
#ifndef MPP_STREAM_WG_PER_CU
#define MPP_STREAM_WG_PER_CU 0u
#endif

// Tiles per batch of the streaming kernel: about MPP_STREAM_LOADS dwordx4
// loads per lane (R x U x loads-per-tile), at least 1 and at most MAXU tiles.
constexpr int stream_batch(bool src_is_wire, int rank_bucket) {
    const int per_tile = (src_is_wire ? 1 : 2) * rank_bucket;
    const int u = MPP_STREAM_LOADS / per_tile;
    return u < 1 ? 1 : (u > MPP_STREAM_MAXU ? MPP_STREAM_MAXU : u);
}

// Register-staged streaming kernel: ST = non-temporal stores, SLICED = the
// per-rank slice ranges of the broadcast schedule, M = some rank inactive.
#define MPP_STREAM_REG(NAME, ST, SLICED, M)                                                         \
    template <int W, bool SW, int RB>                                                             \
    __global__ __launch_bounds__(kStreamBlock) void NAME(KernelArgs a) {                          \
        reduce_range<W, SW, RB, stream_batch(SW, RB), MPP_STREAM_NT != 0, ST, kStreamBlock, SLICED, M>(a); \
    }
MPP_STREAM_REG(k_stream_reg, false, false, false)
MPP_STREAM_REG(k_stream_reg_nts, true, false, false)
MPP_STREAM_REG(k_stream_reg_sl, false, true, false)
MPP_STREAM_REG(k_stream_reg_nts_sl, true, true, false)
MPP_STREAM_REG(k_stream_reg_m, false, false, true)
MPP_STREAM_REG(k_stream_reg_nts_m, true, false, true)
MPP_STREAM_REG(k_stream_reg_sl_m, false, true, true)
MPP_STREAM_REG(k_stream_reg_nts_sl_m, true, true, true)
#undef MPP_STREAM_REG

// ---------------------------------------------------------------------------
// LDS-staged streaming kernel (one wave per workgroup).  Each wave owns two
// LDS stages of R x U x K blocks of 1 KiB.  global_load_lds_dwordx4 writes a
// lane's 16 B straight into the stage (no VGPRs held while the load is in
// flight); while the wave folds and stores the batch in one stage, the loads
// of its next batch stream into the other.  A lane only ever reads back the
// 16 B it loaded itself, so the stages need no barrier, only the wait on the
// wave's own vector-memory counter.
// ---------------------------------------------------------------------------
#ifndef MPP_LDS_U
#define MPP_LDS_U 1
#endif
#ifndef MPP_LDS_WG_PER_CU
#define MPP_LDS_WG_PER_CU 32u
#endif

// Tiles per stage: MPP_LDS_U, reduced so one stage is at most 32 loads per
// lane (the stage wait uses the 6-bit vector-memory counter).
constexpr int lds_batch(bool src_is_wire, int rank_bucket) {
    const int per_tile = (src_is_wire ? 1 : 2) * rank_bucket;
    const int cap = 32 / per_tile;
    const int u = MPP_LDS_U;
    return u < 1 ? 1 : (u > cap ? (cap < 1 ? 1 : cap) : u);
}

template <int W, bool SW, int RB, int U>
struct LdsStage {
    static constexpr int kBlocks = RB * U * Tile<SW>::kRaw;   // 1 KiB each
};

typedef __attribute__((address_space(3))) void lds_void;

template <int W, bool SW, int RB, int U, bool MASKED>
__device__ __forceinline__ void lds_issue(const KernelArgs &a, size_t t, int lane, u32x4 (*stage)[kWave]) {
    constexpr int K = Tile<SW>::kRaw;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        if ((r < 2 || r < a.R) && rank_active<MASKED>(a, r)) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    const size_t e = SW ? t + u * kWaveTile + 8 * lane : t + u * kWaveTile + 256 * j + 4 * lane;
                    const char *g = static_cast<const char *>(a.src[r]) + e * (SW ? 2 : 4);
                    __builtin_amdgcn_global_load_lds(g, (lds_void *)(&stage[(r * U + u) * K + j][0]),
                                                     16, 0, 0);
                }
            }
        }
    }
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit counter");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The loads of a stage are the oldest `L + (later loads)` in flight when the
// next stage's L loads have just been issued: vector-memory loads retire in
// order, so vmcnt(L) means every load of the older stage has landed in LDS.
// L = R x U x K is only known at run time, hence the table of immediates.
template <int MaxL>
__device__ __forceinline__ void wait_stage(int L) {
    if constexpr (MaxL >= 0) {
        if (L == MaxL) {
            wait_vm<MaxL>();
            return;
        }
        wait_stage<MaxL - 1>(L);
    } else {
        wait_vm<0>();
    }
}

// 16 B read of LDS at byte address `addr`, completed before it returns.  The
// read is opaque to the compiler on purpose: its own wait insertion would
// otherwise drain every outstanding LDS load (both stages) before any read.
__device__ __forceinline__ u32x4 lds_read16(unsigned addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr));
    return v;
}

template <int W, bool SW, int RB, int U, bool ST, bool MASKED>
__device__ __forceinline__ void lds_consume(const KernelArgs &a, size_t t, int lane, u32x4 (*stage)[kWave]) {
    constexpr int K = Tile<SW>::kRaw;
    const unsigned base = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_void *)(&stage[0][lane])));
    u32x4 raw[RB][U][K];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        if ((r < 2 || r < a.R) && rank_active<MASKED>(a, r)) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < K; ++j) raw[r][u][j] = lds_read16(base + ((r * U + u) * K + j) * kWave * 16);
        }
    }
    fold_store<W, SW, RB, U, true, ST, MASKED>(a, t, lane, raw);
}

template <int W, bool SW, int RB, bool ST, bool SLICED, bool MASKED>
__device__ __forceinline__ void stream_lds_as(const KernelArgs &a, u32x4 (*stage0)[kWave], u32x4 (*stage1)[kWave]) {
    constexpr int U = lds_batch(SW, RB);
    const int lane = threadIdx.x;
    const unsigned gw = blockIdx.x;
    const unsigned nw = a.waves;
    size_t off;
    unsigned len;
    range_of<SLICED>(a, off, len);
    constexpr unsigned big = kWaveTile * U;
    const unsigned n_big = len / big;

    // loads per stage (vector-memory instructions): active ranks x U x K
    const unsigned ranks_mask = (a.R < RB ? a.R : RB) >= 32 ? ~0u : ((1u << (a.R < RB ? a.R : RB)) - 1u);
    const int L = __builtin_popcount(a.active & ranks_mask) * U * Tile<SW>::kRaw;
    constexpr int kMaxL = RB * U * Tile<SW>::kRaw;

    unsigned t = gw;
    if (t < n_big) lds_issue<W, SW, RB, U, MASKED>(a, off + (size_t)t * big, lane, stage0);
    while (t < n_big) {
        const unsigned t1 = t + nw;
        if (t1 < n_big) {
            lds_issue<W, SW, RB, U, MASKED>(a, off + (size_t)t1 * big, lane, stage1);
            wait_stage<kMaxL>(L);
        } else {
            wait_vm<0>();
        }
        lds_consume<W, SW, RB, U, ST, MASKED>(a, off + (size_t)t * big, lane, stage0);
        if (t1 >= n_big) break;
        const unsigned t2 = t1 + nw;
        if (t2 < n_big) {
            lds_issue<W, SW, RB, U, MASKED>(a, off + (size_t)t2 * big, lane, stage0);
            wait_stage<kMaxL>(L);
        } else {
            wait_vm<0>();
        }
        lds_consume<W, SW, RB, U, ST, MASKED>(a, off + (size_t)t1 * big, lane, stage1);
        t = t2;
    }
    reduce_rest<W, SW, RB, U, true, ST, MASKED>(a, off, len, n_big * big, gw, nw, lane);
}

template <int W, bool SW, int RB, bool ST, bool SLICED, bool MASKED>
__device__ __forceinline__ void stream_lds(const KernelArgs &a) {
    constexpr int NB = LdsStage<W, SW, RB, lds_batch(SW, RB)>::kBlocks;
    __shared__ u32x4 stage0[NB][kWave];
    __shared__ u32x4 stage1[NB][kWave];
    stream_lds_as<W, SW, RB, ST, SLICED, MASKED>(a, stage0, stage1);
}

#define MPP_STREAM_LDS(NAME, ST, SLICED, M)                                  \
    template <int W, bool SW, int RB>                                      \
    __global__ __launch_bounds__(kLdsBlock) void NAME(KernelArgs a) {      \
        stream_lds<W, SW, RB, ST, SLICED, M>(a);                           \
    }
MPP_STREAM_LDS(k_stream_lds, false, false, false)
MPP_STREAM_LDS(k_stream_lds_nts, true, false, false)
MPP_STREAM_LDS(k_stream_lds_sl, false, true, false)
MPP_STREAM_LDS(k_stream_lds_nts_sl, true, true, false)
MPP_STREAM_LDS(k_stream_lds_m, false, false, true)
MPP_STREAM_LDS(k_stream_lds_nts_m, true, false, true)
MPP_STREAM_LDS(k_stream_lds_sl_m, false, true, true)
MPP_STREAM_LDS(k_stream_lds_nts_sl_m, true, true, true)
#undef MPP_STREAM_LDS

// ---------------------------------------------------------------------------
// Dispatch tables.  Combination index: 0 (f32 wire, f32 src), 1 (bf16 wire,
// f32 src), 2 (f16 wire, f32 src), 3 (bf16 wire, bf16 src), 4 (f16 wire,
// f16 src).  Rank bucket index: 0 -> R <= 2, 1 -> <= 4, 2 -> <= 8, 3 -> <= 16.
// ---------------------------------------------------------------------------
#define MPP_ROW(KERNEL, W, SW) \
    {reinterpret_cast<const void *>(&KERNEL<W, SW, 2>), reinterpret_cast<const void *>(&KERNEL<W, SW, 4>), \
     reinterpret_cast<const void *>(&KERNEL<W, SW, 8>), reinterpret_cast<const void *>(&KERNEL<W, SW, 16>)}

#define MPP_TABLE(KERNEL)                                                                          \
    {MPP_ROW(KERNEL, AR_F32, false), MPP_ROW(KERNEL, AR_BF16, false), MPP_ROW(KERNEL, AR_F16, false), \
     MPP_ROW(KERNEL, AR_BF16, true), MPP_ROW(KERNEL, AR_F16, true)}

// [masked][combination][rank bucket]
const void *const kSingleShot[2][5][4] = {MPP_TABLE(k_single_shot), MPP_TABLE(k_single_shot_m)};
// [masked][store_nt][sliced][combination][rank bucket]
const void *const kStreamReg[2][2][2][5][4] = {
    {{MPP_TABLE(k_stream_reg), MPP_TABLE(k_stream_reg_sl)},
     {MPP_TABLE(k_stream_reg_nts), MPP_TABLE(k_stream_reg_nts_sl)}},
    {{MPP_TABLE(k_stream_reg_m), MPP_TABLE(k_stream_reg_sl_m)},
     {MPP_TABLE(k_stream_reg_nts_m), MPP_TABLE(k_stream_reg_nts_sl_m)}}};
const void *const kStreamLds[2][2][2][5][4] = {
    {{MPP_TABLE(k_stream_lds), MPP_TABLE(k_stream_lds_sl)},
     {MPP_TABLE(k_stream_lds_nts), MPP_TABLE(k_stream_lds_nts_sl)}},
    {{MPP_TABLE(k_stream_lds_m), MPP_TABLE(k_stream_lds_sl_m)},
     {MPP_TABLE(k_stream_lds_nts_m), MPP_TABLE(k_stream_lds_nts_sl_m)}}};

int combo_index(int wire, bool src_is_wire) {
    if (wire == AR_F32) return 0;
    if (!src_is_wire) return wire == AR_BF16 ? 1 : 2;
    return wire == AR_BF16 ? 3 : 4;
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

}  // namespace

unsigned stream_tile_elems(Family family, bool src_is_wire, int R) {
    return kWaveTile * batch_tiles(family, src_is_wire, R);
}

LaunchShape plan_shape(Family family, int wire, bool src_is_wire, int R, unsigned max_slice_len,
                       unsigned n_slices, int cu_count, int grid_override) {
    (void)wire;
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
    s.block = family == Family::StreamLds ? kLdsBlock : kStreamBlock;
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

hipError_t launch(Family family, int wire, bool src_is_wire, bool sliced, KernelArgs a,
                  const LaunchShape &shape, hipStream_t stream) {
    const int c = combo_index(wire, src_is_wire);
    const int b = bucket_index(a.R);
    const int nt = a.store_nt ? 1 : 0;
    const int sl = sliced ? 1 : 0;
    const unsigned full = a.R >= 32 ? ~0u : ((1u << a.R) - 1u);
    const int m = (a.active & full) == full ? 0 : 1;   // some rank inactive
    const void *fn = nullptr;
    switch (family) {
    case Family::SingleShot:
        if (sliced) return hipErrorNotSupported;
        fn = kSingleShot[m][c][b];
        break;
    case Family::StreamReg: fn = kStreamReg[m][nt][sl][c][b]; break;
    case Family::StreamLds: fn = kStreamLds[m][nt][sl][c][b]; break;
    default: return hipErrorNotSupported;
    }
    if (shape.block % kWave != 0) return hipErrorInvalidValue;
    a.waves = shape.grid_x * (shape.block / kWave);
    void *kargs[] = {&a};
    return hipLaunchKernel(fn, dim3(shape.grid_x, shape.grid_y, 1), dim3(shape.block, 1, 1), kargs,
                           shape.lds_bytes, stream);
}

}  // namespace mpp
