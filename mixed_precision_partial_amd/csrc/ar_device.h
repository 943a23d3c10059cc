// ar_device.h -- gfx950 device code of the mixed-precision partial-sum reduce
// (templates only; the ar_k_*.hip files instantiate them into kernel tables).
//
// Every kernel computes, for each element i of its range and every
// destination d:
//     acc = wire(src_0[i]); acc = RN_D(acc + wire(src_r[i])) for r = 1 .. R-1
//     acc = RN_D(acc + res[i])         (with a residual only)
//     dst_d[i] = acc
// where wire(x) rounds a binary32 partial to the wire type (RNE) and widens it
// back exactly, or just widens when the source already holds the wire type,
// and RN_D is one rounding to the destination type (binary32, or binary16 /
// bfloat16 when destination, wire and sources share that type).
//   * The fold runs in rank order with one rounding per add ("Hexagon
//     allreduce-ops.c" page, allreduce_thread_dma_1d: s0 + s1, then + s2 ...),
//     and the local partial is rounded like the peers' ("CUDA allreduce.cu"
//     page, "Chunked kernel AllReduce" comment block, phase 3).
//   * The residual is added after the last rank, element-wise or as one row
//     broadcast to every row (Hexagon page, the HAS_ADD / IS_ROW_BCAST forms),
//     in the destination type, never rounded through the wire.
//   * Narrow destinations accumulate in their own type (CUDA page, the half /
//     nv_bfloat16 chunked-kernel instances; Hexagon page, the f16 instances):
//     the add is done in binary32 and rounded once to the 16-bit type, which
//     is the correctly rounded 16-bit add (binary32 has >= 2p + 2 bits).
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
//   * The streaming kernel gives each wave a batch of U tiles, issuing all
//     R x U x 16 B loads of the batch before the first add so that many
//     independent loads are in flight per lane.
//   * The rank count is a template bucket (2, 4, 8, 16) with the real R tested
//     against compile-time rank indices, so every kernarg access uses a
//     constant offset (no private-memory copies) and all loads of a batch can
//     issue back to back.
#pragma once

#include "ar_internal.h"

namespace mpp {
namespace {

constexpr int kWave = 64;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Compile-time description of one kernel instance.
//   W      wire type (ar_dtype)
//   SW     sources already hold the wire type (16-bit loads)
//   DN     narrow destination: destination type == W (16-bit stores); implies SW
//   RB     rank bucket: the kernel handles R <= RB
//   MASKED some rank may be inactive (bit r of LaunchArgs::active clear)
//   RES    a residual is added after the fold
template <int W_, bool SW_, bool DN_, int RB_, bool MASKED_, bool RES_>
struct Cfg {
    static constexpr int W = W_;
    static constexpr bool SW = SW_;
    static constexpr bool DN = DN_;
    static constexpr int RB = RB_;
    static constexpr bool MASKED = MASKED_;
    static constexpr bool RES = RES_;
    static_assert(!DN || (SW && W != AR_F32), "a narrow destination has 16-bit sources of its own type");
    static constexpr int kSrcRaw = SW ? 1 : 2;   // dwordx4 loads per lane per source per tile
    static constexpr int kResRaw = DN ? 1 : 2;   // dwordx4 loads per lane of the residual per tile
    static constexpr int kDstBytes = DN ? 2 : 4;
};

// Bit casts take their operand by value.  With this compiler (AMD clang 22,
// ROCm 7.2), __builtin_bit_cast applied directly to a vector subscript such as
// `v[q]` reads element 0 whatever q is; passing the element through a scalar
// parameter first, as these helpers do, gives the intended element.
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

// Destination store policies (a template value along the store path):
//   kStoreKeep   through the caches: device-scope write-through (sc1) for
//                binary32 sources, whose store instructions each write 1 KiB
//                of whole lines; write-back for the 16-bit layouts.  Measured
//                on MI355X, write-through beats write-back for read-dominated
//                calls (prefill reduce 16.2 against 16.8 us, R = 8 fp32
//                partials 368 against 383 us): with write-back the dirty lines
//                wait in L2 and the end-of-kernel writeback of up to the whole
//                L2 runs after the last wave, a 3 us gap before the next
//                kernel; with write-through that traffic overlaps the reads.
//                16-bit sources into binary32 store half lines per
//                instruction, which write-back merges in L2 (write-through
//                doubled their time), and 16-bit destinations measured no
//                gain.  The single-shot kernel keeps its stores too: a decode
//                call then leaves no dirty lines for the end-of-kernel release
//                (R = 2 x 4096 replayed from a graph: 1.61 against 1.75 us).
//   kStoreStream non-temporal stores (calls that write as much as they read).
constexpr int kStoreKeep = 0;
constexpr int kStoreStream = 1;

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Third dword of a raw buffer resource on gfx9-family parts (untyped 32-bit
// data, no swizzle, no thread-id addressing).
constexpr int kRsrcWord3 = 0x00020000;

// 16-byte store with the device-scope write-through cache policy (sc1): a
// buffer store, which the compiler schedules and tracks like any other store,
// through a resource whose base is the wave-uniform start of the stored span
// (`span_bytes` long) and a per-lane byte offset inside it.
__device__ __forceinline__ void store16_wt(void *base, int span_bytes, unsigned off, u32x4 v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, span_bytes, kRsrcWord3);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, static_cast<int>(off), 0, 16);
}

// 16-byte store: SP 0 write-back, 1 non-temporal.
template <int SP>
__device__ __forceinline__ void store16(void *p, u32x4 v) {
    if constexpr (SP == 1) {
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
    } else {
        *reinterpret_cast<u32x4 *>(p) = v;
    }
}

// Round two binary32 values to the 16-bit type W (round to nearest even,
// subnormals kept, NaN stays NaN: gfx950's v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32 under the default mode) and return them packed, x in the
// low half.
template <int W>
__device__ __forceinline__ uint32_t round_pack(float x, float y) {
    if constexpr (W == AR_BF16) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, bf16x2));
    } else {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x, y}, f16x2));
    }
}

// Widen a pair of 16-bit values packed in one dword (element 2k in the low
// half, 2k+1 in the high half); exact.
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

// round_W then widen, two binary32 values at a time; the identity for a
// binary32 wire.
template <int W>
__device__ __forceinline__ void wire_pair(float &x, float &y) {
    if constexpr (W != AR_F32) widen_pair<W>(round_pack<W>(x, y), x, y);
}

// One element of a source, scalar path (range remainders).
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
//   binary32 sources, and their destinations and residual:
//       part j in {0,1}: elements t + 256 j + 4 lane + {0..3}
//   16-bit sources: elements t + 8 lane + {0..7} (one dwordx4)
//       binary32 destinations / residual: t + 8 lane + 4 j + {0..3}
//       16-bit destinations / residual:   t + 8 lane + {0..7} (one dwordx4)
// Values v[0..7] of a lane are ordered as v[4 j + k] for the binary32 forms
// and v[k] = element t + 8 lane + k for the 16-bit forms.
// ---------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ size_t part_elem(size_t t, int lane, int j) {
    return C::SW ? t + 8 * lane + 4 * j : t + 256 * j + 4 * lane;
}

template <class C, bool NT>
__device__ __forceinline__ void tile_load(const void *src, size_t t, int lane, u32x4 (&raw)[C::kSrcRaw]) {
    if constexpr (C::SW) {
        raw[0] = load16<NT>(reinterpret_cast<const uint16_t *>(src) + t + 8 * lane);
    } else {
        const float *s = reinterpret_cast<const float *>(src) + t + 4 * lane;
        raw[0] = load16<NT>(s);
        raw[1] = load16<NT>(s + 256);
    }
}

// Load j of a tile's kSrcRaw loads (the same addresses as tile_load's).
template <class C, bool NT>
__device__ __forceinline__ u32x4 part_load(const void *src, size_t t, int lane, int j) {
    if constexpr (C::SW) {
        return load16<NT>(reinterpret_cast<const uint16_t *>(src) + t + 8 * lane);
    } else {
        return load16<NT>(reinterpret_cast<const float *>(src) + t + 256 * j + 4 * lane);
    }
}

// Loads of a binary32-source tile are issued part by part across the ranks
// (part 0 of every rank, then part 1) rather than rank by rank.  Measured on
// MI355X, same machine, bit-identical outputs: 4 ranks with one inactive
// 20.97 against 21.29-21.33 us, R = 8 [8192 x 8192] 366.7-367.5 against
// 370.3-371.4 us; the prefill call unchanged (16.05-16.07 us).
#ifndef MPP_PART_MAJOR
#define MPP_PART_MAJOR 1
#endif

template <class C>
__device__ __forceinline__ void tile_values(const u32x4 (&raw)[C::kSrcRaw], float (&v)[8]) {
    if constexpr (C::SW) {
#pragma unroll
        for (int k = 0; k < 4; ++k) widen_pair<C::W>(raw[0][k], v[2 * k], v[2 * k + 1]);
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int k = 0; k < 4; k += 2) {
                float x = f32_from_bits(raw[j][k]);
                float y = f32_from_bits(raw[j][k + 1]);
                wire_pair<C::W>(x, y);
                v[4 * j + k] = x;
                v[4 * j + k + 1] = y;
            }
        }
    }
}

// Where one gridDim.y range of a launch starts in each tensor: element
// offsets of the range's first element in the sources, the destinations and
// an element-wise residual (they differ when the tensors are row-strided),
// and the range's position in the whole call (for a broadcast row's column).
struct RangeOff {
    size_t src;
    size_t dst;
    size_t res;
    uint64_t pos;
};

// Column of call position `pos` in a broadcast row of res_len elements (a
// multiple of 8, so the 4 or 8 consecutive elements of one lane part never
// straddle a row boundary).  Calls can pass 2^32 elements: those positions
// take a 64-bit remainder, all others the cheaper 32-bit one.
template <class A>
__device__ __forceinline__ size_t res_column(const A &a, uint64_t pos) {
    const uint64_t x = pos + a.res_phase;
    if (x < (uint64_t(1) << 32)) return static_cast<unsigned>(x) % a.res_len;
    return x % a.res_len;
}

// Residual element of range element e: element-wise (o.res + e, which is the
// same row for every range when the residual's row stride is 0), or the
// column of a 1-D broadcast row.
template <class A>
__device__ __forceinline__ size_t res_index(const A &a, const RangeOff &o, size_t e) {
    return a.res_len == 0 ? o.res + e : res_column(a, o.pos + e);
}

// Residual loads of one tile: streaming loads when each residual element is
// read once, ordinary cached loads when a row is read by every row.  Both
// forms issue the same number of loads, so the branch does not change how
// many loads are outstanding after it.
template <class C, bool NT>
__device__ __forceinline__ void res_load(const LaunchArgs<C::RB> &a, const RangeOff &o, size_t t, int lane,
                                         u32x4 (&raw)[C::kResRaw]) {
    size_t e[C::kResRaw];
#pragma unroll
    for (int j = 0; j < C::kResRaw; ++j) e[j] = res_index(a, o, part_elem<C>(t, lane, j));
    const char *base = static_cast<const char *>(a.res);
    if (a.res_reuse) {
#pragma unroll
        for (int j = 0; j < C::kResRaw; ++j) raw[j] = load16<false>(base + e[j] * C::kDstBytes);
    } else {
#pragma unroll
        for (int j = 0; j < C::kResRaw; ++j) raw[j] = load16<NT>(base + e[j] * C::kDstBytes);
    }
}

template <class C>
__device__ __forceinline__ void res_values(const u32x4 (&raw)[C::kResRaw], float (&v)[8]) {
    if constexpr (C::DN) {
#pragma unroll
        for (int k = 0; k < 4; ++k) widen_pair<C::W>(raw[0][k], v[2 * k], v[2 * k + 1]);
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k) v[4 * j + k] = f32_from_bits(raw[j][k]);
    }
}

// One rounding of every accumulator to the destination type (no-op for
// binary32 destinations).
template <class C>
__device__ __forceinline__ void round_dst(float (&acc)[8]) {
    if constexpr (C::DN) {
#pragma unroll
        for (int k = 0; k < 8; k += 2) wire_pair<C::W>(acc[k], acc[k + 1]);
    }
}

// Store policy of tile_store as a value: 0 write-back, 1 non-temporal, 2
// device-scope write-through.
template <class C, int ST>
constexpr int store_policy() {
    return ST == kStoreStream ? 1 : (ST == kStoreKeep && !C::SW ? 2 : 0);
}

template <class C, int ST>
__device__ __forceinline__ void tile_store(void *dst, size_t t, int lane, const float (&acc)[8]) {
    // write-through for the binary32-source layout (each store instruction
    // covers 1 KiB contiguous); the 16-bit layouts measured better with
    // write-back
    constexpr int SP = store_policy<C, ST>();
    if constexpr (C::DN) {
        // the values already lie in the destination type: the packing is exact
        const u32x4 v = {round_pack<C::W>(acc[0], acc[1]), round_pack<C::W>(acc[2], acc[3]),
                         round_pack<C::W>(acc[4], acc[5]), round_pack<C::W>(acc[6], acc[7])};
        store16<SP>(static_cast<uint16_t *>(dst) + t + 8 * lane, v);
    } else if constexpr (C::SW) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4 v = {bits_from_f32(acc[4 * j]), bits_from_f32(acc[4 * j + 1]),
                             bits_from_f32(acc[4 * j + 2]), bits_from_f32(acc[4 * j + 3])};
            store16<SP>(static_cast<float *>(dst) + part_elem<C>(t, lane, j), v);
        }
    } else {
        // binary32 layout: the tile's 2 KiB start at the wave-uniform element t
        float *base = static_cast<float *>(dst) + t;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4 v = {bits_from_f32(acc[4 * j]), bits_from_f32(acc[4 * j + 1]),
                             bits_from_f32(acc[4 * j + 2]), bits_from_f32(acc[4 * j + 3])};
            if constexpr (SP == 2) {
                store16_wt(base, kWaveTile * 4, (256 * j + 4 * lane) * 4, v);
            } else {
                store16<SP>(base + 256 * j + 4 * lane, v);
            }
        }
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
template <class C>
__device__ __forceinline__ bool rank_active(const LaunchArgs<C::RB> &a, int r) {
    if constexpr (C::MASKED) {
        return (a.active >> r) & 1u;
    } else {
        return true;
    }
}

template <class C>
__device__ __forceinline__ bool rank_used(const LaunchArgs<C::RB> &a, int r) {
    return r < 2 || r < a.R;
}

// A launch argument read where it is used: the empty asm keeps the compiler
// from hoisting work on it above the batch's loads, which would make every
// wave wait for its scalar fetch before issuing them (the destinations after
// the first are not among the preloaded parameters).
__device__ __forceinline__ void *at_use(void *p) {
    const uint64_t v = reinterpret_cast<uintptr_t>(p);
    unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v));
    unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(v >> 32));
    asm volatile("" : "+s"(lo), "+s"(hi));
    return reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Registers of one batch of U wave tiles.
template <class C, int U>
struct Batch {
    u32x4 src[C::RB][U][C::kSrcRaw];
    u32x4 res[U][C::kResRaw];
};

// Issue every load of a batch of U consecutive wave tiles starting at range
// element `t` for the first R of RB sources, tile by tile (and within a tile
// part by part, see MPP_PART_MAJOR): the loads of tile 0 are the oldest in
// flight, so tile 0 can be folded and stored while the later tiles' loads are
// still arriving.  The residual loads of the batch come last.
template <class C, int U, bool NT>
__device__ __forceinline__ void load_batch(const LaunchArgs<C::RB> &a, const RangeOff &o, size_t t, int lane,
                                           Batch<C, U> &b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#if MPP_PART_MAJOR
        // part by part across the ranks: a 1 KiB part can be folded and
        // stored as soon as its R loads are in
#pragma unroll
        for (int j = 0; j < C::kSrcRaw; ++j) {
#pragma unroll
            for (int r = 0; r < C::RB; ++r) {
                if (rank_used<C>(a, r) && rank_active<C>(a, r)) {
                    b.src[r][u][j] = part_load<C, NT>(a.src[r], o.src + t + u * kWaveTile, lane, j);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#else
#pragma unroll
        for (int r = 0; r < C::RB; ++r) {
            if (rank_used<C>(a, r) && rank_active<C>(a, r)) {
                tile_load<C, NT>(a.src[r], o.src + t + u * kWaveTile, lane, b.src[r][u]);
            }
        }
#endif
        // keep tile order: the scheduler must not hoist a later tile's loads
        // above this one's
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (C::RES) {
#pragma unroll
        for (int u = 0; u < U; ++u) res_load<C, NT>(a, o, t + u * kWaveTile, lane, b.res[u]);
    }
}

// Binary32-source tiles of the 8- and 16-rank buckets fold and store each
// 1 KiB part as soon as its R loads are in (fold_store_part); smaller buckets
// fold the whole tile first.  Measured on MI355X, same machine, bit-identical
// outputs: R = 8 [8192 x 8192] 364.6-365.0 against 366.7-367.5 us (whole
// tiles); with parts stored early at R = 2 the prefill call took 16.24 against
// 16.15 us and the decode call 2.01 against 1.75 us.
#ifndef MPP_PART_STORE
#define MPP_PART_STORE 1
#endif
#ifndef MPP_PART_STORE_MIN_RB
#define MPP_PART_STORE_MIN_RB 8
#endif

// Fold part j of a binary32-source tile (elements td + 256 j + 4 lane + 0..3)
// in rank order, add its residual, and store it to every destination.  The
// same arithmetic per element as fold_store_tile; a part is stored as soon as
// its R loads are in, ahead of the tile's other part.
template <class C, int ST>
__device__ __forceinline__ void fold_store_part(const LaunchArgs<C::RB> &a, size_t td, int lane, int j,
                                                const u32x4 (&src)[C::RB][C::kSrcRaw], const u32x4 *res) {
    static_assert(!C::SW && !C::DN, "binary32 sources and destinations only");
    float acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = 0.0f;
    if (rank_active<C>(a, 0)) {
#pragma unroll
        for (int k = 0; k < 4; k += 2) {
            float x = f32_from_bits(src[0][j][k]);
            float y = f32_from_bits(src[0][j][k + 1]);
            wire_pair<C::W>(x, y);
            acc[k] = x;
            acc[k + 1] = y;
        }
    }
#pragma unroll
    for (int r = 1; r < C::RB; ++r) {
        if (rank_used<C>(a, r)) {
            float w[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (rank_active<C>(a, r)) {
#pragma unroll
                for (int k = 0; k < 4; k += 2) {
                    float x = f32_from_bits(src[r][j][k]);
                    float y = f32_from_bits(src[r][j][k + 1]);
                    wire_pair<C::W>(x, y);
                    w[k] = x;
                    w[k + 1] = y;
                }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] = acc[k] + w[k];
        }
    }
    if constexpr (C::RES) {
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = acc[k] + f32_from_bits(res[j][k]);
    }
    const u32x4 v = {bits_from_f32(acc[0]), bits_from_f32(acc[1]), bits_from_f32(acc[2]), bits_from_f32(acc[3])};
    constexpr int SP = store_policy<C, ST>();
    auto put = [&](void *dst) {
        float *base = static_cast<float *>(dst) + td;
        if constexpr (SP == 2) {
            store16_wt(base, kWaveTile * 4, (256 * j + 4 * lane) * 4, v);
        } else {
            store16<SP>(base + 256 * j + 4 * lane, v);
        }
    };
    // every launch writes destination 0 (the host never launches without one);
    // the others sit behind a single branch: per-destination tests around the
    // first destination's stores cost the prefill call 0.3 us on MI355X
    // (16.09-16.11 against 15.78-15.79 us, same machine)
    put(a.dst[0]);
    if (a.n_dst > 1) {
#pragma unroll
        for (int d = 1; d < C::RB; ++d) {
            if (d < a.n_dst) put(at_use(a.dst[d]));
        }
    }
}

// Fold one tile in rank order (one rounding to the destination type per add),
// add the residual, and store to every destination at element `td`.
template <class C, int ST>
__device__ __forceinline__ void fold_store_tile(const LaunchArgs<C::RB> &a, size_t td, int lane,
                                                const u32x4 (&src)[C::RB][C::kSrcRaw], const u32x4 *res) {
    if constexpr (MPP_PART_STORE && !C::SW && !C::DN && C::RB >= MPP_PART_STORE_MIN_RB) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            fold_store_part<C, ST>(a, td, lane, j, src, res);
            // keep part order: part 1's work must not be hoisted above part 0's stores
            __builtin_amdgcn_sched_barrier(0);
        }
        return;
    }
    float acc[8];
    if (rank_active<C>(a, 0)) {
        tile_values<C>(src[0], acc);
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
    }
#pragma unroll
    for (int r = 1; r < C::RB; ++r) {
        if (rank_used<C>(a, r)) {
            float w[8];
            if (rank_active<C>(a, r)) {
                tile_values<C>(src[r], w);
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) w[k] = 0.0f;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] = acc[k] + w[k];
            round_dst<C>(acc);
        }
    }
    if constexpr (C::RES) {
        u32x4 rr[C::kResRaw];
#pragma unroll
        for (int j = 0; j < C::kResRaw; ++j) rr[j] = res[j];
        float rv[8];
        res_values<C>(rr, rv);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = acc[k] + rv[k];
        round_dst<C>(acc);
    }
    // destination 0 always, the others behind one branch (see fold_store_part)
    tile_store<C, ST>(a.dst[0], td, lane, acc);
    if (a.n_dst > 1) {
#pragma unroll
        for (int d = 1; d < C::RB; ++d) {
            if (d < a.n_dst) tile_store<C, ST>(at_use(a.dst[d]), td, lane, acc);
        }
    }
}

// Fold each tile of the batch and store it before the next tile is folded.
// Stores use the policy ST (streaming for calls that write at least as much
// as they read, kept in the cache hierarchy otherwise; see kStoreKeep).  The
// policy is a template parameter: two stores that differ only in their cache
// hint would be merged into one by the compiler.
template <class C, int U, int ST>
__device__ __forceinline__ void fold_store(const LaunchArgs<C::RB> &a, const RangeOff &o, size_t t, int lane,
                                           const Batch<C, U> &b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        u32x4 src[C::RB][C::kSrcRaw];
#pragma unroll
        for (int r = 0; r < C::RB; ++r)
#pragma unroll
            for (int j = 0; j < C::kSrcRaw; ++j) src[r][j] = b.src[r][u][j];
        fold_store_tile<C, ST>(a, o.dst + t + u * kWaveTile, lane, src, b.res[u]);
    }
}

template <class C, int U, bool NT, int ST>
__device__ __forceinline__ void reduce_tiles(const LaunchArgs<C::RB> &a, const RangeOff &o, size_t t, int lane) {
    Batch<C, U> b;
    load_batch<C, U, NT>(a, o, t, lane, b);
    fold_store<C, U, ST>(a, o, t, lane, b);
}

// Range elements [begin, end), one per lane per step (end - begin is below one
// wave tile, so this is at most 8 steps).
template <class C>
__device__ __forceinline__ void reduce_tail(const LaunchArgs<C::RB> &a, const RangeOff &o, size_t begin,
                                            size_t end, int lane) {
    // end - begin < one wave tile, so a lane owns at most kTileLane elements
    // (begin + lane + kWave k).  The tail's loads are issued without a branch,
    // KB elements' worth at a time (at most 16 per lane), and folded
    // afterwards; the stores come after every fold, guarded.  With a load and
    // its use inside one guarded branch per element, every element waited for
    // its own loads: the tail then cost one memory round trip per element (up
    // to 1.8 us on a prefill-sized call).  The sources are read through buffer
    // loads over [begin, end) of each, so a lane's load past the end returns 0
    // (the hardware's range check); the residual at an index clamped into the
    // range.  Each element is read and written by this lane alone and every
    // load precedes every store, so in-place calls stay exact.
    constexpr int kTileLane = kWaveTile / kWave;
    constexpr int KB = C::RB >= 16 ? 1 : (16 / C::RB < kTileLane ? 16 / C::RB : kTileLane);
    float acc[kTileLane];
    constexpr unsigned kSrcBytes = C::SW ? 2u : 4u;
    const unsigned span = static_cast<unsigned>(end - begin) * kSrcBytes;
#pragma unroll
    for (int k0 = 0; k0 < kTileLane; k0 += KB) {
        float v[KB][C::RB];
        float rv[KB];
#pragma unroll
        for (int q = 0; q < KB; ++q) {
            const size_t e0 = begin + lane + static_cast<size_t>(kWave) * (k0 + q);
            const size_t e = e0 < end ? e0 : end - 1;
            const int off = (lane + kWave * (k0 + q)) * static_cast<int>(kSrcBytes);
#pragma unroll
            for (int r = 0; r < C::RB; ++r) {
                v[q][r] = 0.0f;
                if (rank_used<C>(a, r) && rank_active<C>(a, r)) {
                    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                        const_cast<char *>(static_cast<const char *>(a.src[r])) + (o.src + begin) * kSrcBytes, 0,
                        span, kRsrcWord3);
                    if constexpr (C::SW) {
                        v[q][r] = f32_from_bits(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
                    } else {
                        v[q][r] = f32_from_bits(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
                    }
                }
            }
            rv[q] = 0.0f;
            if constexpr (C::RES) {
                const size_t ri = res_index(a, o, e);
                if constexpr (C::DN) {
                    rv[q] = f32_from_bits(static_cast<const uint16_t *>(a.res)[ri]);
                } else {
                    rv[q] = static_cast<const float *>(a.res)[ri];
                }
            }
        }
#pragma unroll
        for (int q = 0; q < KB; ++q) {
            // the raw values become the wire-rounded terms (16-bit sources and a
            // narrow residual were loaded as their bit patterns)
            float term[C::RB];
#pragma unroll
            for (int r = 0; r < C::RB; ++r) {
                if constexpr (C::SW) {
                    float x, unused;
                    widen_pair<C::W>(bits_from_f32(v[q][r]), x, unused);
                    term[r] = x;
                } else {
                    float x = v[q][r], y = 0.0f;
                    wire_pair<C::W>(x, y);
                    term[r] = x;
                }
            }
            float t0 = rank_active<C>(a, 0) ? term[0] : 0.0f;
#pragma unroll
            for (int r = 1; r < C::RB; ++r) {
                if (rank_used<C>(a, r)) {
                    t0 = t0 + (rank_active<C>(a, r) ? term[r] : 0.0f);
                    if constexpr (C::DN) {
                        float y = 0.0f;
                        wire_pair<C::W>(t0, y);
                    }
                }
            }
            if constexpr (C::RES) {
                if constexpr (C::DN) {
                    float x, unused;
                    widen_pair<C::W>(bits_from_f32(rv[q]), x, unused);
                    t0 = t0 + x;
                    float y = 0.0f;
                    wire_pair<C::W>(t0, y);
                } else {
                    t0 = t0 + rv[q];
                }
            }
            acc[k0 + q] = t0;
        }
    }
#pragma unroll
    for (int k = 0; k < kTileLane; ++k) {
        const size_t e = begin + lane + static_cast<size_t>(kWave) * k;
        if (e < end) {
            const size_t ed = o.dst + e;
#pragma unroll
            for (int d = 0; d < C::RB; ++d) {
                if (d < a.n_dst) {
                    if constexpr (C::DN) {
                        static_cast<uint16_t *>(a.dst[d])[ed] =
                            static_cast<uint16_t>(round_pack<C::W>(acc[k], 0.0f));
                    } else {
                        static_cast<float *>(a.dst[d])[ed] = acc[k];
                    }
                }
            }
        }
    }
}

// The tail one element at a time, each element's loads, fold and stores in
// turn: the LDS-staged kernels keep this form.  Inlined into them, the
// batched tail above keeps the backend from folding the LDS stage pointers'
// address-space casts in the plain (unmasked, no residual) instances, and the
// compare against the shared aperture it leaves fails to compile for gfx950
// ("Operand has incorrect register class"); out of line it gives every
// LDS-staged kernel a private stack.
template <class C>
__device__ __forceinline__ void reduce_tail_each(const LaunchArgs<C::RB> &a, const RangeOff &o, size_t begin,
                                                 size_t end, int lane) {
    for (size_t e = begin + lane; e < end; e += kWave) {
        const size_t es = o.src + e;
        float acc = rank_active<C>(a, 0) ? wire_one<C::W, C::SW>(a.src[0], es) : 0.0f;
#pragma unroll
        for (int r = 1; r < C::RB; ++r) {
            if (rank_used<C>(a, r)) {
                acc = acc + (rank_active<C>(a, r) ? wire_one<C::W, C::SW>(a.src[r], es) : 0.0f);
                if constexpr (C::DN) {
                    float y = 0.0f;
                    wire_pair<C::W>(acc, y);
                }
            }
        }
        if constexpr (C::RES) {
            const size_t ri = res_index(a, o, e);
            if constexpr (C::DN) {
                acc = acc + wire_one<C::W, true>(a.res, ri);
                float y = 0.0f;
                wire_pair<C::W>(acc, y);
            } else {
                acc = acc + static_cast<const float *>(a.res)[ri];
            }
        }
        const size_t ed = o.dst + e;
#pragma unroll
        for (int d = 0; d < C::RB; ++d) {
            if (d < a.n_dst) {
                if constexpr (C::DN) {
                    static_cast<uint16_t *>(a.dst[d])[ed] = static_cast<uint16_t>(round_pack<C::W>(acc, 0.0f));
                } else {
                    static_cast<float *>(a.dst[d])[ed] = acc;
                }
            }
        }
    }
}

template <class C, bool LDS_FAMILY>
__device__ __forceinline__ void reduce_scalar(const LaunchArgs<C::RB> &a, const RangeOff &o, size_t begin,
                                              size_t end, int lane) {
    if constexpr (LDS_FAMILY) {
        reduce_tail_each<C>(a, o, begin, end, lane);
    } else {
        reduce_tail<C>(a, o, begin, end, lane);
    }
}

// Offsets and length of this workgroup's gridDim.y range.  Slice ranges
// (broadcast schedule): [slice_start[y], + slice_len[y]) of every tensor.
// Strided ranges (everything else): range y has min(cols, n - y * cols)
// elements starting at element y * stride of each tensor class -- 1-D chunks
// (stride = cols) and the rows of row-strided tensors alike.  Both forms only
// read launch arguments at fixed offsets (blockIdx.y is known at wave
// start), so a wave fetches everything it needs in one batch of scalar loads.
// Kernels call it on their own argument block for slice ranges (an indexed
// read of kernel arguments is one scalar load) and never on a local copy of
// the block, whose arrays would then have to live in scratch memory.
template <bool SLICED, class A>
__device__ __forceinline__ void range_of(const A &a, RangeOff &o, unsigned &len) {
    const unsigned y = blockIdx.y;
    if constexpr (SLICED) {
        o.src = o.dst = o.res = a.slice_start[y];
        o.pos = a.slice_start[y];
        len = a.slice_len[y];
    } else {
        const uint64_t start = static_cast<uint64_t>(y) * a.cols;
        const uint64_t left = a.n - start;
        len = left < a.cols ? static_cast<unsigned>(left) : a.cols;
        o.src = static_cast<size_t>(y) * a.src_stride;
        o.dst = static_cast<size_t>(y) * a.dst_stride;
        o.res = static_cast<size_t>(y) * a.res_stride;
        o.pos = start;
    }
}

// Whole wave tiles after the batched part, then the element remainder on
// wave 0 of workgroup 0 of the range.
template <class C, int U, bool NT, int ST, bool LDS_FAMILY = false>
__device__ __forceinline__ void reduce_rest(const LaunchArgs<C::RB> &a, const RangeOff &o, unsigned len,
                                            unsigned done, unsigned gw, unsigned nw, int lane) {
    if constexpr (U > 1) {
        const unsigned n_one = (len - done) / kWaveTile;
        for (unsigned t = gw; t < n_one; t += nw) {
            reduce_tiles<C, 1, NT, ST>(a, o, done + (size_t)t * kWaveTile, lane);
        }
    }
    const unsigned vec_end = (len / kWaveTile) * kWaveTile;
    if (vec_end < len && gw == 0) {
        reduce_scalar<C, LDS_FAMILY>(a, o, vec_end, len, lane);
    }
}

// Walk the wave tiles of this workgroup's range: batches of U tiles strided
// over the `a.waves` waves of the range, then the remainder.  BLOCK is the
// workgroup size the kernel is always launched with (no read of blockDim).
template <class C, int U, bool NT, int ST, int BLOCK, bool SLICED>
__device__ __forceinline__ void reduce_range(const LaunchArgs<C::RB> &a, const RangeOff &o, unsigned len) {
    constexpr unsigned wpb = BLOCK / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const unsigned nw = a.waves;
    // the wave's index, read from lane 0 so the compiler keeps it (and every
    // tile address derived from it) in scalar registers; the workgroup's
    // index is its place in the XCD placement map
    const unsigned gw = xcd_virtual_block(blockIdx.x, nw / wpb, a.map_lc) * wpb +
                        __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

    constexpr unsigned big = kWaveTile * U;
    const unsigned n_big = len / big;
    // one-shot grid over whole batches (the common case): a wave's single
    // batch, then nothing -- no loop back-edge and no remainder tests on its
    // path.  Measured on MI355X, same machine: prefill 15.70-15.72 against
    // 15.72-15.74 us; for the 8- and 16-rank buckets the loop form is kept
    // (R = 8: 370 against 363 us with the shortcut)
    if (C::RB <= 4 && n_big * big == len && n_big <= nw) {
        if (gw < n_big) reduce_tiles<C, U, NT, ST>(a, o, (size_t)gw * big, lane);
        return;
    }
    for (unsigned t = gw; t < n_big; t += nw) {
        reduce_tiles<C, U, NT, ST>(a, o, (size_t)t * big, lane);
    }
    reduce_rest<C, U, NT, ST>(a, o, len, n_big * big, gw, nw, lane);
}

constexpr int kSingleShotBlock = 64;
constexpr int kLdsBlock = 64;

// Workgroup size of the register-staged streaming kernel per rank bucket
// (measured on MI355X, with the XCD placement runs): one wave per workgroup
// up to the 8-rank bucket -- small workgroups pack the CUs more evenly and
// keep each XCD's run of tiles spread over its CUs (same machine against 256
// threads, bit-identical: 4 ranks 25.71 against 25.94 us, 3 ranks 20.11
// against 20.40, 4 ranks with one inactive 20.33 against 20.69, two-rank
// slice + broadcast 23.99 against 24.56, row-strided block + bias 16.12
// against 16.28, 3 ranks + bias row 20.63 against 20.95; 4 bf16 partials
// 17.51 against 17.63; the prefill call and 3-rank narrow destinations
// unchanged); 256 threads for the 16-rank bucket (27.52 against 27.92 us with
// one wave per workgroup on a quarter of the prefill shape).  The host takes
// the same function for the launch shape, and the launcher refuses a shape
// that differs from it.
#ifndef MPP_STREAM_BLOCK
#define MPP_STREAM_BLOCK 0
#endif
constexpr int stream_block(int rank_bucket, bool res, bool src_is_wire) {
    return MPP_STREAM_BLOCK > 0 ? MPP_STREAM_BLOCK : (rank_bucket == 16 ? 256 : 64);
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
// loads per lane (R x U x loads-per-tile) for 16-bit sources and
// MPP_STREAM_LOADS_F32 for binary32 sources, at least 1 and at most MAXU
// tiles.  With binary32 sources that makes one tile per wave at every bucket:
// measured on MI355X, same machine, against two tiles at R = 2 (8 loads):
// prefill 15.74-15.75 against 15.78-15.81 us, prefill + bias row 16.64
// against 16.99 us, row-strided block + bias 16.39-16.40 against 16.97-17.00
// us, element-wise residual 20.44 against 20.31 us.  16-bit sources keep 8
// (4 measured 17.5 against 15.9-16.0 us at R = 3).
#ifndef MPP_STREAM_LOADS_F32
#define MPP_STREAM_LOADS_F32 4
#endif
constexpr int stream_batch(bool src_is_wire, int rank_bucket) {
    const int per_tile = (src_is_wire ? 1 : 2) * rank_bucket;
    const int u = (src_is_wire ? MPP_STREAM_LOADS : MPP_STREAM_LOADS_F32) / per_tile;
    return u < 1 ? 1 : (u > MPP_STREAM_MAXU ? MPP_STREAM_MAXU : u);
}

template <class C, int ST, bool SLICED>
__device__ __forceinline__ void stream_reg(const LaunchArgs<C::RB> &a, const RangeOff &o, unsigned len) {
    constexpr int block = stream_block(C::RB, C::RES, C::SW);
    reduce_range<C, stream_batch(C::SW, C::RB), MPP_STREAM_NT != 0, ST, block, SLICED>(a, o, len);
}

// ---------------------------------------------------------------------------
// LDS-staged streaming kernel (one wave per workgroup).  Each wave owns two
// LDS stages of R x U x K blocks of 1 KiB.  global_load_lds_dwordx4 writes a
// lane's 16 B straight into the stage (no VGPRs held while the load is in
// flight); while the wave folds and stores the batch in one stage, the loads
// of its next batch stream into the other.  A lane only ever reads back the
// 16 B it loaded itself, so the stages need no barrier, only the wait on the
// wave's own vector-memory counter.  A residual is staged the same way, as
// U x kResRaw more blocks after the ranks' (cached loads for a broadcast row,
// which every row reads; non-temporal for an element-wise residual).
// ---------------------------------------------------------------------------
#ifndef MPP_LDS_U
#define MPP_LDS_U 1
#endif
// Grid of the LDS-staged kernel: 0 = one-shot (one batch per wave, the
// hardware back-fills CUs as waves retire; measured best on MI355X), k > 0 =
// persistent grid of k workgroups per CU that double-buffers its batches.
#ifndef MPP_LDS_WG_PER_CU
#define MPP_LDS_WG_PER_CU 0u
#endif
// Cache-policy bits of the LDS-staged loads: 2 = non-temporal (streaming
// data read once; with cached loads the kernel only looked faster when the
// inputs were still in the Infinity Cache), 0 = default.
#ifndef MPP_LDS_AUX
#define MPP_LDS_AUX 2
#endif

// Tiles per stage: MPP_LDS_U, reduced so one stage is at most 32 loads per
// lane (the stage wait uses the 6-bit vector-memory counter).
constexpr int lds_batch(bool src_is_wire, int rank_bucket) {
    const int per_tile = (src_is_wire ? 1 : 2) * rank_bucket;
    const int cap = 32 / per_tile;
    const int u = MPP_LDS_U;
    return u < 1 ? 1 : (u > cap ? (cap < 1 ? 1 : cap) : u);
}

typedef __attribute__((address_space(3))) void lds_void;

// 1 KiB blocks of one LDS stage: the ranks' RB x U x K, then the residual's U x kResRaw.
template <class C, int U>
constexpr int lds_rank_blocks() { return C::RB * U * C::kSrcRaw; }
template <class C, int U>
constexpr int lds_stage_blocks() { return lds_rank_blocks<C, U>() + (C::RES ? U * C::kResRaw : 0); }

template <class C, int U>
__device__ __forceinline__ void lds_issue(const LaunchArgs<C::RB> &a, const RangeOff &o, size_t t, int lane,
                                          u32x4 (*stage)[kWave]) {
    constexpr int K = C::kSrcRaw;
#pragma unroll
    for (int r = 0; r < C::RB; ++r) {
        if (rank_used<C>(a, r) && rank_active<C>(a, r)) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    const size_t e = o.src + (C::SW ? t + u * kWaveTile + 8 * lane : t + u * kWaveTile + 256 * j + 4 * lane);
                    const char *g = static_cast<const char *>(a.src[r]) + e * (C::SW ? 2 : 4);
                    __builtin_amdgcn_global_load_lds(g, (lds_void *)(&stage[(r * U + u) * K + j][0]),
                                                     16, 0, MPP_LDS_AUX);
                }
            }
        }
    }
    if constexpr (C::RES) {
        constexpr int B0 = lds_rank_blocks<C, U>();
        const char *base = static_cast<const char *>(a.res);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int j = 0; j < C::kResRaw; ++j) {
                const char *g = base + res_index(a, o, part_elem<C>(t + u * kWaveTile, lane, j)) * C::kDstBytes;
                lds_void *l = (lds_void *)(&stage[B0 + u * C::kResRaw + j][0]);
                if (a.res_reuse) {
                    __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
                } else {
                    __builtin_amdgcn_global_load_lds(g, l, 16, 0, MPP_LDS_AUX);
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

template <class C, int U, int ST>
__device__ __forceinline__ void lds_consume(const LaunchArgs<C::RB> &a, const RangeOff &o, size_t t, int lane,
                                            u32x4 (*stage)[kWave]) {
    constexpr int K = C::kSrcRaw;
    const unsigned base = static_cast<unsigned>(reinterpret_cast<uintptr_t>((lds_void *)(&stage[0][lane])));
    Batch<C, U> b;
#pragma unroll
    for (int r = 0; r < C::RB; ++r) {
        if (rank_used<C>(a, r) && rank_active<C>(a, r)) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < K; ++j) b.src[r][u][j] = lds_read16(base + ((r * U + u) * K + j) * kWave * 16);
        }
    }
    if constexpr (C::RES) {
        constexpr int B0 = lds_rank_blocks<C, U>();
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < C::kResRaw; ++j) b.res[u][j] = lds_read16(base + (B0 + u * C::kResRaw + j) * kWave * 16);
    }
    fold_store<C, U, ST>(a, o, t, lane, b);
}

// One-shot fast path of the LDS-staged kernel (ranges of whole batches, 2-
// and 4-rank buckets): the wave's single stage without the double-buffer
// bookkeeping and the remainder tests.  Measured on MI355X, same machine:
// bf16 partials into a bf16 destination on the prefill shape 8.85 against
// 9.09-9.10 us; the 4-rank broadcasts unchanged.
#ifndef MPP_LDS_FAST
#define MPP_LDS_FAST 1
#endif

template <class C, int ST, bool SLICED>
__device__ __forceinline__ void stream_lds_as(const LaunchArgs<C::RB> &a, const RangeOff &o, unsigned len,
                                              u32x4 (*stage0)[kWave], u32x4 (*stage1)[kWave]) {
    constexpr int U = lds_batch(C::SW, C::RB);
    const int lane = threadIdx.x;
    const unsigned nw = a.waves;
    const unsigned gw = xcd_virtual_block(blockIdx.x, nw, a.map_lc);
    constexpr unsigned big = kWaveTile * U;
    const unsigned n_big = len / big;
#if MPP_LDS_FAST
    // one-shot grid over whole batches: the wave's single stage, then nothing
    if (C::RB <= 4 && n_big * big == len && n_big <= nw) {
        if (gw < n_big) {
            lds_issue<C, U>(a, o, (size_t)gw * big, lane, stage0);
            wait_vm<0>();
            lds_consume<C, U, ST>(a, o, (size_t)gw * big, lane, stage0);
        }
        return;
    }
#endif

    // loads per stage (vector-memory instructions): active ranks x U x K
    const int RU = a.R < C::RB ? a.R : C::RB;
    const unsigned ranks_mask = RU >= 32 ? ~0u : ((1u << RU) - 1u);
    const int L = __builtin_popcount(a.active & ranks_mask) * U * C::kSrcRaw + (C::RES ? U * C::kResRaw : 0);
    constexpr int kMaxL = lds_stage_blocks<C, U>();

    unsigned t = gw;
    if (t < n_big) lds_issue<C, U>(a, o, (size_t)t * big, lane, stage0);
    while (t < n_big) {
        const unsigned t1 = t + nw;
        if (t1 < n_big) {
            lds_issue<C, U>(a, o, (size_t)t1 * big, lane, stage1);
            wait_stage<kMaxL>(L);
        } else {
            wait_vm<0>();
        }
        lds_consume<C, U, ST>(a, o, (size_t)t * big, lane, stage0);
        if (t1 >= n_big) break;
        const unsigned t2 = t1 + nw;
        if (t2 < n_big) {
            lds_issue<C, U>(a, o, (size_t)t2 * big, lane, stage0);
            wait_stage<kMaxL>(L);
        } else {
            wait_vm<0>();
        }
        lds_consume<C, U, ST>(a, o, (size_t)t1 * big, lane, stage1);
        t = t2;
    }
    reduce_rest<C, U, true, ST, true>(a, o, len, n_big * big, gw, nw, lane);
}

template <class C, int ST, bool SLICED>
__device__ __forceinline__ void stream_lds(const LaunchArgs<C::RB> &a, const RangeOff &o, unsigned len) {
    constexpr int NB = lds_stage_blocks<C, lds_batch(C::SW, C::RB)>();   // 1 KiB blocks per stage
    __shared__ u32x4 stage0[NB][kWave];
    __shared__ u32x4 stage1[NB][kWave];
    stream_lds_as<C, ST, SLICED>(a, o, len, stage0, stage1);
}

// ---------------------------------------------------------------------------
// Kernel parameters.  The fields a wave reads before its first load of a
// strided range -- the launch length, the range length, the wave count, the
// source and destination strides, the first two sources and the first
// destination, and one "shape" dword (bits 0-23 the wave count, 24-27 the
// destination count minus one, 28-31 the XCD placement exponent map_lc) --
// come first, as plain scalars (14 dwords), so that the dispatcher preloads
// them into SGPRs (the non-residual streaming tables are built with kernarg
// preloading for the leading parameters; an aggregate parameter is never
// preloaded).  The argument block that follows holds every field, these
// included.  Measured on MI355X with a minimal kernel of the prefill access
// pattern: 15.53 against 15.85 us per call -- every wave of a one-shot grid
// starts together, so the scalar fetch of its arguments sits once on the
// critical path of the call.
// ---------------------------------------------------------------------------
#define MPP_HOT_PARAMS uint64_t hot_n, unsigned hot_cols, unsigned hot_shape, uint64_t hot_src_stride, \
                       uint64_t hot_dst_stride, const void *hot_src0, const void *hot_src1, void *hot_dst0

template <int NR>
__device__ __forceinline__ LaunchArgs<NR> with_hot(const LaunchArgs<NR> &a, uint64_t n, unsigned cols,
                                                   unsigned shape, uint64_t src_stride, uint64_t dst_stride,
                                                   const void *src0, const void *src1, void *dst0) {
    LaunchArgs<NR> b = a;
    b.n = n;
    b.cols = cols;
    b.waves = shape & 0xffffffu;
    b.n_dst = static_cast<int>((shape >> 24) & 15u) + 1;
    b.map_lc = shape >> 28;
    b.src_stride = src_stride;
    b.dst_stride = dst_stride;
    b.src[0] = src0;
    b.src[1] = src1;
    b.dst[0] = dst0;
    return b;
}
#define MPP_HOT_ARGS hot_n, hot_cols, hot_shape, hot_src_stride, hot_dst_stride, hot_src0, hot_src1, hot_dst0

// Entry of a kernel with preloaded fields: its working copy of the arguments
// with those fields substituted, and its workgroup's range -- slice ranges
// read from the argument block itself, strided ranges from the copy.
template <class C, bool SLICED, class F>
__device__ __forceinline__ void hot_entry(const LaunchArgs<C::RB> &a, uint64_t n, unsigned cols, unsigned shape,
                                          uint64_t src_stride, uint64_t dst_stride, const void *src0,
                                          const void *src1, void *dst0, F &&run) {
    const LaunchArgs<C::RB> h = with_hot(a, n, cols, shape, src_stride, dst_stride, src0, src1, dst0);
    RangeOff o;
    unsigned len;
    if constexpr (SLICED) {
        range_of<true>(a, o, len);
    } else {
        range_of<false>(h, o, len);
    }
    run(h, o, len);
}

// ---------------------------------------------------------------------------
// Kernels.  Single-shot: one wave tile per wave.  Streaming (register-staged
// or LDS-staged): ST = the store policy (kStoreKeep / kStoreStream), SLICED =
// the per-rank slice ranges of the broadcast schedule.  The plain streaming
// kernels and the residual ones (`_res`) differ only in their parameters:
// the plain ones take the preloaded leading fields; the residual and
// single-shot kernels take the argument block alone and are built without
// preloading.  Measured on MI355X: the substituted copies held live through
// the residual loop cost 8 VGPRs and one wave per SIMD (prefill + bias row
// 17.5 against 17.3 us, the row-strided block + bias 17.7 against 17.4 us),
// and the decode call does not gain (1.77 against 1.74 us per graph-replayed
// call), while the plain reduce does (R = 8: 371-378 against 378-386 us;
// 4-destination fp16 broadcast: 45.7-46.4 against 46.7-47.1 us; prefill:
// 16.09-16.16 against 16.16-16.20 us).
// ---------------------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(kSingleShotBlock) void k_single_shot(LaunchArgs<C::RB> a) {
    RangeOff o;
    unsigned len;
    range_of<false>(a, o, len);
    reduce_range<C, 1, false, kStoreKeep, kSingleShotBlock, false>(a, o, len);
}

#define MPP_STREAM_KERNELS(NAME, BLOCK, BODY, ST, SLICED)                                  \
    template <class C>                                                                  \
    __global__ __launch_bounds__(BLOCK) void NAME(MPP_HOT_PARAMS, LaunchArgs<C::RB> a) {   \
        hot_entry<C, SLICED>(a, MPP_HOT_ARGS,                                           \
                             [](const LaunchArgs<C::RB> &x, const RangeOff &o, unsigned len) { \
                                 BODY<C, ST, SLICED>(x, o, len);                        \
                             });                                                        \
    }                                                                                   \
    template <class C>                                                                  \
    __global__ __launch_bounds__(BLOCK) void NAME##_res(LaunchArgs<C::RB> a) {           \
        RangeOff o;                                                                     \
        unsigned len;                                                                   \
        range_of<SLICED>(a, o, len);                                                    \
        BODY<C, ST, SLICED>(a, o, len);                                                 \
    }
MPP_STREAM_KERNELS(k_stream_reg, stream_block(C::RB, C::RES, C::SW), stream_reg, kStoreKeep, false)
MPP_STREAM_KERNELS(k_stream_reg_nts, stream_block(C::RB, C::RES, C::SW), stream_reg, kStoreStream, false)
MPP_STREAM_KERNELS(k_stream_reg_sl, stream_block(C::RB, C::RES, C::SW), stream_reg, kStoreKeep, true)
MPP_STREAM_KERNELS(k_stream_reg_nts_sl, stream_block(C::RB, C::RES, C::SW), stream_reg, kStoreStream, true)
MPP_STREAM_KERNELS(k_stream_lds, kLdsBlock, stream_lds, kStoreKeep, false)
MPP_STREAM_KERNELS(k_stream_lds_nts, kLdsBlock, stream_lds, kStoreStream, false)
MPP_STREAM_KERNELS(k_stream_lds_sl, kLdsBlock, stream_lds, kStoreKeep, true)
MPP_STREAM_KERNELS(k_stream_lds_nts_sl, kLdsBlock, stream_lds, kStoreStream, true)
#undef MPP_STREAM_KERNELS
#undef MPP_HOT_ARGS
#undef MPP_HOT_PARAMS

// ---------------------------------------------------------------------------
// Two-rank contiguous kernels: the commonest call -- two active binary32
// partials, one binary32 destination, one contiguous range (the pages' own
// tensor-parallel case is two ranks) -- as a 1-D grid whose leading
// parameters are all a wave needs before its loads, every one preloaded into
// SGPRs: the tile count, the remainder, the destination, the two sources and
// the placement exponent (then, for the residual forms, the residual and its
// length, also preloaded, and the launch piece's phase in the row, read from
// the argument block while the partials' loads are in flight).  A wave reduces one wave tile with the
// arithmetic of the streaming kernels' binary32 path (acc = wire(src0),
// acc = RN32(acc + wire(src1)), then acc = RN32(acc + res[i]) with a
// residual; write-through stores); the wave after the last tile reduces the
// remainder element by element.  One wave per workgroup: measured on MI355X
// on the prefill call, 15.44-15.45 us against 15.48-15.50 us with four waves
// per workgroup, and 15.62 against 15.86-15.89 us with a 4096-element row
// (the four-wave form was also the more sensitive to where the buffers sit
// relative to each other).  Against the general streaming kernels
// (bit-identical outputs) the register-staged kernel's range, rank-mask and
// destination bookkeeping costs 0.3-0.45 us per prefill call, and both
// general families lose 0.9 us and more once a residual is fused.
//
// RK: 0 no residual, 1 element-wise residual (read once, non-temporal), 2-4
// a broadcast row of res_len elements (a multiple of 8; cached loads, the row
// is read by every row of the call): element i adds res[(i + phase) mod
// res_len].  The column of a lane part takes one AND for a power-of-two row
// (4), at most one wrap for a row of at least one wave tile (2), a remainder
// for a shorter row (3); the wave's first column takes one scalar remainder.
// The row loads follow the partials' loads: a part's fold waits for every
// load issued before its own, and row loads issued first or interleaved
// measured slower on MI355X.
// ---------------------------------------------------------------------------
constexpr int kPairBlock = 64;

template <int W>
__device__ __forceinline__ u32x4 pair_part(u32x4 a, u32x4 b) {
    float x[4], y[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        x[k] = f32_from_bits(a[k]);
        y[k] = f32_from_bits(b[k]);
    }
    wire_pair<W>(x[0], x[1]);
    wire_pair<W>(x[2], x[3]);
    wire_pair<W>(y[0], y[1]);
    wire_pair<W>(y[2], y[3]);
    return u32x4{bits_from_f32(x[0] + y[0]), bits_from_f32(x[1] + y[1]), bits_from_f32(x[2] + y[2]),
                 bits_from_f32(x[3] + y[3])};
}

__device__ __forceinline__ u32x4 add_res(u32x4 v, u32x4 r) {
    return u32x4{bits_from_f32(f32_from_bits(v[0]) + f32_from_bits(r[0])),
                 bits_from_f32(f32_from_bits(v[1]) + f32_from_bits(r[1])),
                 bits_from_f32(f32_from_bits(v[2]) + f32_from_bits(r[2])),
                 bits_from_f32(f32_from_bits(v[3]) + f32_from_bits(r[3]))};
}

// Column of element i + phase in a row of res_len elements, as the row kind
// RK computes it: c0 = the wave's first column (t + phase, below 2^31: both
// are below one launch piece), off < one wave tile.
template <int RK>
__device__ __forceinline__ unsigned pair_column(unsigned c0, unsigned off, unsigned res_len) {
    const unsigned c = c0 + off;
    if constexpr (RK == 4) return c & (res_len - 1);
    if constexpr (RK == 2) return c >= res_len ? c - res_len : c;
    return c % res_len;
}

template <int W, int RK>
__device__ __forceinline__ void pair_body(unsigned tiles, unsigned rem, float *dst, const float *src0,
                                          const float *src1, unsigned lc, const float *res, unsigned res_len,
                                          unsigned res_phase) {
    constexpr unsigned wpb = kPairBlock / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    // the grid size from the preloaded counts (the dispatch's own grid size
    // is a hidden argument past the preloaded dwords of the residual forms)
    const unsigned grid = (tiles + (rem != 0 ? 1u : 0u) + wpb - 1) / wpb;
    const unsigned w = xcd_virtual_block(blockIdx.x, grid, lc) * wpb +
                       __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (w >= tiles) {
        if (w == tiles && rem != 0) {
            // the tail: every load issued unguarded at a clamped index, then the
            // folds, then the guarded stores (see reduce_scalar)
            constexpr int K = kWaveTile / kWave;
            const size_t t = static_cast<size_t>(tiles) * kWaveTile;
            float x[K], y[K], r[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const unsigned e0 = lane + kWave * k;
                const unsigned e = e0 < rem ? e0 : rem - 1;
                x[k] = src0[t + e];
                y[k] = src1[t + e];
                if constexpr (RK == 1) r[k] = res[t + e];
                if constexpr (RK >= 2) r[k] = res[(static_cast<unsigned>(t) + e + res_phase) % res_len];
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float z = 0.0f, u = 0.0f;
                wire_pair<W>(x[k], z);
                wire_pair<W>(y[k], u);
                x[k] = x[k] + y[k];
                if constexpr (RK != 0) x[k] = x[k] + r[k];
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const unsigned e = lane + kWave * k;
                if (e < rem) dst[t + e] = x[k];
            }
        }
        return;
    }
    const size_t t = static_cast<size_t>(w) * kWaveTile;
    u32x4 a[2], b[2], r[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        a[j] = load16<true>(src0 + t + 256 * j + 4 * lane);
        b[j] = load16<true>(src1 + t + 256 * j + 4 * lane);
    }
    if constexpr (RK == 1) {
#pragma unroll
        for (int j = 0; j < 2; ++j) r[j] = load16<true>(res + t + 256 * j + 4 * lane);
    } else if constexpr (RK >= 2) {
        const unsigned base = static_cast<unsigned>(t) + res_phase;
        const unsigned c0 = RK == 4 ? base : base % res_len;
#pragma unroll
        for (int j = 0; j < 2; ++j) r[j] = load16<false>(res + pair_column<RK>(c0, 256 * j + 4 * lane, res_len));
    }
    float *out = dst + t;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        u32x4 v = pair_part<W>(a[j], b[j]);
        if constexpr (RK != 0) v = add_res(v, r[j]);
        store16_wt(out, kWaveTile * 4, (256 * j + 4 * lane) * 4, v);
    }
}

template <int W>
__global__ __launch_bounds__(kPairBlock) void k_pair(unsigned tiles, unsigned rem, float *dst, const float *src0,
                                                     const float *src1, unsigned lc) {
    pair_body<W, 0>(tiles, rem, dst, src0, src1, lc, nullptr, 1, 0);
}

template <int W, int RK>
__global__ __launch_bounds__(kPairBlock) void k_pair_res(unsigned tiles, unsigned rem, float *dst,
                                                         const float *src0, const float *src1, unsigned lc,
                                                         const float *res, unsigned res_len, unsigned res_phase) {
    pair_body<W, RK>(tiles, rem, dst, src0, src1, lc, res, res_len, res_phase);
}

// Kernels for two to four active binary32 partials (A) among more ranks, or
// for three or four ranks, into one binary32 destination, contiguous, no
// residual: the two-rank kernels' grid, preloaded parameters, placement and
// stores, with the active partials passed compacted in rank order.  An
// inactive rank contributes +0.0 at its place in the fold; adding +0.0 leaves
// every value but -0.0 unchanged (-0.0 becomes +0.0), and adding -0.0 leaves
// every value unchanged, so the fold adds z[g] = +0.0 or -0.0 at each gap g
// (before active partial g, and after the last at g = A) according to
// whether an inactive rank lies there (bit g of zmask): bit-identical with
// the fold over all R ranks, with no branch between the loads.  RES: an
// element-wise binary32 residual added after the fold, read once like the
// partials.
template <int W, int A>
__device__ __forceinline__ u32x4 few_part(const u32x4 (&v)[A], const float (&z)[A + 1]) {
    float x[A][4];
#pragma unroll
    for (int a = 0; a < A; ++a) {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[a][k] = f32_from_bits(v[a][k]);
        wire_pair<W>(x[a][0], x[a][1]);
        wire_pair<W>(x[a][2], x[a][3]);
    }
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float acc = x[0][k] + z[0];
#pragma unroll
        for (int a = 1; a < A; ++a) acc = (acc + z[a]) + x[a][k];
        o[k] = bits_from_f32(acc + z[A]);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
}

template <int W, int A, bool RES>
__global__ __launch_bounds__(kPairBlock) void k_few(unsigned tiles, unsigned rem, float *dst, const float *s0,
                                                    const float *s1, unsigned lc, const float *s2,
                                                    const float *s3, unsigned zmask, const float *res) {
    static_assert(A >= 2 && A <= 4, "two to four active partials");
    const int lane = threadIdx.x & (kWave - 1);
    const unsigned grid = tiles + (rem != 0 ? 1u : 0u);
    const unsigned w = xcd_virtual_block(blockIdx.x, grid, lc);
    const float *const s[4] = {s0, s1, s2, s3};
    float z[A + 1];
#pragma unroll
    for (int g = 0; g <= A; ++g) z[g] = ((zmask >> g) & 1u) != 0 ? 0.0f : -0.0f;
    if (w >= tiles) {
        if (w == tiles && rem != 0) {
            // the tail: every load issued unguarded at a clamped index, then the
            // folds, then the guarded stores (see reduce_scalar)
            constexpr int K = kWaveTile / kWave;
            const size_t t = static_cast<size_t>(tiles) * kWaveTile;
            float x[A][K], r[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const unsigned e0 = lane + kWave * k;
                const unsigned e = e0 < rem ? e0 : rem - 1;
#pragma unroll
                for (int a = 0; a < A; ++a) x[a][k] = s[a][t + e];
                if constexpr (RES) r[k] = res[t + e];
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
#pragma unroll
                for (int a = 0; a < A; ++a) {
                    float unused = 0.0f;
                    wire_pair<W>(x[a][k], unused);
                }
                float acc = x[0][k] + z[0];
#pragma unroll
                for (int a = 1; a < A; ++a) acc = (acc + z[a]) + x[a][k];
                x[0][k] = acc + z[A];
                if constexpr (RES) x[0][k] = x[0][k] + r[k];
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const unsigned e = lane + kWave * k;
                if (e < rem) dst[t + e] = x[0][k];
            }
        }
        return;
    }
    const size_t t = static_cast<size_t>(w) * kWaveTile;
    u32x4 v[2][A], rv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int a = 0; a < A; ++a) v[j][a] = load16<true>(s[a] + t + 256 * j + 4 * lane);
    if constexpr (RES) {
#pragma unroll
        for (int j = 0; j < 2; ++j) rv[j] = load16<true>(res + t + 256 * j + 4 * lane);
    }
    float *out = dst + t;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        u32x4 o = few_part<W, A>(v[j], z);
        if constexpr (RES) o = add_res(o, rv[j]);
        store16_wt(out, kWaveTile * 4, (256 * j + 4 * lane) * 4, o);
    }
}

// Two-rank kernels over row-strided tensors whose rows are whole wave tiles
// (cols a multiple of 512): the same per-tile work as the contiguous ones,
// over one 1-D grid of every row's tiles, so that the XCD placement runs span
// consecutive rows (a 2-D grid of a few workgroups per row would give each
// XCD the same column block of every row: the hardware's one-by-one order).
// Tile w is column block w mod tpr of row w / tpr (a shift when tpr, the
// tiles per row, is a power of two: P2, `tpr` then holding its log2).  The
// strides are in elements and below 2^32.  RK: 0 no residual, 1 an
// element-wise residual with its own row stride, 2 one bias row of cols
// elements (cached loads).
template <int W, int RK, bool P2>
__device__ __forceinline__ void pair_rows_body(unsigned tiles, unsigned tpr, unsigned src_stride,
                                               unsigned dst_stride, float *dst, const float *src0,
                                               const float *src1, unsigned lc, const float *res,
                                               unsigned res_stride) {
    const int lane = threadIdx.x & (kWave - 1);
    const unsigned w = xcd_virtual_block(blockIdx.x, tiles, lc);
    if (w >= tiles) return;
    const unsigned row = P2 ? w >> tpr : w / tpr;
    const unsigned col = (w - (P2 ? row << tpr : row * tpr)) * kWaveTile;
    const size_t s_off = static_cast<size_t>(row) * src_stride + col;
    u32x4 a[2], b[2], r[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        a[j] = load16<true>(src0 + s_off + 256 * j + 4 * lane);
        b[j] = load16<true>(src1 + s_off + 256 * j + 4 * lane);
    }
    if constexpr (RK == 1) {
        const size_t r_off = static_cast<size_t>(row) * res_stride + col;
#pragma unroll
        for (int j = 0; j < 2; ++j) r[j] = load16<true>(res + r_off + 256 * j + 4 * lane);
    } else if constexpr (RK == 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j) r[j] = load16<false>(res + col + 256 * j + 4 * lane);
    }
    float *out = dst + static_cast<size_t>(row) * dst_stride + col;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        u32x4 v = pair_part<W>(a[j], b[j]);
        if constexpr (RK != 0) v = add_res(v, r[j]);
        store16_wt(out, kWaveTile * 4, (256 * j + 4 * lane) * 4, v);
    }
}

// Two-rank kernel for 16-bit partials into a destination of the same 16-bit
// type W (bf16 or fp16; no residual): per element, both values widened
// exactly, one binary32 add, one rounding to W (binary32 has more than
// 2p + 2 bits for both types, so this is the correctly rounded add in W).
// One wave tile is 512 elements, lane l holding elements t + 8 l .. t + 8 l
// + 7 of each source in one 16-byte load; stores write-back, as the 16-bit
// layouts of the general kernels.  The same 1-D grid of one-wave workgroups,
// preloaded parameters and placement as k_pair; the wave after the last tile
// does the remainder.
template <int W>
__global__ __launch_bounds__(kPairBlock) void k_pair16(unsigned tiles, unsigned rem, uint16_t *dst,
                                                       const uint16_t *src0, const uint16_t *src1, unsigned lc) {
    const int lane = threadIdx.x & (kWave - 1);
    const unsigned grid = tiles + (rem != 0 ? 1u : 0u);
    const unsigned w = xcd_virtual_block(blockIdx.x, grid, lc);
    if (w >= tiles) {
        if (w == tiles && rem != 0) {
            // the tail: every load issued unguarded at a clamped index, then the
            // adds, then the guarded stores (see reduce_scalar)
            constexpr int K = kWaveTile / kWave;
            const size_t t = static_cast<size_t>(tiles) * kWaveTile;
            uint32_t p[K], q[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const unsigned e0 = lane + kWave * k;
                const unsigned e = e0 < rem ? e0 : rem - 1;
                p[k] = src0[t + e];
                q[k] = src1[t + e];
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float x, y, unused;
                widen_pair<W>(p[k], x, unused);
                widen_pair<W>(q[k], y, unused);
                p[k] = round_pack<W>(x + y, 0.0f);
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const unsigned e = lane + kWave * k;
                if (e < rem) dst[t + e] = static_cast<uint16_t>(p[k]);
            }
        }
        return;
    }
    const size_t e0 = static_cast<size_t>(w) * kWaveTile + 8 * lane;
    const u32x4 a = load16<true>(src0 + e0);
    const u32x4 b = load16<true>(src1 + e0);
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float x0, x1, y0, y1;
        widen_pair<W>(a[k], x0, x1);
        widen_pair<W>(b[k], y0, y1);
        v[k] = round_pack<W>(x0 + y0, x1 + y1);
    }
    store16<0>(dst + e0, v);
}

template <int W, int RK, bool P2>
__global__ __launch_bounds__(kPairBlock) void k_pair_rows(unsigned tiles, unsigned tpr, unsigned src_stride,
                                                          unsigned dst_stride, float *dst, const float *src0,
                                                          const float *src1, unsigned lc, const float *res,
                                                          unsigned res_stride) {
    pair_rows_body<W, RK, P2>(tiles, tpr, src_stride, dst_stride, dst, src0, src1, lc, res, res_stride);
}

}  // namespace

// ---------------------------------------------------------------------------
// Kernel tables.  Combination index (element types):
//   0 f32 wire, f32 src       1 bf16 wire, f32 src     2 f16 wire, f32 src
//   3 bf16 wire, bf16 src     4 f16 wire, f16 src
//   5 bf16 src / wire / dst   6 f16 src / wire / dst
// Rank bucket index: 0 -> R <= 2, 1 -> <= 4, 2 -> <= 8, 3 -> <= 16.
// ---------------------------------------------------------------------------
constexpr int kCombos = 7;
constexpr int kBuckets = 4;

#define MPP_ROW(KERNEL, W, SW, DN, M, RES)                                                   \
    {reinterpret_cast<const void *>(&KERNEL<Cfg<W, SW, DN, 2, M, RES>>),                   \
     reinterpret_cast<const void *>(&KERNEL<Cfg<W, SW, DN, 4, M, RES>>),                   \
     reinterpret_cast<const void *>(&KERNEL<Cfg<W, SW, DN, 8, M, RES>>),                   \
     reinterpret_cast<const void *>(&KERNEL<Cfg<W, SW, DN, 16, M, RES>>)}

#define MPP_TABLE(KERNEL, M, RES)                                                            \
    {MPP_ROW(KERNEL, AR_F32, false, false, M, RES), MPP_ROW(KERNEL, AR_BF16, false, false, M, RES), \
     MPP_ROW(KERNEL, AR_F16, false, false, M, RES), MPP_ROW(KERNEL, AR_BF16, true, false, M, RES),  \
     MPP_ROW(KERNEL, AR_F16, true, false, M, RES), MPP_ROW(KERNEL, AR_BF16, true, true, M, RES),    \
     MPP_ROW(KERNEL, AR_F16, true, true, M, RES)}

// Defined in the ar_k_*.hip files (one table group per file, so the files
// compile in parallel).  Indices of the streaming tables: [store_nt][sliced]
// [combination][rank bucket]; the name says residual (Res) and masked (M)
// instances.  The single-shot table is [residual][masked][combination]
// [rank bucket].
typedef const void *const StreamTable[2][2][kCombos][kBuckets];
extern const void *const kSingleShot[2][2][kCombos][kBuckets];
// two-rank contiguous kernels, indexed by [residual kind][wire type (ar_dtype)]
extern const void *const kPair[5][3];
extern const void *const kPair16[2];   // [0] fp16, [1] bf16
// kernels for two to four active binary32 partials, [element-wise residual][active partials - 2][wire type]
extern const void *const kFew[2][3][3];
// two-rank row-strided kernels, [residual kind][power-of-two tiles per row][wire type]
extern const void *const kPairRows[3][2][3];
extern StreamTable kStreamReg, kStreamRegM, kStreamRegRes, kStreamRegResM, kStreamLds, kStreamLdsM, kStreamLdsRes,
    kStreamLdsResM;

#define MPP_STREAM_TABLE(FAMILY, M, RES, SUFFIX)                                                      \
    {{MPP_TABLE(k_stream_##FAMILY##SUFFIX, M, RES), MPP_TABLE(k_stream_##FAMILY##_sl##SUFFIX, M, RES)},     \
     {MPP_TABLE(k_stream_##FAMILY##_nts##SUFFIX, M, RES), MPP_TABLE(k_stream_##FAMILY##_nts_sl##SUFFIX, M, RES)}}

}  // namespace mpp
