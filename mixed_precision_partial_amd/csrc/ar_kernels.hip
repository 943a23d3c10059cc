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
__device__ __forceinline__ void tile_store(float *dst, size_t t, int lane, const float (&acc)[8]) {
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

// U consecutive wave tiles starting at element `t` (already slice-relative
// plus slice offset).  All loads of the batch are issued before the fold.
template <int W, bool SW, int RB, int U, bool NT>
__device__ __forceinline__ void reduce_tiles(const KernelArgs &a, size_t t, int lane) {
    constexpr int K = Tile<SW>::kRaw;
    u32x4 raw[RB][U][K];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        if (r < 2 || r < a.R) {
#pragma unroll
            for (int u = 0; u < U; ++u) tile_load<W, SW, NT>(a.src[r], t + u * kWaveTile, lane, raw[r][u]);
        }
    }
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) tile_values<W, SW>(raw[0][u], acc[u]);
#pragma unroll
    for (int r = 1; r < RB; ++r) {
        if (r < 2 || r < a.R) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float w[8];
                tile_values<W, SW>(raw[r][u], w);
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[u][k] = acc[u][k] + w[k];
            }
        }
    }
#pragma unroll
    for (int d = 0; d < RB; ++d) {
        if (d < a.n_dst) {
#pragma unroll
            for (int u = 0; u < U; ++u) tile_store<SW, NT>(a.dst[d], t + u * kWaveTile, lane, acc[u]);
        }
    }
}

// Elements [begin, end) of the launch, one per lane per step (end - begin is
// below one wave tile, so this is at most 8 steps).
template <int W, bool SW, int RB>
__device__ __forceinline__ void reduce_scalar(const KernelArgs &a, size_t begin, size_t end, int lane) {
    for (size_t e = begin + lane; e < end; e += kWave) {
        float acc = wire_one<W, SW>(a.src[0], e);
#pragma unroll
        for (int r = 1; r < RB; ++r) {
            if (r < 2 || r < a.R) acc = acc + wire_one<W, SW>(a.src[r], e);
        }
#pragma unroll
        for (int d = 0; d < RB; ++d) {
            if (d < a.n_dst) a.dst[d][e] = acc;
        }
    }
}

// Walk the wave tiles of this workgroup's slice: batches of U tiles first,
// then single tiles, then the element remainder on wave 0 of workgroup 0.
template <int W, bool SW, int RB, int U, bool NT>
__device__ __forceinline__ void reduce_slice(const KernelArgs &a) {
    const int lane = threadIdx.x & (kWave - 1);
    const unsigned wpb = blockDim.x / kWave;
    const unsigned gw = blockIdx.x * wpb + threadIdx.x / kWave;
    const unsigned nw = gridDim.x * wpb;
    size_t off;
    unsigned len;
    if (a.chunk_elems != 0) {
        const unsigned start = blockIdx.y * a.chunk_elems;
        off = start;
        len = (a.n - start) < a.chunk_elems ? (a.n - start) : a.chunk_elems;
    } else {
        off = a.slice_start[blockIdx.y];
        len = a.slice_len[blockIdx.y];
    }

    const unsigned big = kWaveTile * U;
    const unsigned n_big = len / big;
    for (unsigned t = gw; t < n_big; t += nw) {
        reduce_tiles<W, SW, RB, U, NT>(a, off + (size_t)t * big, lane);
    }
    const unsigned done = n_big * big;
    if constexpr (U > 1) {
        const unsigned n_one = (len - done) / kWaveTile;
        for (unsigned t = gw; t < n_one; t += nw) {
            reduce_tiles<W, SW, RB, 1, NT>(a, off + done + (size_t)t * kWaveTile, lane);
        }
    }
    const unsigned vec_end = (len / kWaveTile) * kWaveTile;
    if (vec_end < len && blockIdx.x == 0 && threadIdx.x < kWave) {
        reduce_scalar<W, SW, RB>(a, off + vec_end, off + len, lane);
    }
}

template <int W, bool SW, int RB>
__global__ __launch_bounds__(256) void k_single_shot(KernelArgs a) {
    reduce_slice<W, SW, RB, 1, false>(a);
}

// Tiles per batch of the streaming kernel: about 16 dwordx4 loads in flight
// per lane (R x U x loads-per-tile), at least 1 and at most 4 tiles.
constexpr int stream_batch(bool src_is_wire, int rank_bucket) {
    const int per_tile = (src_is_wire ? 1 : 2) * rank_bucket;
    const int u = 16 / per_tile;
    return u < 1 ? 1 : (u > 4 ? 4 : u);
}

template <int W, bool SW, int RB>
__global__ __launch_bounds__(256) void k_stream_reg(KernelArgs a) {
    reduce_slice<W, SW, RB, stream_batch(SW, RB), true>(a);
}

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

const void *const kSingleShot[5][4] = MPP_TABLE(k_single_shot);
const void *const kStreamReg[5][4] = MPP_TABLE(k_stream_reg);

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
        s.block = 64;
        const unsigned tiles = (max_slice_len + kWaveTile - 1) / kWaveTile;
        unsigned g = tiles == 0 ? 1 : tiles;
        const unsigned cap = static_cast<unsigned>(cu_count) * 16u;
        if (g > cap) g = cap;
        s.grid_x = grid_override > 0 ? static_cast<unsigned>(grid_override) : g;
        return s;
    }
    s.block = 256;
    const unsigned wpb = s.block / kWave;
    const unsigned per_wave = stream_tile_elems(family, src_is_wire, R);
    const unsigned batches = (max_slice_len + per_wave - 1) / per_wave;
    unsigned g = (batches + wpb - 1) / wpb;
    if (g == 0) g = 1;
    // resident-grid cap: 8 workgroups of 4 waves per CU, shared by the slices
    unsigned cap = static_cast<unsigned>(cu_count) * 8u / (n_slices ? n_slices : 1u);
    if (cap < 1) cap = 1;
    if (g > cap) g = cap;
    s.grid_x = grid_override > 0 ? static_cast<unsigned>(grid_override) : g;
    return s;
}

hipError_t launch(Family family, int wire, bool src_is_wire, const KernelArgs &args,
                  const LaunchShape &shape, hipStream_t stream) {
    const int c = combo_index(wire, src_is_wire);
    const int b = bucket_index(args.R);
    const void *fn = nullptr;
    switch (family) {
    case Family::SingleShot: fn = kSingleShot[c][b]; break;
    case Family::StreamReg:  fn = kStreamReg[c][b]; break;
    default:                 return hipErrorNotSupported;
    }
    KernelArgs a = args;
    void *kargs[] = {&a};
    return hipLaunchKernel(fn, dim3(shape.grid_x, shape.grid_y, 1), dim3(shape.block, 1, 1), kargs,
                           shape.lds_bytes, stream);
}

}  // namespace mpp
