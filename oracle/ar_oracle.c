/*
 * ar_oracle.c -- plain scalar CPU oracle for the mixed-precision partial-sum
 * reduce.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU
 * baseline leg of the benchmark are the only callers.  It shares no code,
 * header, table or helper with the HIP library and must never be linked into
 * it.
 *
 * What it computes, for 0 <= i < n and every destination d < n_dst:
 *
 *     w_r      = widen(round_W(src_r[i]))        r = 0 .. R-1
 *     acc      = w_0
 *     acc      = RN_D(acc + w_r)                 r = 1 .. R-1, rank order
 *     acc      = RN_D(acc + res[i mod L])        only with a residual
 *     dst_d[i] = acc                             (not re-rounded to the wire)
 *
 * RN_D is one rounding to the destination type D: binary32 (the common
 * case), or binary16 / bfloat16 when the destination, the wire and the
 * sources all have that type.
 *
 * Sources (the pages are cited by title and passage):
 *   - "CUDA allreduce.cu" page (toy 0.8.0 diff of ggml-cuda/allreduce.cu),
 *     comment block "Chunked kernel AllReduce", phase 1: every rank casts its
 *     caller-typed partial to the wire type before it leaves the device.
 *   - same page, phase 3 and the "Combined load-convert-add kernel": the
 *     receiver rounds its *own* partial through the wire type as well, adds
 *     the two in float and stores the caller's type, so every rank produces
 *     the same bits.
 *   - "Hexagon allreduce-ops.c" page (llama.cpp fork, ggml-hexagon/htp),
 *     allreduce_thread_dma_1d: the sources are summed in the fixed order
 *     s0 + s1, then + s2, ... and the block is written to every destination
 *     (n_dsts defaults to n_ranks in op_allreduce).
 *
 * Inactive ranks: a NULL source is a rank that skipped its compute; its
 * partial is all +0.0, which the CUDA page obtains by zeroing such a shard
 * before the same reduce runs (comments on inactive shards and NCCL /
 * meta-backend semantics in ggml_cuda_ar_allreduce).  Its wire value is
 * therefore +0.0 and it still takes part in the fold (so -0 + inactive = +0).
 *
 * Readings where the pages leave a step open (all pinned by the tests):
 *   - round_W is IEEE round-to-nearest-ties-to-even for both bf16 and fp16
 *     (the conversion routine itself is not printed on the pages).  NaN maps
 *     to a quiet NaN of the same sign; the NaN payload is not part of the
 *     contract.
 *   - The fold starts from w_0 (not from +0.0), so [-0, -0] gives -0.
 *   - The accumulator is binary32 with one rounding per add; no wider or
 *     compensated arithmetic.
 *   - Subnormals are kept everywhere (no flush-to-zero on input or output).
 *   - A narrow destination (binary16 / bfloat16, with the same wire and
 *     source type, the only narrow combinations the CUDA page launches)
 *     rounds to its type after every add, the residual add included; for
 *     R = 2 this is the CUDA page's float add followed by the cast to T_dst.
 *   - The residual is added once, after the last rank, in the destination
 *     type, and is not rounded through the wire type.
 *
 * Build with:  gcc -O2 -fno-fast-math -ffp-contract=off -shared -fPIC
 * The float additions below are ordinary C float additions; on x86-64
 * (SSE, FLT_EVAL_METHOD == 0) each one is a single binary32 RN addition.
 * The entry points clear MXCSR's FTZ and DAZ bits for the duration of the
 * call so a caller that set them cannot change the result.
 */
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#include <xmmintrin.h>

#if !defined(FLT_EVAL_METHOD)
#include <float.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* ---------------------------------------------------------------------------
 * binary32 <-> raw bits
 * ------------------------------------------------------------------------- */
static float orc_bits_to_float(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t orc_float_to_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* ---------------------------------------------------------------------------
 * binary32 -> bfloat16, round to nearest, ties to even.
 *
 * bfloat16 is binary32 with the low 16 significand bits removed, so the
 * narrowing keeps the upper half and rounds on the dropped half: above one
 * half-ulp rounds up, below rounds down, exactly one half rounds to the even
 * neighbour.  A carry out of the significand increments the exponent, which
 * is the correct result, including the step from the largest finite value to
 * infinity.  NaN is handled first so that a NaN whose payload sits only in
 * the dropped bits cannot turn into infinity.
 * ------------------------------------------------------------------------- */
uint16_t orc_round_bf16(uint32_t x) {
    const uint32_t exp_field = x & 0x7F800000u;
    const uint32_t frac      = x & 0x007FFFFFu;
    if (exp_field == 0x7F800000u && frac != 0) {
        return (uint16_t)((x >> 16) | 0x0040u);          /* quiet NaN, sign kept */
    }
    uint32_t kept    = x >> 16;
    uint32_t dropped = x & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) {
        kept += 1u;
    }
    return (uint16_t)kept;
}

uint32_t orc_widen_bf16(uint16_t h) {
    return (uint32_t)h << 16;                             /* exact */
}

/* ---------------------------------------------------------------------------
 * binary32 -> binary16, IEEE 754 convertFormat with roundTiesToEven.
 *
 * binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Normal range 2^-14 .. 65504; subnormals are multiples of 2^-24.
 * ------------------------------------------------------------------------- */
uint16_t orc_round_f16(uint32_t x) {
    const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    const int      e    = (int)((x >> 23) & 0xFFu);
    const uint32_t m    = x & 0x007FFFFFu;

    if (e == 0xFF) {                                      /* Inf or NaN */
        if (m != 0) {
            return (uint16_t)(sign | 0x7C00u | 0x0200u | (m >> 13));
        }
        return (uint16_t)(sign | 0x7C00u);
    }
    if (e == 0) {
        /* zero or a binary32 subnormal: magnitude < 2^-126, far below half of
         * the smallest binary16 subnormal (2^-25), so it rounds to zero. */
        return sign;
    }

    const int E = e - 127;                                /* unbiased exponent */
    if (E > 15) {
        return (uint16_t)(sign | 0x7C00u);                /* >= 2^16: overflow */
    }

    if (E >= -14) {
        /* normal binary16 candidate: keep 10 of 23 fraction bits. */
        uint32_t kept    = m >> 13;
        uint32_t dropped = m & 0x1FFFu;
        uint32_t out     = ((uint32_t)(E + 15) << 10) | kept;
        if (dropped > 0x1000u || (dropped == 0x1000u && (kept & 1u))) {
            out += 1u;                                    /* may carry to Inf */
        }
        return (uint16_t)(sign | out);
    }

    /* binary16 subnormal range: the value is sig * 2^(E-23) with the hidden
     * bit restored; expressed in units of 2^-24 that is sig * 2^(E+1), i.e.
     * sig shifted right by s = -(E+1) >= 14 places. */
    const uint64_t sig = (uint64_t)(m | 0x00800000u);
    int s = -(E + 1);
    if (s > 40) s = 40;                                   /* all bits dropped */
    uint64_t kept    = sig >> s;
    uint64_t dropped = sig & ((1ull << s) - 1ull);
    uint64_t half    = 1ull << (s - 1);
    if (dropped > half || (dropped == half && (kept & 1ull))) {
        kept += 1ull;                                     /* may become 0x400 */
    }
    return (uint16_t)(sign | (uint16_t)kept);
}

uint32_t orc_widen_f16(uint16_t h) {
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    int            e    = (h >> 10) & 0x1F;
    uint32_t       m    = h & 0x03FFu;

    if (e == 0x1F) {
        return sign | 0x7F800000u | (m << 13);            /* Inf / NaN */
    }
    if (e == 0) {
        if (m == 0) {
            return sign;                                  /* signed zero */
        }
        /* subnormal m * 2^-24: normalise so the leading one is bit 10 */
        e = 1;
        while ((m & 0x0400u) == 0) {
            m <<= 1;
            e -= 1;
        }
        m &= 0x03FFu;
    }
    return sign | ((uint32_t)(e + 112) << 23) | (m << 13);
}

/* ---------------------------------------------------------------------------
 * The wire value of one source element: round through the wire type, then
 * widen back exactly.  When the source already holds the wire type the
 * rounding is the identity and only the widening remains.
 * ------------------------------------------------------------------------- */
static float orc_wire_value(const void *src, size_t i, int src_type, int wire_type) {
    if (src == NULL) {
        return 0.0f;                                      /* inactive rank */
    }
    if (src_type == ORC_F32) {
        const uint32_t bits = ((const uint32_t *)src)[i];
        switch (wire_type) {
        case ORC_F32:  return orc_bits_to_float(bits);
        case ORC_BF16: return orc_bits_to_float(orc_widen_bf16(orc_round_bf16(bits)));
        case ORC_F16:  return orc_bits_to_float(orc_widen_f16(orc_round_f16(bits)));
        default:       return 0.0f;
        }
    }
    const uint16_t h = ((const uint16_t *)src)[i];
    return orc_bits_to_float(src_type == ORC_BF16 ? orc_widen_bf16(h) : orc_widen_f16(h));
}

/* MXCSR bit 15 = FTZ, bit 6 = DAZ. */
static unsigned orc_enter_ieee(void) {
    const unsigned saved = _mm_getcsr();
    _mm_setcsr(saved & ~((1u << 15) | (1u << 6)));
    return saved;
}

static void orc_leave_ieee(unsigned saved) {
    _mm_setcsr(saved);
}

/* ---------------------------------------------------------------------------
 * Narrowing of a binary32 value to the destination type and back (exact
 * widening): the identity for binary32, RNE for binary16 / bfloat16.
 * ------------------------------------------------------------------------- */
static float orc_to_dst(float x, int dst_type) {
    const uint32_t bits = orc_float_to_bits(x);
    switch (dst_type) {
    case ORC_BF16: return orc_bits_to_float(orc_widen_bf16(orc_round_bf16(bits)));
    case ORC_F16:  return orc_bits_to_float(orc_widen_f16(orc_round_f16(bits)));
    default:       return x;
    }
}

/* Element i of a destination-typed array, widened exactly. */
static float orc_dst_value(const void *p, size_t i, int dst_type) {
    if (dst_type == ORC_F32) return ((const float *)p)[i];
    const uint16_t h = ((const uint16_t *)p)[i];
    return orc_bits_to_float(dst_type == ORC_BF16 ? orc_widen_bf16(h) : orc_widen_f16(h));
}

/* Store a value that already lies in the destination type. */
static void orc_store_dst(void *p, size_t i, float v, int dst_type) {
    if (dst_type == ORC_F32) {
        ((float *)p)[i] = v;
    } else {
        const uint32_t bits = orc_float_to_bits(v);
        ((uint16_t *)p)[i] = dst_type == ORC_BF16 ? orc_round_bf16(bits) : orc_round_f16(bits);
    }
}

/* ---------------------------------------------------------------------------
 * The reduce, general form.
 *   dst      : n_dst arrays of dst_type, n elements each.
 *   srcs     : R arrays of src_type (a NULL entry is an inactive rank
 *              contributing +0.0).
 *   residual : NULL, or residual_len elements of dst_type added after the
 *              last rank ("Hexagon allreduce-ops.c" page, the HAS_ADD forms
 *              of allreduce_thread_dma_1d / _2d: once the ranks are summed,
 *              src[2 * n_ranks] is added, element-wise, or one row added to
 *              every row in the IS_ROW_BCAST form).  residual_len == n is the
 *              element-wise form; a smaller residual_len that divides n is
 *              one row broadcast over the n / residual_len rows, element i
 *              taking residual[i mod residual_len].  The residual is local to
 *              the receiving rank and never crosses the wire, so it is not
 *              rounded through the wire type.
 *   dst_type : binary32, or binary16 / bfloat16 with wire_type == dst_type.
 *              A narrow destination accumulates in its own type: every add
 *              is rounded to dst_type ("CUDA allreduce.cu" page, the
 *              half / nv_bfloat16 instances of the chunked kernel, whose sum
 *              is cast to T_dst; "Hexagon allreduce-ops.c" page, the f16
 *              instances adding natively in __fp16).  The add is done in
 *              binary32 and then rounded once to dst_type; binary32 has at
 *              least 2p + 2 significand bits for p = 11 and p = 8, so this
 *              equals a correctly rounded add in dst_type.
 * Returns 0 on success, -1 on an argument the oracle does not define.
 * ------------------------------------------------------------------------- */
int orc_reduce_ex(void *const *dst, int n_dst, int dst_type, const void *const *srcs, int R,
                  size_t n, int src_type, int wire_type, const void *residual, size_t residual_len) {
    if (R < 1 || n_dst < 1 || dst == NULL || srcs == NULL) return -1;
    if (wire_type < ORC_F32 || wire_type > ORC_BF16) return -1;
    if (src_type != ORC_F32 && src_type != wire_type) return -1;
    if (dst_type != ORC_F32 && (dst_type != wire_type || src_type != wire_type)) return -1;
    if (residual != NULL && (residual_len == 0 || n % residual_len != 0)) return -1;

    const unsigned saved = orc_enter_ieee();
    for (size_t i = 0; i < n; ++i) {
        float acc = orc_wire_value(srcs[0], i, src_type, wire_type);
        for (int r = 1; r < R; ++r) {
            const float w = orc_wire_value(srcs[r], i, src_type, wire_type);
            acc = acc + w;
            if (dst_type != ORC_F32) acc = orc_to_dst(acc, dst_type);
        }
        if (residual != NULL) {
            acc = acc + orc_dst_value(residual, i % residual_len, dst_type);
            if (dst_type != ORC_F32) acc = orc_to_dst(acc, dst_type);
        }
        for (int d = 0; d < n_dst; ++d) {
            orc_store_dst(dst[d], i, acc, dst_type);
        }
    }
    orc_leave_ieee(saved);
    return 0;
}

/* The reduce into binary32 destinations without a residual. */
int orc_reduce(float *const *dst, int n_dst, const void *const *srcs, int R,
               size_t n, int src_type, int wire_type) {
    return orc_reduce_ex((void *const *)dst, n_dst, ORC_F32, srcs, R, n, src_type, wire_type, NULL, 0);
}

/* ---------------------------------------------------------------------------
 * The reduce over row-strided tensors ("Hexagon allreduce-ops.c" page,
 * allreduce_thread_dma_2d: each rank's rows are fetched with the tensor's
 * row stride nb[1] and ne0 elements per row; with IS_ROW_BCAST one residual
 * row is added to every row).  Row i, column j of a tensor lives at element
 * i * stride + j; the columns cols .. stride-1 of each row are not part of
 * the tensor and are never written.  The arithmetic of every element is that
 * of orc_reduce_ex.  res_stride 0 with a residual is the broadcast row.
 * ------------------------------------------------------------------------- */
int orc_reduce_rows(void *const *dst, int n_dst, int dst_type, const void *const *srcs, int R,
                    size_t rows, size_t cols, size_t src_stride, size_t dst_stride, int src_type,
                    int wire_type, const void *residual, size_t res_stride) {
    if (R < 1 || n_dst < 1 || dst == NULL || srcs == NULL) return -1;
    if (wire_type < ORC_F32 || wire_type > ORC_BF16) return -1;
    if (src_type != ORC_F32 && src_type != wire_type) return -1;
    if (dst_type != ORC_F32 && (dst_type != wire_type || src_type != wire_type)) return -1;
    if (src_stride < cols || dst_stride < cols) return -1;
    if (residual != NULL && res_stride != 0 && res_stride < cols) return -1;

    const unsigned saved = orc_enter_ieee();
    for (size_t i = 0; i < rows; ++i) {
        for (size_t j = 0; j < cols; ++j) {
            const size_t si = i * src_stride + j;
            float acc = orc_wire_value(srcs[0], si, src_type, wire_type);
            for (int r = 1; r < R; ++r) {
                acc = acc + orc_wire_value(srcs[r], si, src_type, wire_type);
                if (dst_type != ORC_F32) acc = orc_to_dst(acc, dst_type);
            }
            if (residual != NULL) {
                acc = acc + orc_dst_value(residual, i * res_stride + j, dst_type);
                if (dst_type != ORC_F32) acc = orc_to_dst(acc, dst_type);
            }
            for (int d = 0; d < n_dst; ++d) {
                orc_store_dst(dst[d], i * dst_stride + j, acc, dst_type);
            }
        }
    }
    orc_leave_ieee(saved);
    return 0;
}

/* Array forms of the conversions, used by the exhaustive pins. */
void orc_round_bf16_array(const uint32_t *x, uint16_t *out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_round_bf16(x[i]);
}

void orc_round_f16_array(const uint32_t *x, uint16_t *out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_round_f16(x[i]);
}

void orc_widen_bf16_array(const uint16_t *h, uint32_t *out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_widen_bf16(h[i]);
}

void orc_widen_f16_array(const uint16_t *h, uint32_t *out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_widen_f16(h[i]);
}

/* One binary32 addition under the same IEEE settings as orc_reduce. */
void orc_add_f32_array(const float *a, const float *b, float *out, size_t n) {
    const unsigned saved = orc_enter_ieee();
    for (size_t i = 0; i < n; ++i) out[i] = a[i] + b[i];
    orc_leave_ieee(saved);
}

/* Keeps the bit helpers referenced in builds that only use the arrays. */
uint32_t orc_f32_bits(float f) { return orc_float_to_bits(f); }
