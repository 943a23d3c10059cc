/*
 * ar.h -- C ABI of the MI355X (gfx950) mixed-precision partial-sum reduce.
 *
 * The operation: R partial activations (one per tensor-parallel rank) are
 * summed element-wise into a binary32 result (or, for 16-bit tensors, a
 * result of their own type).  Every partial -- the receiving rank's own
 * included -- is first rounded through a possibly narrower "wire" type, and
 * the rounded values are added in the destination type in the fixed rank
 * order 0, 1, ..., R-1, so every rank computes the same bits.
 *
 *   for 0 <= i < n, for every destination d:
 *       w_r       = widen(round_W(src_r[i]))          r = 0 .. R-1
 *       acc       = w_0
 *       acc       = RN_D(acc + w_r)                   r = 1 .. R-1
 *       acc       = RN_D(acc + res[i mod L])          ar_reduce_add only
 *       dst_d[i]  = acc
 *   RN_D rounds to nearest even in the destination type D: binary32, or
 *   binary16 / bfloat16 when destination, wire and sources share that type.
 *
 * Passages this follows (page title, then the passage):
 *   - "CUDA allreduce.cu" page (toy 0.8.0 diff of ggml-cuda/allreduce.cu):
 *     the comment block "Chunked kernel AllReduce" (phase 1 casts the
 *     caller-typed partial to the wire type; phase 3 rounds the local
 *     partial through the same type and adds in float) and the comment on
 *     the "Combined load-convert-add kernel".
 *   - "Hexagon allreduce-ops.c" page (llama.cpp fork, ggml-hexagon/htp):
 *     allreduce_thread_dma_1d (fixed-order sum s0+s1, then +s2 ..., and the
 *     write of each block to every destination; each rank reduces its own
 *     element range), its HAS_ADD forms and the 2-D IS_ROW_BCAST form (a
 *     residual added after the ranks, element-wise or one row per row), the
 *     f16 instances (sums kept in the tensor's own 16-bit type), and
 *     op_allreduce (rank-count checks, n_dsts).
 *   - "CUDA allreduce.cu" page, the chunked kernel's (half, half) and
 *     (nv_bfloat16, nv_bfloat16) instances: 16-bit tensors are reduced in
 *     their own type, the float sum cast back to it.
 *   - "llama.cpp commit log" page: the Vulkan comm hook commit (partials
 *     narrowed to F16 before the host transfer and added into the fp32
 *     result; a chunked pipeline for prefill and a single-shot path for
 *     decode) and the SYCL tensor-parallel commit (BF16-compressed large
 *     path, no per-call host synchronisation).
 *
 * All R ranks live on one GPU here: each rank's partial is a separate
 * buffer, in HBM or (host-staged mode) in pinned host memory.
 *
 * Conventions shared by every entry point:
 *   - Return value: an ar_status code.  Nothing aborts the process.
 *   - A call that fails validation enqueues no GPU work.
 *   - ar_reduce is asynchronous: work is enqueued on `hip_stream` (a
 *     hipStream_t, NULL = the null stream) and the call returns without
 *     waiting.  No host synchronisation happens inside it.
 *   - The caller owns every dst / src buffer; they must stay alive and
 *     unmodified until the enqueued work completes in stream order.
 *   - A context is not thread-safe: one host thread at a time per ar_ctx.
 */
#ifndef MPP_AR_H
#define MPP_AR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque, library-owned state: device, internal copy stream and events,
 * lazily allocated HBM scratch for host-staged mode. */
typedef struct ar_ctx ar_ctx;

/* Element types.  A 16-bit dst_type needs wire_type == dst_type (its sources
 * hold that type too). */
typedef enum { AR_F32 = 0, AR_F16 = 1, AR_BF16 = 2 } ar_dtype;

/* Schedules, in the low 8 bits of `mode`.
 *   AR_MODE_AUTO         SINGLE_SHOT when the wire bytes of all ranks,
 *                        R * n * sizeof(wire), are below twice the
 *                        single-shot limit (the limit is per rank at
 *                        R = 2), CHUNKED otherwise; sources in pinned host
 *                        memory select HOST_STAGED.
 *   AR_MODE_SINGLE_SHOT  one low-latency launch for decode-sized vectors.
 *   AR_MODE_CHUNKED      one bandwidth-bound launch over the whole tensor,
 *                        work planned in chunks of `chunk_bytes` wire bytes
 *                        per rank.
 *   AR_MODE_RS_BCAST     per-rank slice schedule: simulated rank r reduces
 *                        its own slice and writes it to all R destinations
 *                        (n_dst = R; `dst` holds R pointers).
 *   AR_MODE_HOST_STAGED  sources are pinned host buffers; by default the add
 *                        kernel reads them directly through their device
 *                        mapping; with host_path 1, chunks are copied to HBM
 *                        scratch on an internal copy stream while the add
 *                        kernel runs on `hip_stream`.
 * The result bytes do not depend on the mode, the chunk size or the launch
 * shape. */
enum {
    AR_MODE_AUTO        = 0,
    AR_MODE_SINGLE_SHOT = 1,
    AR_MODE_CHUNKED     = 2,
    AR_MODE_RS_BCAST    = 3,
    AR_MODE_HOST_STAGED = 4
};
#define AR_MODE_MASK 0xFFu
/* Flag: the sources already hold wire_type values (a peer narrowed them),
 * so round_W is the identity and each element is read at the wire width. */
#define AR_SRC_WIRE 0x100u
/* Flag: a NULL entry in srcs is an inactive rank (it skipped its compute);
 * its partial is +0.0 everywhere and still takes part in the fold, as the
 * CUDA allreduce.cu page does by zeroing such a shard before reducing.
 * Without the flag a NULL source is AR_ERR_INVALID. */
#define AR_SRC_INACTIVE_NULL 0x200u

#define AR_MAX_RANKS 16

typedef enum {
    AR_OK              = 0,
    AR_ERR_INVALID     = 1,  /* bad argument: see ar_reduce                */
    AR_ERR_UNSUPPORTED = 2,  /* valid request the library does not implement */
    AR_ERR_NOMEM       = 3,  /* allocation failed                           */
    AR_ERR_RUNTIME     = 4   /* a HIP runtime call failed                   */
} ar_status;

/* Optional tuning, read once by ar_init.  Zero fields take the defaults;
 * environment variables AR_SINGLE_SHOT_MAX_BYTES, AR_CHUNK_BYTES,
 * AR_HOST_CHUNK_BYTES, AR_HOST_SLOTS, AR_GRID_WGS, AR_STREAM_KERNEL,
 * AR_STORE_POLICY, AR_HOST_PATH, AR_XCD_RUN_ELEMS and AR_OCCUPANCY_HOLD
 * override the defaults when cfg is NULL or the field is zero. */
typedef struct {
    size_t single_shot_max_bytes; /* AUTO threshold, wire bytes per rank at R = 2
                                     (2x this over all ranks); 0 -> 1 MiB */
    size_t chunk_bytes;           /* CHUNKED / RS_BCAST plan unit, wire bytes per rank; 0 -> 4 MiB */
    size_t host_chunk_bytes;      /* HOST_STAGED copy unit, source bytes per rank;
                                     0 -> clamp(bytes/2, 512 KiB, 64 MiB) per call */
    int    host_slots;            /* HOST_STAGED scratch slots (>= 1); 0 -> 3 */
    int    grid_wgs;              /* CHUNKED / RS_BCAST workgroups; 0 -> tuned per shape */
    int    stream_kernel;         /* 0 auto (the family measured faster on MI355X
                                     for the call's schedule, source and
                                     destination widths, residual and rank count;
                                     ar_plan_query reports the choice),
                                     1 register-staged, 2 LDS-staged */
    int    store_policy;          /* destination stores: 0 auto (streaming when the
                                     call writes at least as many bytes as it
                                     reads, kept otherwise), 1 kept in the cache
                                     hierarchy (device-scope write-through for fp32
                                     sources, write-back for 16-bit ones), 2 streaming
                                     (non-temporal) */
    int    host_path;             /* HOST_STAGED: 0 auto (= 2), 1 copy-engine chunks
                                     into HBM scratch on the internal copy stream,
                                     overlapped with the add kernel (the CUs stay
                                     free while bytes cross PCIe), 2 the kernel reads
                                     the pinned buffers directly over PCIe (no
                                     scratch, lowest latency) */
    size_t xcd_run_elems;         /* workgroup placement of the streaming kernels
                                     over MI355X's 8 XCDs (the dispatcher gives
                                     workgroup b to XCD b mod 8): workgroups are
                                     renumbered so that each XCD streams runs of
                                     about this many elements of every source, the
                                     8 XCDs' runs side by side, round after round.
                                     0 -> automatic (for R <= 4: 2^17, or 2^18 in the
                                     broadcast schedule; none beyond);
                                     a value below one workgroup's share (e.g. 1)
                                     -> no renumbering.  No effect on any result */
    int    occupancy_hold;        /* resident waves per CU the streaming launches
                                     are held to, by dynamic LDS the kernels do
                                     not use (asked for only when a launch's grid
                                     fills every CU beyond the hold): 0 automatic
                                     (the binary32 two-rank kernels 18, 14 with
                                     a residual, the kernels for two to four
                                     active partials 18, 14 or 10, with a
                                     residual 14, 10 or 8 -- fewer
                                     loads in flight per CU stream faster on
                                     MI355X -- and the general kernels and the
                                     16-bit two-rank kernel unheld), -1 no
                                     hold, 1..32 every register-, LDS-staged,
                                     two-rank and few-partial launch held to
                                     that many (single-shot launches are never
                                     held).  No effect on any result */
} ar_config;

/* Create a context on HIP device `hip_device`.
 * Follows the "CUDA allreduce.cu" page's ggml_cuda_ar_pipeline_init: set-up
 * either yields a usable handle or reports failure (that function returns
 * nullptr so the caller falls back, and releases whatever it had created
 * first); here the failure is a status code and nothing is left allocated.
 *   out  : receives the context (set to NULL on failure).
 *   cfg  : NULL for defaults (plus AR_* environment overrides).
 * Errors: AR_ERR_INVALID (out NULL, device index out of range, negative or
 *         inconsistent cfg fields), AR_ERR_UNSUPPORTED (the device is not a
 *         gfx950 part: the library holds gfx950 code only), AR_ERR_RUNTIME
 *         (stream / event creation), AR_ERR_NOMEM.  Nothing leaks on failure.
 * The context makes `hip_device` current on the calling thread while it
 * creates its resources and restores the previous device afterwards. */
int ar_init(ar_ctx **out, int hip_device, const ar_config *cfg);

/* Enqueue one reduce.
 * The operation is the one in this file's header, as the "CUDA
 * allreduce.cu" page's ggml_cuda_ar_allreduce performs it between two ranks
 * (the accepted element types F32 / F16 / BF16, a non-empty tensor, the
 * wire-type narrowing of large F32 inputs) and the "Hexagon allreduce-ops.c"
 * page's allreduce_thread_dma_1d for any rank count (fixed-order sum, each
 * block written to every destination).  Where that page asserts on a bad
 * argument, this call returns a status and enqueues nothing.
 *   dst       : array of n_dst pointers to buffers of n dst_type elements
 *               (n_dst = R for AR_MODE_RS_BCAST, else 1); device memory of
 *               the context's device.
 *   srcs      : array of R pointers to the partials, n elements each, of
 *               dst_type (default) or wire_type (with AR_SRC_WIRE).  Device
 *               memory, or pinned host memory for AR_MODE_HOST_STAGED.
 *   R         : 2 .. AR_MAX_RANKS.
 *   n         : elements per partial; 0 is a no-op returning AR_OK.
 *   dst_type  : AR_F32; or AR_F16 / AR_BF16 with wire_type == dst_type, in
 *               which case the sources hold dst_type and every add is
 *               rounded to it (a different wire -> AR_ERR_UNSUPPORTED).
 *   wire_type : AR_F32, AR_F16 or AR_BF16; not wider than dst_type.
 *   mode      : AR_MODE_* | optional AR_SRC_WIRE | optional AR_SRC_INACTIVE_NULL.
 *   hip_stream: hipStream_t to enqueue on (NULL = null stream).
 * Graph capture: every schedule enqueues kernel launches only (no memsets,
 * no host synchronisation), so calls can be captured into a HIP graph and
 * replayed -- except the host-staged copy-engine pipeline, which is refused
 * under capture (the direct host reads, the default, can be captured).
 * Errors (all detected on the host before anything is enqueued):
 *   AR_ERR_INVALID for a NULL ctx / array / entry, R outside 2..16, a
 *   pointer not 16-byte aligned, an unknown type / mode / flag, a wire type
 *   wider than the destination, a destination that overlaps another
 *   destination or a source other than exactly in place (dst[d] equal to
 *   some srcs[r], same element width), n * element size overflowing size_t, or
 *   memory of the wrong kind for the mode (device pointers of another device,
 *   pageable host memory, host sources outside AR_MODE_HOST_STAGED);
 *   AR_ERR_UNSUPPORTED for a 16-bit dst_type with a different wire_type,
 *   and for a host-staged call on the copy-engine path (host_path 1) while
 *   hip_stream is being captured into a graph;
 *   AR_ERR_NOMEM if host-staged scratch cannot be allocated;
 *   AR_ERR_RUNTIME if a launch or copy cannot be enqueued.  Faults of
 *   enqueued work surface at the caller's next synchronisation. */
int ar_reduce(ar_ctx *ctx, void *const *dst, const void *const *srcs, int R, size_t n,
              ar_dtype dst_type, ar_dtype wire_type, unsigned mode, void *hip_stream);

/* For callers that cannot allocate device memory (code under graph-free
 * tight loops, harnesses that forbid hipMalloc): the host-staged reduce of
 * ar_reduce through the copy-engine pipeline, with its staging ring in the
 * library's static device array (64 MiB per device, part of the code object,
 * held until the process ends) instead of the context's hipMalloc'd ring.
 * It calls no hipMalloc / hipFree and allocates nothing else.
 *   Arguments, ownership and results are those of ar_reduce for a
 *   host-staged call; mode must be AR_MODE_HOST_STAGED (or AR_MODE_AUTO
 *   with pinned host sources) plus optional AR_SRC_WIRE /
 *   AR_SRC_INACTIVE_NULL, whatever the context's host_path.
 *   The array is one staging slot: the copy chunk is the largest whose R
 *   rank chunks fit it (any n is accepted; host_slots does not apply); a
 *   host_chunk_bytes set in the context's ar_config whose R chunks would not
 *   fit -> AR_ERR_NOMEM, nothing enqueued.
 *   Every call on a device shares that device's array: calls through one
 *   context are ordered by the context's event on the array, but calls of
 *   different contexts that overlap on one device race on the array.  Nothing in it needs to
 *   start at zero (every byte a kernel reads was copied in by the same call).
 * Errors: those of ar_reduce; another resolved mode -> AR_ERR_INVALID; under
 * stream capture -> AR_ERR_UNSUPPORTED. */
int ar_reduce_staged_static(ar_ctx *ctx, void *const *dst, const void *const *srcs, int R, size_t n,
                            ar_dtype dst_type, ar_dtype wire_type, unsigned mode, void *hip_stream);

/* Enqueue one reduce followed by a residual add: after the last rank,
 * res[i mod residual_len] is added in the destination type, element-wise
 * (residual_len == n) or as one row broadcast to every row (residual_len
 * divides n), as the "Hexagon allreduce-ops.c" page's HAS_ADD forms of
 * allreduce_thread_dma_1d / _2d and its IS_ROW_BCAST form do.  The residual
 * is the receiving rank's own tensor: it is not rounded through the wire.
 *   residual     : residual_len elements of dst_type in device memory of the
 *                  context's device, 16-byte aligned (also for host-staged
 *                  sources).  It may be exactly one of the destinations when
 *                  element-wise (x += reduce(partials)); any other overlap
 *                  with a destination is invalid.  It may overlap sources.
 *   residual_len : n (element-wise), or a divisor of n that is a multiple of
 *                  8 (broadcast row; other divisors -> AR_ERR_UNSUPPORTED).
 * Every other argument, the ownership rules and the error codes are those
 * of ar_reduce; residual NULL, residual_len 0 or not dividing n ->
 * AR_ERR_INVALID (n = 0 is a no-op and checks only residual != NULL).  Calls
 * with a residual run on the two-rank kernels (two fp32 partials into one
 * fp32 destination, CHUNKED or SINGLE_SHOT), on the kernels for two to four
 * active fp32 partials (an element-wise residual, three or four ranks or
 * inactive ones among more, CHUNKED or SINGLE_SHOT), on the single-shot
 * kernel in other SINGLE_SHOT calls, on the LDS-staged kernels in the
 * broadcast schedule, and on the register-staged kernels otherwise (unless
 * stream_kernel forces a family). */
int ar_reduce_add(ar_ctx *ctx, void *const *dst, const void *const *srcs, int R, size_t n,
                  ar_dtype dst_type, ar_dtype wire_type, unsigned mode, const void *residual,
                  size_t residual_len, void *hip_stream);

/* Row-strided tensors ("Hexagon allreduce-ops.c" page, allreduce_thread_dma_2d:
 * rows of ne0 elements fetched with the tensor's row stride nb[1]).  Row i of
 * every source starts at element i * src_stride, of every destination at
 * i * dst_stride, of an element-wise residual at i * res_stride; the elements
 * from cols up to the stride of each row are neither read nor written. */
typedef struct {
    size_t rows;
    size_t cols;        /* elements per row (at most 2^30)                        */
    size_t src_stride;  /* >= cols; src_stride * source element size % 16 == 0   */
    size_t dst_stride;  /* >= cols; dst_stride * destination element size % 16 == 0 */
    size_t res_stride;  /* residual: >= cols (element-wise, same alignment rule),
                           or 0 = one residual row of cols elements added to every
                           row (the page's IS_ROW_BCAST form); ignored without one */
} ar_rows;

/* Enqueue one reduce of row-strided tensors: for every row i and column
 * j < cols the element at row i, column j is computed exactly as ar_reduce
 * computes one element (followed, when `residual` is not NULL, by the residual
 * add of ar_reduce_add with the residual's row i -- or its only row when
 * res_stride is 0).  n = rows * cols; rows = 0 or cols = 0 is a no-op.
 *   shape    : the row layout above.
 *   residual : NULL, or a device buffer of dst_type laid out as shape says.
 * Every base pointer must be 16-byte aligned and every stride keep row starts
 * 16-byte aligned (AR_ERR_INVALID otherwise).  AR_MODE_RS_BCAST writes every
 * row to all R destinations (the rows are spread over the workgroups, not cut
 * into per-rank slices; the bytes are the same).  AR_MODE_HOST_STAGED reads the
 * pinned rows directly, or (host_path 1) copies chunks of whole rows with 2-D
 * copy-engine transfers.  Exactly in place needs equal strides;
 * overlaps are judged on each tensor's span from its first to its last
 * element.  Ownership and the remaining error codes are those of ar_reduce
 * and ar_reduce_add; cols > 2^30 -> AR_ERR_UNSUPPORTED. */
int ar_reduce_rows(ar_ctx *ctx, void *const *dst, const void *const *srcs, int R,
                   const ar_rows *shape, ar_dtype dst_type, ar_dtype wire_type, unsigned mode,
                   const void *residual, void *hip_stream);

/* Drain the context's internal stream and release everything it owns.
 * NULL is accepted and returns AR_OK.  Work already enqueued by ar_reduce
 * on caller streams must be complete or ordered before any reuse of the
 * buffers, as usual; ar_free waits for the context's own copy stream.
 * Follows the "CUDA allreduce.cu" page's ggml_cuda_ar_pipeline_free, which
 * returns at once for a null handle and synchronises its streams before it
 * frees buffers and events. */
int ar_free(ar_ctx *ctx);

/* Static, human-readable name of a status code ("AR_OK", ...).  The codes
 * follow the status style of the "Hexagon allreduce-ops.c" page's
 * validate_allreduce / op_allreduce: invalid parameters, a valid request the
 * implementation does not support (the caller falls back), not enough memory,
 * and an internal (runtime) error are distinct results. */
const char *ar_status_str(int status);

/* ---------------------------------------------------------------------
 * Host-only helpers (no HIP calls; usable without a GPU).
 * ------------------------------------------------------------------- */

/* The plan ar_reduce would execute for these arguments. */
typedef struct {
    int    mode;          /* resolved AR_MODE_* (never AUTO)               */
    int    n_dst;         /* destinations written                           */
    int    src_bytes;     /* bytes per source element                       */
    int    wire_bytes;    /* bytes per wire element                         */
    size_t chunk_elems;   /* plan unit in elements per rank                 */
    size_t n_chunks;      /* ceil(n / chunk_elems)                          */
    size_t slice_start[AR_MAX_RANKS]; /* RS_BCAST: first element of rank r  */
    size_t slice_len[AR_MAX_RANKS];   /* RS_BCAST: elements of rank r       */
    size_t algo_bytes;    /* algorithmic bytes: A*n*src_bytes + n_dst*n*dst_bytes
                             (+ residual_len*dst_bytes with a residual), A =
                             active ranks (an inactive rank is not read)     */
    int    store_nt;      /* 1: streaming (non-temporal) destination stores */
    int    host_direct;   /* HOST_STAGED: 1 = kernel reads host memory directly */
    int    stream_kernel; /* 0 single-shot, 1 register-staged, 2 LDS-staged,
                             3 the two-rank kernels (two active binary32
                             partials, one binary32 destination, contiguous
                             or rows of whole 512-element tiles with strides
                             below 2^32, optionally an element-wise or
                             broadcast-row residual; or two active 16-bit
                             partials into a contiguous destination of
                             their type, no residual),
                             4 the kernels for two to four active binary32
                             partials (three or four ranks, or inactive
                             ranks among more; one binary32 destination,
                             contiguous, no residual or an element-wise
                             one); 3 and 4 for CHUNKED
                             or SINGLE_SHOT calls with kept stores and no
                             forced grid, chosen automatically           */
    unsigned active_mask; /* bit r set: rank r has a partial (not inactive)   */
    int    dst_bytes;     /* bytes per destination element                  */
    int    residual_kind; /* 0 none, 1 element-wise, 2 broadcast row        */
    int    hold_waves;    /* resident waves per CU the launch is held to when
                             its grid fills every CU beyond that (0: none;
                             see ar_config.occupancy_hold)                  */
} ar_plan;

/* Validate the arguments exactly as ar_reduce does, except the memory-kind
 * checks (which need the HIP runtime), and fill `plan` (may be NULL).
 * `srcs_on_host` != 0 tells AUTO that the sources are pinned host memory.
 * `cfg` NULL means defaults.  Returns an ar_status code. */
int ar_plan_query(const ar_config *cfg, void *const *dst, const void *const *srcs, int R,
                  size_t n, ar_dtype dst_type, ar_dtype wire_type, unsigned mode, int srcs_on_host,
                  ar_plan *plan);

/* The same for ar_reduce_rows (slice_start / slice_len stay 0: row-strided
 * calls are not cut into per-rank slices; chunk_elems is one row on the
 * device, or the rows of one host-staged copy chunk times cols). */
int ar_plan_query_rows(const ar_config *cfg, void *const *dst, const void *const *srcs, int R,
                       const ar_rows *shape, ar_dtype dst_type, ar_dtype wire_type, unsigned mode,
                       const void *residual, int srcs_on_host, ar_plan *plan);

/* The same for ar_reduce_add (residual checks included). */
int ar_plan_query_add(const ar_config *cfg, void *const *dst, const void *const *srcs, int R,
                      size_t n, ar_dtype dst_type, ar_dtype wire_type, unsigned mode,
                      const void *residual, size_t residual_len, int srcs_on_host,
                      ar_plan *plan);

#ifdef __cplusplus
}
#endif

#endif /* MPP_AR_H */
