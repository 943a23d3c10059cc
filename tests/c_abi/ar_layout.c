/*
 * A plain C99 client of include/ar.h, built by the CPU tests with gcc: it
 * checks that the header compiles as C, links against libmpp_ar.so, and
 * prints the structure layouts the C compiler chose and one host-only plan,
 * so the tests can compare them with the Python binding's ctypes structures.
 * Nothing here needs a GPU.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>

#include "ar.h"

#define FIELD(T, f) printf("%s.%s %zu %zu\n", #T, #f, offsetof(T, f), sizeof(((T *)0)->f))

int main(void) {
    printf("sizeof ar_config %zu\n", sizeof(ar_config));
    FIELD(ar_config, single_shot_max_bytes);
    FIELD(ar_config, chunk_bytes);
    FIELD(ar_config, host_chunk_bytes);
    FIELD(ar_config, host_slots);
    FIELD(ar_config, grid_wgs);
    FIELD(ar_config, stream_kernel);
    FIELD(ar_config, store_policy);
    FIELD(ar_config, host_path);
    FIELD(ar_config, xcd_run_elems);
    FIELD(ar_config, occupancy_hold);
    printf("sizeof ar_plan %zu\n", sizeof(ar_plan));
    FIELD(ar_plan, mode);
    FIELD(ar_plan, n_dst);
    FIELD(ar_plan, src_bytes);
    FIELD(ar_plan, wire_bytes);
    FIELD(ar_plan, chunk_elems);
    FIELD(ar_plan, n_chunks);
    FIELD(ar_plan, slice_start);
    FIELD(ar_plan, slice_len);
    FIELD(ar_plan, algo_bytes);
    FIELD(ar_plan, store_nt);
    FIELD(ar_plan, host_direct);
    FIELD(ar_plan, stream_kernel);
    FIELD(ar_plan, active_mask);
    FIELD(ar_plan, dst_bytes);
    FIELD(ar_plan, residual_kind);
    FIELD(ar_plan, hold_waves);
    printf("sizeof ar_rows %zu\n", sizeof(ar_rows));
    FIELD(ar_rows, rows);
    FIELD(ar_rows, cols);
    FIELD(ar_rows, src_stride);
    FIELD(ar_rows, dst_stride);
    FIELD(ar_rows, res_stride);

    for (int s = 0; s <= 5; ++s) printf("status %d %s\n", s, ar_status_str(s));
    printf("free_null %d\n", ar_free(NULL));
    printf("init_null %d\n", ar_init(NULL, 0, NULL));

    /* the 4-rank slice + broadcast plan of 2048 x 8192 elements, fp16 wire,
       on made-up (never dereferenced) 16-byte aligned addresses */
    const void *srcs[4];
    void *dst[4];
    for (int r = 0; r < 4; ++r) {
        srcs[r] = (const void *)(uintptr_t)(((uint64_t)(r + 1)) << 36);
        dst[r] = (void *)(uintptr_t)(((uint64_t)(r + 9)) << 36);
    }
    ar_plan p;
    const int rc = ar_plan_query(NULL, dst, srcs, 4, (size_t)2048 * 8192, AR_F32, AR_F16, AR_MODE_RS_BCAST, 0, &p);
    printf("plan rc %d mode %d n_dst %d src_bytes %d wire_bytes %d chunk_elems %zu n_chunks %zu algo_bytes %zu "
           "store_nt %d stream_kernel %d active_mask %u slice1 %zu %zu\n",
           rc, p.mode, p.n_dst, p.src_bytes, p.wire_bytes, p.chunk_elems, p.n_chunks, p.algo_bytes, p.store_nt,
           p.stream_kernel, p.active_mask, p.slice_start[1], p.slice_len[1]);
    return 0;
}
