// ar_k_pair.hip -- two-rank kernel instances: contiguous [residual kind][wire type], row-strided
// [residual kind][power-of-two tiles per row][wire type], 16-bit into 16-bit [fp16, bf16]; and the
// kernels for two to four active binary32 partials [element-wise residual][active partials - 2][wire type].
#include "ar_device.h"

namespace mpp {

#define MPP_PAIR_ROW(RK)                                                                              \
    {reinterpret_cast<const void *>(&k_pair_res<AR_F32, RK>), reinterpret_cast<const void *>(&k_pair_res<AR_F16, RK>), \
     reinterpret_cast<const void *>(&k_pair_res<AR_BF16, RK>)}
const void *const kPair[5][3] = {{reinterpret_cast<const void *>(&k_pair<AR_F32>),
                                  reinterpret_cast<const void *>(&k_pair<AR_F16>),
                                  reinterpret_cast<const void *>(&k_pair<AR_BF16>)},
                                 MPP_PAIR_ROW(1), MPP_PAIR_ROW(2), MPP_PAIR_ROW(3),
                                 MPP_PAIR_ROW(4)};
#undef MPP_PAIR_ROW

#define MPP_PAIR_ROWS_W(RK, P2)                                                           \
    {reinterpret_cast<const void *>(&k_pair_rows<AR_F32, RK, P2>),                      \
     reinterpret_cast<const void *>(&k_pair_rows<AR_F16, RK, P2>),                      \
     reinterpret_cast<const void *>(&k_pair_rows<AR_BF16, RK, P2>)}
#define MPP_PAIR_ROWS(RK) {MPP_PAIR_ROWS_W(RK, false), MPP_PAIR_ROWS_W(RK, true)}
const void *const kPairRows[3][2][3] = {MPP_PAIR_ROWS(0), MPP_PAIR_ROWS(1), MPP_PAIR_ROWS(2)};
#undef MPP_PAIR_ROWS
#undef MPP_PAIR_ROWS_W

const void *const kPair16[2] = {reinterpret_cast<const void *>(&k_pair16<AR_F16>),
                                reinterpret_cast<const void *>(&k_pair16<AR_BF16>)};

#define MPP_FEW_ROW(A, RES)                                                                       \
    {reinterpret_cast<const void *>(&k_few<AR_F32, A, RES>), reinterpret_cast<const void *>(&k_few<AR_F16, A, RES>), \
     reinterpret_cast<const void *>(&k_few<AR_BF16, A, RES>)}
const void *const kFew[2][3][3] = {{MPP_FEW_ROW(2, false), MPP_FEW_ROW(3, false), MPP_FEW_ROW(4, false)},
                                   {MPP_FEW_ROW(2, true), MPP_FEW_ROW(3, true), MPP_FEW_ROW(4, true)}};
#undef MPP_FEW_ROW

}  // namespace mpp
