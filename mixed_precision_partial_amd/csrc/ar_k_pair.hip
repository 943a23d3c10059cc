// ar_k_pair.hip -- two-rank contiguous kernel instances: [residual kind][wire type].
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

}  // namespace mpp
