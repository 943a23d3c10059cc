// ar_k_lds_res_m.hip -- LDS-staged streaming instances with a residual add and an inactive rank.
#include "ar_device.h"

namespace mpp {

StreamTable kStreamLdsResM = MPP_STREAM_TABLE(lds, true, true, _res);

}  // namespace mpp
