// ar_k_lds_res.hip -- LDS-staged streaming instances with a residual add, every rank active.
#include "ar_device.h"

namespace mpp {

StreamTable kStreamLdsRes = MPP_STREAM_TABLE(lds, false, true, _res);

}  // namespace mpp
