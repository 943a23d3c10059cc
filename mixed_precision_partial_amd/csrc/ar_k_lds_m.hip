// ar_k_lds_m.hip -- LDS-staged streaming instances for launches with an inactive rank.
#include "ar_device.h"

namespace mpp {

StreamTable kStreamLdsM = MPP_STREAM_TABLE(lds, true, false, );

}  // namespace mpp
