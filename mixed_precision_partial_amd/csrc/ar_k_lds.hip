// ar_k_lds.hip -- LDS-staged streaming instances, every rank active.
#include "ar_device.h"

namespace mpp {

StreamTable kStreamLds = MPP_STREAM_TABLE(lds, false, false, );

}  // namespace mpp
