// ar_k_reg_m.hip -- register-staged streaming instances for launches with an inactive rank, no residual.
#include "ar_device.h"

namespace mpp {

StreamTable kStreamRegM = MPP_STREAM_TABLE(reg, true, false, );

}  // namespace mpp
