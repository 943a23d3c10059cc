// ar_k_reg.hip -- register-staged streaming instances, every rank active, no residual.
#include "ar_device.h"

namespace mpp {

StreamTable kStreamReg = MPP_STREAM_TABLE(reg, false, false, );

}  // namespace mpp
