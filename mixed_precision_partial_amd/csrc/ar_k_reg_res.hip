// ar_k_reg_res.hip -- register-staged streaming instances that add a residual, every rank active.
#include "ar_device.h"

namespace mpp {

StreamTable kStreamRegRes = MPP_STREAM_TABLE(reg, false, true, _res);

}  // namespace mpp
