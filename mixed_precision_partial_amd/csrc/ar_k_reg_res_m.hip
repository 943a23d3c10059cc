// ar_k_reg_res_m.hip -- register-staged streaming instances that add a residual, some rank inactive.
#include "ar_device.h"

namespace mpp {

StreamTable kStreamRegResM = MPP_STREAM_TABLE(reg, true, true, _res);

}  // namespace mpp
