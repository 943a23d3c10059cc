// ar_k_pair.hip -- two-rank contiguous kernel instances, one per wire type.
#include "ar_device.h"

namespace mpp {

const void *const kPair[3] = {reinterpret_cast<const void *>(&k_pair<AR_F32>),
                              reinterpret_cast<const void *>(&k_pair<AR_F16>),
                              reinterpret_cast<const void *>(&k_pair<AR_BF16>)};

}  // namespace mpp
