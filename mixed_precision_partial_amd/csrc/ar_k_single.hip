// ar_k_single.hip -- single-shot kernel instances (decode-sized vectors).
#include "ar_device.h"

namespace mpp {

const void *const kSingleShot[2][2][kCombos][kBuckets] = {
    {MPP_TABLE(k_single_shot, false, false), MPP_TABLE(k_single_shot, true, false)},
    {MPP_TABLE(k_single_shot, false, true), MPP_TABLE(k_single_shot, true, true)}};

}  // namespace mpp
