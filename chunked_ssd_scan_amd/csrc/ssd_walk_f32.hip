// General walk instantiations for fp32 inputs (ssd_walk_kernel; see ssd_kernels.h).
#include "ssd_select.h"

namespace ssd_detail {

void* select_walk_f32(bool rot, int mode, int P, int NP) {
    if (rot) return mode ? walk_ptr_p<float, true, 1>(P, NP) : walk_ptr_p<float, true, 0>(P, NP);
    return mode ? walk_ptr_p<float, false, 1>(P, NP) : walk_ptr_p<float, false, 0>(P, NP);
}

}  // namespace ssd_detail
