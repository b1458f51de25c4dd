// General walk instantiations for bf16 inputs (ssd_walk_kernel; see ssd_kernels.h).
#include "ssd_select.h"

namespace ssd_detail {

void* select_walk_bf16(bool rot, int mode, int P, int NP) {
    if (rot) return mode ? walk_ptr_p<uint16_t, true, 1>(P, NP) : walk_ptr_p<uint16_t, true, 0>(P, NP);
    return mode ? walk_ptr_p<uint16_t, false, 1>(P, NP) : walk_ptr_p<uint16_t, false, 0>(P, NP);
}

}  // namespace ssd_detail
