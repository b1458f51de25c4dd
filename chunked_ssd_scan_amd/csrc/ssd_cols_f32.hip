// Column-block walk instantiations for fp32 inputs (ssd_cols_kernel, shared
// B/C) and the fp32 C B^T pack; see ssd_kernels.h.
#include "ssd_select.h"

namespace ssd_detail {

void* select_cols_f32(int mode, int w, int NP, bool ysub) {
    if (mode) return cols_ptr_w<float, 1>(w, NP);
    return ysub ? cols_ptr_w<float, 0, true>(w, NP) : cols_ptr_w<float, 0>(w, NP);
}

void* cb_pack_f32(int NP) { return cb_pack_ptr<float>(NP); }

}  // namespace ssd_detail
