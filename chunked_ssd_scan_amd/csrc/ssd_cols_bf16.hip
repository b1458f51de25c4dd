// Column-block walk instantiations for bf16 inputs (ssd_cols_kernel, shared
// B/C and rotating) and the bf16 C B^T pack; see ssd_kernels.h.
#include "ssd_select.h"

namespace ssd_detail {

// ysub selects the output-pass instantiations that keep only odd steps of y
void* select_cols_bf16(int mode, int w, int NP, bool ysub) {
    if (mode) return cols_ptr_w<uint16_t, 1>(w, NP);
    return ysub ? cols_ptr_w<uint16_t, 0, true>(w, NP) : cols_ptr_w<uint16_t, 0>(w, NP);
}

// Rotating column walk: one head (headdim 64 or 128) per block, dstate 64 or
// 128 (one table lane per state pair).
void* select_cols_rot_bf16(int mode, int w, int NP, bool ysub) {
    if (w == 4) {
        switch (NP) {
            case 64: return mode ? (ysub ? cols_ptr<uint16_t, 64, 4, 1, true, true>() : cols_ptr<uint16_t, 64, 4, 1, true>())
                                 : ysub ? cols_ptr<uint16_t, 64, 4, 0, true, true>() : cols_ptr<uint16_t, 64, 4, 0, true>();
            case 128: return mode ? (ysub ? cols_ptr<uint16_t, 128, 4, 1, true, true>() : cols_ptr<uint16_t, 128, 4, 1, true>())
                                  : ysub ? cols_ptr<uint16_t, 128, 4, 0, true, true>() : cols_ptr<uint16_t, 128, 4, 0, true>();
        }
    } else if (w == 8) {
        switch (NP) {
            case 64: return mode ? (ysub ? cols_ptr<uint16_t, 64, 8, 1, true, true>() : cols_ptr<uint16_t, 64, 8, 1, true>())
                                 : ysub ? cols_ptr<uint16_t, 64, 8, 0, true, true>() : cols_ptr<uint16_t, 64, 8, 0, true>();
            case 128: return mode ? (ysub ? cols_ptr<uint16_t, 128, 8, 1, true, true>() : cols_ptr<uint16_t, 128, 8, 1, true>())
                                  : ysub ? cols_ptr<uint16_t, 128, 8, 0, true, true>() : cols_ptr<uint16_t, 128, 8, 0, true>();
        }
    }
    return nullptr;
}

void* cb_pack_bf16(int NP) { return cb_pack_ptr<uint16_t>(NP); }

}  // namespace ssd_detail
