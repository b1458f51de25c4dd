// Kernel selection templates: the address of the instantiation for a launch
// plan (nullptr when none fits). Included by the instantiation units.
#ifndef SSD_SELECT_H
#define SSD_SELECT_H

#include "ssd_kernels.h"

namespace {

constexpr int kLdsLimitSel = 160 * 1024;

template <typename TI, int P, int NP, bool ROT, int MODE>
void* walk_ptr() {
    return reinterpret_cast<void*>(&ssd_walk_kernel<TI, P, NP, ROT, MODE>);
}

template <typename TI, int P, bool ROT, int MODE>
void* walk_ptr_np(int NP) {
    switch (NP) {
        case 32: return walk_ptr<TI, P, 32, ROT, MODE>();
        case 64: return walk_ptr<TI, P, 64, ROT, MODE>();
        case 128: return walk_ptr<TI, P, 128, ROT, MODE>();
        case 256: return walk_ptr<TI, P, 256, ROT, MODE>();
    }
    return nullptr;
}

template <typename TI, bool ROT, int MODE>
void* walk_ptr_p(int P, int NP) {
    switch (P) {
        case 16: return walk_ptr_np<TI, 16, ROT, MODE>(NP);
        case 32: return walk_ptr_np<TI, 32, ROT, MODE>(NP);
        case 64: return walk_ptr_np<TI, 64, ROT, MODE>(NP);
        case 128: return walk_ptr_np<TI, 128, ROT, MODE>(NP);
    }
    return nullptr;
}


template <typename TI, int NP, int W, int MODE, bool ROT, bool YS = false>
void* cols_ptr() {
    if constexpr (cols_lds_bytes<TI, NP, W, ROT>(MODE) <= kLdsLimitSel)
        return reinterpret_cast<void*>(&ssd_cols_kernel<TI, NP, W, MODE, ROT, YS>);
    else
        return nullptr;  // does not fit one CU's LDS
}

template <typename TI, int W, int MODE, bool ROT, bool YS = false>
void* cols_ptr_np(int NP) {
    switch (NP) {
        case 32: return cols_ptr<TI, 32, W, MODE, ROT, YS>();
        case 64: return cols_ptr<TI, 64, W, MODE, ROT, YS>();
        case 128: return cols_ptr<TI, 128, W, MODE, ROT, YS>();
        case 256: return cols_ptr<TI, 256, W, MODE, ROT, YS>();
    }
    return nullptr;
}

template <typename TI, int MODE, bool YS = false>
void* cols_ptr_w(int w, int NP) {
    switch (w) {
        case 1: return cols_ptr_np<TI, 1, MODE, false, YS>(NP);
        case 2: return cols_ptr_np<TI, 2, MODE, false, YS>(NP);
        case 4: return cols_ptr_np<TI, 4, MODE, false, YS>(NP);
        case 6: return cols_ptr_np<TI, 6, MODE, false, YS>(NP);
        case 8: return cols_ptr_np<TI, 8, MODE, false, YS>(NP);
        case 10: return cols_ptr_np<TI, 10, MODE, false, YS>(NP);
    }
    return nullptr;
}

template <typename TI>
void* cb_pack_ptr(int NP) {
    switch (NP) {
        case 32: return reinterpret_cast<void*>(&ssd_cb_pack_kernel<TI, 32>);
        case 64: return reinterpret_cast<void*>(&ssd_cb_pack_kernel<TI, 64>);
        case 128: return reinterpret_cast<void*>(&ssd_cb_pack_kernel<TI, 128>);
        case 256: return reinterpret_cast<void*>(&ssd_cb_pack_kernel<TI, 256>);
    }
    return nullptr;
}

}  // namespace

#endif  // SSD_SELECT_H
