// Dispatch of the row-gather GEMV to its instantiations (weight dtype x block size, each
// compiled in its own translation unit).
#include "common.hpp"

namespace djv {

hipError_t launch_gemv_f32(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f32_side(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f16(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f16_side(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f32_dyn(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f32_side_dyn(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f16_dyn(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f16_side_dyn(const GemvArgs& a, hipStream_t s);

static hipError_t launch_valu(bool f16, const GemvArgs& a, hipStream_t s);

hipError_t launch_gemv(bool f16, const GemvArgs& a, hipStream_t s) {
    if (a.nseg < 1 || a.nseg > kMaxSeg || a.nside < 0 || a.nside > kMaxSide || a.nattn < 0)
        return hipErrorInvalidValue;
    for (int i = 0; i < a.nseg; ++i)
        if (a.seg[i].epi < kEpiStore || a.seg[i].epi > kEpiQkv) return hipErrorInvalidValue;
    if (a.mfma) {
        // matrix-core form: side selections run first, on their own (their inputs are ready
        // before the launch, so the results are the same).  Attention chunks are left to the
        // caller: their unmerged partials feed only the vector-ALU O-projection.
        if (!f16 || !a.mfma_part || a.nattn > 0) return hipErrorInvalidValue;
        if (a.nside > 0) {
            const hipError_t e = launch_select(a.side, a.nside, a.B, s, 0);
            if (e != hipSuccess) return e;
        }
        return launch_gemv_mfma(a, a.mfma_part, s);
    }
    if (a.B > kMaxBatch) return hipErrorInvalidValue;
    GemvArgs d = a;
    d.dyn = false;
    if (a.nseg > 1 && a.nattn == 0) {
        bool counted = false, same = true;
        for (int i = 0; i < a.nseg; ++i) {
            counted = counted || a.seg[i].list.count != nullptr;
            same = same && same_row_input(a.seg[i].in, a.seg[0].in);
        }
        d.dyn = counted && same;
    }
    return launch_valu(f16, d, s);
}

static hipError_t launch_valu(bool f16, const GemvArgs& a, hipStream_t s) {
    bool long_rows = false;
    for (int i = 0; i < a.nside; ++i) long_rows = long_rows || a.side[i].n_out > kShortRows;
    if (long_rows && (a.nattn > 0 || a.B > 1)) {
        // no side-block form for this launch: the selections run first, on their own (their
        // inputs are ready before the launch, so the results are the same)
        hipError_t e = launch_select(a.side, a.nside, a.B, s, 0);
        if (e != hipSuccess) return e;
        GemvArgs b = a;
        b.nside = 0;
        if (a.dyn) return f16 ? launch_gemv_f16_dyn(b, s) : launch_gemv_f32_dyn(b, s);
        return f16 ? launch_gemv_f16(b, s) : launch_gemv_f32(b, s);
    }
    if (a.dyn && (long_rows || a.nside == 0)) {
        if (f16) return long_rows ? launch_gemv_f16_side_dyn(a, s) : launch_gemv_f16_dyn(a, s);
        return long_rows ? launch_gemv_f32_side_dyn(a, s) : launch_gemv_f32_dyn(a, s);
    }
    GemvArgs b = a;
    b.dyn = false;  // short-row side selections run in the static form
    if (f16) return long_rows ? launch_gemv_f16_side(b, s) : launch_gemv_f16(b, s);
    return long_rows ? launch_gemv_f32_side(b, s) : launch_gemv_f32(b, s);
}

}  // namespace djv
