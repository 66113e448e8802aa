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
hipError_t launch_gemv_f32_own(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f32_side_own(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f16_own(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f16_side_own(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f32_dyn_own(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f32_side_dyn_own(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f16_dyn_own(const GemvArgs& a, hipStream_t s);
hipError_t launch_gemv_f16_side_dyn_own(const GemvArgs& a, hipStream_t s);

namespace {
// The four launch forms of one weight dtype and input kind.
using LaunchFn = hipError_t (*)(const GemvArgs&, hipStream_t);
struct Forms {
    LaunchFn plain, side, dyn, side_dyn;
};
Forms forms(bool f16, bool own) {
    if (f16) {
        if (own) return {launch_gemv_f16_own, launch_gemv_f16_side_own, launch_gemv_f16_dyn_own,
                         launch_gemv_f16_side_dyn_own};
        return {launch_gemv_f16, launch_gemv_f16_side, launch_gemv_f16_dyn, launch_gemv_f16_side_dyn};
    }
    if (own) return {launch_gemv_f32_own, launch_gemv_f32_side_own, launch_gemv_f32_dyn_own,
                     launch_gemv_f32_side_dyn_own};
    return {launch_gemv_f32, launch_gemv_f32_side, launch_gemv_f32_dyn, launch_gemv_f32_side_dyn};
}
}  // namespace

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
    // LN(x) with moments summed by the kernel runs in its own instantiations: all segments
    // of a launch read the same kind of input
    const bool own = !a.seg[0].in.y && a.seg[0].in.own_stats;
    for (int i = 1; i < a.nseg; ++i)
        if ((!a.seg[i].in.y && a.seg[i].in.own_stats) != own) return hipErrorInvalidValue;
    const Forms F = forms(f16, own);
    bool long_rows = false;
    for (int i = 0; i < a.nside; ++i) long_rows = long_rows || a.side[i].n_out > kShortRows;
    if (long_rows && (a.nattn > 0 || a.B > 1)) {
        // no side-block form for this launch: the selections run first, on their own (their
        // inputs are ready before the launch, so the results are the same)
        hipError_t e = launch_select(a.side, a.nside, a.B, s, 0);
        if (e != hipSuccess) return e;
        GemvArgs b = a;
        b.nside = 0;
        return a.dyn ? F.dyn(b, s) : F.plain(b, s);
    }
    if (a.dyn && (long_rows || a.nside == 0)) return long_rows ? F.side_dyn(a, s) : F.dyn(a, s);
    GemvArgs b = a;
    b.dyn = false;  // short-row side selections run in the static form
    return long_rows ? F.side(b, s) : F.plain(b, s);
}

}  // namespace djv
