// kernel_stubs.cpp -- stand-ins for the device-side entry points of libbsattn,
// so that the host code (api.cpp) links into a sanitizer-instrumented test
// program built with a plain host compiler.  The schedule and layout code
// under test never reaches them; every stub reports "not supported".
#include "internal.h"

namespace bsattn {

hipError_t launch_fwd_bf16(const FwdArgs&, int, int, hipStream_t, hipEvent_t, hipEvent_t) {
    return hipErrorNotSupported;
}
int fwd_bf16_ctas_per_cu(int head_dim, bool two_wave) { return head_dim == 64 ? (two_wave ? 4 : 1) : 2; }
hipError_t launch_topr_select(const void*, const void*, uint64_t*, int, int, int, int, hipStream_t, hipEvent_t,
                              hipEvent_t) {
    return hipErrorNotSupported;
}
hipError_t launch_adaptive_select(const void*, const void*, double*, double*, int32_t*, int, int, int, int,
                                  hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_fill_tiles(const int32_t*, int32_t*, const int4*, const int32_t*, const int32_t*, int,
                             const int32_t*, int, int, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_gather_global(const FwdArgs&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fwd_f32(const FwdArgs&, const int32_t*, int, int, hipStream_t, hipEvent_t, hipEvent_t) {
    return hipErrorNotSupported;
}
size_t route_workspace_bytes(int32_t B, int32_t H, int32_t L, int32_t) { return (size_t)B * H * L * sizeof(double); }
hipError_t launch_route_topk(const void*, const float*, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t*, void*,
                             hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_bwd_dq(const BwdArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_dkdv(const BwdArgs&, int, int, hipStream_t, hipEvent_t, hipEvent_t) {
    return hipErrorNotSupported;
}
hipError_t launch_bwd_sum(const BwdArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_routed_sum(const BwdArgs&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_tok_bwd_extra(const BwdArgs&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_cand_positions(const void*, const float*, const float*, int, int, int, int, int32_t*, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_cand_attention(const void*, const void*, const void*, const int32_t*, int, int, int, int, int, int,
                                 float, void*, float*, int32_t*, hipStream_t, hipEvent_t, hipEvent_t) {
    return hipErrorNotSupported;
}
hipError_t launch_split_heads(const float*, const void*, void*, void*, void*, int, int, int, int, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_merge_heads(const void*, void*, int, int, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bias_out(const float*, const void*, void*, size_t, int, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_layout_build(const RowRule&, int, int32_t, int32_t, int32_t, int32_t*, int32_t*, uint8_t*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace bsattn
