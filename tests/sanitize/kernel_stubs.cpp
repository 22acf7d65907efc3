// Host-only stand-ins for the kernel launchers of libns.so, for the
// sanitizer build of the host code (tests/test_host_sanitizers.py). That
// build exercises argument validation, planning and the rank planner, which
// never launch; every launcher here fails with hipErrorNotSupported.
#include "ns_kernels.h"

namespace ns {

hipError_t launch_small(int, int, const SmallMat*, int, const int32_t*, int, int, int, const SmallCoeffs&,
                        hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t launch_norm_partial(int, const LargeMat*, int, const int32_t*, int, float*, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t launch_norm_final(int, const int32_t*, const float*, int, float*, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t launch_prep(int, const LargeMat*, int, const int32_t*, int, const float*, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t launch_scale_out(int, const LargeMat*, int, const int32_t*, int, const float*, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t launch_gemm(int, int, const LargeMat*, const Tile*, int, int, int, int, float, float, float,
                       hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace ns
