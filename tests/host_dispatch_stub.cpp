// host_dispatch_stub.cpp -- TEST INFRASTRUCTURE for the host-sanitizer build
// of the C ABI (tests/test_host_sanitizers.py).  fa_capi.cpp validates every
// argument on the host and only then calls these kernel-dispatch functions;
// the sanitizer build compiles fa_capi.cpp with gcc (no device code) against
// these definitions, which launch nothing and report hipErrorNotSupported.
// The host tests make invalid calls only, so none of them is reached; a call
// that got here would come back as FA_ERR_HIP.  The product library never
// links this file.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace fa {
hipError_t fwd_dispatch(const void *, const void *, const void *, float *, float *, int, int, int, int, int,
                        float, int, int, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t decode_dispatch(const void *, const void *, const void *, const int32_t *, const int32_t *, void *,
                           int, int, int, int, int, float, int, void *, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t decode_noalloc_dispatch(const void *, const void *, const void *, const int32_t *, const int32_t *,
                                   void *, int, int, int, int, int, float, int, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t bwd_dispatch(const void *, const void *, const void *, const float *, const float *, const void *,
                        float *, float *, float *, int, int, int, int, int, float, int, int, void *, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t fwd_ext_dispatch(const void *, const void *, const void *, float *, float *, int, int, int, int, int,
                            int, float, int, int, int, const uint8_t *, int64_t, int64_t, int, const uint32_t *,
                            int, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t fwd_paged_dispatch(const void *, const void *, const void *, const int32_t *, const int32_t *, float *,
                              float *, int, int, int, int, int, uint64_t, float, int, int, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t mask_blocks_dispatch(const uint8_t *, int, int, int, int, int64_t, int64_t, int, uint32_t *,
                                hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t quant_fp8_dispatch(const void *, int, int, int, int, int, int, void *, int32_t *, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t fwd_fp8_dispatch(const void *, const void *, const void *, const int32_t *, const int32_t *,
                            const int32_t *, float *, float *, int, int, int, int, float, int, hipStream_t)
{
    return hipErrorNotSupported;
}
}  // namespace fa
