// Stand-in for the kernel layer of libkda.so (kda_launch.h) in the host-only
// build the sanitizer tier makes: there is no device, so every call that
// passes validation and planning stops at the device check, as it does on a
// machine without a gfx950.
#include "kda_launch.h"

namespace kda_internal {

kda_status device_ready()
{
    return KDA_ERR_DEVICE;
}

kda_status launch_decode(const DecodeCall &)
{
    return KDA_ERR_LAUNCH;
}

kda_status launch_gated_rmsnorm(const void *, const void *, const void *, void *, int64_t, int32_t, float, void *)
{
    return KDA_ERR_LAUNCH;
}

}  // namespace kda_internal
