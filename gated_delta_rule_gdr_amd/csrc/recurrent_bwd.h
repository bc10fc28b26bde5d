// Tokenwise backward of the gated delta / gated linear rules
// (recurrent_bwd.hip): fp32 state checkpoints and per-token partial sums in
// the caller's workspace. Not part of the public ABI (include/gdr.h is).
#pragma once

#include "gdr_internal.h"

namespace gdr {

size_t recurrent_bwd_workspace(const gdr_args &a);
hipError_t launch_recurrent_bwd(const gdr_args &a, const void *dout, void *dq, void *dk, void *dv, float *dbeta,
                                float *dg, float *dstate0, void *ws, hipStream_t stream);

}  // namespace gdr
