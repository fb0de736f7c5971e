// Merged RMS layer norm of node features (norm.hip), host launcher.
#pragma once

#include "common.h"

namespace so2 {

so2_status launch_merged_rms_norm(const void* x, const float* gamma, void* y, int n_atoms, int L, int C,
                                  float eps, int dtype, hipStream_t stream);

}  // namespace so2
