// SwiGLU-S2 activation of node features (swiglu.hip), host launcher.
#pragma once

#include "common.h"

namespace so2 {

// Workspace bytes of launch_swiglu_s2 for n_atoms nodes of degree <= L and C
// channels: u, v, the gate and the gated grid product s, sized for fp32.
size_t swiglu_s2_workspace_bytes(int n_atoms, int L, int C, int dtype);

// stages: SO2_STAGE_SW_* bits; the steps run in order maps, grid, output.
so2_status launch_swiglu_s2(uint32_t stages, const void* x, const void* w_a, const void* w_b, const void* w_g,
                            const void* w_o, float* y, int n_atoms, int L, int C, int dtype, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

}  // namespace so2
