// forms.h -- launchers of the standalone dequantized matvec and of an expert's fused
// gate/up + SwiGLU in four forms of the per-weight arithmetic (kernels_forms.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmoe {

// form: 0 naive, 1 per-weight fma recast, 2 group-factored, 3 table of c*s+b in LDS
constexpr int kForms = 4;
hipError_t launch_qmatvec_form(int bits, int form, const uint8_t *blob, int rows, int cols, const float *x, float *y,
                               hipStream_t s);
// h[r] = silu(gate_r . x) * (up_r . x) for one expert's interleaved gate/up region, in
// the same four forms
hipError_t launch_expert_gateup_form(int bits, int form, const uint8_t *gu, int hidden, int inter, const float *x,
                                     float *h, hipStream_t s);

}  // namespace fmoe
