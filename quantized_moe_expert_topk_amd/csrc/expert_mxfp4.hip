// expert_mxfp4.hip -- the MXFP4 (e8m0 per 32, native scaled FP4 MFMA) instantiations of the
// streaming expert kernels.  This file is compiled with the backend's memory-clause scheduling
// (build.py), which measured faster for these kernels and slower for the other formats' (MI355X,
// steps of 200: the DeepSeek-V4-Flash-shaped layer at T = 256 378.5 -> 376.3 us, at T = 1
// 40.5 -> 38.0 us; the NVFP4 decode layer at T = 64 63.9 -> 66.4 us).
#include "expert_kernels.h"

namespace qmoe {

void launch_gate_up_mxfp4(const GateUpArgs &a, int n_shared_sub, hipStream_t s) {
  launch_gate_up_grid<MOE_FMT_MXFP4_E8M0>(a, n_shared_sub, s);
}

void launch_down_mxfp4(const DownArgs &a, dim3 grid, hipStream_t s) { launch_down_fmt<MOE_FMT_MXFP4_E8M0>(a, grid, s); }

void launch_down_t1_mxfp4(const DownArgs &a, const float *topk_w, void *out, int out_bf16, hipStream_t s) {
  launch_down_t1_fmt<MOE_FMT_MXFP4_E8M0>(a, topk_w, out, out_bf16, s);
}

}  // namespace qmoe
