// Decode prologue in one launch (MXFP4 weights, small problems): workgroup 0
// groups the routed slots (the one-workgroup align), workgroups 1..T split
// the token rows of x for the block-scaled MFMA, in token order (MX8: as
// MXFP8 activations). GEMM1 then reads a sorted row's split activations
// through the permutation. The two parts are independent, so the split runs
// beside the align instead of after it, on T rows instead of T*k.
#pragma once

#include "align.hpp"
#include "gemm_skinny.hpp"

namespace moe {

template <bool MX8>
__global__ __launch_bounds__(256) void k_align_fused_quant(const int32_t* ids, const float* w, int M, int E,
                                                           int nbits, int BM, AlignOut o,
                                                           const uint16_t* __restrict__ x, int T, int H,
                                                           skinny::QRows xq) {
  if (blockIdx.x == 0) {
    align_fused_body(ids, w, M, E, nbits, BM, o);
    return;
  }
  const int r = blockIdx.x - 1;
  if (r < T) skinny::quant_row<MX8>(x, (size_t)r, r, H, xq);
}

}  // namespace moe
