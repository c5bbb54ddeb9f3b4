// Route weight on the input: routed rows x * w, in sorted row order.
//
// moonep_experts page, MoonEPExperts.apply: with input-weighted routing (top-1,
// e.g. Llama 4) the route weight has already scaled the activations before
// dispatch, and the experts step does not multiply the activation by it. Here
// the experts step does that scaling itself: sorted row p gets
// bf16(x[perm[p] / div] * w[p]) (bf16, as the activations handed to the GEMMs
// are), and GEMM1 then reads these rows in order, with no weight in its
// epilogue.
#pragma once

#include "common.hpp"

namespace moe {

// One workgroup per row, 8 values per thread and step. With perm, rows at or
// past status[1] (the valid sorted rows) are skipped: no GEMM reads them.
__global__ __launch_bounds__(256) void k_scale_rows(const uint16_t* __restrict__ x, const int32_t* perm, int div,
                                                    const float* __restrict__ w, const int32_t* status, int rows,
                                                    int H, uint16_t* __restrict__ xs) {
  const int r = blockIdx.x;
  if (r >= rows || (perm && r >= status[1])) return;
  const size_t src = perm ? (size_t)(perm[r] / div) : (size_t)r;
  const float s = w[r];
  for (int h = threadIdx.x * 8; h < H; h += 256 * 8) {
    const u32x4 v = *(const u32x4*)(x + src * H + h);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack_bf16x2(bf16_bits_to_f32(v[i] & 0xffffu) * s, bf16_bits_to_f32(v[i] >> 16) * s);
    *(u32x4*)(xs + (size_t)r * H + h) = o;
  }
}

}  // namespace moe
