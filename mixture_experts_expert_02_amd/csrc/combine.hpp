// Back to token order.
//
// flashinfer_moe_ep page, module docstring and FlashInferMoeEpExperts
// (finalize_weight_and_reduce_impl is a no-op): the experts step itself
// reduces each token's k slot results, and the output is written, not
// accumulated. Here the sum runs over j = 0..k-1 in that order, in fp32, so
// the result does not depend on scheduling (no atomics).
#pragma once

#include "common.hpp"

namespace moe {

// The down projection may come in S partial outputs over K ranges (S from
// split_k_count with the GEMM's own arguments; 1 when s_cap is 1).
struct SplitSum {
  const int32_t* status;  // status[2] = row tiles of the GEMM
  int32_t n_tiles;        // GEMM2 column tiles
  int32_t kt;             // GEMM2 K stages
  int32_t ncu;
  int32_t s_cap;
  int64_t stride;         // elements between partial outputs
};

// One workgroup per token and 2048 columns (blockIdx.y); each thread sums 8
// consecutive columns, slot j outer and K range s inner, both ascending. The
// (j, s) rows are fetched eight at a time before any is added, so a thread
// has up to eight loads in flight instead of one; the additions keep the
// order above. Each slot row is read once: non-temporal loads.
__global__ __launch_bounds__(256) void k_combine(const uint16_t* y, const int32_t* inv_perm, int T, int k,
                                                 int H, const SplitSum ss, uint16_t* out) {
  const int t = blockIdx.x;
  if (t >= T) return;
  const int h0 = blockIdx.y * 256 * 8;
  const int S = ss.s_cap > 1 ? split_k_count(ss.status[2] * ss.n_tiles, ss.kt, ss.ncu, ss.s_cap) : 1;
  const int n = k * S;  // (j, s) pairs, j-major
  const int32_t* ip = inv_perm + (size_t)t * k;
  for (int h = h0 + threadIdx.x * 8; h < min(H, h0 + 256 * 8); h += 256 * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int base = 0; base < n; base += 8) {
      u32x4 v[8];
      bool ok[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = base + u;
        const int j = idx / S, sp = idx - j * S;
        const int p = idx < n ? ip[j] : -1;
        ok[u] = p >= 0;
        if (ok[u]) v[u] = __builtin_nontemporal_load((const u32x4*)(y + (size_t)sp * ss.stride + (size_t)p * H + h));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (!ok[u]) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += bf16_bits_to_f32(v[u][i] & 0xffffu);
          acc[2 * i + 1] += bf16_bits_to_f32(v[u][i] >> 16);
        }
      }
    }
    u32x4 o;
    o[0] = pack_bf16x2(acc[0], acc[1]);
    o[1] = pack_bf16x2(acc[2], acc[3]);
    o[2] = pack_bf16x2(acc[4], acc[5]);
    o[3] = pack_bf16x2(acc[6], acc[7]);
    *(u32x4*)(out + (size_t)t * H + h) = o;
  }
}

// Pre-grouped entry: zero rows [status[1], NvS) of out (moonep_experts page,
// MoonEPExperts.apply: padding rows past the last segment come out zero).
__global__ __launch_bounds__(256) void k_zero_tail(uint16_t* out, const int32_t* status, int NvS, int H) {
  const int first = status[1];
  const int row = blockIdx.x;
  if (row < first || row >= NvS) return;
  for (int h = threadIdx.x * 8; h < H; h += 256 * 8) *(u32x4*)(out + (size_t)row * H + h) = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace moe
