// Grouped GEMM for few rows per segment (decode): weights streamed from HBM
// straight into MFMA operand registers, no LDS.
//
// Same grouped-GEMM definition as the prefill kernel (moonep_experts page,
// moonep_grouped_gemm; route weight on the activation per the module
// docstring). Weights may be bf16 or MXFP4 (trtllm_mxfp4_moe page,
// TrtLlmMxfp4ExpertsBase._supports_quant_scheme: MXFP4 weights with
// unquantized activations): e2m1 codes with an e8m0 scale per 32 K elements
// (OCP Microscaling v1.0 reading). MXFP4 codes are decoded to bf16 in
// registers with v_cvt_scalef32_pk_bf16_fp4; every e2m1 value times a power of
// two in the bf16 range is exact in bf16, so the MFMA sees the exact weights.
//
// Tile: 16 rows x 16 output columns per wave, 4 waves per workgroup side by
// side (64 columns). v_mfma_f32_16x16x32_bf16 with the activations as the A
// operand (row = lane & 15) and the weights as the B operand (column =
// lane & 15). The K order inside the dot product is free as long as A and B
// agree, so lane group q = lane >> 4 of step s owns the 32-element scale block
// kb = 4 s + q: one 16-byte load carries a lane's 32 MXFP4 codes and a single
// scale, which feed four MFMAs (8 K values each).
#pragma once

#include "common.hpp"

namespace moe {
namespace skinny {

constexpr int BM = 16;   // rows per tile
constexpr int WN = 16;   // columns per wave
constexpr int NW = 4;    // waves per workgroup
constexpr int NT = NW * 64;
constexpr int UNR = 4;   // K steps in flight per wave

enum WFmt { W_BF16 = 0, W_MXFP4 = 1 };

struct Params {
  const uint16_t* A;      // rows [*, K] bf16
  const int32_t* a_perm;  // sorted row -> flat slot, or nullptr
  int32_t a_div;
  const void* B0;         // gate / down: bf16 [G, N, K] or e2m1 codes [G, N, K/2]
  const void* B1;         // up (GEMM1)
  const uint8_t* S0;      // e8m0 scales [G, N, K/32] (MXFP4)
  const uint8_t* S1;
  int32_t N, K;
  const int32_t* tile_seg;
  const int32_t* tile_row0;
  const int32_t* seg_end;
  const int32_t* status;  // status[2] = number of row tiles
  int32_t mt_cap;
  int32_t n_tiles;        // ceil(N / 64)
  uint16_t* C;
  const float* row_w;
  ActParams act;
};

__device__ __forceinline__ float e8m0_to_f32(uint32_t v) {
  if (v == 0) return __uint_as_float(0x00400000u);  // 2^-127
  if (v == 255) return __uint_as_float(0x7fc00000u);
  return __uint_as_float(v << 23);
}

// 8 e2m1 codes (one dword, element 2i in the low nibble of byte i) -> 8 bf16
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// The weights of one lane for one K step: 32 consecutive K values of row n.
template <int FMT>
struct WChunk {
  u32x4 q[FMT == W_BF16 ? 4 : 1];
  uint32_t s;
};

template <int FMT>
__device__ __forceinline__ void load_w(WChunk<FMT>& w, const void* Bm, const uint8_t* Sm, size_t row, int K,
                                       int kb, bool ok) {
  if (FMT == W_BF16) {
    const u32x4* src = (const u32x4*)((const uint16_t*)Bm + row * K + (size_t)kb * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) w.q[i] = ok ? src[i] : u32x4{0u, 0u, 0u, 0u};
    w.s = 0;
  } else {
    const u32x4* src = (const u32x4*)((const uint8_t*)Bm + row * (K / 2) + (size_t)kb * 16);
    w.q[0] = ok ? *src : u32x4{0u, 0u, 0u, 0u};
    w.s = ok ? Sm[row * (K / 32) + kb] : 127u;
  }
}

template <int FMT>
__device__ __forceinline__ bf16x8 w_operand(const WChunk<FMT>& w, int i, float scale) {
  if (FMT == W_BF16) {
    return *(const bf16x8*)&w.q[i];
  } else {
    const uint32_t d = i == 0 ? w.q[0][0] : i == 1 ? w.q[0][1] : i == 2 ? w.q[0][2] : w.q[0][3];
    return fp4x8_to_bf16(d, scale);
  }
}

template <int FMT, bool GATED>
__global__ __launch_bounds__(NT) void k_gemm(const Params p) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mt = blockIdx.x / p.n_tiles;
  const int nt = blockIdx.x - mt * p.n_tiles;
  if (mt >= p.status[2]) return;
  const int seg = p.tile_seg[mt];
  const int row0 = p.tile_row0[mt];
  const int rows = min(BM, p.seg_end[seg] - row0);
  const int N = p.N, K = p.K;
  const int KB = K / 32;
  const int n0 = nt * (NW * WN) + wave * WN;
  if (n0 >= N) return;  // wave-uniform, no barriers in this kernel

  const int l16 = lane & 15, q = lane >> 4;
  const int n = min(n0 + l16, N - 1);
  const size_t wrow = (size_t)seg * N + n;
  const bool arow_ok = l16 < rows;
  const int arow = arow_ok ? (p.a_perm ? p.a_perm[row0 + l16] / p.a_div : row0 + l16) : 0;
  const uint16_t* a_src = p.A + (size_t)arow * K;

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int steps = (KB + 3) / 4;
  for (int s0 = 0; s0 < steps; s0 += UNR) {
    WChunk<FMT> w0[UNR], w1[UNR];
    u32x4 xa[UNR][4];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int kb = 4 * (s0 + u) + q;
      const bool ok = (s0 + u < steps) && kb < KB;
      load_w<FMT>(w0[u], p.B0, p.S0, wrow, K, kb, ok);
      if (GATED) load_w<FMT>(w1[u], p.B1, p.S1, wrow, K, kb, ok);
      const u32x4* xs = (const u32x4*)(a_src + (size_t)kb * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[u][i] = (ok && arow_ok) ? xs[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const float sc0 = FMT == W_MXFP4 ? e8m0_to_f32(w0[u].s) : 1.f;
      const float sc1 = (FMT == W_MXFP4 && GATED) ? e8m0_to_f32(w1[u].s) : 1.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 a = *(const bf16x8*)&xa[u][i];
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w_operand<FMT>(w0[u], i, sc0), acc0, 0, 0, 0);
        if (GATED)
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w_operand<FMT>(w1[u], i, sc1), acc1, 0, 0, 0);
      }
    }
  }

  // 16x16 result layout: lane holds column (lane & 15), rows 4 (lane >> 4) + r.
  const int col = n0 + l16;
  if (col < N) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = q * 4 + r;
      if (row >= rows) continue;
      uint16_t* dst = p.C + (size_t)(row0 + row) * N + col;
      if (GATED)
        *dst = f32_to_bf16_rne(gated_act(p.act, acc0[r], acc1[r]) * p.row_w[row0 + row]);
      else
        *dst = f32_to_bf16_rne(acc0[r]);
    }
  }
}

}  // namespace skinny
}  // namespace moe
