// Shared device helpers for the gfx950 MoE experts kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 with round-to-nearest-even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

// 1 / (1 + e^-x) with v_exp_f32 and v_rcp_f32 (about 1 ulp each); for very
// negative x the reciprocal of +inf is 0, so x * sigmoid(x) stays finite.
__device__ __forceinline__ float sigmoidf_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// Activation of the gate/up pair, in fp32.
//   act 0: silu(g) * u                       (moonep_experts page, module docstring)
//   act 1: SwiGLU-OAI, g' = min(g, limit), u' = clamp(u, -limit, limit),
//          g' * sigmoid(alpha g') * (u' + beta)   (trtllm_mxfp4_moe page,
//          TrtLlmMxfp4ExpertsBase parameters; formula is the gpt-oss reading)
//   act 2: SiTu, alpha tanh(g / alpha) sigmoid(g) * beta tanh(u / beta)
struct ActParams {
  int32_t kind;
  float alpha, beta, limit;
};

// AK >= 0: the kind fixed at compile time (the prefill GEMMs' epilogues, which
// evaluate it for 64 values per lane, are instantiated per kind so that each
// carries one formula's code); AK < 0: a.kind at run time.
template <int AK>
__device__ __forceinline__ float gated_act_k(const ActParams& a, float g, float u) {
  const int kind = AK >= 0 ? AK : a.kind;
  if (kind == 0) return g * sigmoidf_fast(g) * u;
  if (kind == 2)  // SiTu (trtllm_mxfp4_moe page, TrtLlmMxfp4ExpertsBase constructor comment)
    return a.alpha * tanhf(g / a.alpha) * sigmoidf_fast(g) * (a.beta * tanhf(u / a.beta));
  g = fminf(g, a.limit);
  u = fminf(fmaxf(u, -a.limit), a.limit);
  return g * sigmoidf_fast(a.alpha * g) * (u + a.beta);
}

__device__ __forceinline__ float gated_act(const ActParams& a, float g, float u) { return gated_act_k<-1>(a, g, u); }

// Per-expert parameters: device float32 arrays of one value per expert
// (segment), or nullptr where the problem's scalar (or 1 for the scales)
// holds for every expert. trtllm_mxfp4_moe page, TrtLlmMxfp4ExpertsBase
// constructor: the activation's alpha, beta and clamp limit are per-expert
// tensors; flashinfer_moe_ep page, epilogue_from_quant_config: one fc1 and one
// fc2 alpha per expert, scaling the gate/up products and the down product.
struct ExpertParams {
  const float* alpha;
  const float* beta;
  const float* limit;
  const float* fc1;
  const float* fc2;
};

__device__ __forceinline__ ActParams act_for(const ActParams& a, const ExpertParams& e, int seg) {
  ActParams r = a;
  if (e.alpha) r.alpha = e.alpha[seg];
  if (e.beta) r.beta = e.beta[seg];
  if (e.limit) r.limit = e.limit[seg];
  return r;
}

__device__ __forceinline__ float scale_for(const float* s, int seg) { return s ? s[seg] : 1.f; }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const uint32_t lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Mask of the lanes of this wave whose key equals this lane's key. Every lane
// of the wave must call it (keys of idle lanes should be a sentinel).
__device__ __forceinline__ uint64_t match_key(int key, int nbits) {
  uint64_t m = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const int bit = (key >> b) & 1;
    const uint64_t s = __ballot(bit);
    m &= bit ? s : ~s;
  }
  return m;
}

// Split of the down projection's K range (GEMM2 of the big-tile path): the
// number of K ranges S (1..s_cap) that minimises rounds x stages per block,
// where a round is one tile per compute unit and each block carries a fixed
// cost worth about 12 stages (first loads, epilogue, and the partial output
// written and read back by the combine; fitted to Mixtral-shaped timings,
// where 3 ranges beat 4). Pure function of its arguments: the GEMM and the
// combine that sums the S partial outputs both call it and get the same S.
__host__ __device__ inline int split_k_count(int tiles, int kt, int ncu, int s_cap) {
  int best = 1;
  long long best_cost = -1;
  for (int s = 1; s <= s_cap && s <= kt; ++s) {
    const long long rounds = ((long long)tiles * s + ncu - 1) / ncu;
    const long long cost = rounds * ((kt + s - 1) / s + 12);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}


}  // namespace moe
