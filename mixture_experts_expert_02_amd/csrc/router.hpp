// Router step: per-token expert logits -> top-k expert ids and route weights.
//
// trtllm_mxfp4_moe page, TrtLlmMxfp4ExpertsMonolithic: the routing methods
// Renormalize / RenormalizeNaive and DeepSeekV3 (score-correction bias,
// expert groups, groups kept, routed scaling factor). Readings of the
// unprinted formulas: Renormalize weights are a softmax over the k largest
// logits (the full softmax renormalised over the picks is the same number);
// DeepSeekV3 scores are sigmoids, the bias only steers selection, groups are
// scored by the sum of their two best selection scores, and the weights are
// the picked scores normalised to sum 1 times the scaling factor.
//
// One wave per token, four tokens per workgroup. Lane l holds experts
// l, l + 64, ... (PER of them), so a token's logits load as whole 256-byte
// rows. Selection works on order-preserving 32-bit keys of the scores: a
// radix select with wave ballots (32 rounds, no cross-lane data movement)
// finds the k-th largest key, the picks (ties to the lower index) are
// compacted into a per-wave LDS row, and pick j's output slot is the number
// of picks that beat it. Group scores go through a per-wave LDS row and are
// selected the same way. No workgroup barrier is used, so a wave with no
// token may exit at once.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kRouteMaxE = 1024;
constexpr int kRouteMaxK = 32;
constexpr int kRouteMaxGroups = 64;

struct RouteParams {
  const float* logits;  // [T, E]
  const float* bias;    // [E] or nullptr (DeepSeekV3)
  int32_t T, E, k;
  int32_t method;       // 0 Renormalize, 1 DeepSeekV3
  int32_t n_group, topk_group;
  float scale;
  int32_t* ids;         // [T, k]
  float* w;             // [T, k]
};

// Order-preserving 32-bit key of a float (larger float, larger key); finite
// values map above 0x007fffff, so 0 marks "not a candidate".
__device__ __forceinline__ uint32_t route_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Rank of this lane's bit among the set bits of a wave mask below it.
__device__ __forceinline__ int route_rank(uint64_t m) { return __popcll(m & lanemask_lt()); }

// Radix select over the wave: the k-th largest key thr among the P keys of
// every lane, and how many keys equal to thr belong to the top k (rem).
// 32 rounds of ballots; every lane gets the same answer.
template <int P>
__device__ __forceinline__ void route_kth(const uint32_t (&key)[P], int k, uint32_t& thr, int& rem) {
  uint32_t prefix = 0;
  rem = k;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = prefix | (1u << b);
    const uint32_t hi = ~((1u << b) - 1u);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) cnt += __popcll(__ballot((key[i] & hi) == cand));
    if (cnt >= rem) prefix = cand;
    else rem -= cnt;
  }
  thr = prefix;
}

// Top-k membership in index order e = lane + 64 i (ties at thr to the lower
// index); returns the number of members before slot i of this lane in that
// order in pos[i] (compact slot), -1 for non-members.
template <int P>
__device__ __forceinline__ void route_members(const uint32_t (&key)[P], uint32_t thr, int rem, int (&pos)[P]) {
  int ties = 0, taken = 0;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const uint64_t tm = __ballot(key[i] == thr);
    const bool in = key[i] > thr || (key[i] == thr && ties + route_rank(tm) < rem);
    ties += __popcll(tm);
    const uint64_t im = __ballot(in);
    pos[i] = in ? taken + route_rank(im) : -1;
    taken += __popcll(im);
  }
}

template <int PER>
__global__ __launch_bounds__(256) void k_route(const RouteParams p) {
  __shared__ float sel_lds[4][kRouteMaxE];
  __shared__ uint32_t pk_key[4][kRouteMaxK];
  __shared__ int32_t pk_idx[4][kRouteMaxK];
  __shared__ float pk_sc[4][kRouteMaxK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= p.T) return;
  const float* row = p.logits + (size_t)t * p.E;
  const bool ds = p.method == 1;
  constexpr float kMax = 3.402823466e38f;

  uint32_t key[PER];  // selection key (0: not a candidate)
  float v[PER];       // selection score
  float sc[PER];      // logit (Renormalize) or sigmoid score (DeepSeekV3)
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    v[i] = 0.f;
    sc[i] = 0.f;
    if (e < p.E) {
      float x = row[e];
      x = x != x ? -kMax : fminf(fmaxf(x, -kMax), kMax);
      if (ds) {
        const float s = (float)(1.0 / (1.0 + exp(-(double)x)));
        sc[i] = s;
        v[i] = s + (p.bias ? p.bias[e] : 0.f);
      } else {
        sc[i] = x;
        v[i] = x;
      }
    }
    key[i] = e < p.E ? route_key(v[i]) : 0u;
  }
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  if (ds && p.n_group > 1) {
    // group scores: lane g < n_group sums the two largest selection scores
    // of experts g*G .. g*G + G - 1; the topk_group best groups stay
    float* srow = sel_lds[wave];
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (lane + 64 * i < p.E) srow[lane + 64 * i] = v[i];
    wave_sync();
    const int G = p.E / p.n_group;
    uint32_t gkey[1] = {0u};
    if (lane < p.n_group) {
      float m1 = -INFINITY, m2 = -INFINITY;
      for (int j = 0; j < G; ++j) {
        const float x = srow[lane * G + j];
        if (x > m1) {
          m2 = m1;
          m1 = x;
        } else if (x > m2) {
          m2 = x;
        }
      }
      gkey[0] = route_key(m1 + m2);
    }
    uint32_t gthr;
    int grem, gpos[1];
    route_kth<1>(gkey, p.topk_group, gthr, grem);
    route_members<1>(gkey, gthr, grem, gpos);
    const uint64_t kept = __ballot(gpos[0] >= 0);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + 64 * i;
      if (e < p.E && !((kept >> (e / G)) & 1ull)) key[i] = 0u;
    }
  }

  // the k picks, compacted in index order into this wave's LDS rows
  uint32_t thr;
  int rem, pos[PER];
  route_kth<PER>(key, p.k, thr, rem);
  route_members<PER>(key, thr, rem, pos);
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (pos[i] >= 0) {
      pk_key[wave][pos[i]] = key[i];
      pk_idx[wave][pos[i]] = lane + 64 * i;
      pk_sc[wave][pos[i]] = sc[i];
    }
  wave_sync();
  // lane j < k takes pick j: its output slot is the number of picks that beat
  // it (larger key, or equal key and lower index); Renormalize also needs the
  // largest picked logit
  if (lane < p.k) {
    const uint32_t mk = pk_key[wave][lane];
    const int mi = pk_idx[wave][lane];
    const float ms = pk_sc[wave][lane];
    int slot = 0;
    float top = -INFINITY;
    for (int m = 0; m < p.k; ++m) {
      const uint32_t ok = pk_key[wave][m];
      const int oi = pk_idx[wave][m];
      slot += ok > mk || (ok == mk && oi < mi);
      top = fmaxf(top, pk_sc[wave][m]);
    }
    // weights: sums over the picks in compact (index) order, the same in every lane
    float w;
    if (ds) {
      float tot = 0.f;
      for (int m = 0; m < p.k; ++m) tot += pk_sc[wave][m];
      w = tot > 0.f ? ms / tot * p.scale : 0.f;
    } else {
      float tot = 0.f;
      for (int m = 0; m < p.k; ++m) tot += expf(pk_sc[wave][m] - top);
      w = expf(ms - top) / tot;
    }
    p.ids[(size_t)t * p.k + slot] = mi;
    p.w[(size_t)t * p.k + slot] = w;
  }
}

}  // namespace moe
