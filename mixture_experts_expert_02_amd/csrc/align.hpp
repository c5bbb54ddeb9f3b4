// Grouping of routed slots by expert: histogram, prefix sum, stable scatter.
//
// moonep_experts page, MoonEPExperts.apply: the segment end offsets are the
// cumulative sum of the per-weight-row token counts (int32, one per row,
// empty rows included). Module docstring: rows are contiguous per weight row
// and empty segments are skipped. Inside a segment the rows keep ascending
// flat slot order t*k + j, which makes the permutation unique.
//
// The slot range is cut into chunks, one per wave. Counting and scattering a
// chunk is done 64 slots at a time: lanes holding the same expert find each
// other with ballots on the bits of the id (match_key), so one leader lane
// updates the LDS counter of each expert and every lane gets its stable rank
// from a popcount. No global atomics; every result is deterministic.
#pragma once

#include "common.hpp"

namespace moe {

struct AlignOut {
  int32_t* counts;     // [E]
  int32_t* cu;         // [E]   end offsets
  int32_t* offsets;    // [E]   start offsets (workspace)
  int32_t* perm;       // [M]
  int32_t* inv_perm;   // [M]
  float* w_sorted;     // [M] or nullptr
  int32_t* tile_seg;   // [mt_cap] tile -> segment
  int32_t* tile_row0;  // [mt_cap] tile -> first sorted row
  int32_t* status;     // [5]: bad ids, valid rows, tiles, wait-timeout flag, cold segments
  int32_t* cold_seg;   // [E] segments of 1..cold_max rows, listed apart from the tiles; nullptr = none
  int32_t cold_max;
  int32_t* sync;       // counters the single-launch decode step expects zero, or nullptr
  int32_t n_sync;
};

__device__ __forceinline__ int slot_key(const int32_t* ids, int i, int end, int E, int& bad) {
  if (i >= end) return E;
  const int e = ids[i];
  if (e >= 0 && e < E) return e;
  if (e != -1) ++bad;
  return E;
}

// Histogram of one chunk into hist[E] (LDS, zeroed by the caller).
__device__ __forceinline__ int wave_count(const int32_t* ids, int begin, int end, int E, int nbits,
                                          int32_t* hist) {
  int bad = 0;
  for (int b = begin; b < end; b += kWave) {
    const int key = slot_key(ids, b + (int)__lane_id(), end, E, bad);
    const uint64_t peers = match_key(key, nbits);
    if (key < E && (peers & lanemask_lt()) == 0) hist[key] += __popcll(peers);
  }
  // wave sum of bad ids
  for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off);
  return bad;
}

// Stable scatter of one chunk; base[E] (LDS) holds each expert's next row.
__device__ __forceinline__ void wave_scatter(const int32_t* ids, const float* w, int begin, int end,
                                             int E, int nbits, int32_t* base, const AlignOut& o) {
  int unused = 0;
  for (int b = begin; b < end; b += kWave) {
    const int i = b + (int)__lane_id();
    const int key = slot_key(ids, i, end, E, unused);
    const uint64_t peers = match_key(key, nbits);
    if (key < E) {
      const uint64_t lower = peers & lanemask_lt();
      const int pos = base[key] + __popcll(lower);
      o.perm[pos] = i;
      o.inv_perm[i] = pos;
      if (o.w_sorted) o.w_sorted[pos] = w[i];
      if (lower == 0) base[key] = pos + __popcll(peers);
    } else if (i < end) {
      o.inv_perm[i] = -1;
    }
  }
}

// Exclusive scan of v[0..n) in LDS by the whole block (NT threads); returns
// the total. scratch needs NT/64 ints of LDS.
template <int NT>
__device__ int block_exclusive_scan(int32_t* v, int n, int32_t* scratch) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int per = (n + NT - 1) / NT;
  const int lo = min(tid * per, n), hi = min(lo + per, n);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += v[i];
  int x = s;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int t = lane < NT / 64 ? scratch[lane] : 0;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(t, off);
      if (lane >= off) t += y;
    }
    if (lane < NT / 64) scratch[lane] = t;
  }
  __syncthreads();
  int run = (wid ? scratch[wid - 1] : 0) + x - s;
  for (int i = lo; i < hi; ++i) {
    const int t = v[i];
    v[i] = run;
    run += t;
  }
  const int total = scratch[NT / 64 - 1];
  __syncthreads();
  return total;
}

// After counts (cnt) and start offsets (off) are known: end offsets, the tile
// table for BM-row tiles, unused perm entries, status. With o.cold_seg, the
// segments of 1..o.cold_max rows get no tiles and are listed in o.cold_seg
// instead (ascending), their number in status[4].
template <int NT>
__device__ void finish_tables(const int32_t* cnt, const int32_t* off, int32_t* mt_scan, int E, int M,
                              int total, int BM, int bad, const AlignOut& o, int32_t* scratch) {
  const int tid = threadIdx.x;
  const int cmax = o.cold_seg ? o.cold_max : 0;
  for (int e = tid; e < E; e += NT) {
    o.counts[e] = cnt[e];
    o.cu[e] = off[e] + cnt[e];
    o.offsets[e] = off[e];
    mt_scan[e] = cnt[e] <= cmax ? 0 : (cnt[e] + BM - 1) / BM;
  }
  __syncthreads();
  const int n_tiles = block_exclusive_scan<NT>(mt_scan, E, scratch);
  for (int e = tid; e < E; e += NT) {
    const int t0 = mt_scan[e];
    const int nt = cnt[e] <= cmax ? 0 : (cnt[e] + BM - 1) / BM;
    for (int t = 0; t < nt; ++t) {
      o.tile_seg[t0 + t] = e;
      o.tile_row0[t0 + t] = off[e] + t * BM;
    }
  }
  int n_cold = 0;
  if (o.cold_seg) {
    __syncthreads();  // every thread has read its tile offsets
    for (int e = tid; e < E; e += NT) mt_scan[e] = (cnt[e] > 0 && cnt[e] <= cmax) ? 1 : 0;
    __syncthreads();
    n_cold = block_exclusive_scan<NT>(mt_scan, E, scratch);
    for (int e = tid; e < E; e += NT)
      if (cnt[e] > 0 && cnt[e] <= cmax) o.cold_seg[mt_scan[e]] = e;
  }
  for (int p = total + tid; p < M; p += NT) o.perm[p] = -1;
  if (tid == 0) {
    o.status[0] = bad;
    o.status[1] = total;
    o.status[2] = n_tiles;
    o.status[3] = 0;
    o.status[4] = n_cold;
  }
}

// ------------------------------------------------------------------------
// One-workgroup path (small M, E <= 1024): count, scan and scatter in one launch.
// LDS: hist[4][E] + cnt[E] + off[E] + mt[E] + 16 ints.
// ------------------------------------------------------------------------
__device__ __forceinline__ void align_fused_body(const int32_t* ids, const float* w, int M, int E, int nbits,
                                                 int BM, const AlignOut& o) {
  extern __shared__ int32_t lds[];
  int32_t* hist = lds;            // [4][E]
  int32_t* cnt = hist + 4 * E;    // [E]
  int32_t* off = cnt + E;         // [E]
  int32_t* mts = off + E;         // [E]
  int32_t* scratch = mts + E;     // [16]
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  for (int i = tid; i < 4 * E; i += 256) hist[i] = 0;
  if (o.sync)
    for (int i = tid; i < o.n_sync; i += 256) o.sync[i] = 0;
  __syncthreads();
  const int chunk = ((M + 3) / 4 + 63) / 64 * 64;
  const int begin = min(wid * chunk, M), end = min(begin + chunk, M);
  const int bad = wave_count(ids, begin, end, E, nbits, hist + wid * E);
  if (lane == 0) scratch[8 + wid] = bad;
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    int run = 0;
    for (int c = 0; c < 4; ++c) {
      const int v = hist[c * E + e];
      hist[c * E + e] = run;
      run += v;
    }
    cnt[e] = run;
    off[e] = run;
  }
  const int total_bad = scratch[8] + scratch[9] + scratch[10] + scratch[11];
  __syncthreads();
  const int total = block_exclusive_scan<256>(off, E, scratch);
  for (int e = tid; e < E; e += 256)
    for (int c = 0; c < 4; ++c) hist[c * E + e] += off[e];
  __syncthreads();
  wave_scatter(ids, w, begin, end, E, nbits, hist + wid * E, o);
  finish_tables<256>(cnt, off, mts, E, M, total, BM, total_bad, o, scratch);
}

__global__ __launch_bounds__(256) void k_align_fused(const int32_t* ids, const float* w, int M, int E,
                                                     int nbits, int BM, AlignOut o) {
  align_fused_body(ids, w, M, E, nbits, BM, o);
}

// ------------------------------------------------------------------------
// Multi-workgroup path: count per chunk, one-workgroup scan, scatter per chunk.
// blkcnt is [nch][E]; the scan turns it into each chunk's running prefix.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_align_count(const int32_t* ids, int M, int E, int nbits,
                                                     int chunk, int nch, int32_t* blkcnt,
                                                     int32_t* blkbad) {
  extern __shared__ int32_t lds[];
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + wid;
  if (c >= nch) return;  // wave-uniform; no block barrier below
  int32_t* hist = lds + wid * E;
  for (int e = lane; e < E; e += 64) hist[e] = 0;
  const int begin = c * chunk, end = min(begin + chunk, M);
  const int bad = wave_count(ids, begin, end, E, nbits, hist);
  for (int e = lane; e < E; e += 64) blkcnt[(size_t)c * E + e] = hist[e];
  if (lane == 0) blkbad[c] = bad;
}

__global__ __launch_bounds__(1024) void k_align_scan(int32_t* blkcnt, const int32_t* blkbad, int nch,
                                                     int M, int E, int BM, AlignOut o) {
  extern __shared__ int32_t lds[];
  int32_t* cnt = lds;          // [E]
  int32_t* off = cnt + E;      // [E]
  int32_t* mts = off + E;      // [E]
  int32_t* scratch = mts + E;  // [32]
  const int tid = threadIdx.x;
  // per expert, an exclusive scan over the chunks; the counts are read eight
  // chunks at a time so that the loads overlap
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int c0 = 0; c0 < nch; c0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = c0 + u < nch ? blkcnt[(size_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c0 + u < nch) {
          blkcnt[(size_t)(c0 + u) * E + e] = run;
          run += v[u];
        }
    }
    cnt[e] = run;
    off[e] = run;
  }
  int bad = 0;
  for (int c = tid; c < nch; c += 1024) bad += blkbad[c];
  for (int s = 32; s > 0; s >>= 1) bad += __shfl_xor(bad, s);
  if ((tid & 63) == 0) scratch[16 + (tid >> 6)] = bad;
  __syncthreads();
  int total_bad = 0;
  for (int i = 0; i < 16; ++i) total_bad += scratch[16 + i];
  __syncthreads();
  const int total = block_exclusive_scan<1024>(off, E, scratch);
  finish_tables<1024>(cnt, off, mts, E, M, total, BM, total_bad, o, scratch);
}

__global__ __launch_bounds__(256) void k_align_scatter(const int32_t* ids, const float* w, int M, int E,
                                                       int nbits, int chunk, int nch,
                                                       const int32_t* blkcnt, AlignOut o) {
  extern __shared__ int32_t lds[];
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + wid;
  if (c >= nch) return;
  int32_t* base = lds + wid * E;
  for (int e = lane; e < E; e += 64) base[e] = o.offsets[e] + blkcnt[(size_t)c * E + e];
  const int begin = c * chunk, end = min(begin + chunk, M);
  wave_scatter(ids, w, begin, end, E, nbits, base, o);
}

// ------------------------------------------------------------------------
// Pre-grouped entry: segment tables from caller-given end offsets.
// moonep_experts page, MoonEPExperts.apply / moonep_grouped_gemm (int32 end
// offsets, one per weight row). Malformed offsets (decreasing, negative, or
// past NvS) set status[0] = 1 and leave every segment empty.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_grouped_prep(const int32_t* cu_in, int G, int NvS, int BM,
                                                       AlignOut o) {
  extern __shared__ int32_t lds[];
  int32_t* cnt = lds;          // [G]
  int32_t* off = cnt + G;      // [G]
  int32_t* mts = off + G;      // [G]
  int32_t* scratch = mts + G;  // [32]
  __shared__ int bad_flag;
  const int tid = threadIdx.x;
  if (tid == 0) bad_flag = 0;
  __syncthreads();
  for (int g = tid; g < G; g += 1024) {
    const int prev = g ? cu_in[g - 1] : 0;
    const int cur = cu_in[g];
    if (cur < prev || cur > NvS || prev < 0) bad_flag = 1;
  }
  __syncthreads();
  const int bad = bad_flag;
  for (int g = tid; g < G; g += 1024) {
    const int prev = g ? cu_in[g - 1] : 0;
    cnt[g] = bad ? 0 : cu_in[g] - prev;
    off[g] = bad ? 0 : prev;
  }
  __syncthreads();
  const int total = bad ? 0 : cu_in[G - 1];
  finish_tables<1024>(cnt, off, mts, G, 0, total, BM, bad, o, scratch);
}

}  // namespace moe
