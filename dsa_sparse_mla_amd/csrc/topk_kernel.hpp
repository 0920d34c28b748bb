// Top-k index selection: per query token, the topk best-scoring candidate
// keys of its score row, written as ascending column ids padded with -1 (the
// index rows the sparse MLA forward consumes).
//
// Pages: "feat: add XTuner TileLang sparse MLA backend" (lmdeploy PR 4904),
// Summary (DSA index production kept for short prefill), per-file overview
// (prefill scores over chunks of query rows; the short-prefill scoring skip)
// and Validation (-1-padded index rows); "[Feature] Add optional FlashMLA
// backend for DSA Sparse MLA" (xtuner PR 2083), Changes (an indexer in front
// of the sparse kernel). The score function itself is an input.
//
// Order: larger score first; equal scores (-0 == +0) by smaller column; NaN
// after every number. Each score maps to a 32-bit key whose unsigned order
// is that order (ties aside), so selection is an exact radix select:
//   1. four passes over the row's keys, each a 256-bin histogram of one byte
//      (most significant first) among the keys that match the bytes fixed so
//      far; the bin where the count from the top reaches the remaining k fixes
//      the next byte. After four passes the k-th key K is known, and so is how
//      many keys equal to K are taken (the first ones by column).
//   2. one ordered pass: key > K, or key == K among the first of them, is
//      selected; a workgroup-wide prefix count over 512-column chunks gives
//      each selected column its place, so the row comes out ascending.
// A row with at most topk candidates skips all of this and is written as its
// whole range (no score is read).
//
// One workgroup (8 waves) per token row. Rows of up to kTkCache candidates
// keep their keys in LDS after the first pass; longer rows read their scores
// again in each pass (from L2 or beyond).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace dsa {

struct TopkArgs {
  const float* scores;       // fp32 [T, num_cols] (row t at scores + t * score_st); may be null
  int64_t score_st;
  int64_t num_cols;
  const int32_t* key_start;  // int32 [T]
  const int32_t* key_end;    // int32 [T]
  int64_t num_tokens;
  int32_t topk;
  int32_t* out;              // int32 [T, topk] (row t at out + t * out_st)
  int64_t out_st;
};

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkCache = 16384;   // candidate keys held in LDS (64 KB)

// Unsigned order of the result = selection order of the scores: NaN -> 0
// (below -inf, whose key is 0x007fffff), -0 -> +0, negatives reversed below
// positives.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// lanes below this one whose bit is set in m
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__global__ void __launch_bounds__(kTkThreads) topk_select_kernel(const TopkArgs a) {
  __shared__ uint32_t s_key[kTkCache];
  __shared__ uint32_t s_hist[kTkWaves][256];
  __shared__ uint32_t s_wsum[2][kTkWaves];
  __shared__ uint32_t s_state[2];   // next byte's digit, keys still to take from it

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t t = blockIdx.x;
  const int k = a.topk;
  int32_t* orow = a.out + t * a.out_st;

  int64_t lo = a.key_start[t], hi = a.key_end[t];
  lo = lo < 0 ? 0 : lo;
  hi = hi > a.num_cols ? a.num_cols : hi;
  const int64_t n = hi > lo ? hi - lo : 0;

  // ---------------------------------------------------------------- short rows
  if (n <= k || a.scores == nullptr) {
    for (int j = tid; j < k; j += kTkThreads) orow[j] = (n <= k && j < n) ? (int32_t)(lo + j) : -1;
    return;
  }

  const float* srow = a.scores + t * a.score_st + lo;
  const bool cached = n <= kTkCache;
  auto key_at = [&](int64_t j) -> uint32_t { return cached ? s_key[j] : score_key(srow[j]); };

  // ---------------------------------------------------------------- 1. radix select
  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kTkWaves * 256; i += kTkThreads) (&s_hist[0][0])[i] = 0u;
    __syncthreads();
    if (pass == 0) {
      for (int64_t j = tid; j < n; j += kTkThreads) {
        const uint32_t key = score_key(srow[j]);
        if (cached) s_key[j] = key;
        atomicAdd(&s_hist[wave][key >> 24], 1u);
      }
    } else {
      for (int64_t j = tid; j < n; j += kTkThreads) {
        const uint32_t key = key_at(j);
        if (((key ^ prefix) & mask) == 0u) atomicAdd(&s_hist[wave][(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    // bin totals, then the bin where the count from the top reaches `remaining`
    if (tid < 256) {
      uint32_t c = 0;
#pragma unroll
      for (int w = 0; w < kTkWaves; ++w) c += s_hist[w][tid];
      uint32_t incl = c;   // suffix sum over the wave's 64 bins (bins tid .. 64 wave + 63)
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(incl, off, 64);
        if (lane + off < 64) incl += o;
      }
      if (lane == 0) s_wsum[0][wave] = incl;
      s_hist[0][tid] = c;         // wave 0's copy is no longer needed: keep the totals
      s_hist[1][tid] = incl - c;  // and the count above each bin inside its wave
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t above = s_hist[1][tid];
      for (int w = wave + 1; w < 4; ++w) above += s_wsum[0][w];
      const uint32_t c = s_hist[0][tid];
      if (above < remaining && remaining <= above + c) {
        s_state[0] = (uint32_t)tid;
        s_state[1] = remaining - above;
      }
    }
    __syncthreads();
    prefix |= s_state[0] << shift;
    mask |= 255u << shift;
    remaining = s_state[1];
    __syncthreads();   // s_state and s_hist are rewritten by the next pass
  }
  const uint32_t K = prefix;    // the k-th key; `remaining` keys equal to it are taken

  // ---------------------------------------------------------------- 2. ordered compaction
  uint32_t eq_base = 0, sel_base = 0;
  int par = 0;
  for (int64_t c0 = 0; c0 < n; c0 += kTkThreads, par ^= 1) {
    const int64_t j = c0 + tid;
    const uint32_t key = j < n ? key_at(j) : 0u;
    const bool in = j < n;
    const bool gt = in && key > K;
    const bool eq = in && key == K;
    const uint64_t eqm = __ballot(eq);
    if (lane == 0) s_wsum[par][wave] = (uint32_t)__builtin_popcountll(eqm);
    __syncthreads();
    uint32_t eq_before = eq_base + lanes_below(eqm), eq_all = 0;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
      const uint32_t v = s_wsum[par][w];
      eq_before += w < wave ? v : 0u;
      eq_all += v;
    }
    const bool sel = gt || (eq && eq_before < remaining);
    const uint64_t selm = __ballot(sel);
    __syncthreads();   // every wave has read s_wsum[par]
    if (lane == 0) s_wsum[par][wave] = (uint32_t)__builtin_popcountll(selm);
    __syncthreads();
    uint32_t pos = sel_base + lanes_below(selm), sel_all = 0;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
      const uint32_t v = s_wsum[par][w];
      pos += w < wave ? v : 0u;
      sel_all += v;
    }
    if (sel && pos < (uint32_t)k) orow[pos] = (int32_t)(lo + j);   // exactly k are selected
    eq_base += eq_all;
    sel_base += sel_all;
  }
}

}  // namespace dsa
