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
//      selected; workgroup-wide prefix counts over 4096-column chunks (8
//      consecutive columns per thread) give each selected column its place,
//      so the row comes out ascending.
// A row with at most topk candidates skips all of this and is written as its
// whole range (no score is read).
//
// One workgroup (8 waves) per token row. Rows of up to kTkCache candidates
// keep their keys in LDS after the first pass; longer rows read their scores
// again in each pass (from L2 or beyond).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

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
constexpr int kTkPer = 8;         // consecutive columns per thread in a chunk
constexpr int kTkCopies = 8;      // copies of each histogram bin (lane & 7 picks one)
constexpr int kTkChunk = kTkThreads * kTkPer;   // columns per chunk (4096)
static_assert(kTkCache % kTkChunk == 0, "cached rows end on a chunk boundary");

// Unsigned order of the result = selection order of the scores: NaN -> 0
// (below -inf, whose key is 0x007fffff), -0 -> +0, negatives reversed below
// positives.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t hist_at(uint32_t b, uint32_t c) { return 256u * c + ((b + 8u * c) & 255u); }

// lanes below this one whose bit is set in m
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__global__ void __launch_bounds__(kTkThreads) topk_select_kernel(const TopkArgs a) {
  __shared__ uint32_t s_key[kTkCache];
  // copy c of bin b at s_hist[hist_at(b, c)]: the copies of one bin fall in
  // eight different banks, and the 64 bins 4l + i that wave 0's lanes read
  // for one (i, c) spread over 16 banks
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[256 * kTkCopies];   // 16-byte reads below
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
  // kTkPer entries j0 + i * stride (i < kTkPer), read without branches:
  // indices past the row are clamped to its last column (the caller masks
  // them), so the loads are issued together. From LDS they are keys; from
  // the scores, raw score bits that to_key turns into keys when used.
  // Offsets are 32-bit: the host caps num_cols at INT32_MAX, so n - 1 and
  // j0 + i * stride (below n + kTkPer * kTkThreads) fit.
  const uint32_t last = (uint32_t)(n - 1);
  auto load_raw = [&](auto lds_tag, int64_t j0, int64_t stride, uint32_t* raw) {
    const uint32_t b = (uint32_t)j0, st = (uint32_t)stride;
    if constexpr (decltype(lds_tag)::value) {
#pragma unroll
      for (int i = 0; i < kTkPer; ++i) raw[i] = s_key[min(b + i * st, last)];
    } else {
      const uint32_t* sr = reinterpret_cast<const uint32_t*>(srow);
#pragma unroll
      for (int i = 0; i < kTkPer; ++i) raw[i] = sr[min(b + i * st, last)];
    }
  };
  auto to_key = [](auto lds_tag, uint32_t raw) {
    if constexpr (decltype(lds_tag)::value) return raw;
    else return score_key(__uint_as_float(raw));
  };

  // ---------------------------------------------------------------- 1. radix select
  // Two barriers per pass: counts complete, then the chosen digit published.
  // Lane l counts into copy l & 7 of each bin: scores concentrate in a few
  // values of the top byte, and one copy per bin would serialise most of a
  // wave's atomics on a handful of addresses. The copies are shared by all
  // waves, so only wave 0 touches them between the two barriers: it reads
  // each count and writes 0 back, which leaves the histogram clear for the
  // next pass.
  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)k;
  const uint32_t copy = (uint32_t)lane & (kTkCopies - 1);
#pragma unroll
  for (int i = 0; i < 4; ++i) s_hist[256 * wave + 64 * i + lane] = 0u;
  __syncthreads();   // clear before any wave counts
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    // kTkPer keys per thread and round; the next round's entries are
    // loaded before this round's are counted (one loop per source)
    auto count = [&](auto lds_tag) {
      constexpr int64_t kRound = (int64_t)kTkThreads * kTkPer;
      uint32_t nxt[kTkPer];
      load_raw(lds_tag, tid, kTkThreads, nxt);
      for (int64_t j0 = tid; j0 < n; j0 += kRound) {
        uint32_t key[kTkPer];
#pragma unroll
        for (int i = 0; i < kTkPer; ++i) key[i] = to_key(lds_tag, nxt[i]);
        if (j0 + kRound < n) load_raw(lds_tag, j0 + kRound, kTkThreads, nxt);
#pragma unroll
        for (int i = 0; i < kTkPer; ++i) {
          const int64_t j = j0 + (int64_t)i * kTkThreads;
          if (j < n) {
            if (pass == 0 && cached) s_key[j] = key[i];
            if (((key[i] ^ prefix) & mask) == 0u) atomicAdd(&s_hist[hist_at((key[i] >> shift) & 255u, copy)], 1u);
          }
        }
      }
    };
    if (pass > 0 && cached) count(std::true_type{});
    else count(std::false_type{});
    __syncthreads();   // every wave's counts are in
    if (wave == 0) {
      // lane l takes bins 4l .. 4l+3: their totals over the copies (copy cp
      // of the four bins is four consecutive words at a 16-byte boundary),
      // the keys in higher bins (a suffix sum over the lanes), then the bin
      // where the count from the top reaches `remaining`
      uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int cp = 0; cp < kTkCopies; ++cp) {
        uint4* w = reinterpret_cast<uint4*>(&s_hist[hist_at(4 * lane, cp)]);
        const uint4 v = *w;
        *w = make_uint4(0u, 0u, 0u, 0u);
        c[0] += v.x;
        c[1] += v.y;
        c[2] += v.z;
        c[3] += v.w;
      }
      const uint32_t tot = (c[0] + c[1]) + (c[2] + c[3]);
      uint32_t incl = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(incl, off, 64);
        if (lane + off < 64) incl += o;
      }
      uint32_t above = incl - tot;   // keys in bins 4l + 4 ..
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (above < remaining && remaining <= above + c[i]) {
          s_state[0] = (uint32_t)(4 * lane + i);
          s_state[1] = remaining - above;
        }
        above += c[i];
      }
    }
    __syncthreads();   // the digit is published; the histogram is clear again
    prefix |= s_state[0] << shift;
    mask |= 255u << shift;
    remaining = s_state[1];
  }
  const uint32_t K = prefix;    // the k-th key; `remaining` keys equal to it are taken

  // ---------------------------------------------------------------- 2. ordered compaction
  // Chunks of kTkChunk columns; thread tid takes columns kTkPer tid .. +kTkPer-1
  // of the chunk, so thread order is column order. One workgroup prefix count
  // per chunk, of the pair (keys > K, keys == K) packed in one word (each at
  // most kTkChunk): a column's place is the keys > K before it plus the keys
  // == K before it, capped at `remaining` (the first of those are taken). The
  // next two chunks' keys are in flight.
  // Exclusive prefix of v over the threads and its total (s_wsum[buf]).
  auto wg_scan = [&](uint32_t v, int buf, uint32_t& total) -> uint32_t {
    uint32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) s_wsum[buf][wave] = incl;
    __syncthreads();
    uint32_t before = incl - v;
    total = 0;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
      const uint32_t x = s_wsum[buf][w];
      before += w < wave ? x : 0u;
      total += x;
    }
    return before;
  };
  static_assert(kTkChunk < 65536, "both counts of a chunk fit 16 bits");
  auto load_chunk = [&](auto lds_tag, int64_t c0, uint32_t* raw) { load_raw(lds_tag, c0 + (int64_t)kTkPer * tid, 1, raw); };
  uint32_t gt_base = 0, eq_base = 0;
  auto taken = [&] { return gt_base + min(eq_base, remaining); };   // columns placed so far
  auto compact = [&](auto lds_tag) {
    // chunks c+1 and c+2 are in flight while chunk c is placed
    uint32_t cur[kTkPer], nxt[kTkPer], nxt2[kTkPer];
    load_chunk(lds_tag, 0, cur);
    if (kTkChunk < n) load_chunk(lds_tag, kTkChunk, nxt);
    int buf = 0;
    for (int64_t c0 = 0; c0 < n && taken() < (uint32_t)k; c0 += kTkChunk) {
#pragma unroll
      for (int i = 0; i < kTkPer; ++i) cur[i] = to_key(lds_tag, cur[i]);
      if (c0 + 2 * kTkChunk < n) load_chunk(lds_tag, c0 + 2 * kTkChunk, nxt2);
      const int64_t jt = c0 + (int64_t)kTkPer * tid;   // this thread's first column
      uint32_t ngt = 0, neq = 0;
#pragma unroll
      for (int i = 0; i < kTkPer; ++i) {
        const bool in = jt + i < n;
        ngt += (in && cur[i] > K) ? 1u : 0u;
        neq += (in && cur[i] == K) ? 1u : 0u;
      }
      uint32_t all;
      const uint32_t before = wg_scan((ngt << 16) | neq, buf, all);   // chunks alternate buffers
      buf ^= 1;
      uint32_t e = eq_base + (before & 0xffffu);                      // keys == K before this thread
      uint32_t pos = gt_base + (before >> 16) + min(e, remaining);
#pragma unroll
      for (int i = 0; i < kTkPer; ++i) {
        const bool in = jt + i < n;
        const bool eq = in && cur[i] == K;
        const bool sel = (in && cur[i] > K) || (eq && e < remaining);
        e += eq ? 1u : 0u;
        if (sel) {
          if (pos < (uint32_t)k) orow[pos] = (int32_t)(lo + jt + i);   // exactly k are selected
          ++pos;
        }
      }
      gt_base += all >> 16;
      eq_base += all & 0xffffu;
#pragma unroll
      for (int i = 0; i < kTkPer; ++i) {
        cur[i] = nxt[i];
        nxt[i] = nxt2[i];
      }
    }
  };
  if (cached) compact(std::true_type{});
  else compact(std::false_type{});
}

}  // namespace dsa
