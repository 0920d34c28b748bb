// dkv pass of the split backward schedule (more than 16 heads).
//
// The dq pass (bwd_dq_kernel.hpp) visits each (token, named row) pair once
// and stores P and s*dS of the pair, bf16, for every head: per token and
// head group of 32, the token's named rows in row order (their rank, from the
// prepass), 128 bytes each (P of the 32 heads, then s*dS). This pass forms
// the rows' gradient from those values alone:
//   dkv[r]       += sum over (t, h) of s dS[t,h,r] q[t,h,:]   (576 columns)
//   dkv[r, :512] += sum over (t, h) of P[t,h,r] dO[t,h,:]
// with no recomputation of S or dP. A token's named rows inside a block of
// rows form one run of ranks, pre .. pre + cnt - 1 (pre from the prepass, cnt
// the popcount of the token's mask words over the block), so the pass copies
// that run.
//
// One work item = (256 kv rows r0 .., column half ch, chunk of 64 tokens):
// latent columns 256ch .. 256ch+255 and rope columns 512 + 32ch .. +31. It
// collects the chunk's tokens whose masks name any of its rows and takes
// them in steps of one token and one head group. A step has two parts, each
// behind one barrier: the q part (dkv += (s dS)^T q over the 32 heads) and
// the dO part (dkv[:, :512] += P^T dO). Wave (rq, cw) of the 8 owns rows r0 +
// 64rq .. +63 (four row tiles) and column tiles 8cw .. 8cw+7 of the half's
// latent part plus its rope tile cw: 144 accumulators, added once per item.
//   * A operand (rows x heads): lane (g, n) of row tile rt reads the 16-byte
//     unit g of its row's entry (heads 8g .. 8g+7), or zero when the token
//     does not name the row;
//   * B operand (heads x columns): q^T / dO^T read transposed from LDS
//     (ds_read_b64_tr_b16 of head rows 8g + n/4 and 8g + 4 + n/4 give the
//     same k-slot order); each read feeds the four row tiles.
// A half of the columns per item halves the q and dO bytes each step copies
// for the same products (the copies, not the MFMAs, bound this pass); the
// two halves of a row block are neighbours in the work queue, so the second
// finds the entry runs in L2.
//
// The parts go HBM -> LDS by global_load_lds through a ring of three
// buffers; a step's run of entries is copied with its q part into one of
// two list buffers, as many 1 KB copies as the run needs.
//
// LDS: q part = [32 heads][512 B] (the latent half) + [32][128 B] (the
// whole rope part), 20 KB; the dO part uses the latent layout. Granule G
// (16 B) of head row h sits at G ^ dk_swz(h) within its 256-byte group (rope:
// G ^ dk_swz_r(h)): a transposed read serves a half-wave's 8 head rows
// (8g + 0..3 for two g) in one pass when their 32-byte pieces fall on
// distinct bank groups, which these swizzles give (checked with a bank
// probe); unit G of list entry e sits at G ^ (e & 7), so that the 16 rows of
// a row tile (consecutive entries when named) spread over the banks.
//
// Pages: the prime-rl pull request 4078 that adds a `cudnn_flashmla` DSA
// backend (a separate DSA backward kernel, timed per call); "[Feature] Add
// optional FlashMLA backend for DSA Sparse MLA" (xtuner PR 2083), Motivation
// (the forward's output and LSE feed the backward).
#pragma once

#include <type_traits>

#include "bwd_kernel.hpp"

namespace dsa {

constexpr int kDkRows = 256;                      // kv rows per work item (eight mask words)
constexpr int kDkWords = kDkRows / 32;
constexpr int kDkChunk = 64;                      // tokens per work item (one ballot)
constexpr int kDkBallots = kDkChunk / 64;
static_assert(kDkChunk % 64 == 0 && kDkBallots <= 4, "waves 0 .. kDkBallots-1 collect the chunk's tokens");
constexpr int kDkWaves = 8;
constexpr int kDkHeads = 32;                      // heads per step (one head group)
constexpr int kDkQR = kDkHeads * 512;             // rope rows within a q part
constexpr int kDkPart = kDkQR + kDkHeads * 128;   // one part buffer (20 KB)
constexpr int kDkParts = 3;                       // part ring
constexpr int kDkEnt = 128;                       // one named row's P and s dS of a head group
constexpr int kDkList = kDkRows * kDkEnt;         // one step's entry run, at most (32 KB)
constexpr int kDkQueues = 8;                      // work queues (one per XCD)
static_assert(kDkPart % 1024 == 0 && kDkList % 1024 == 0, "buffers keep the 1 KB copy alignment");

typedef __attribute__((address_space(3))) const uint8_t dk_lds;
__device__ __forceinline__ bf16x8_t dk_b128(const dk_lds* p) {
  return *(__attribute__((address_space(3))) const bf16x8_t*)p;
}
__device__ __forceinline__ short4_t dk_tr(const dk_lds* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)p);
}

// Swizzles of the part buffers (in 16-byte granules): latent rows of 512 B,
// rope rows of 128 B.
__device__ __forceinline__ constexpr int dk_swz(int h) { return 2 * ((h & 3) | (((h >> 3) & 1) << 2)); }
__device__ __forceinline__ constexpr int dk_swz_r(int h) { return 2 * (((h >> 1) & 1) | (((h >> 3) & 1) << 1)); }

// Wait until at most nl + Q of this wave's copies are outstanding (nl in 0..4).
template <int Q>
__device__ __forceinline__ void dk_wait(int nl) {
  switch (nl) {
    case 0: wait_vmem<Q>(); break;
    case 1: wait_vmem<Q + 1>(); break;
    case 2: wait_vmem<Q + 2>(); break;
    case 3: wait_vmem<Q + 3>(); break;
    default: wait_vmem<Q + 4>(); break;
  }
}

// Persistent: one workgroup per CU. Workgroup b serves queue b % 8 first
// (the XCD it runs on when workgroups are dealt to the XCDs in turn): queue
// x holds the items of the chunks c = x, x + 8, ..., row block by row block
// and half by half, so that the XCD's workgroups take one chunk's items
// together and read each token's q and dO at about the same time (from that
// XCD's L2). A workgroup whose queue is empty takes items from the next
// queues. Short items (64 tokens) keep the last round short: with 256-token
// items the last of them ran alone for about a sixth of the pass. Counters
// start at 0 (the prepass clears them); each ends past its queue's length,
// so every workgroup leaves the loop.
__global__ void __launch_bounds__(64 * kDkWaves)
sparse_mla_bwd_dkv_kernel(const BwdArgs a, const KvMajorArgs m) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_part[kDkParts][kDkPart];
  __shared__ __attribute__((aligned(1024))) uint8_t s_list[2][kDkList];
  __shared__ int s_tok[kDkChunk];
  __shared__ uint4 s_msk[kDkChunk][2];
  __shared__ int s_pre[kDkChunk];
  __shared__ int s_wcnt[4];
  __shared__ int s_item[3];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int nblk = m.num_blk;
  const int64_t T = a.num_tokens;
  const int nchunks = (int)((T + kDkChunk - 1) / kDkChunk);
  const int xq = (int)(blockIdx.x % kDkQueues);
  const int rq = wave >> 1, cw = wave & 1;
  int qi = 0;   // queues xq, xq + 1, ... in turn (an empty one is not visited again)

  for (;;) {
  __syncthreads();   // the previous item's LDS reads are done
  if (tid == 0) {
    int chunk = -1, bk = 0, half = 0;
    for (; qi < kDkQueues; ++qi) {
      const int y = (xq + qi) % kDkQueues;
      const int len = (nchunks - y + kDkQueues - 1) / kDkQueues * 2 * nblk;   // chunks y, y + 8, ...
      if (len <= 0) continue;
      const int i = (int)atomicAdd(m.queue + y, 1u);
      if (i < len) {
        chunk = y + kDkQueues * (i / (2 * nblk));
        bk = (i % (2 * nblk)) >> 1;
        half = i & 1;
        break;
      }
    }
    s_item[0] = chunk;
    s_item[1] = bk;
    s_item[2] = half;
  }
  __syncthreads();
  if (s_item[0] < 0) break;   // uniform: every queue is exhausted
  const int blk = s_item[1];
  const int ch = s_item[2];
  const int64_t t0 = (int64_t)s_item[0] * kDkChunk;
  const int64_t r0 = (int64_t)blk * kDkRows;

  // ---- the chunk's tokens that name rows of the block, in token order
  {
    uint32_t w[kDkWords];
    uint64_t act = 0;
    const int64_t t = t0 + 64 * wave + lane;
    if (wave < kDkBallots) {
      uint32_t any = 0u;
#pragma unroll
      for (int i = 0; i < kDkWords; ++i) {
        w[i] = (t < T && kDkWords * blk + i < m.num_words) ? m.mask[(int64_t)(kDkWords * blk + i) * T + t] : 0u;
        any |= w[i];
      }
      act = __ballot(any != 0u);
      if (lane == 0) s_wcnt[wave] = __popcll(act);
    }
    __syncthreads();
    if (wave < kDkBallots && ((act >> lane) & 1ull)) {
      int base = 0;
      for (int i = 0; i < wave; ++i) base += s_wcnt[i];
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(act >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)act, 0u));
      s_tok[pos] = 64 * wave + lane;
      s_msk[pos][0] = (uint4){w[0], w[1], w[2], w[3]};
      s_msk[pos][1] = (uint4){w[4], w[5], w[6], w[7]};
      s_pre[pos] = m.pre[(int64_t)blk * T + t];
    }
  }
  int np = 0;
#pragma unroll
  for (int i = 0; i < kDkBallots; ++i) np += s_wcnt[i];
  if (np == 0) continue;   // uniform over the workgroup
  __syncthreads();

  const int num_heads = a.num_heads;
  const int groups = m.groups;
  const uint16_t* const q_ptr = a.q;
  const uint16_t* const do_ptr = a.dout;
  const int64_t q_st = a.q_st, q_sh = a.q_sh, do_st = a.do_st, do_sh = a.do_sh;
  const uint8_t* const pds = reinterpret_cast<const uint8_t*>(m.pds);
  const int64_t cap = m.cap;

  // ---- copies. The latent half of part i (q or dO) into ring buffer
  // i % 3: wave w copies head rows 2j, 2j + 1 for j = w, w + 8 (one copy per
  // pair: lanes 0..31 the first row, 32..63 the second; lane L fetches
  // logical granule (L & 31) ^ dk_swz(row) of the half). For a q part waves
  // 0..3 also copy the whole rope part, rows 8w .. 8w+7 (lane L: row 8w +
  // L/8, rope granule (L & 7) ^ dk_swz_r(row)). Padded heads copy the
  // group's last head. A plan holds a part's scalars; copy k issues the
  // wave's k-th copy, so that the copies can be spread over the products.
  struct PartPlan {
    const uint16_t* base;   // the token's q or dO row, head h0
    int64_t sh;
    const uint16_t* rope;   // the token's q row, head h0, rope columns
    int hmax;
    uint32_t dst;
  };
  auto part_plan = [&](int i) {
    PartPlan pl;
    const int s = i >> 1;
    const int p = s / groups, hg = s - p * groups;
    const int64_t tok = t0 + __builtin_amdgcn_readfirstlane(s_tok[p]);
    const int h0 = kDkHeads * hg;
    pl.hmax = min(kDkHeads - 1, num_heads - 1 - h0);
    pl.dst = lds_offset(&s_part[i % kDkParts][0]);
    const bool isq = (i & 1) == 0;
    pl.sh = isq ? q_sh : do_sh;
    pl.base = (isq ? q_ptr + tok * q_st : do_ptr + tok * do_st) + (int64_t)h0 * pl.sh;
    pl.rope = q_ptr + tok * q_st + (int64_t)h0 * q_sh + kDv;
    return pl;
  };
  auto part_copy = [&](const PartPlan& pl, int k) {   // k < 2: latent head pairs; k = 2: rope (waves 0..3)
    if (k < 2) {
      const int h = 2 * (wave + 8 * k) + (lane >> 5);
      dma_16b(pl.base + (int64_t)min(h, pl.hmax) * pl.sh + 256 * ch + 8 * ((lane & 31) ^ dk_swz(h)),
              pl.dst + (uint32_t)((2 * (wave + 8 * k)) * 512));
    } else {
      const int h = 8 * wave + (lane >> 3);
      dma_16b(pl.rope + (int64_t)min(h, pl.hmax) * q_sh + 8 * ((lane & 7) ^ dk_swz_r(h)),
              pl.dst + (uint32_t)(kDkQR + 8 * wave * 128));
    }
  };
  const int qcopies = wave < 4 ? 3 : 2;   // copies of a q part per wave (a dO part: 2)
  // The entry run of step s into list buffer s & 1: copy k (k < ceil(cnt / 8))
  // holds entries 8k .. 8k+7 and is issued by wave k % 8 (lane L: entry 8k +
  // L/8, stored unit L & 7 holds unit (L & 7) ^ (entry & 7)); entries past
  // the run copy its last entry (the run is never empty: the token names a
  // row of the block). nl is the wave's number of copies.
  struct ListPlan {
    const uint8_t* run;
    int cnt, nl;
    uint32_t dst;
  };
  auto list_plan = [&](int s) {
    ListPlan lp;
    const int p = s / groups, hg = s - p * groups;
    const int64_t tok = t0 + __builtin_amdgcn_readfirstlane(s_tok[p]);
    const uint4 m0 = s_msk[p][0], m1 = s_msk[p][1];
    lp.cnt = __builtin_amdgcn_readfirstlane(__popc(m0.x) + __popc(m0.y) + __popc(m0.z) + __popc(m0.w) +
                                            __popc(m1.x) + __popc(m1.y) + __popc(m1.z) + __popc(m1.w));
    const int pre = __builtin_amdgcn_readfirstlane(s_pre[p]);
    lp.run = pds + ((tok * groups + hg) * cap + pre) * kDkEnt;
    lp.dst = lds_offset(&s_list[s & 1][0]);
    const int ncp = (lp.cnt + 7) >> 3;
    lp.nl = max(0, (ncp - wave + 7) >> 3);   // copies k = wave, wave + 8, .. < ncp
    return lp;
  };
  auto list_copy = [&](const ListPlan& lp, int i) {
    const int k = wave + 8 * i;
    const int e = 8 * k + (lane >> 3);
    const int u = (lane & 7) ^ (e & 7);
    dma_16b(lp.run + (int64_t)min(e, lp.cnt - 1) * kDkEnt + 16 * u, lp.dst + (uint32_t)(k * 1024));
  };

  // dkv of the wave's rows and columns: acc[rt][k], lane (g, n) holds
  // column n of tile k (k < 8: latent columns 256ch + 128cw + 16k ..; k = 8:
  // rope columns 512 + 32ch + 16cw ..) for rows 64rq + 16rt + 4g + e
  float4_t acc[4][9];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int k = 0; k < 9; ++k) acc[rt][k] = (float4_t){0.f, 0.f, 0.f, 0.f};

  // Transposed reads of head rows hr = 8g + n/4 and hr + 4: latent column
  // tile 8cw + k of the half at t_lat[k] (the second read: +4 rows), the
  // rope tile 2ch + cw at t_rope. Both rows share the swizzle's bits 0, 1
  // and 3, so the second read's granule is the first's.
  uint32_t t_lat[8], t_rope;
  {
    const int hr = 8 * g + (n >> 2), hb = (n >> 1) & 1;
    static_assert(dk_swz(0) == dk_swz(4) && dk_swz_r(0) == dk_swz_r(4) && dk_swz(9) == dk_swz(13) &&
                  dk_swz_r(11) == dk_swz_r(15), "rows h and h + 4 (h & 4 == 0) share a swizzle");
#pragma unroll
    for (int k = 0; k < 8; ++k)
      t_lat[k] = (uint32_t)(hr * 512 + 256 * cw + 16 * ((2 * k + hb) ^ dk_swz(hr)) + 8 * (n & 1));
    t_rope = (uint32_t)(kDkQR + hr * 128 + 16 * ((2 * (2 * ch + cw) + hb) ^ dk_swz_r(hr)) + 8 * (n & 1));
  }

  {
    const ListPlan lp = list_plan(0);
    for (int i = 0; i < lp.nl; ++i) list_copy(lp, i);
    const PartPlan q0 = part_plan(0), d0 = part_plan(1);
    for (int k = 0; k < qcopies; ++k) part_copy(q0, k);
    part_copy(d0, 0);
    part_copy(d0, 1);
  }
  wait_vmem<2>();   // the run and q part of step 0 (the dO part may still fly)
  __syncthreads();

  // per-lane list offsets of the current token's rows (row tile rt: row
  // 64rq + 16rt + n): byte offsets of unit g (P) and unit 4 + g (s dS) of
  // the row's entry, and whether the token names the row
  uint32_t off_p[4], off_d[4];
  bool named[4];
  auto row_offsets = [&](int p) {
    const uint4 m0 = s_msk[p][0], m1 = s_msk[p][1];
    const uint32_t wv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    int below = 0;   // named rows in the words below the wave's rows (rq is wave-uniform)
#pragma unroll
    for (int i = 0; i < 6; ++i) below += i < 2 * rq ? __popc(wv[i]) : 0;
    const uint32_t lo = rq == 0 ? wv[0] : rq == 1 ? wv[2] : rq == 2 ? wv[4] : wv[6];
    const uint32_t hi = rq == 0 ? wv[1] : rq == 1 ? wv[3] : rq == 2 ? wv[5] : wv[7];
    const int blo = below, bhi = below + __popc(lo);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const uint32_t word = rt < 2 ? lo : hi;
      const int bit = 16 * (rt & 1) + n;
      const int e = (rt < 2 ? blo : bhi) + __popc(word & ((1u << bit) - 1u));
      named[rt] = (word >> bit) & 1u;
      off_p[rt] = (uint32_t)(e * kDkEnt + 16 * (g ^ (e & 7)));
      off_d[rt] = (uint32_t)(e * kDkEnt + 16 * ((4 + g) ^ (e & 7)));
    }
  };
  constexpr int kRing = 4;
  auto b_read = [&](const dk_lds* part, int k) -> bf16x8_t {
    if (k < 8) {
      const dk_lds* o = part + t_lat[k];
      return join4(dk_tr(o), dk_tr(o + 4 * 512));
    }
    const dk_lds* o = part + t_rope;
    return join4(dk_tr(o), dk_tr(o + 4 * 128));
  };
  // dkv[4 row tiles x NT column tiles] += A^T B over the 32 heads of a part;
  // copy(k) runs after the products of column tile k
  auto products = [&](const dk_lds* part, const dk_lds* list, const uint32_t (&off)[4], auto nt, auto&& copy) {
    constexpr int NT = decltype(nt)::value;
    bf16x8_t av[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const bf16x8_t v = dk_b128(list + off[rt]);
      av[rt] = named[rt] ? v : (bf16x8_t){};
    }
    bf16x8_t ring[kRing];
#pragma unroll
    for (int k = 0; k < kRing; ++k) ring[k] = b_read(part, k);
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      const bf16x8_t b = ring[k % kRing];
      if (k + kRing < NT) ring[k % kRing] = b_read(part, k + kRing);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[rt], b, acc[rt][k], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      copy(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nsteps = np * groups;
  int cur_p = -1;
  for (int s = 0; s < nsteps; ++s) {
    const int p = s / groups;
    if (p != cur_p) {
      cur_p = p;
      row_offsets(p);
    }
    const dk_lds* const list = (const dk_lds*)&s_list[s & 1][0];
    // ---- q part (part 2s): dkv[:, all 9 tiles] += (s dS)^T q. The next
    // step's run and q part are copied meanwhile (their buffers were left at
    // the last barrier).
    const bool more = s + 1 < nsteps;
    int nl = 0;
    if (more) {
      const ListPlan lp = list_plan(s + 1);
      nl = lp.nl;
      for (int i = 0; i < nl; ++i) list_copy(lp, i);
      const PartPlan qn = part_plan(2 * s + 2);
      for (int k = 0; k < qcopies; ++k) part_copy(qn, k);
    }
    products((const dk_lds*)&s_part[(2 * s) % kDkParts][0], list, off_d, std::integral_constant<int, 9>(),
             [](int) {});
    // the dO part of this step landed in this wave; the copies issued above may still fly
    if (!more) wait_vmem<0>();
    else if (qcopies == 3) dk_wait<3>(nl);
    else dk_wait<2>(nl);
    __syncthreads();
    // ---- dO part (part 2s + 1): dkv[:, latent tiles] += P^T dO
    if (more) {
      const PartPlan dn = part_plan(2 * s + 3);
      part_copy(dn, 0);
      part_copy(dn, 1);
    }
    products((const dk_lds*)&s_part[(2 * s + 1) % kDkParts][0], list, off_p, std::integral_constant<int, 8>(),
             [](int) {});
    // the next step's run and q part landed
    if (more) wait_vmem<2>();
    else wait_vmem<0>();
    __syncthreads();
  }

  // ---- the rows' dkv, once per item (other chunks add to the same rows)
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      const int col = k < 8 ? 256 * ch + 128 * cw + 16 * k + n : kDv + 32 * ch + 16 * cw + n;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t r = r0 + 64 * rq + 16 * rt + 4 * g + e;
        if (r < a.num_kv) unsafeAtomicAdd(a.dkv + r * a.dkv_st + col, acc[rt][k][e]);
      }
    }
  }
}

}  // namespace dsa
