// dq pass of the split backward schedule (more than 16 heads): for every
// token whose index row repeats no entry, dq = s dS K over the token's valid
// keys (the notation of bwd_kernel.hpp), and P and s dS of every (key, head)
// stored for the dkv pass (bwd_dkv_kernel.hpp), which forms dkv of the same
// tokens from them.
//
// One workgroup of 8 waves = (token, block of 64 heads; 32 at up to 32
// heads), two waves per SIMD with split roles. The index row is compacted
// per 2048-entry segment as in the forward, into the named row ids. Tiles
// of 32 keys are copied HBM -> LDS with global_load_lds_dwordx4 by the dq
// waves into a ring of four stages (swizzled latent and rope parts). Per
// tile j:
//   S waves (4): wave w forms S^T = K Q^T and dP^T = V dO^T of head tile w
//            over both 16-key blocks (at 32 heads: key block w & 1 of head
//            tile w >> 1) on 16x16x32 MFMA, with Q^T and dO^T in registers
//            and each K-row read feeding both products; then P = exp(s S -
//            LSE) and s dS = s P (dP - D) (D = dO . O, formed once per token
//            from O and the dO registers), s dS into LDS as bf16 [head][32
//            keys] in the dq product's k-slot order, and P and s dS
//            transposed over lane quads into per-key rows, stored at each
//            key's rank (read from the prepass one tile ahead) during the
//            next tile's products;
//   dq waves (4): dq column tiles 4k + w (k = 0..8) of every head tile +=
//            (s dS) K for tile j - 1, K^T read transposed from the stage,
//            and the copies of tile j + 2.
// One barrier per tile (s dS of tile j written; tile j + 1 landed).
//
// Pages: "[Feature] Add optional FlashMLA backend for DSA Sparse MLA"
// (xtuner PR 2083), Motivation (forward output and LSE feed the backward);
// the prime-rl pull request 4078 that adds a `cudnn_flashmla` DSA backend
// (a separate DSA backward kernel, timed per call).
#pragma once

#include "bwd_kernel.hpp"

namespace dsa {

constexpr int kDqWaves = 8;                                   // 4 S waves, 4 dq waves: two per SIMD
constexpr int kDqStages = 4;                                  // LDS ring depth
constexpr int kDqDmaPerWave = kTileKeys / 4 + 1;              // per dq wave: 8 latent rows + 8 rope rows, 9 copies
static_assert(kBwStage % 1024 == 0, "stages keep the 1 KB copy alignment");

// Copy tile t into stage t % kDqStages: wave w takes latent rows 8w .. 8w+7
// (one 1 KB row per copy; lane i fetches logical granule i ^ bw_swz(row))
// and rope rows 8w .. 8w+7 (one copy; lane i fetches rope granule
// (i & 7) ^ bw_swz_r(row) of row 8w + i/8).
__device__ __forceinline__ void dq_issue_tile(const BwdArgs& a, const uint32_t* s_rows, uint32_t stage_lds, int t,
                                              int wave, int lane) {
  const uint32_t base = stage_lds + (uint32_t)((t % kDqStages) * kBwStage);
  const uint4* gl = (const uint4*)(s_rows + t * kTileKeys + 8 * wave);
  uint32_t go[8];
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const uint4 v = gl[q2];   // same address in every lane: a broadcast read
    go[4 * q2 + 0] = v.x;
    go[4 * q2 + 1] = v.y;
    go[4 * q2 + 2] = v.z;
    go[4 * q2 + 3] = v.w;
  }
  const int rrow = 8 * wave + (lane >> 3);
  const uint32_t gr = s_rows[t * kTileKeys + rrow];
  const uint32_t lane16 = (uint32_t)lane * 16u;
  const uint64_t kvb = (uint64_t)a.kv, rb = (uint64_t)a.kv_st * 2u;   // row stride in bytes
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = 8 * wave + u;
    const uint64_t sb = kvb + (uint64_t)__builtin_amdgcn_readfirstlane(go[u]) * rb;
    dma_16b_sbase(sb, lane16 ^ (uint32_t)(bw_swz(row) * 16), base + (uint32_t)(row * 1024));
  }
  const uint32_t g = (uint32_t)((lane & 7) ^ bw_swz_r(rrow));
  dma_16b((const void*)(kvb + (uint64_t)gr * rb + (uint64_t)(2 * kDv) + 16u * g),
          base + (uint32_t)(kBwLat + wave * 1024));
}

// s dS row swizzle (8-byte units; rows of 64 bytes)
__device__ __forceinline__ constexpr int dst_swz(int n) { return (n & 6) | ((n >> 3) & 1); }

// 4 x 4 transpose of bf16 values over the lanes of a quad (i = lane & 3).
// On entry lane i holds row i: x0 = (v0, v1), x1 = (v2, v3); on exit it holds
// element i of rows 0 .. 3, packed the same way. Two quad permutes (DPP).
__device__ __forceinline__ uint2 quad_transpose_bf16(uint32_t x0, uint32_t x1, int i) {
  const bool b1 = (i & 2) != 0, b0 = (i & 1) != 0;
  // exchange with lane i ^ 2: lanes 0, 1 keep elements 0, 1; lanes 2, 3 elements 2, 3
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(b1 ? x0 : x1), 0x4E, 0xF, 0xF, false);
  const uint32_t A = b1 ? r1 : x0;   // row i & 1
  const uint32_t B = b1 ? x1 : r1;   // row (i & 1) + 2
  // exchange with lane i ^ 1: an even lane keeps the low elements, an odd lane the high ones
  const uint32_t send = b0 ? ((A & 0xFFFFu) | (B << 16)) : ((A >> 16) | (B & 0xFFFF0000u));
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
  uint2 o;
  o.x = b0 ? ((r2 & 0xFFFFu) | (A & 0xFFFF0000u)) : ((A & 0xFFFFu) | (r2 << 16));
  o.y = b0 ? ((r2 >> 16) | (B & 0xFFFF0000u)) : ((B & 0xFFFFu) | (r2 & 0xFFFF0000u));
  return o;
}

// HT head tiles of 16 per workgroup (2 or 4). With 2, S wave w takes key
// block w & 1 of head tile w >> 1; with 4, S wave w takes both key blocks
// of head tile w (each Q^T / dO^T operand then serves twice as many
// products, and each tile is gathered once for 64 heads).
// blockIdx.x = token * head_blocks + head block, over the tokens with
// only[token] == 0 (only_nonzero = 0).
template <int HT>
__global__ void __launch_bounds__(64 * kDqWaves)
sparse_mla_bwd_dq_kernel(const BwdArgs a, const KvMajorArgs m) {
  static_assert(HT == 2 || HT == 4, "32 or 64 heads per workgroup");
  constexpr int KBW = HT / 2;   // key blocks per S wave
  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[kDqStages * kBwStage];
  // s dS, bf16 [16 HT heads][32 keys], one buffer per tile parity: logical
  // 8-byte unit 2q of a head's row holds keys 4q .. 4q+3, unit 2q+1 keys
  // 16+4q .. 16+4q+3; unit u of head row h sits at u ^ dst_swz(h % 16), so
  // that the 16 lanes a b64 write serves together hit distinct banks
  __shared__ __attribute__((aligned(16))) uint8_t s_dst[2][16 * HT * 64];
  __shared__ __attribute__((aligned(16))) uint32_t s_rows[kSegment];   // compacted row ids
  // the index stage's chunk counts share the s dS buffers (160 KB of LDS
  // in all at 64 heads); a barrier ends each index segment, so no wave still
  // reads s dS when the next segment's index stage writes them
  int* const s_cnt = reinterpret_cast<int*>(&s_dst[1][0]);
  static_assert(kChunks * 4 <= 16 * HT * 64, "the chunk counts fit a s dS buffer");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool is_s = wave < 4;   // role (uniform per wave)
  const int sw = wave & 3;      // index within the role
  const int n = lane & 15, g = lane >> 4;   // MFMA column / k-group of the lane
  const int64_t token = blockIdx.x / a.head_blocks;
  const int h0 = (int)(blockIdx.x % a.head_blocks) * 16 * HT;
  if (a.only && ((a.only[token] != 0u) != (a.only_nonzero != 0))) return;   // uniform over the workgroup

  FwdArgs fa = {};   // the forward's index stage, with row ids as the offsets
  fa.idx = a.idx;
  fa.idx_st = a.idx_st;
  fa.num_kv = a.num_kv;
  fa.kv_row_gran = 1;
  fa.topk = a.topk;
  fa.seg_len = kSegment;
  const uint32_t stage_lds = lds_offset(s_stage);
  const int nseg = (a.topk + kSegment - 1) / kSegment;

  // Barrier sequence per index segment, every wave: the index stage's two;
  // tile 0 landed; then after iteration j < ntiles: s dS of tile j written
  // and tile j+1 landed; the dq waves' last products done. In iteration j the S waves form s dS of tile j and
  // the dq waves take the dq products of tile j - 1 and copy tile j + 2
  // into the stage of tile j - 2.
  if (is_s) {
    // ============================================================ S waves
    // Key blocks kb0 .. kb0 + KBW - 1, head tile ht; the lane's head is h0 + 16ht + n.
    const int kb0 = HT == 2 ? (sw & 1) : 0, ht = HT == 2 ? (sw >> 1) : sw;
    const int head = h0 + 16 * ht + n;
    const bool head_ok = head < a.num_heads;
    // Q^T and dO^T as the MFMA B operand: lane holds columns 32c + 8g .. +7 of its head
    bf16x8_t bq[kDqk / 32], bdo[kDv / 32];
    {
      const int hh = head_ok ? head : 0;
      const uint16_t* qp = a.q + token * a.q_st + (int64_t)hh * a.q_sh + 8 * g;
      const uint16_t* dp = a.dout + token * a.do_st + (int64_t)hh * a.do_sh + 8 * g;
#pragma unroll
      for (int c = 0; c < kDqk / 32; ++c) {
        const bf16x8_t v = *(const bf16x8_t*)(qp + 32 * c);
        bq[c] = head_ok ? v : (bf16x8_t){};
      }
#pragma unroll
      for (int c = 0; c < kDv / 32; ++c) {
        const bf16x8_t v = *(const bf16x8_t*)(dp + 32 * c);
        bdo[c] = head_ok ? v : (bf16x8_t){};
      }
    }
    // D = dO . O of the lane's head, with dO from the operand registers (the
    // four lanes of a head hold its 512 columns); LSE in log2 units, +inf
    // for padded heads (P = 0 there)
    float Dh;
    {
      const uint16_t* op = a.out + token * a.o_st + (int64_t)(head_ok ? head : 0) * a.o_sh + 8 * g;
      float d = 0.f;
#pragma unroll
      for (int c = 0; c < kDv / 32; ++c) {
        const bf16x8_t o = *(const bf16x8_t*)(op + 32 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) d += (float)o[e] * (float)bdo[c][e];
      }
      d += __shfl_xor(d, 16);
      d += __shfl_xor(d, 32);
      Dh = head_ok ? d : 0.f;
    }
    const float l2 = head_ok ? a.lse[token * a.lse_st + head] * 1.4426950408889634f : INFINITY;
    // P and s dS for the dkv pass: after the quad transpose, lane (g, n)
    // holds key 16kb + 4g + (n & 3) and heads 16ht + 4(n >> 2) .. +3; they go
    // to the key's rank in the head group's run, heads in order (the four
    // lanes of a key write the head tile's 32 contiguous bytes)
    const int hg = (h0 + 16 * ht) >> 5;
    const bool pds_ok = hg < m.groups;
    uint8_t* const pds_tok = reinterpret_cast<uint8_t*>(m.pds) + ((token * m.groups + hg) * m.cap) * 128 +
                             32 * (ht & 1) + 8 * (n >> 2);
    const int32_t* const rank_tok = m.rank + token * m.cap;
    int cbase = 0;   // valid entries of the earlier index segments
    // A-operand offsets of key block kb0 + b: key 16(kb0 + b) + n, logical
    // granule c' = 4c + g; latent c = 4i + c'' at a_lat[b][c''] + 256i, rope
    // c = 16 + c'' at a_rope[b][c''].
    uint32_t a_lat[KBW][4], a_rope[KBW][2];
#pragma unroll
    for (int b = 0; b < KBW; ++b) {
      const int r = (kb0 + b) * 16 + n;
#pragma unroll
      for (int c = 0; c < 4; ++c) a_lat[b][c] = (uint32_t)(r * 1024 + 16 * ((4 * c + g) ^ bw_swz(r)));
#pragma unroll
      for (int c = 0; c < 2; ++c) a_rope[b][c] = (uint32_t)(kBwLat + r * 128 + 16 * ((4 * c + g) ^ bw_swz_r(r)));
    }

    for (int seg = 0; seg < nseg; ++seg) {
      const int nvalid = build_key_list<false, kDqWaves>(fa, token, seg, wave, lane, s_rows, s_cnt, [] {});
      const int ntiles = (nvalid + kTileKeys - 1) / kTileKeys;
      if (ntiles == 0) continue;   // uniform
      // ranks of the keys this lane stores in phase 2 of tile j, read one
      // tile ahead and before the stores of the tile in between (the wait
      // for a read would otherwise also wait for those stores)
      auto read_ranks = [&](int j, int (&rk)[KBW]) {
#pragma unroll
        for (int b = 0; b < KBW; ++b) {
          const int kk = j * kTileKeys + 16 * (kb0 + b) + 4 * g + (n & 3);
          rk[b] = rank_tok[cbase + (kk < nvalid ? kk : 0)];
        }
      };
      int rk[KBW], rk_next[KBW];
      read_ranks(0, rk);
      // P and s dS of the previous tile, stored during this tile's products
      // (issued at the end of phase 2 they waited, before the barrier, behind
      // the dq waves' copies in the CU's memory queue)
      uint2 pend_p[KBW], pend_d[KBW];
      int pend_rk[KBW];
      bool pend_ok[KBW];
#pragma unroll
      for (int b = 0; b < KBW; ++b) pend_ok[b] = false;
      auto store_pending = [&](int b) {
        if (pend_ok[b]) {
          uint8_t* const d = pds_tok + (int64_t)pend_rk[b] * 128;
          *(uint2*)d = pend_p[b];
          *(uint2*)(d + 64) = pend_d[b];
        }
      };
      __syncthreads();             // tile 0 landed
      for (int j = 0; j < ntiles; ++j) {
        const uint8_t* st = s_stage + (j % kDqStages) * kBwStage;
        const int lim = nvalid - j * kTileKeys;
        // ---- phase 1: S^T and dP^T of key blocks kb0 .., head tile ht
        float4_t acc_s[KBW], acc_dp[KBW];
#pragma unroll
        for (int b = 0; b < KBW; ++b) acc_s[b] = acc_dp[b] = (float4_t){0.f, 0.f, 0.f, 0.f};
        {
          // read i: chunk i / KBW of key block kb0 + i % KBW
          constexpr int kReads = KBW * (kDqk / 32);
          auto a_read = [&](int i) {
            const int c = i / KBW, b = i % KBW;
            return lds16(c < 16 ? st + a_lat[b][c & 3] + 256 * (c >> 2) : st + a_rope[b][c - 16]);
          };
          // A operands read 6 ahead (pinned order: the scheduler would
          // otherwise sink each read next to its products)
          constexpr int kRing = 6;
          bf16x8_t ring[kRing];
#pragma unroll
          for (int i = 0; i < kRing; ++i) ring[i] = a_read(i);
#pragma unroll
          for (int i = 0; i < kReads; ++i) {
            const int c = i / KBW, b = i % KBW;
            const bf16x8_t av = ring[i % kRing];
            if (i + kRing < kReads) ring[i % kRing] = a_read(i + kRing);
            acc_s[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bq[c], acc_s[b], 0, 0, 0);
            if (c < kDv / 32) acc_dp[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bdo[c], acc_dp[b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (i % 8 == 3 && i / 8 < KBW) store_pending(i / 8);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // ---- phase 2: P and s*dS (lane: head 16ht + n, keys 16kb + 4g + e)
#pragma unroll
        for (int b = 0; b < KBW; ++b) {
          const int kb = kb0 + b;
          float pv[4], ds[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool ok = kb * 16 + 4 * g + e < lim;
            pv[e] = ok ? __builtin_amdgcn_exp2f(acc_s[b][e] * a.scale_log2 - l2) : 0.f;
            ds[e] = pv[e] * (acc_dp[b][e] - Dh) * a.scale;
          }
          const uint32_t d01 = pack_bf16x2(ds[0], ds[1]), d23 = pack_bf16x2(ds[2], ds[3]);
          *(uint2*)(s_dst[j & 1] + (16 * ht + n) * 64 + 8 * ((2 * g + kb) ^ dst_swz(n))) = (uint2){d01, d23};
          if (b == 0) read_ranks(j + 1 < ntiles ? j + 1 : j, rk_next);
          pend_p[b] = quad_transpose_bf16(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), n & 3);
          pend_d[b] = quad_transpose_bf16(d01, d23, n & 3);
          pend_rk[b] = rk[b];
          pend_ok[b] = pds_ok && kb * 16 + 4 * g + (n & 3) < lim;
        }
#pragma unroll
        for (int b = 0; b < KBW; ++b) rk[b] = rk_next[b];
        __syncthreads();   // s dS of tile j written; tile j+1 landed
      }
#pragma unroll
      for (int b = 0; b < KBW; ++b) store_pending(b);   // the last tile's
      __syncthreads();     // the dq waves' last products are done
      cbase += nvalid;
    }
  } else {
    // ============================================================ dq waves
    // dq column tiles m = 4k + sw (k = 0 .. 8) of head tile t: lane holds
    // column 16m + n of heads 16t + 4g .. +3
    float4_t dq_acc[HT][9];
#pragma unroll
    for (int t = 0; t < HT; ++t)
#pragma unroll
      for (int k = 0; k < 9; ++k) dq_acc[t][k] = (float4_t){0.f, 0.f, 0.f, 0.f};
    // K^T operand of column tile m = 4k + sw: lane (g, n) points at key
    // 4g + n/4 (and 16 + 4g + n/4), columns 16m + 4(n % 4) ..; latent tile
    // k at t_lat[k % 2] + 256 (k / 2), the rope tile (k = 8) at t_rope.
    uint32_t t_lat[2], t_rope;
    {
      const int r = 4 * g + (n >> 2), hb = (n >> 1) & 1;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        t_lat[i] = (uint32_t)(r * 1024 + 16 * ((2 * (sw + 4 * i) + hb) ^ bw_swz(r)) + 8 * (n & 1));
      t_rope = (uint32_t)(kBwLat + r * 128 + 16 * ((2 * sw + hb) ^ bw_swz_r(r)) + 8 * (n & 1));
    }
    // ---- phase 3 of tile j: dq tiles 4k + sw += (s dS)[16 heads x 32 keys] K[32 keys x 16 columns],
    //      k slots 8g .. 8g+7 = keys 4g .. 4g+3, 16+4g .. 16+4g+3
    auto phase3 = [&](int j) {
      const uint8_t* st = s_stage + (j % kDqStages) * kBwStage;
      bf16x8_t ads[HT];
#pragma unroll
      for (int t = 0; t < HT; ++t) {
        // units 2g, 2g+1 share a granule; an odd swizzle stores them swapped
        const bf16x8_t v = lds16(s_dst[j & 1] + (16 * t + n) * 64 + 16 * (g ^ (dst_swz(n) >> 1)));
        ads[t] = (dst_swz(n) & 1) ? __builtin_shufflevector(v, v, 4, 5, 6, 7, 0, 1, 2, 3) : v;
      }
      constexpr int kRA = 4;
      bf16x8_t kb_ring[kRA];
      auto kt_read = [&](int k) {
        if (k < 8) {
          const uint8_t* p = st + t_lat[k & 1] + 256 * (k >> 1);
          return join4(lds_read_tr16(p), lds_read_tr16(p + 16 * 1024));
        }
        const uint8_t* p = st + t_rope;
        return join4(lds_read_tr16(p), lds_read_tr16(p + 16 * 128));
      };
#pragma unroll
      for (int k = 0; k < kRA; ++k) kb_ring[k] = kt_read(k);
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        const bf16x8_t b = kb_ring[k % kRA];
        if (k + kRA < 9) kb_ring[k % kRA] = kt_read(k + kRA);
#pragma unroll
        for (int t = 0; t < HT; ++t)
          dq_acc[t][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ads[t], b, dq_acc[t][k], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    for (int seg = 0; seg < nseg; ++seg) {
      const int nvalid = build_key_list<false, kDqWaves>(fa, token, seg, wave, lane, s_rows, s_cnt, [] {});
      const int ntiles = (nvalid + kTileKeys - 1) / kTileKeys;
      if (ntiles == 0) continue;   // uniform
      dq_issue_tile(a, s_rows, stage_lds, 0, sw, lane);
      if (ntiles > 1) {
        dq_issue_tile(a, s_rows, stage_lds, 1, sw, lane);
        wait_vmem<kDqDmaPerWave>();
      } else {
        wait_vmem<0>();
      }
      __syncthreads();   // tile 0 landed
      for (int j = 0; j < ntiles; ++j) {
        // stage (j + 2) % 4 held tile j - 2: every wave left it at the last barrier
        if (j + 2 < ntiles) dq_issue_tile(a, s_rows, stage_lds, j + 2, sw, lane);
        if (j > 0) phase3(j - 1);
        // tile j+1 landed in this wave (tile j+2 may still fly)
        if (j + 2 < ntiles) wait_vmem<kDqDmaPerWave>();
        else wait_vmem<0>();
        __syncthreads();   // s dS of tile j written; tile j+1 landed
      }
      phase3(ntiles - 1);
      __syncthreads();   // s dS and the stages are free for the next segment
    }

    // ---------------------------------------------------------------- dq (fp32)
#pragma unroll
    for (int t = 0; t < HT; ++t)
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        const int d = 16 * (4 * k + sw) + n;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int h = h0 + 16 * t + 4 * g + e;
          if (h < a.num_heads) a.dq[token * a.dq_st + (int64_t)h * a.dq_sh + d] = dq_acc[t][k][e];
        }
      }
  }
}

}  // namespace dsa
