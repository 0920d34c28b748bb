// Sparse MLA forward for blocks of 64 heads: two waves per SIMD with split roles.
//
// Same steps as sparse_mla_fwd_kernel (index stage, gather ring, QK^T, online
// softmax, PV, epilogue). The work split targets the MFMA-bound regime. With
// one wave per SIMD, in-order issue exposes every LDS round trip (~250
// clocks), barrier and dependent VALU chain to the matrix pipe. A second wave
// on the SIMD lets the hardware fill those gaps. Eight waves fit in 256
// registers each only if their state is split by role:
//
//   S waves (w = 0..3): head half hh = w & 1, key block kd = (w >> 1) & 1.
//     QK^T of 32 heads against keys 16kd .. 16kd+15 of a tile: 36 16x16x32
//     MFMAs, two head tiles per K read, Q^T mostly in the accumulator file.
//     Raw fp32 scores go to LDS. The S waves also issue the gather.
//   PV waves (w = 4..7): head half hh, value half kd.
//     The online softmax of all 32 keys of a tile for 32 heads: each lane
//     reads the 16 scores that form its P^T operand. Then O^T[256 columns x
//     32 heads] += V^T P^T: 16 32x32x16 MFMAs, O^T in the accumulator file.
//     The two PV waves of a head half compute the same reference maxima from
//     the same scores, so they scale P and O identically without talking.
// The hardware places wave w on SIMD w % 4, so each SIMD runs one S wave and
// one PV wave. Per tile every SIMD has 36 x 16 + 16 x 32 = 1088 MFMA clocks.
//
// Pipeline: in iteration j the S waves score tile j+1 while the PV waves
// finish tile j. One workgroup barrier per tile publishes the scores and the
// gathered rows.
//
// LDS (exactly 160 KB): the 4-stage tile ring (kStages x 36 KB), plus two
// score buffers of 8 KB (tile parity). During the index stage the first
// holds the compacted key list and the second the chunk counts.
//
// Pages: "feat: add XTuner TileLang sparse MLA backend" (lmdeploy PR 4904),
// Performance > Isolated sparse MLA forward (64-head operation of the other
// kernel); "[Feature] Add optional FlashMLA backend for DSA Sparse MLA"
// (xtuner PR 2083), Runtime constraints.
#pragma once

#include "fwd_kernel.hpp"

namespace dsa {

typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kWsWaves = 8;
constexpr int kScoreBytes = 2 * 32 * 32 * 4;   // one tile: [hh 2][32 heads][32 keys] fp32
static_assert(kScoreBytes == kSegment * 4, "a score buffer doubles as the key list");

// Latent-row swizzle of this kernel's tiles: granule G of latent row r is
// stored at G ^ swz_ws(r). A bijection of r & 15 (16 consecutive rows read at
// one logical granule hit distinct banks), and the 4 rows x 4 granules of a
// half-wave transposed V read also hit distinct banks.
__host__ __device__ constexpr int swz_ws(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Score buffer: 16-byte group g (keys 4g .. 4g+3) of head h sits at group
// g ^ ((h >> 1) & 7) of the head's 128-byte row, so that 16 consecutive heads
// at one group use 16 distinct 4-bank groups.
__host__ __device__ constexpr int score_off(int h, int g) { return h * 128 + 16 * (g ^ ((h >> 1) & 7)); }

__device__ __forceinline__ short4_t lds_tr16_at(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(uintptr_t)addr);
}
__device__ __forceinline__ bf16x8_t lds_b128_at(uint32_t addr) {
  return *(__attribute__((address_space(3))) const bf16x8_t*)(uintptr_t)addr;
}
__device__ __forceinline__ float4_t lds_f4_at(uint32_t addr) {
  return *(__attribute__((address_space(3))) const float4_t*)(uintptr_t)addr;
}
__device__ __forceinline__ void lds_f4_write_at(uint32_t addr, float4_t v) {
  *(__attribute__((address_space(3))) float4_t*)(uintptr_t)addr = v;
}

// Combine over lanes l and l ^ 32 with the gfx950 lane swap (VALU, no LDS
// round trip). The swap reads VGPRs that the previous VALU instruction may
// have just written, so s_nop guards both sides of it.
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_halves(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);   // a holds the low half's value in both halves, b the high half's
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float sum_halves(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Lazy reference (log2 units): it moves only when a tile maximum exceeds it
// by more than kRescaleSlack, so O is rescaled rarely after the first tile.
__device__ __forceinline__ float next_ref(float m_run, float m_tile) {
  return m_tile > m_run + kRescaleSlack ? fmaxf(m_run, m_tile) : m_run;
}
__device__ __forceinline__ float ref_factor(float m_old, float m_new) {
  return m_new == m_old ? 1.f : fast_exp2(m_old - m_new);   // m_old = -inf gives 0
}

template <bool PAGED>
__global__ void __launch_bounds__(64 * kWsWaves)
sparse_mla_fwd_ws_kernel(const FwdArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[kStages * kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_score[2][kScoreBytes];   // tile parity

  uint32_t* s_goff = (uint32_t*)s_score[0];   // index stage only
  int* s_cnt = (int*)s_score[1];              // index stage only

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool is_s = wave < 4;     // role (uniform per wave)
  const int sw = wave & 3;        // index within the role
  const int hh = sw & 1;          // head half
  const int kd = sw >> 1;         // S: key block; PV: value half

  const int64_t per_token = (int64_t)a.splits * a.head_blocks;
  const int64_t bid = blockIdx.x;
  const int64_t token = a.num_tokens - 1 - bid / per_token;   // longest rows first in causal prefill
  const int rem = (int)(bid % per_token);
  const int split = rem / a.head_blocks;
  const int hblock = rem % a.head_blocks;

  // ---------------------------------------------------------------- 1. index stage
  const int nvalid = build_key_list<PAGED, kWsWaves>(a, token, split, wave, lane, s_goff, s_cnt);
  const int ntiles = (nvalid + kTileKeys - 1) / kTileKeys;

  // S waves keep the offsets of rows 8sw .. 8sw+7 of every tile in registers:
  // row r of tile t in lane 8(t & 7) + r of klist[t >> 3].
  constexpr int kListRegs = kSegment / kTileKeys / 8;
  uint32_t klist[kListRegs];
#pragma unroll
  for (int k = 0; k < kListRegs; ++k) {
    const int n = 64 * k + lane, t = n >> 3, r = n & 7;
    klist[k] = is_s && t < ntiles ? s_goff[t * kTileKeys + 8 * sw + r] : 0u;
  }
  __syncthreads();   // the score buffers are free from here on
  const uint32_t stage_lds = lds_offset(s_stage);
  const uint32_t score_lds = lds_offset(s_score[0]);
  auto stage_of = [&](int t) { return stage_lds + (uint32_t)(t % kStages) * kStageBytes; };
  // this head half's scores of tile t: [32 heads][32 keys]
  auto scores_of = [&](int t) { return score_lds + (uint32_t)(t & 1) * kScoreBytes + (uint32_t)hh * (kScoreBytes / 2); };

  // Barrier sequence, every wave:
  //   prologue: tiles 0..2 gathered, tile 0 landed | scores of tile 0 written, tile 1 landed
  //   tile j (j + 1 < ntiles): scores of tile j+1 written, tile j+2 landed
  if (is_s) {
    // ============================================================ S waves
    const int hcol = lane & 15;   // 16x16 MFMA row / column
    const int kq = lane >> 4;     // 16x16 MFMA k-group
    // Q^T, head tile ht: dims 32c + 8kq .. +7 of head 16ht + hcol. Chunks 0..14
    // in the accumulator file (the MFMA reads them from there), which with the
    // QK^T accumulator (8) fills this wave's 128.
    bf16x8_t qreg[2][kDqk / 32];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int h = hblock * 64 + hh * 32 + ht * 16 + hcol;
      const bool ok = h < a.num_heads;
      const uint16_t* qp = a.q + token * a.q_st + (int64_t)(ok ? h : 0) * a.q_sh + 8 * kq;
#pragma unroll
      for (int c = 0; c < kDqk / 32; ++c) {
        bf16x8_t v = *(const bf16x8_t*)(qp + 32 * c);
        qreg[ht][c] = ok ? v : (bf16x8_t){};
      }
    }
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int c = 0; c < kDqk / 32; ++c) {
        if (c < 15) asm volatile("" : "+a"(qreg[ht][c]));
        else asm volatile("" : "+v"(qreg[ht][c]));
      }
    // K operand, latent chunk c: row 16kd + hcol, logical granule 4c + kq:
    //   (kb0 ^ 64(c & 3)) + 256(c >> 2);  rope chunk 16 + cr: rb0 ^ 64cr
    const int kr_row = 16 * kd + hcol;
    const uint32_t kb0 = kr_row * 1024 + 16 * (kq ^ swz_ws(kr_row));
    const uint32_t rb0 = kRopeOff + kr_row * 128 + 16 * (kq ^ ((kr_row >> 1) & 7));
    auto kread = [&](uint32_t st, int c) {
      return c < 16 ? lds_b128_at(((st + kb0) ^ (64u * (c & 3))) + 256u * (c >> 2))
                    : lds_b128_at((st + rb0) ^ (64u * (c - 16)));
    };
    const uint32_t lane16 = (uint32_t)lane * 16u;
    uint32_t grope = 0;
    auto gather_rows = [&](int t, uint32_t* go, bool live) {
      if (live && (t & 7) == 0 && t > 0) {
#pragma unroll
        for (int k = 0; k + 1 < kListRegs; ++k) klist[k] = klist[k + 1];
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) go[r] = __builtin_amdgcn_readlane(klist[0], 8 * (t & 7) + r);
      grope = (uint32_t)__builtin_amdgcn_ds_bpermute((8 * (t & 7) + (lane >> 3)) * 4, (int)klist[0]);
    };
    // copy d of this wave's share of tile t: latent row 8sw + d (d < 8), or
    // rope rows 8sw .. 8sw+7 (lane i: rope granule (i & 7) ^ ((row >> 1) & 7) of row 8sw + i/8)
    auto gather_copy = [&](int t, const uint32_t* go, int d) {
      const uint32_t base = stage_of(t);
      if (d < 8) {
        const int row = 8 * sw + d;
        dma_16b_sbase((uint64_t)a.kv + (uint64_t)go[d] * 16ull, lane16 ^ (uint32_t)(swz_ws(row) * 16),
                      base + row * 1024);
      } else {
        const int rrow = 8 * sw + (lane >> 3);
        const int g = (lane & 7) ^ ((rrow >> 1) & 7);
        dma_16b(a.kv + ((uint64_t)grope + 64u + (uint32_t)g) * 16ull, base + kRopeOff + sw * 1024);
      }
    };
    auto issue = [&](int t) {   // all of this wave's copies of tile t (prologue)
      uint32_t go[8];
      gather_rows(t, go, true);
#pragma unroll
      for (int d = 0; d < kDmaPerWave; ++d) gather_copy(t, go, d);
    };
    // QK^T of tile ts (the gather of tile ti spread over it); the raw scores
    // of head 16ht + hcol, keys 16kd + 4kq .. +3 (group 4kd + kq) go to the
    // score buffer of tile ts.
    auto s_step = [&](int ts, int ti) {
      constexpr int kS = 36;    // chunk t >> 1, head tile t & 1
      constexpr int kKA = 8;    // K chunks read ahead (about 256 MFMA clocks)
      const uint32_t st = stage_of(ts);
      uint32_t go[8];
      gather_rows(ti >= 0 ? ti : 0, go, ti >= 0);
      bf16x8_t kr[kKA + 1];
      float4_t sacc[2];
#pragma unroll
      for (int c = 0; c < kKA; ++c) kr[c] = kread(st, c);
#pragma unroll
      for (int t = 0; t < kS; ++t) {
        const int c = t >> 1;
        if ((t & 1) == 0 && c + kKA < kS / 2) kr[(c + kKA) % (kKA + 1)] = kread(st, c + kKA);
        sacc[t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[c % (kKA + 1)], qreg[t & 1][c],
                                                              c == 0 ? (float4_t){0.f, 0.f, 0.f, 0.f} : sacc[t & 1], 0, 0, 0);
        if (ti >= 0 && t % 4 == 1 && t / 4 < kDmaPerWave) gather_copy(ti, go, t / 4);   // copies at MFMA 1, 5, .., 33
        __builtin_amdgcn_sched_barrier(0);
      }
      const uint32_t sb = scores_of(ts);
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) lds_f4_write_at(sb + score_off(16 * ht + hcol, 4 * kd + kq), sacc[ht]);
    };

    if (ntiles > 0) {
      issue(0);
      if (ntiles > 1) issue(1);
      if (ntiles > 2) issue(2);
      if (ntiles > 2) wait_vmem<2 * kDmaPerWave>();
      else if (ntiles > 1) wait_vmem<kDmaPerWave>();
      else wait_vmem<0>();
      __syncthreads();
      s_step(0, -1);
      if (ntiles > 2) wait_vmem<kDmaPerWave>();   // tile 1 landed
      else wait_vmem<0>();
      __syncthreads();
      for (int j = 0; j + 1 < ntiles; ++j) {
        // QK^T of tile j+1; the gather of tile j+3 goes into the stage of tile
        // j-1 and the scores into the buffer of tile j-1, both of which the PV
        // waves left at the last barrier
        s_step(j + 1, j + 3 < ntiles ? j + 3 : -1);
        if (j + 3 < ntiles) wait_vmem<kDmaPerWave>();   // tile j+2 landed; tile j+3 may still fly
        else wait_vmem<0>();
        __syncthreads();
      }
    }
  } else {
    // ============================================================ PV waves
    const int col = lane & 31;   // 32x32 MFMA column: head col of the head half
    const int kh = lane >> 5;    // 32x32 MFMA k half
    float m_run = -INFINITY;     // reference of head col, log2 units
    float l_run = 0.f;           // sum over this lane's keys (16 of every tile)
    float16_t oacc[8];           // O^T: value tile u of this half; lane holds head col
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      oacc[u] = (float16_t){};
      asm volatile("" : "+a"(oacc[u]));
    }
    // V^T operand of value tile u and key block m, read rd: the lane (group
    // vg = (lane >> 4) & 1, index vj = lane & 15) points at row 16m + 8kh + 4rd + vj/4,
    // columns 256kd + 32u + 16vg + 4(vj & 3) .. +3; the transposed read returns
    // column 256kd + 32u + 16vg + vj (operand row col) of keys 16m + 8kh + 4rd .. +3
    // (operand slots 4rd .. 4rd+3). Address: ((vb0[rd] ^ 64(u & 3)) + 16384m + 256(u >> 2))
    const int vj = lane & 15, vg = (lane >> 4) & 1;
    uint32_t vb0[2];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int r = 8 * kh + 4 * rd + (vj >> 2);
      vb0[rd] = r * 1024 + 512 * kd + 16 * ((2 * vg + ((vj & 3) >> 1)) ^ swz_ws(r)) + 8 * (vj & 1);
    }
    auto vread = [&](uint32_t st, int u, int m) {
      const uint32_t off = 16384u * m + 256u * (u >> 2);
      const short4_t lo = lds_tr16_at(((st + vb0[0]) ^ (64u * (u & 3))) + off);
      const short4_t hi = lds_tr16_at(((st + vb0[1]) ^ (64u * (u & 3))) + off);
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // Tile t: online softmax of this lane's 16 scores (head col; slot 8m + e
    // holds key 16m + 8kh + e) into the P^T operands, then PV.
    auto pv_tile = [&](int t) {
      constexpr int kP = 16;   // PV MFMAs: key block s >> 3, value tile s & 7
      constexpr int kVA = 6;   // V^T operands read ahead (12 LDS operations)
      const uint32_t st = stage_of(t);
      const uint32_t sb = scores_of(t);
      float4_t sc[4];   // group 4(q >> 1) + 2kh + (q & 1): keys 16(q >> 1) + 8kh + 4(q & 1) .. +3
#pragma unroll
      for (int q = 0; q < 4; ++q) sc[q] = lds_f4_at(sb + score_off(col, 4 * (q >> 1) + 2 * kh + (q & 1)));
      bf16x8_t vr[kVA + 1];
#pragma unroll
      for (int s = 0; s < kVA; ++s) vr[s] = vread(st, s & 7, s >> 3);
      float sv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[4 * q + i] = sc[q][i];
      const bool partial = (t + 1) * kTileKeys > nvalid;   // uniform
      auto key_ok = [&](int k) { return t * kTileKeys + 16 * (k >> 3) + 8 * kh + (k & 7) < nvalid; };
      if (partial) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if (!key_ok(k)) sv[k] = -INFINITY;
      }
      float mx = sv[0];
#pragma unroll
      for (int k = 1; k < 16; ++k) mx = fmaxf(mx, sv[k]);
      mx = max_halves(mx);   // all 32 keys of the tile, which holds at least one valid key
      mx = mx == -INFINITY ? -INFINITY : mx * a.scale_log2;   // the scale may be 0
      const float m_new = next_ref(m_run, mx);
      const float alpha = ref_factor(m_run, m_new);
      m_run = m_new;
      float p[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) p[k] = fast_exp2(__builtin_fmaf(sv[k], a.scale_log2, -m_run));
      if (partial) {   // a masked slot has weight 0, also when the scale is 0
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if (!key_ok(k)) p[k] = 0.f;
      }
      float ps = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) ps += p[k];
      l_run = l_run * alpha + ps;
      bf16x8_t pk[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        uint4 w;
        w.x = pack_bf16x2(p[8 * m + 0], p[8 * m + 1]);
        w.y = pack_bf16x2(p[8 * m + 2], p[8 * m + 3]);
        w.z = pack_bf16x2(p[8 * m + 4], p[8 * m + 5]);
        w.w = pack_bf16x2(p[8 * m + 6], p[8 * m + 7]);
        pk[m] = __builtin_bit_cast(bf16x8_t, w);
      }
      if (__ballot(alpha != 1.f)) {   // some reference moved: rescale O
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          float16_t x = oacc[u];
          asm volatile("" : "+v"(x));
          x *= alpha;
          asm volatile("" : "+a"(x));
          oacc[u] = x;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < kP; ++s) {
        if (s + kVA < kP) vr[(s + kVA) % (kVA + 1)] = vread(st, (s + kVA) & 7, (s + kVA) >> 3);
        oacc[s & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[s % (kVA + 1)], pk[s >> 3], oacc[s & 7], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) asm volatile("" : "+a"(oacc[u]));
    };

    if (ntiles > 0) {
      __syncthreads();   // tile 0 landed
      __syncthreads();   // scores of tile 0 written, tile 1 landed
      for (int j = 0; j + 1 < ntiles; ++j) {
        pv_tile(j);
        __syncthreads();
      }
      pv_tile(ntiles - 1);
    }

    // ---------------------------------------------------------------- 6. epilogue
    const float L = sum_halves(l_run);   // all keys of head col
    const float inv_l = L > 0.f ? 1.f / L : 0.f;
    const int head = hblock * 64 + hh * 32 + col;
    if (head < a.num_heads) {
      if (a.splits == 1) {
        uint16_t* op = a.out + token * a.o_st + (int64_t)head * a.o_sh + 256 * kd + 4 * kh;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float16_t x = oacc[u] * inv_l;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            uint2 w;
            w.x = pack_bf16x2(x[4 * q4], x[4 * q4 + 1]);
            w.y = pack_bf16x2(x[4 * q4 + 2], x[4 * q4 + 3]);
            *(uint2*)(op + 32 * u + 8 * q4) = w;   // O[head][256kd + 32u + 8q4 + 4kh .. +3]
          }
        }
        if (kd == 0 && kh == 0) a.lse[token * a.lse_st + head] = L > 0.f ? (m_run + __log2f(L)) * kLn2 : -INFINITY;
      } else {
        const int64_t prow = (token * a.splits + split) * a.num_heads + head;
        float* pp = a.part_o + prow * kDv + 256 * kd + 4 * kh;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float16_t x = oacc[u] * inv_l;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *(float4_t*)(pp + 32 * u + 8 * q4) = (float4_t){x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]};
        }
        if (kd == 0 && kh == 0) {
          a.part_ml[prow * 2] = m_run;
          a.part_ml[prow * 2 + 1] = L;
        }
      }
    }
  }
}

}  // namespace dsa
