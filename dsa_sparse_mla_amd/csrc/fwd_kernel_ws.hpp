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
//     Then the softmax numerators of those scores: each exponential is taken
//     once, by the wave that holds the score. They go to LDS as bf16 P.
//   PV waves (w = 4..7): value quarter pw = w & 3, all 64 heads.
//     O^T[128 columns x 64 heads] += V^T P^T: 16 32x32x16 MFMAs, each V^T
//     operand used for two head tiles (every V element is read from LDS
//     once), O^T in the accumulator file. The PV waves also issue the gather.
// The hardware places wave w on SIMD w % 4, so each SIMD runs one S wave and
// one PV wave. Per tile every SIMD has 36 x 16 + 16 x 32 = 1088 MFMA clocks.
//
// Reference maxima. P must use one reference per head across both key blocks
// and all PV waves, and it must be known before the scores that it scales:
// the S waves use the reference of the tiles before (lagged). A tile whose
// scaled score exceeds its head's reference by more than kWsSlack (log2
// units; always the case for the first tile) is settled in one extra step:
// the S waves agree on new references from the published block maxima,
// rewrite that tile's P, and publish the factors by which the PV waves
// rescale O. Between such steps P <= 2^kWsSlack, far from the bf16 and fp32
// ranges, and bf16 keeps its relative precision at any magnitude.
//
// Pipeline: in iteration j the S waves settle tile j and score tile j+1,
// while the PV waves accumulate tile j and gather tile j+3. One workgroup
// barrier per tile publishes P, the flags and the gathered rows.
//
// LDS: the 4-stage tile ring (kStages x 36 KB), two P buffers of 4 KB (tile
// parity), block maxima, flags, factors and row sums (157472 bytes in all).
// During the index stage the P buffers hold the compacted key list and the
// block maxima the chunk counts.
//
// Pages: "feat: add XTuner TileLang sparse MLA backend" (lmdeploy PR 4904),
// Performance > Isolated sparse MLA forward (64-head operation of the other
// kernel); "[Feature] Add optional FlashMLA backend for DSA Sparse MLA"
// (xtuner PR 2083), Runtime constraints.
#pragma once

#include <type_traits>

#include "fwd_kernel.hpp"

namespace dsa {

typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kWsWaves = 8;
constexpr int kPBytes = 64 * kTileKeys * 2;   // P of one tile: [64 heads][32 keys] bf16
static_assert(2 * kPBytes == kSegment * 4, "the two P buffers double as the key list");
constexpr float kWsSlack = 16.f;              // log2 units: P <= 65536 between reference moves

// Latent-row swizzle of this kernel's tiles: granule G of latent row r is
// stored at G ^ swz_ws(r). A bijection of r & 15 (16 consecutive rows read at
// one logical granule hit distinct banks), and the 4 rows x 4 granules of a
// half-wave transposed V read also hit distinct banks.
__host__ __device__ constexpr int swz_ws(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Key rows of the QK^T operand. Lane i of a 16x16x32 MFMA operand supplies
// row i & 15; the lane reading row i loads key 4 sigma(i >> 2) + (i & 3) of
// its 16-key block, so output row 4q + e holds key 4 sigma(q) + e. The
// permutation matters for LDS banks: a ds_read_b128 serves in one cycle the
// 16 lanes of a half-wave whose quad index (lane bits 2..4) has one parity,
// and with sigma = (2, 0, 1, 3) those lanes hit 16 distinct slots under
// swz_ws (with the identity they pair up: a 2-way conflict on every K read).
__host__ __device__ constexpr int key_sigma(int q) { return (0x3102 >> (4 * q)) & 15; }
__host__ __device__ constexpr int key_rho(int i) { return 4 * key_sigma(i >> 2) + (i & 3); }

// P buffer: the 16-byte group g (keys 8g .. 8g+7) of head h sits at group
// g ^ ((h >> 2) & 3) of the head's 64-byte row. 16 consecutive heads at one
// group then cover all 64 banks (PV operand reads), and so do the 8-byte
// writes of 16 heads x 2 half-groups (S waves).
__host__ __device__ constexpr int p_off(int h, int g) { return h * 64 + 16 * (g ^ ((h >> 2) & 3)); }

__device__ __forceinline__ short4_t lds_tr16_at(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(uintptr_t)addr);
}
__device__ __forceinline__ bf16x8_t lds_b128_at(uint32_t addr) {
  return *(__attribute__((address_space(3))) const bf16x8_t*)(uintptr_t)addr;
}
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void lds_write_b64_at(uint32_t addr, u32x2_t v) {
  *(__attribute__((address_space(3))) u32x2_t*)(uintptr_t)addr = v;
}

// Lane swaps of gfx950 (VALU, no LDS round trip): swap16 exchanges the odd
// 16-lane rows of a with the even rows of b, swap32 the high half of a with
// the low half of b. They read VGPRs that the previous VALU instruction may
// have just written, so s_nop guards both sides.
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
// sum over the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float sum_kgroups(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap16(a, b);
  x = __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  a = __builtin_bit_cast(uint32_t, x), b = a;
  swap32(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// New reference from the old one and a tile maximum (log2 units): it moves
// only beyond the slack.
__device__ __forceinline__ float next_ref(float m_run, float m_tile) {
  return m_tile > m_run + kWsSlack ? fmaxf(m_run, m_tile) : m_run;
}
__device__ __forceinline__ float ref_factor(float m_old, float m_new) {
  return m_new == m_old ? 1.f : fast_exp2(m_old - m_new);   // m_old = -inf gives 0
}

template <bool PAGED>
__global__ void __launch_bounds__(64 * kWsWaves)
sparse_mla_fwd_ws_kernel(const FwdArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[kStages * kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[2][kPBytes];    // tile parity
  __shared__ __attribute__((aligned(16))) float s_mx[2][2][64];       // [parity][key block][head]
  __shared__ __attribute__((aligned(16))) int s_flag[2][4];           // [parity][S wave]
  __shared__ float s_alpha[64];                                       // O factors of a settle step
  __shared__ float s_l[2][64];                                        // [key block][head] row sums

  uint32_t* s_goff = (uint32_t*)&s_p[0][0];   // index stage only (both P buffers)
  int* s_cnt = (int*)&s_mx[0][0][0];          // index stage only

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool is_s = wave < 4;     // role (uniform per wave)
  const int sw = wave & 3;        // index within the role

  const int64_t per_token = (int64_t)a.splits * a.head_blocks;
  const int64_t bid = blockIdx.x;
  const int64_t token = a.num_tokens - 1 - bid / per_token;   // longest rows first in causal prefill
  const int rem = (int)(bid % per_token);
  const int split = rem / a.head_blocks;
  const int hblock = rem % a.head_blocks;

  // S waves: head half hh, key block kd; lane = (hcol, kq) of the 16x16 MFMAs
  const int hh = sw & 1, kd = sw >> 1;
  const int hcol = lane & 15, kq = lane >> 4;
  // Q^T (S waves), head tile ht: dims 32c + 8kq .. +7 of head 32hh + 16ht + hcol.
  // Its loads are issued with the index loads so that the two latencies overlap.
  bf16x8_t qreg[2][kDqk / 32];
  auto load_q = [&] {
    if (!is_s) return;
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
  };

  // ---------------------------------------------------------------- 1. index stage
  const int nvalid = build_key_list<PAGED, kWsWaves>(a, token, split, wave, lane, s_goff, s_cnt, load_q);
  const int ntiles = (nvalid + kTileKeys - 1) / kTileKeys;

  // PV waves keep the offsets of rows 8sw .. 8sw+7 of every tile in registers:
  // row r of tile t in lane 8(t & 7) + r of klist[t >> 3].
  constexpr int kListRegs = kSegment / kTileKeys / 8;
  uint32_t klist[kListRegs];
#pragma unroll
  for (int k = 0; k < kListRegs; ++k) {
    const int n = 64 * k + lane, t = n >> 3, r = n & 7;
    klist[k] = !is_s && t < ntiles ? s_goff[t * kTileKeys + 8 * sw + r] : 0u;
  }
  __syncthreads();   // the P buffers and block maxima are free from here on
  const uint32_t stage_lds = lds_offset(s_stage);
  const uint32_t p_lds = lds_offset(&s_p[0][0]);
  auto stage_of = [&](int t) { return stage_lds + (uint32_t)(t % kStages) * kStageBytes; };
  auto p_of = [&](int t) { return p_lds + (uint32_t)(t & 1) * kPBytes; };

  // Barrier sequence, every wave:
  //   prologue: tiles 0..2 gathered, tile 0 landed | tile 0 scored, tile 1 landed
  //   tile j: [settle step, if a flag of tile j is set] | tile j+1 scored, tile j+2 landed (j + 1 < ntiles)
  //   epilogue: row sums published
  if (is_s) {
    // ============================================================ S waves
    // Q^T chunks 0..14 in the accumulator file (the MFMA reads them from
    // there), which with the QK^T accumulator (8) fills this wave's 128.
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int c = 0; c < kDqk / 32; ++c) {
        if (c < 15) asm volatile("" : "+a"(qreg[ht][c]));
        else asm volatile("" : "+v"(qreg[ht][c]));
      }
    // K operand, latent chunk c: row 16kd + key_rho(hcol), logical granule 4c + kq:
    //   (kb0 ^ 64(c & 3)) + 256(c >> 2);  rope chunk 16 + cr: rb0 ^ 64cr
    const int kr_row = 16 * kd + key_rho(hcol);
    const int kq_key = 4 * key_sigma(kq);   // this lane's scores: keys 16kd + kq_key .. +3
    const int kpos = 16 * kd + kq_key;      // ... at positions kpos .. +3 of the tile
    const uint32_t kb0 = kr_row * 1024 + 16 * (kq ^ swz_ws(kr_row));
    const uint32_t rb0 = kRopeOff + kr_row * 128 + 16 * (kq ^ ((kr_row >> 1) & 7));
    auto kread = [&](uint32_t st, int c) {
      return c < 16 ? lds_b128_at(((st + kb0) ^ (64u * (c & 3))) + 256u * (c >> 2))
                    : lds_b128_at((st + rb0) ^ (64u * (c - 16)));
    };

    // per head tile ht (head 32hh + 16ht + hcol): reference, row sum of the
    // settled tiles, and the last scored tile's raw scores q.k (keys
    // 16kd + kq_key .. +3, masked = -inf) with their numerator sum
    float m_ref[2] = {-INFINITY, -INFINITY};
    // Scale used here: a zero scale becomes 1e-30, which leaves every weight
    // 2^(s * 1e-30 - m) equal to 1 in fp32 but keeps -inf * scale = -inf, so a
    // masked score (-inf) gives weight 0 without a separate mask.
    const float sc = fmaxf(a.scale_log2, 1e-30f);
    // A raw score q.k above thr flags its tile: in log2 units it exceeds the
    // reference by more than kWsSlack (with scale 0 every score is 0).
    auto raw_threshold = [&](float m) {
      const float t = m + kWsSlack;
      return t / sc;
    };
    float thr[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};
    float sv[2][4];
    float psum[2] = {0.f, 0.f};
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[ht][i] = -INFINITY;

    // numerators of the scored tile t under the current references -> P buffer
    auto make_p = [&](int t) {
      const uint32_t pb = p_of(t);
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = fast_exp2(__builtin_fmaf(sv[ht][i], sc, -m_ref[ht]));   // masked: 0
        psum[ht] = (p[0] + p[1]) + (p[2] + p[3]);
        const u32x2_t w = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
        lds_write_b64_at(pb + p_off(32 * hh + 16 * ht + hcol, (16 * kd + kq_key) >> 3) + 2 * (kq_key & 7), w);
      }
    };
    // settle tile t (its P written, flags published at the last barrier)
    auto settle = [&](int t, int4 fl) {
      if ((fl.x | fl.y | fl.z | fl.w) != 0) {   // same in every wave of the workgroup
        const int b = t & 1;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          const int h = 32 * hh + 16 * ht + hcol;
          const float mn = next_ref(m_ref[ht], fmaxf(s_mx[b][0][h], s_mx[b][1][h]));
          const float al = ref_factor(m_ref[ht], mn);
          m_ref[ht] = mn;
          thr[ht] = raw_threshold(mn);
          l_run[ht] *= al;
          if (kd == 0 && kq == 0) s_alpha[h] = al;
        }
        make_p(t);
        __syncthreads();   // new P and O factors visible
      }
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) l_run[ht] += psum[ht];
    };
    // QK^T of tile ts, then its scaled scores, block maxima, flag and P;
    // tile tsettle (if any) is settled once the first K operands are in flight
    auto s_step = [&](int ts, int tsettle) {
      constexpr int kS = 36;    // chunk t >> 1, head tile t & 1
      constexpr int kKA = 10;   // K chunks read ahead (about 320 MFMA clocks)
      const uint32_t st = stage_of(ts);
      int4 fl = {0, 0, 0, 0};
      if (tsettle >= 0) fl = *(const int4*)&s_flag[tsettle & 1][0];
      __builtin_amdgcn_sched_barrier(0);
      bf16x8_t kr[kKA + 1];
#pragma unroll
      for (int c = 0; c < kKA; ++c) kr[c] = kread(st, c);
      __builtin_amdgcn_sched_barrier(0);
      if (tsettle >= 0) settle(tsettle, fl);
      float4_t sacc[2];
#pragma unroll
      for (int t = 0; t < kS; ++t) {
        const int c = t >> 1;
        if ((t & 1) == 0 && c + kKA < kS / 2) kr[(c + kKA) % (kKA + 1)] = kread(st, c + kKA);
        sacc[t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[c % (kKA + 1)], qreg[t & 1][c],
                                                              c == 0 ? (float4_t){0.f, 0.f, 0.f, 0.f} : sacc[t & 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // raw scores, masked = -inf (the scale >= 0 is applied to maxima and
      // inside the exponent only)
      const int lim = nvalid - ts * kTileKeys;   // keys of this tile in the list (>= 32 unless it is the last)
      auto scaled = [&](float x) { return x * sc; };
      bool exceed = false;
      float ml[2];
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[ht][i] = kpos + i >= lim ? -INFINITY : sacc[ht][i];
        ml[ht] = fmaxf(fmaxf(sv[ht][0], sv[ht][1]), fmaxf(sv[ht][2], sv[ht][3]));
        exceed = exceed || ml[ht] > thr[ht];
      }
      // block maxima of both head tiles in two lane swaps: after them rows
      // 0 and 2 (kq even) hold head tile 0's maximum, rows 1 and 3 tile 1's
      {
        uint32_t x0 = __builtin_bit_cast(uint32_t, ml[0]), x1 = __builtin_bit_cast(uint32_t, ml[1]);
        swap16(x0, x1);   // x0: rows (t0 r0, t1 r0, t0 r2, t1 r2), x1: (t0 r1, t1 r1, t0 r3, t1 r3)
        uint32_t y0 = __builtin_bit_cast(uint32_t, fmaxf(__builtin_bit_cast(float, x0), __builtin_bit_cast(float, x1)));
        uint32_t y1 = y0;
        swap32(y0, y1);   // y0: low half twice, y1: high half twice
        const float mx = fmaxf(__builtin_bit_cast(float, y0), __builtin_bit_cast(float, y1));
        s_mx[ts & 1][kd][32 * hh + 16 * (kq & 1) + hcol] = scaled(mx);   // rows 2, 3 repeat rows 0, 1
      }
      const bool any = __ballot(exceed) != 0;
      if (lane == 0) s_flag[ts & 1][sw] = any ? 1 : 0;
      make_p(ts);
    };

    if (ntiles > 0) {
      __syncthreads();   // tile 0 landed
      s_step(0, -1);
      __syncthreads();   // tile 0 scored, tile 1 landed
      for (int j = 0; j + 1 < ntiles; ++j) {
        s_step(j + 1, j);
        __syncthreads();
      }
      settle(ntiles - 1, *(const int4*)&s_flag[(ntiles - 1) & 1][0]);
    }

    // ---------------------------------------------------------------- 6. epilogue (LSE)
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const float lw = sum_kgroups(l_run[ht]);   // this key block's keys of the head
      if (kq == 0) s_l[kd][32 * hh + 16 * ht + hcol] = lw;
    }
    __syncthreads();   // row sums published
    if (kd == 0 && kq == 0) {
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const int h = 32 * hh + 16 * ht + hcol;
        const int head = hblock * 64 + h;
        if (head < a.num_heads) {
          const float L = s_l[0][h] + s_l[1][h];
          if (a.splits == 1) {
            a.lse[token * a.lse_st + head] = L > 0.f ? (m_ref[ht] + __log2f(L)) * kLn2 : -INFINITY;
          } else {
            const int64_t prow = (token * a.splits + split) * a.num_heads + head;
            a.part_ml[prow * 2] = m_ref[ht];
            a.part_ml[prow * 2 + 1] = L;
          }
        }
      }
    }
  } else {
    // ============================================================ PV waves
    const int pw = sw;           // value columns 128pw .. 128pw+127
    const int col = lane & 31;   // 32x32 MFMA column: head 32ht2 + col
    const int kh = lane >> 5;    // 32x32 MFMA k half
    float16_t oacc[2][4];        // O^T: [head tile ht2][value tile u]
#pragma unroll
    for (int ht2 = 0; ht2 < 2; ++ht2)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        oacc[ht2][u] = (float16_t){};
        asm volatile("" : "+a"(oacc[ht2][u]));
      }
    // V^T operand of value tile u and key block m, read rd: the lane (group
    // vg = (lane >> 4) & 1, index vj = lane & 15) points at row 16m + 8kh + 4rd + vj/4,
    // columns 128pw + 32u + 16vg + 4(vj & 3) .. +3; the transposed read returns
    // column 128pw + 32u + 16vg + vj (operand row col) of keys 16m + 8kh + 4rd .. +3
    // (operand slots 4rd .. 4rd+3). Address: (vb0[rd] ^ 64u) + 16384m
    const int vj = lane & 15, vg = (lane >> 4) & 1;
    uint32_t vb0[2];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int r = 8 * kh + 4 * rd + (vj >> 2);
      vb0[rd] = r * 1024 + 256 * pw + 16 * ((2 * vg + ((vj & 3) >> 1)) ^ swz_ws(r)) + 8 * (vj & 1);
    }
    auto vread = [&](uint32_t st, int u, int m) {
      const uint32_t off = 16384u * m;
      const short4_t lo = lds_tr16_at(((st + vb0[0]) ^ (64u * u)) + off);
      const short4_t hi = lds_tr16_at(((st + vb0[1]) ^ (64u * u)) + off);
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
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
    // copy d of this wave's share of tile t: latent row 8pw + d (d < 8), or
    // rope rows 8pw .. 8pw+7 (lane i: rope granule (i & 7) ^ ((row >> 1) & 7) of row 8pw + i/8)
    auto gather_copy = [&](uint32_t base, const uint32_t* go, int d) {   // base: the stage, in SGPRs
      if (d < 8) {
        const int row = 8 * pw + d;
        dma_16b_sbase((uint64_t)a.kv + (uint64_t)go[d] * 16ull, lane16 ^ (uint32_t)(swz_ws(row) * 16),
                      base + row * 1024);
      } else {
        const int rrow = 8 * pw + (lane >> 3);
        const int g = (lane & 7) ^ ((rrow >> 1) & 7);
        dma_16b(a.kv + ((uint64_t)grope + 64u + (uint32_t)g) * 16ull, base + kRopeOff + pw * 1024);
      }
    };
    auto issue = [&](int t) {   // all of this wave's copies of tile t (prologue)
      uint32_t go[8];
      gather_rows(t, go, true);
      const uint32_t base = __builtin_amdgcn_readfirstlane(stage_of(t));
#pragma unroll
      for (int d = 0; d < kDmaPerWave; ++d) gather_copy(base, go, d);
    };
    // P^T operand of head tile ht2 and key block m: head 32ht2 + col, keys 16m + 8kh .. +7
    auto read_p = [&](uint32_t pb, bf16x8_t (*pk)[2]) {
#pragma unroll
      for (int ht2 = 0; ht2 < 2; ++ht2)
#pragma unroll
        for (int m = 0; m < 2; ++m) pk[ht2][m] = lds_b128_at(pb + p_off(32 * ht2 + col, 2 * m + kh));
    };
    // PV of tile t, with the gather of tile tg spread over it if G (one copy
    // of the body per case, so the MFMA stream carries no branches)
    auto pv_tile = [&](auto gather, int t, int tg) {
      constexpr bool G = decltype(gather)::value;
      constexpr int kO = 8;    // V^T operands: key block o >> 2, value tile o & 3
      constexpr int kVA = 4;   // operands read ahead (8 LDS operations)
      const uint32_t st = stage_of(t);
      const uint32_t pb = p_of(t);
      // The first kEarly copies of the next gather go out before this wave's
      // P and V^T reads: the LDS serves requests in arrival order, and the S
      // waves' K reads at the same barrier are on the tile's critical path
      // while these reads are not (the PV MFMAs fill the S waves' softmax tail).
      constexpr int kEarly = 4;
      const int4 fl = *(const int4*)&s_flag[t & 1][0];
      uint32_t go[8];
      uint32_t gbase = 0;
      if (G) {
        gather_rows(tg, go, true);
        gbase = __builtin_amdgcn_readfirstlane(stage_of(tg));
#pragma unroll
        for (int d = 0; d < kEarly; ++d) gather_copy(gbase, go, d);
      }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8_t pk[2][2];
      read_p(pb, pk);
      bf16x8_t vr[kVA + 1];
#pragma unroll
      for (int o = 0; o < kVA; ++o) vr[o] = vread(st, o & 3, o >> 2);
      if ((fl.x | fl.y | fl.z | fl.w) != 0) {   // settle step: new P, O factors
        __syncthreads();
        float al[2];
#pragma unroll
        for (int ht2 = 0; ht2 < 2; ++ht2) al[ht2] = s_alpha[32 * ht2 + col];
        read_p(pb, pk);
        if (__ballot(al[0] != 1.f || al[1] != 1.f)) {
#pragma unroll
          for (int ht2 = 0; ht2 < 2; ++ht2)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              float16_t x = oacc[ht2][u];
              asm volatile("" : "+v"(x));
              x *= al[ht2];
              asm volatile("" : "+a"(x));
              oacc[ht2][u] = x;
            }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 2 * kO; ++s) {
        const int o = s >> 1, ht2 = s & 1;
        if (ht2 == 0 && o + kVA < kO) vr[(o + kVA) % (kVA + 1)] = vread(st, (o + kVA) & 3, (o + kVA) >> 2);
        oacc[ht2][o & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[o % (kVA + 1)], pk[ht2][o >> 2], oacc[ht2][o & 3], 0, 0, 0);
        if (G && s + kEarly < kDmaPerWave) gather_copy(gbase, go, s + kEarly);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int ht2 = 0; ht2 < 2; ++ht2)
#pragma unroll
        for (int u = 0; u < 4; ++u) asm volatile("" : "+a"(oacc[ht2][u]));
    };

    if (ntiles > 0) {
      issue(0);
      if (ntiles > 1) issue(1);
      if (ntiles > 2) issue(2);
      if (ntiles > 2) wait_vmem<2 * kDmaPerWave>();
      else if (ntiles > 1) wait_vmem<kDmaPerWave>();
      else wait_vmem<0>();
      __syncthreads();   // tile 0 landed
      if (ntiles > 2) wait_vmem<kDmaPerWave>();
      else wait_vmem<0>();
      __syncthreads();   // tile 0 scored, tile 1 landed
      // the gather of tile j+3 goes into the stage of tile j-1, which every
      // wave left at the last barrier
      int j = 0;
      for (; j + 3 < ntiles; ++j) {
        pv_tile(std::true_type{}, j, j + 3);
        wait_vmem<kDmaPerWave>();   // tile j+2 landed; tile j+3 may still fly
        __syncthreads();
      }
      for (; j + 1 < ntiles; ++j) {
        pv_tile(std::false_type{}, j, -1);
        wait_vmem<0>();
        __syncthreads();
      }
      pv_tile(std::false_type{}, ntiles - 1, -1);
    }

    // ---------------------------------------------------------------- 6. epilogue (O)
    // Normalised O goes to LDS (the tile ring is idle now) as [head][column]
    // rows, so that the global stores below write whole rows. bf16: 1 KB per
    // head, 16-byte granule G at G ^ (head & 15); fp32 partials: 2 KB per head.
    __syncthreads();   // row sums published; every stage read and copy done
#pragma unroll
    for (int ht2 = 0; ht2 < 2; ++ht2) {
      const int h = 32 * ht2 + col;
      const float L = s_l[0][h] + s_l[1][h];
      const float inv_l = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float16_t x = oacc[ht2][u] * inv_l;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int c0 = 128 * pw + 32 * u + 8 * q4 + 4 * kh;   // columns c0 .. c0+3
          if (a.splits == 1) {
            const u32x2_t w = {pack_bf16x2(x[4 * q4], x[4 * q4 + 1]), pack_bf16x2(x[4 * q4 + 2], x[4 * q4 + 3])};
            lds_write_b64_at(stage_lds + h * 1024 + 16 * ((c0 >> 3) ^ (h & 15)) + 2 * (c0 & 7), w);
          } else {
            *(__attribute__((address_space(3))) float4_t*)(uintptr_t)(stage_lds + h * 2048 + 16 * ((c0 >> 2) ^ (h & 15))) =
                (float4_t){x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]};
          }
        }
      }
    }
  }

  // ---------------------------------------------------------------- 7. O stores (all waves)
  __syncthreads();   // O staged
  const int tid = threadIdx.x;
  if (a.splits == 1) {
#pragma unroll
    for (int k = 0; k < 64 * 64 / (64 * kWsWaves); ++k) {
      const int flat = k * 64 * kWsWaves + tid, h = flat >> 6, g = flat & 63;   // one head row per wave
      const int head = hblock * 64 + h;
      const bf16x8_t v = lds_b128_at(lds_offset(s_stage) + h * 1024 + 16 * (g ^ (h & 15)));
      if (head < a.num_heads) *(bf16x8_t*)(a.out + token * a.o_st + (int64_t)head * a.o_sh + 8 * g) = v;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 64 * 128 / (64 * kWsWaves); ++k) {
      const int flat = k * 64 * kWsWaves + tid, h = flat >> 7, g = flat & 127;
      const int head = hblock * 64 + h;
      const float4_t v = *(__attribute__((address_space(3))) const float4_t*)(uintptr_t)(lds_offset(s_stage) + h * 2048 + 16 * (g ^ (h & 15)));
      if (head < a.num_heads) {
        const int64_t prow = (token * a.splits + split) * a.num_heads + head;
        *(float4_t*)(a.part_o + prow * kDv + 4 * g) = v;
      }
    }
  }
}

}  // namespace dsa
