// dkv pass of the split backward schedule (more than 16 heads).
//
// Above 16 heads the token-major kernel's dkv atomics (576 floats per token,
// key and 32-head block) bound the backward. The split schedule computes the
// two gradients in separate passes, each written by its owner: dq by the
// dq pass (bwd_dq_kernel.hpp: one workgroup owns a token's heads), and dkv
// by this kv-major pass (one workgroup owns 64 kv rows). Each pass
// recomputes P from the forward's LSE.
//
// One workgroup = 4 waves = (64 kv rows r0 .., chunk of 256 tokens). It
// collects the chunk's tokens whose occupancy masks name any of its rows and
// takes them in steps of one token and 32 heads (a head group; 64 heads take
// two steps per token). The waves pair up: wave (rh, ch) owns rows
// r0 + 32rh .. +31 for the whole chunk and head tile ch of each step:
//   * its K rows (all 576 columns) stay in registers as MFMA B operands;
//   * S^T = q K^T (16x16x32 MFMA, heads as M, the rows as N) and
//     dP^T = dO V^T of head tile ch, with q and dO of the step read from LDS
//     as A operands, each read feeding the two row tiles;
//   * P and s*dS in the accumulator layout: lane (g, n) holds row n and
//     heads 4g .. 4g+3 of its head tile. The pair swaps them through LDS, so
//     that each wave holds heads 4g .. 4g+3 and 16+4g .. 16+4g+3: the A
//     operand of a 16x16x32 MFMA over the 32 heads with its k-slots permuted
//     the same way;
//   * dkv[32 rows x half ch of the columns] += (s dS) q + P dO (the latter on
//     the first 512 columns), with q^T and dO^T read transposed from LDS
//     (ds_read_b64_tr_b16, rows 4g.. and 16+4g.. give the permuted k-slots).
// dkv stays in registers over the chunk and is added once per workgroup.
// Each step's q, dO, LSE and D are copied HBM -> LDS by the 4 waves
// (global_load_lds) during the previous step. Two barriers per step: the
// copies landed, and the P/dS swap.
//
// Masked rows (not named by the step's token) and padded heads (beyond
// num_heads: they alias the last head, with LSE = +inf) get P = 0 and dS = 0.
// Tokens whose index row repeats an entry have all-zero masks (the prepass):
// the token-major kernel handles them, dq and dkv.
//
// LDS per step buffer: q latent [32 heads][1024 B], q rope [32][128 B],
// dO [32][1024 B], then LSE and D [2][32] fp32: 69888 B, two buffers.
// Granule G (16 B) of latent/dO row h sits at G ^ bw_swz(h) (within its
// 256-byte group), rope granule G at G ^ bw_swz_r(h), so that the A-operand
// reads (16 rows at one granule) and the transposed reads (8 rows x 32 B
// per half-wave) are free of bank conflicts.
//
// Pages: the prime-rl pull request 4078 that adds a `cudnn_flashmla` DSA
// backend (a separate DSA backward kernel, timed per call); "[Feature] Add
// optional FlashMLA backend for DSA Sparse MLA" (xtuner PR 2083), Motivation
// (the forward's output and LSE feed the backward).
#pragma once

#include "bwd_kernel.hpp"

namespace dsa {

constexpr int kKwRows = 64;                          // kv rows per workgroup
constexpr int kKwChunk = 256;                        // tokens per workgroup (4 ballots of 64)
constexpr int kKwHeads = 32;                         // heads per step
constexpr int kKwQL = 0;                             // q latent rows
constexpr int kKwQR = kKwQL + kKwHeads * 1024;       // q rope rows
constexpr int kKwDO = kKwQR + kKwHeads * 128;        // dO rows
constexpr int kKwLD = kKwDO + kKwHeads * 1024;       // LSE [32] then D [32], fp32
constexpr int kKwBuf = kKwLD + 2 * kKwHeads * 4;     // one step buffer (69888 B)
static_assert(kKwBuf % 256 == 0, "buffers keep the 256-byte bank alignment");

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) const uint8_t kw_lds;
__device__ __forceinline__ bf16x8_t kw_b128(const kw_lds* p) {
  return *(__attribute__((address_space(3))) const bf16x8_t*)p;
}
__device__ __forceinline__ float4_t kw_f4(const kw_lds* p) {
  return *(__attribute__((address_space(3))) const float4_t*)p;
}
__device__ __forceinline__ short4_t kw_tr(const kw_lds* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)p);
}

// One wave-wide 4-byte-per-lane copy HBM -> LDS: lane L's dword lands at LDS
// byte lds_base + 4 * L (lds_base wave-uniform, in M0).
__device__ __forceinline__ void dma_4b(const void* src, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

// blockIdx.x = chunk * ceil(num_words / 2) + (64-row block)
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
sparse_mla_bwd_kvw_kernel(const BwdArgs a, const KvMajorArgs m) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_buf[2][kKwBuf];
  __shared__ int s_tok[kKwChunk];
  __shared__ uint64_t s_msk[kKwChunk];
  __shared__ int s_wcnt[4];
  __shared__ __attribute__((aligned(16))) uint8_t s_x[4][2048];   // the wave pairs' exchange area

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int nbp = (m.num_words + 1) / 2;
  const int bp = (int)(blockIdx.x % nbp);
  const int64_t t0 = (int64_t)(blockIdx.x / nbp) * kKwChunk;
  const int64_t r0 = (int64_t)bp * kKwRows;

  // ---- the chunk's tokens that name rows of the block, in token order
  {
    const int64_t t = t0 + 64 * wave + lane;
    uint64_t w = 0;
    if (t < a.num_tokens) {
      w = m.mask[(int64_t)(2 * bp) * a.num_tokens + t];
      if (2 * bp + 1 < m.num_words) w |= (uint64_t)m.mask[(int64_t)(2 * bp + 1) * a.num_tokens + t] << 32;
    }
    const uint64_t act = __ballot(w != 0u);
    if (lane == 0) s_wcnt[wave] = __builtin_popcountll(act);
    __syncthreads();
    int base = 0;
    for (int i = 0; i < wave; ++i) base += s_wcnt[i];
    if (w != 0u) {
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(act >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)act, 0u));
      s_tok[pos] = 64 * wave + lane;
      s_msk[pos] = w;
    }
  }
  const int np = s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
  if (np == 0) return;   // uniform over the workgroup
  __syncthreads();

  const int num_heads = a.num_heads;
  const int groups = (num_heads + kKwHeads - 1) / kKwHeads;
  const int nsteps = np * groups;
  const uint16_t* const q_ptr = a.q;
  const uint16_t* const do_ptr = a.dout;
  const float* const lse_ptr = a.lse;
  const float* const d_ptr = m.dbuf;
  const int64_t q_st = a.q_st, q_sh = a.q_sh, do_st = a.do_st, do_sh = a.do_sh, lse_st = a.lse_st;
  const int64_t d_st = m.d_st;
  const float scale = a.scale, scale_log2 = a.scale_log2;

  // Waves pair up: wave (rh, ch) = (w >> 1, w & 1) owns rows r0 + 32rh ..
  // +31 (two row tiles). It forms S^T and dP^T of its rows and head tile ch
  // over all columns, and dkv of its rows on half ch of the columns (latent
  // 256ch .. +255, rope 32ch .. +31). Each q / dO operand read feeds two
  // MFMAs (one per row tile).
  const int rh = wave >> 1, ch = wave & 1;

  // ---- K rows as B operands: kreg[rt][j], lane (g, n) holds row 32rh + 16rt + n,
  // columns 32j + 8g .. +7 (chunks j < 16 latent, 16 and 17 rope)
  bf16x8_t kreg[2][18];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int64_t row = r0 + 32 * rh + 16 * rt + n;
    const bool ok = row < a.num_kv;
    const uint16_t* src = a.kv + (ok ? row : 0) * a.kv_st + 8 * g;
#pragma unroll
    for (int j = 0; j < 18; ++j) {
      const bf16x8_t v = *(const bf16x8_t*)(src + 32 * j);
      kreg[rt][j] = ok ? v : (bf16x8_t){};
    }
  }

  // ---- copies of step s into buffer b: 17 one-KB copies per wave (q latent
  // rows wave + 4k, dO rows wave + 4k, q rope rows 8w .. 8w+7), and wave 0
  // copies LSE and D. A plan holds the step's scalar bases; copy(k) issues
  // copy k (k < 8: q row, k < 16: dO row, 16: rope rows, 17: LSE/D), so that
  // the copies can be spread over the MFMA stream. The latent and dO copies
  // take a scalar base per head row and a fixed lane offset (row h = wave +
  // 4k has the swizzle of h & 15 = wave + 4 (k & 3)); padded heads copy the
  // group's last head.
  uint32_t cp_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cp_off[j] = 16u * (uint32_t)(lane ^ bw_swz(wave + 4 * j));
  const int64_t q_sh2 = 2 * q_sh, do_sh2 = 2 * do_sh;   // bytes
  struct CopyPlan {
    uint64_t qb, db;       // byte addresses of the step's token, head h0
    const uint16_t* qt;    // the token's q row
    int64_t tok;
    int h0, hmax;
    uint32_t bb;           // LDS byte address of the target buffer
  };
  auto plan = [&](int s, int b) {
    CopyPlan c;
    const int p = s / groups, hg = s - p * groups;
    c.tok = t0 + __builtin_amdgcn_readfirstlane(s_tok[p]);
    c.h0 = kKwHeads * hg;
    c.hmax = min(kKwHeads - 1, num_heads - 1 - c.h0);
    c.bb = lds_offset(&s_buf[b][0]);
    c.qt = q_ptr + c.tok * q_st;
    c.qb = (uint64_t)(c.qt + (int64_t)c.h0 * q_sh);
    c.db = (uint64_t)(do_ptr + c.tok * do_st + (int64_t)c.h0 * do_sh);
    return c;
  };
  auto copy = [&](const CopyPlan& c, int k) {
    if (k < 16) {
      const int h = wave + 4 * (k & 7), hr = min(h, c.hmax);
      if (k < 8) dma_16b_sbase(c.qb + (uint64_t)(hr * q_sh2), cp_off[k & 3], c.bb + kKwQL + h * 1024);
      else dma_16b_sbase(c.db + (uint64_t)(hr * do_sh2), cp_off[k & 3], c.bb + kKwDO + h * 1024);
    } else if (k == 16) {
      const int h = 8 * wave + (lane >> 3);
      const int hq = c.h0 + min(h, c.hmax);
      dma_16b(c.qt + hq * q_sh + kDv + 8 * ((lane & 7) ^ bw_swz_r(h)), c.bb + kKwQR + 8 * wave * 128);
    } else if (wave == 0) {
      const int hq = c.h0 + min(lane & 31, c.hmax);
      dma_4b(lane < 32 ? lse_ptr + c.tok * lse_st + hq : d_ptr + c.tok * d_st + hq, c.bb + kKwLD);
    }
  };

  // dkv of the wave's rows and columns: acc[rt][k], lane (g, n) holds column
  // tile k's column n of rows 32rh + 16rt + 4g + e (tiles k < 16: latent
  // columns 256ch + 16k ..; k = 16, 17: rope columns 32ch + 16(k - 16) ..)
  float4_t acc[2][18];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int k = 0; k < 18; ++k) acc[rt][k] = (float4_t){0.f, 0.f, 0.f, 0.f};

  // Per-lane LDS offsets within a step buffer. A-operand reads of row
  // 16ch + n: latent chunk j at 256 (j >> 2) + a_lat[j & 3] (the XOR only
  // touches a granule index's low 4 bits), rope chunk i at a_rope[i].
  // Transposed reads of rows hr = 4g + n/4 and 16 + hr, latent column tile
  // 16ch + k: 256 ((16ch + k) >> 3) + t_lat[k & 7]; rope tiles: t_rope[i].
  uint32_t a_lat[4], a_rope[2], t_lat[8], t_rope[2];
  {
    const int hr = 4 * g + (n >> 2), hb = (n >> 1) & 1;
    const int ar = 16 * ch + n;
#pragma unroll
    for (int c = 0; c < 4; ++c) a_lat[c] = (uint32_t)(ar * 1024 + 16 * ((4 * c + g) ^ bw_swz(ar)));
#pragma unroll
    for (int i = 0; i < 2; ++i) a_rope[i] = (uint32_t)(kKwQR + ar * 128 + 16 * ((4 * i + g) ^ bw_swz_r(ar)));
#pragma unroll
    for (int k = 0; k < 8; ++k)
      t_lat[k] = (uint32_t)(hr * 1024 + 16 * ((2 * k + hb) ^ bw_swz(hr)) + 8 * (n & 1));
#pragma unroll
    for (int i = 0; i < 2; ++i)
      t_rope[i] = (uint32_t)(kKwQR + hr * 128 + 16 * ((2 * (2 * ch + i) + hb) ^ bw_swz_r(hr)) + 8 * (n & 1));
  }
  // exchange area of the pair: region X[w] is wave w's 2 KB
  const kw_lds* const xr_own = (const kw_lds*)&s_x[wave][0];
  // The compiler does not see the asm copies' waits: make the K loads
  // complete here, with a wait it sees, so that it puts none in the loop
  // (there it would wait for the copies of the next step as well).
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  {
    const CopyPlan c0 = plan(0, 0);
#pragma unroll
    for (int k = 0; k < 18; ++k) copy(c0, k);
  }
  for (int s = 0; s < nsteps; ++s) {
    wait_vmem<0>();
    __syncthreads();
    // the next step's copies go into the other buffer (free: its last reads
    // were in the previous step, before this barrier); the last step copies
    // its own token again (valid data nobody reads), so the copy stream has
    // no branch, and the kernel drains it before it ends
    const CopyPlan cn = plan(s + 1 < nsteps ? s + 1 : s, (s + 1) & 1);
    // LDS pointers of this step's buffer: the constant parts of each read's
    // address then fold into the instruction's offset field
    const kw_lds* const buf = (const kw_lds*)&s_buf[s & 1][0];
    const kw_lds* pa[4];
    const kw_lds* pt[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) pa[c] = buf + a_lat[c];
#pragma unroll
    for (int k = 0; k < 8; ++k) pt[k] = buf + t_lat[k];
    const kw_lds* const prope[2] = {buf + a_rope[0], buf + a_rope[1]};
    const int p = s / groups, hg = s - p * groups;
    const int h0 = kKwHeads * hg;
    const uint64_t msk = s_msk[p];
    const float4_t l4[2] = {kw_f4(buf + kKwLD + 16 * g), kw_f4(buf + kKwLD + 64 + 16 * g)};
    const float4_t d4[2] = {kw_f4(buf + kKwLD + 128 + 16 * g), kw_f4(buf + kKwLD + 192 + 16 * g)};

    // ---- S^T and dP^T of head tile ch over all columns: [row tile rt].
    // 34 A-operand reads (q: chunks j = 0..17, dO: j = 0..15), each feeding
    // two MFMAs, kRingA reads ahead; the order is pinned (the scheduler would
    // sink each read next to its products). Read i < 32: chunk i / 2, q
    // (i even) or dO (odd); i = 32, 33: the rope chunks of q.
    constexpr int kReadsA = 34, kRingA = 12;
    auto a_read = [&](int i) -> bf16x8_t {
      if (i < 32) {
        const int j = i >> 1, isdo = i & 1;
        return kw_b128(pa[j & 3] + (isdo ? kKwDO : kKwQL) + 256 * (j >> 2));
      }
      return kw_b128(prope[i - 32]);
    };
    float4_t sc[2], dc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) sc[rt] = dc[rt] = (float4_t){0.f, 0.f, 0.f, 0.f};
    bf16x8_t ra[kRingA];
#pragma unroll
    for (int i = 0; i < kRingA; ++i) ra[i] = a_read(i);
#pragma unroll
    for (int i = 0; i < kReadsA; ++i) {
      const bf16x8_t v = ra[i % kRingA];
      if (i + kRingA < kReadsA) ra[i % kRingA] = a_read(i + kRingA);
      if ((i & 1) == 0) copy(cn, i >> 1);
      if (i == 1) copy(cn, 17);
      const int j = i < 32 ? i >> 1 : i - 16;
      const bool isdo = i < 32 && (i & 1);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        if (isdo)
          dc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, kreg[rt][j], dc[rt], 0, 0, 0);
        else
          sc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, kreg[rt][j], sc[rt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- transposed operands of the dkv product, kRingT column tiles ahead
    // (tile k < 16: q^T and dO^T, 4 reads; rope tiles k = 16, 17: q^T, 2)
    constexpr int kRingT = 4;
    auto t_read = [&](int k, bf16x8_t& bq, bf16x8_t& bo) {
      if (k < 16) {
        const kw_lds* o = pt[k & 7] + 256 * ((16 * ch + k) >> 3);
        bq = join4(kw_tr(o + kKwQL), kw_tr(o + kKwQL + 16 * 1024));
        bo = join4(kw_tr(o + kKwDO), kw_tr(o + kKwDO + 16 * 1024));
      } else {
        const kw_lds* o = buf + t_rope[k - 16];
        bq = join4(kw_tr(o), kw_tr(o + 16 * 128));
        bo = bq;
      }
    };
    bf16x8_t rq[kRingT], ro[kRingT];
#pragma unroll
    for (int k = 0; k < kRingT; ++k) t_read(k, rq[k], ro[k]);

    // ---- P and s*dS of head tile ch: lane (g, n) has rows 32rh + 16rt + n,
    // heads h0 + 16ch + 4g + e; packed bf16 (4 per row tile, P then dS)
    uint32_t own[2][4];   // [rt][P lo, P hi, dS lo, dS hi]
    {
      const float4_t lc = ch ? l4[1] : l4[0], dd = ch ? d4[1] : d4[0];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const bool rowok = (msk >> (32 * rh + 16 * rt + n)) & 1u;
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = rowok && h0 + 16 * ch + 4 * g + e < num_heads;
          pv[e] = ok ? __builtin_amdgcn_exp2f(sc[rt][e] * scale_log2 - lc[e] * 1.4426950408889634f) : 0.f;
          dsv[e] = pv[e] * (dc[rt][e] - dd[e]) * scale;
        }
        own[rt][0] = pack_bf16x2(pv[0], pv[1]);
        own[rt][1] = pack_bf16x2(pv[2], pv[3]);
        own[rt][2] = pack_bf16x2(dsv[0], dsv[1]);
        own[rt][3] = pack_bf16x2(dsv[2], dsv[3]);
      }
    }
    // ... and exchanges them through the pair's region (read from the
    // wave's own, which the pair writes)
    {
      u32x4_t* xo = (u32x4_t*)&s_x[wave ^ 1][0];
      xo[0 * 64 + lane] = (u32x4_t){own[0][0], own[0][1], own[0][2], own[0][3]};
      xo[1 * 64 + lane] = (u32x4_t){own[1][0], own[1][1], own[1][2], own[1][3]};
    }

    __syncthreads();
    bf16x8_t a_p[2], a_ds[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const u32x4_t o = *(__attribute__((address_space(3))) const u32x4_t*)(xr_own + 16 * (rt * 64 + lane));
      // k-slots 8g .. 8g+3: heads 4g .. (head tile 0), 8g+4 .. 8g+7: 16 + 4g .. (tile 1)
      const u32x4_t lo = ch ? o : (u32x4_t){own[rt][0], own[rt][1], own[rt][2], own[rt][3]};
      const u32x4_t hi = ch ? (u32x4_t){own[rt][0], own[rt][1], own[rt][2], own[rt][3]} : o;
      a_p[rt] = __builtin_bit_cast(bf16x8_t, (u32x4_t){lo[0], lo[1], hi[0], hi[1]});
      a_ds[rt] = __builtin_bit_cast(bf16x8_t, (u32x4_t){lo[2], lo[3], hi[2], hi[3]});
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- dkv[2 row tiles x 16 columns] += (s dS) q + P dO over the 32 heads, per column tile
#pragma unroll
    for (int k = 0; k < 18; ++k) {
      const bf16x8_t bq = rq[k % kRingT], bo = ro[k % kRingT];
      if (k + kRingT < 18) t_read(k + kRingT, rq[k % kRingT], ro[k % kRingT]);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) acc[rt][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_ds[rt], bq, acc[rt][k], 0, 0, 0);
      if (k < 16) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) acc[rt][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_p[rt], bo, acc[rt][k], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  wait_vmem<0>();   // the last step's copies land before the workgroup's LDS is released

  // ---- the rows' dkv, once per workgroup (other chunks add to the same rows)
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int k = 0; k < 18; ++k) {
      const int col = k < 16 ? 256 * ch + 16 * k + n : kDv + 32 * ch + 16 * (k - 16) + n;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t r = r0 + 32 * rh + 16 * rt + 4 * g + e;
        if (r < a.num_kv) unsafeAtomicAdd(a.dkv + r * a.dkv_st + col, acc[rt][k][e]);
      }
    }
}

}  // namespace dsa
