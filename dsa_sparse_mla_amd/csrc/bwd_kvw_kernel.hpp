// dkv pass of the split backward schedule (more than 16 heads).
//
// Above 16 heads the token-major kernel's dkv atomics (576 floats per token,
// key and 32-head block) bound the backward. The split schedule computes the
// two gradients in separate passes, each written by its owner: dq by the
// token-major kernel with its dkv phase compiled out (one workgroup owns a
// token's heads), and dkv by this kv-major pass (one workgroup owns 64 kv
// rows). Each pass recomputes P from the forward's LSE.
//
// One workgroup = 4 waves = (64 kv rows r0 .., chunk of 256 tokens). It
// collects the chunk's tokens whose occupancy masks name any of its rows and
// takes them in steps of one token and 32 heads (a head group; 64 heads take
// two steps per token). Wave w owns rows r0 + 16w .. +15 for the whole chunk:
//   * their K rows (all 576 columns) stay in registers as MFMA B operands;
//   * S^T = q K^T (16x16x32 MFMA, heads as M, the wave's rows as N) and
//     dP^T = dO V^T, with q and dO of the step read from LDS as A operands;
//   * P and s*dS in the accumulator layout: lane (g, n) holds row n and
//     heads 4g .. 4g+3, 16+4g .. 16+4g+3. That is exactly the A operand of a
//     16x16x32 MFMA over the 32 heads with its k-slots permuted the same way,
//     so P and dS never go through LDS;
//   * dkv[16 rows x 576] += (s dS) q + P dO (the latter on the first 512
//     columns), with q^T and dO^T read transposed from LDS
//     (ds_read_b64_tr_b16, rows 4g.. and 16+4g.. give the permuted k-slots).
// dkv stays in registers over the chunk and is added once per workgroup.
// Each step's q, dO, LSE and D are copied HBM -> LDS by the 4 waves
// (global_load_lds) during the previous step: one barrier per step, no
// other synchronisation.
//
// Masked rows (not named by the step's token) and padded heads (beyond
// num_heads: they alias the last head, with LSE = +inf) get P = 0 and dS = 0.
// Tokens whose index row repeats an entry have all-zero masks (the prepass):
// the token-major kernel handles them, dq and dkv.
//
// LDS per step buffer: q latent [32 heads][1024 B], q rope [32][128 B],
// dO [32][1024 B], then LSE and D [2][32] fp32: 69888 B, two buffers.
// Granule G (16 B) of latent/dO row h sits at G ^ kw_swz(h) (within its
// 256-byte group), rope granule G at G ^ kw_swz_r(h): the A-operand reads
// (16 rows at one granule) and the transposed reads (8 rows x 32 B) are then
// free of bank conflicts.
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

__host__ __device__ constexpr int kw_swz(int h) { return 2 * ((h & 7) ^ ((h >> 1) & 4)); }
__host__ __device__ constexpr int kw_swz_r(int h) { return 2 * (((h >> 1) & 3) ^ ((h >> 2) & 2)); }

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

  // ---- the wave's K rows as B operands: lane (g, n) holds row 16w + n, columns 32c + 8g .. +7
  bf16x8_t kreg[kDqk / 32];
  {
    const int64_t row = r0 + 16 * wave + n;
    const bool ok = row < a.num_kv;
    const uint16_t* src = a.kv + (ok ? row : 0) * a.kv_st + 8 * g;
#pragma unroll
    for (int c = 0; c < kDqk / 32; ++c) {
      const bf16x8_t v = *(const bf16x8_t*)(src + 32 * c);
      kreg[c] = ok ? v : (bf16x8_t){};
    }
  }

  // ---- copies of step s into buffer b: 17 one-KB copies per wave (q latent
  // rows wave + 4k, dO rows wave + 4k, q rope rows 8w .. 8w+7), and wave 0
  // copies LSE and D
  auto issue = [&](int s, int b) {
    const int p = s / groups, hg = s - p * groups;
    const int64_t tok = t0 + s_tok[p];
    const int h0 = kKwHeads * hg;
    const uint32_t bb = lds_offset(&s_buf[b][0]);
    const uint16_t* qt = q_ptr + tok * q_st;
    const uint16_t* dt = do_ptr + tok * do_st;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int h = wave + 4 * k;
      const int hq = min(h0 + h, num_heads - 1);
      dma_16b(qt + hq * q_sh + 8 * (lane ^ kw_swz(h)), bb + kKwQL + h * 1024);
      dma_16b(dt + hq * do_sh + 8 * (lane ^ kw_swz(h)), bb + kKwDO + h * 1024);
    }
    {
      const int h = 8 * wave + (lane >> 3);
      const int hq = min(h0 + h, num_heads - 1);
      dma_16b(qt + hq * q_sh + kDv + 8 * ((lane & 7) ^ kw_swz_r(h)), bb + kKwQR + 8 * wave * 128);
    }
    if (wave == 0) {
      const int hq = min(h0 + (lane & 31), num_heads - 1);
      dma_4b(lane < 32 ? lse_ptr + tok * lse_st + hq : d_ptr + tok * d_st + hq, bb + kKwLD);
    }
  };

  // dkv of the wave's rows: lane (g, n) holds column 16k + n of rows 16w + 4g + e
  float4_t acc[kDqk / 16];
#pragma unroll
  for (int k = 0; k < kDqk / 16; ++k) acc[k] = (float4_t){0.f, 0.f, 0.f, 0.f};

  // Per-lane LDS offsets (within a step buffer). A-operand reads of row
  // 16ht + n, latent granule 4c + g: 256 (c >> 2) + a_lat[c & 3] (the XOR
  // only touches the granule's low 4 bits); rope granule 4c' + g: a_rope[c'].
  // Transposed reads of rows hr = 4g + n/4 and 16 + hr, columns 16k + 4(n&3):
  // 256 (k >> 3) + t_lat[k & 7]; rope column tile k': t_rope[k'].
  uint32_t a_lat[4], a_rope[2], t_lat[8], t_rope[4];
  {
    const int hr = 4 * g + (n >> 2), hb = (n >> 1) & 1;
#pragma unroll
    for (int c = 0; c < 4; ++c) a_lat[c] = (uint32_t)(n * 1024 + 16 * ((4 * c + g) ^ kw_swz(n)));
#pragma unroll
    for (int c = 0; c < 2; ++c) a_rope[c] = (uint32_t)(kKwQR + n * 128 + 16 * ((4 * c + g) ^ kw_swz_r(n)));
#pragma unroll
    for (int k = 0; k < 8; ++k)
      t_lat[k] = (uint32_t)(hr * 1024 + 16 * ((2 * k + hb) ^ kw_swz(hr)) + 8 * (n & 1));
#pragma unroll
    for (int k = 0; k < 4; ++k)
      t_rope[k] = (uint32_t)(kKwQR + hr * 128 + 16 * ((2 * k + hb) ^ kw_swz_r(hr)) + 8 * (n & 1));
  }
  // The compiler does not see the asm copies' waits: make the K loads
  // complete here, with a wait it sees, so that it puts none in the loop
  // (there it would wait for the copies of the next step as well).
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  issue(0, 0);
  for (int s = 0; s < nsteps; ++s) {
    wait_vmem<0>();
    __syncthreads();
    if (s + 1 < nsteps) issue(s + 1, (s + 1) & 1);
    // LDS pointers of this step's buffer: the constant parts of each read's
    // address then fold into the instruction's offset field
    const kw_lds* const buf = (const kw_lds*)&s_buf[s & 1][0];
    const kw_lds* pa[4];
    const kw_lds* pr[2];
    const kw_lds* pt[8];
    const kw_lds* ptr_[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) pa[c] = buf + a_lat[c];
#pragma unroll
    for (int c = 0; c < 2; ++c) pr[c] = buf + a_rope[c];
#pragma unroll
    for (int k = 0; k < 8; ++k) pt[k] = buf + t_lat[k];
#pragma unroll
    for (int k = 0; k < 4; ++k) ptr_[k] = buf + t_rope[k];
    const int p = s / groups, hg = s - p * groups;
    const int h0 = kKwHeads * hg;
    const uint64_t msk = s_msk[p];
    const float4_t l4[2] = {kw_f4(buf + kKwLD + 16 * g), kw_f4(buf + kKwLD + 64 + 16 * g)};
    const float4_t d4[2] = {kw_f4(buf + kKwLD + 128 + 16 * g), kw_f4(buf + kKwLD + 192 + 16 * g)};

    // ---- S^T (16 heads x 16 rows, per head tile) over 576 columns, dP^T
    // over 512: 68 A-operand reads, each feeding one MFMA, kRingA reads
    // ahead (the order is pinned: the scheduler would otherwise sink each
    // read next to its product). Read i < 64: chunk c = i / 4, head tile
    // i & 1, q (i & 2 == 0) or dO; i >= 64: rope chunk (i - 64) / 2.
    constexpr int kReadsA = 68, kRingA = 12;
    auto a_read = [&](int i) -> bf16x8_t {
      if (i < 64) {
        const int c = i >> 2, ht = i & 1, isdo = (i >> 1) & 1;
        return kw_b128(pa[c & 3] + (isdo ? kKwDO : kKwQL) + 16 * 1024 * ht + 256 * (c >> 2));
      }
      return kw_b128(pr[(i - 64) >> 1] + 16 * 128 * (i & 1));
    };
    float4_t sacc[2], dacc[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) sacc[ht] = dacc[ht] = (float4_t){0.f, 0.f, 0.f, 0.f};
    bf16x8_t ra[kRingA];
#pragma unroll
    for (int i = 0; i < kRingA; ++i) ra[i] = a_read(i);
#pragma unroll
    for (int i = 0; i < kReadsA; ++i) {
      const bf16x8_t v = ra[i % kRingA];
      if (i + kRingA < kReadsA) ra[i % kRingA] = a_read(i + kRingA);
      const int c = i < 64 ? i >> 2 : kDv / 32 + ((i - 64) >> 1);
      const int ht = i & 1;
      if (i < 64 && ((i >> 1) & 1))
        dacc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, kreg[c], dacc[ht], 0, 0, 0);
      else
        sacc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, kreg[c], sacc[ht], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- transposed operands of the dkv product, kRingT column tiles ahead
    // (q^T and dO^T of tile k: 4 reads; rope tiles: 2)
    constexpr int kRingT = 4;
    auto t_read = [&](int k, bf16x8_t& bq, bf16x8_t& bo) {
      if (k < kDv / 16) {
        const kw_lds* o = pt[k & 7] + 256 * (k >> 3);
        bq = join4(kw_tr(o + kKwQL), kw_tr(o + kKwQL + 16 * 1024));
        bo = join4(kw_tr(o + kKwDO), kw_tr(o + kKwDO + 16 * 1024));
      } else {
        const kw_lds* o = ptr_[k - kDv / 16];
        bq = join4(kw_tr(o), kw_tr(o + 16 * 128));
        bo = bq;
      }
    };
    bf16x8_t rq[kRingT], ro[kRingT];
#pragma unroll
    for (int k = 0; k < kRingT; ++k) t_read(k, rq[k], ro[k]);

    // ---- P and s*dS: lane (g, n) has row 16w + n, heads h0 + 16ht + 4g + e
    const bool rowok = (msk >> (16 * wave + n)) & 1u;
    float pv[2][4], dsv[2][4];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = rowok && h0 + 16 * ht + 4 * g + e < num_heads;
        pv[ht][e] = ok ? __builtin_amdgcn_exp2f(sacc[ht][e] * scale_log2 - l4[ht][e] * 1.4426950408889634f) : 0.f;
        dsv[ht][e] = pv[ht][e] * (dacc[ht][e] - d4[ht][e]) * scale;
      }
    const bf16x8_t a_ds = __builtin_bit_cast(
        bf16x8_t, (u32x4_t){pack_bf16x2(dsv[0][0], dsv[0][1]), pack_bf16x2(dsv[0][2], dsv[0][3]),
                            pack_bf16x2(dsv[1][0], dsv[1][1]), pack_bf16x2(dsv[1][2], dsv[1][3])});
    const bf16x8_t a_p = __builtin_bit_cast(
        bf16x8_t, (u32x4_t){pack_bf16x2(pv[0][0], pv[0][1]), pack_bf16x2(pv[0][2], pv[0][3]),
                            pack_bf16x2(pv[1][0], pv[1][1]), pack_bf16x2(pv[1][2], pv[1][3])});
    __builtin_amdgcn_sched_barrier(0);

    // ---- dkv[16 rows x 16 columns] += (s dS) q + P dO over the 32 heads, per
    // column tile; the two products of a tile are a tile apart
    bf16x8_t bo_prev = {};
#pragma unroll
    for (int k = 0; k < kDqk / 16; ++k) {
      const bf16x8_t bq = rq[k % kRingT], bo = ro[k % kRingT];
      if (k + kRingT < kDqk / 16) t_read(k + kRingT, rq[k % kRingT], ro[k % kRingT]);
      acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_ds, bq, acc[k], 0, 0, 0);
      if (k >= 1 && k - 1 < kDv / 16)
        acc[k - 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_p, bo_prev, acc[k - 1], 0, 0, 0);
      bo_prev = bo;
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- the rows' dkv, once per workgroup (other chunks add to the same rows)
#pragma unroll
  for (int k = 0; k < kDqk / 16; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t r = r0 + 16 * wave + 4 * g + e;
      if (r < a.num_kv) unsafeAtomicAdd(a.dkv + r * a.dkv_st + 16 * k + n, acc[k][e]);
    }
}

}  // namespace dsa
