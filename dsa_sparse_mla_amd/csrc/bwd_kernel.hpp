// Backward of the DSA sparse MLA forward for gfx950 (MI355X): gradients with
// respect to q and kv, given the upstream gradient dO, the forward output O
// and the forward LSE.
//
// With J the valid entries of token t's index row, K = kv[J] (|J| x 576),
// V = K[:, :512], s = sm_scale, and per head h:
//   P   = exp(s q.K^T - LSE)          (the forward's softmax, from its LSE)
//   dP  = dO V^T,   D = dO . O,   dS = P (dP - D)
//   dq        = s dS K
//   dkv[J]   += s dS^T q              (all 576 columns: the key use)
//   dkv[J,:512] += P^T dO             (the value use)
// Entries that name no row get nothing; duplicates count once per occurrence.
//
// Two schedules. The token-major kernel (below): one workgroup of 4 waves
// handles one token and a block of 16 heads (32 when the call has more than
// 16 heads: see the kernel's HT). The kv-major pass (further below) serves
// up to 16 heads when index rows name a large share of the kv rows. In the
// token-major kernel the index row is compacted per 2048-entry segment, as in
// the forward. Per tile of 32 keys:
//   phase 1: waves 0,1: S^T = K Q^T on key block 0 / 1 (16x16x32 MFMA, Q^T
//            in registers); waves 2,3: dP^T = V dO^T likewise (dO^T in
//            registers), handed to waves 0,1 through LDS;
//   phase 2: waves 0,1: P and s*dS in bf16 into LDS, [head][32 keys];
//   phase 3: every wave: dq column tiles 4k + w (k = 0..8) += (s dS) K,
//            with K^T read transposed from the tile (ds_read_b64_tr_b16;
//            the k slots of lane group g are keys 4g.., 16+4g..); and
//            dkv tiles [16 keys x 16 columns] = (s dS)^T Q + P^T dO on
//            16x16x16 MFMA over the 16 heads, added to the caller's fp32
//            dkv with atomics (other tokens name the same rows).
// The next tile's rows are loaded into registers while the current one is
// processed and stored to the other LDS stage at its end.
//
// Pages: "[Feature] Add optional FlashMLA backend for DSA Sparse MLA"
// (xtuner PR 2083), Motivation (forward output and LSE feed the backward);
// the prime-rl pull request 4078 that adds a `cudnn_flashmla` DSA backend
// (a separate DSA backward kernel, timed per call).
#pragma once

#include "fwd_kernel.hpp"

namespace dsa {

struct BwdArgs {
  const uint16_t* q;       // bf16 [T, H, 576]
  int64_t q_st, q_sh;
  const uint16_t* kv;      // bf16 [N, 576]
  int64_t kv_st;           // row stride in elements
  int64_t num_kv;
  const int32_t* idx;      // int32 [T, topk]
  int64_t idx_st;
  int64_t num_tokens;
  int32_t num_heads;
  int32_t topk;
  float scale;             // sm_scale
  float scale_log2;        // sm_scale * log2(e)
  const uint16_t* out;     // bf16 [T, H, 512], the forward output
  int64_t o_st, o_sh;
  const float* lse;        // fp32 [T, H], the forward LSE (natural log)
  int64_t lse_st;
  const uint16_t* dout;    // bf16 [T, H, 512]
  int64_t do_st, do_sh;
  float* dq;               // fp32 [T, H, 576]
  int64_t dq_st, dq_sh;
  float* dkv;              // fp32 [N, 576], zeroed before this kernel
  int64_t dkv_st;
  int32_t head_blocks;     // workgroups per token (16 heads each)
  const uint32_t* only;    // if set, tokens are filtered by only[t] (see only_nonzero)
  int32_t only_nonzero;    // 1: run the tokens with only[t] != 0; 0: those with only[t] == 0
};

constexpr int kBwPitch = 1168;                  // LDS row pitch of Q rows (and kv-major K rows): 1152 + 16
constexpr int kBwLat = kTileKeys * kDv * 2;     // stage of one tile: the 32 latent parts (1024 B each),
constexpr int kBwStage = kBwLat + kTileKeys * (kDqk - kDv) * 2;   // then the 32 rope parts (128 B each)

// Swizzles of the key stages (token-major kernel and dq pass): granule G (16 B)
// of the latent part of row r sits at G ^ bw_swz(r) within its 256-byte
// group, rope granule G at G ^ bw_swz_r(r). Chosen by measurement
// (SQ_LDS_BANK_CONFLICT on probes of both read patterns): the transposed
// reads (rows 4g + n/4 and 16 + 4g + n/4, 32 B per row and half-wave) need
// (swizzle >> 1) distinct over rows 0..7 and over 8..15; the A-operand
// reads (16 rows at one logical granule) are conflict-free with these and,
// e.g., with the identity, but not with every XOR that is a bijection on
// 16 rows.
__host__ __device__ constexpr int bw_swz(int r) { return (r & 6) | ((r & 1) << 3); }
__host__ __device__ constexpr int bw_swz_r(int r) { return r & 6; }
constexpr int kBwOPitch = 1040;                 // LDS row pitch of dO rows: 1024 + 16
constexpr int kBwGran = kTileKeys * (kDqk / 8) / 256;   // 16-byte granules per thread per tile (9)
static_assert(kTileKeys * (kDqk / 8) % 256 == 0, "a tile splits evenly over the threads");

__device__ __forceinline__ bf16x8_t lds16(const uint8_t* p) { return *(const bf16x8_t*)p; }
__device__ __forceinline__ bf16x8_t join4(short4_t lo, short4_t hi) {
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// HT head tiles of 16 per workgroup (1 or 2). With 2, each key's dkv row is
// added once per 32 heads instead of once per 16, and each tile is gathered
// once for 32 heads.
template <int HT>
__global__ void __launch_bounds__(256)
sparse_mla_bwd_kernel(const BwdArgs a) {
  constexpr int HB = 16 * HT;   // heads of the workgroup
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[2][kBwStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[HB * kBwPitch];
  __shared__ __attribute__((aligned(16))) uint8_t s_do[HB * kBwOPitch];
  __shared__ __attribute__((aligned(16))) float4_t s_dp[2][HT][64];   // dP^T of key block 0 / 1, head tile
  // P and s*dS, bf16 [head][32 keys], keys in the dq products' k-slot order:
  // bytes 16q .. 16q+7 hold keys 4q .. 4q+3, bytes 16q+8 .. 16q+15 keys 16+4q .. 16+4q+3
  __shared__ __attribute__((aligned(16))) uint8_t s_pt[HB * 64];
  __shared__ __attribute__((aligned(16))) uint8_t s_dst[HB * 64];
  __shared__ __attribute__((aligned(16))) uint32_t s_rows[kSegment];  // compacted row ids
  __shared__ int s_cnt[kChunks];
  __shared__ float s_D[HB], s_lse2[HB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;   // MFMA column / k-group of the lane
  const int64_t token = blockIdx.x / a.head_blocks;
  const int h0 = (int)(blockIdx.x % a.head_blocks) * HB;
  if (a.only && ((a.only[token] != 0u) != (a.only_nonzero != 0))) return;   // uniform over the workgroup

  // ---------------------------------------------------------------- per-token inputs
  // Q (HB x 576) and dO (HB x 512) of the head block into LDS; padded heads are 0.
  for (int i = tid; i < HB * (kDqk / 8); i += 256) {
    const int h = i / (kDqk / 8), c = i % (kDqk / 8);
    bf16x8_t v = {};
    if (h0 + h < a.num_heads) v = *(const bf16x8_t*)(a.q + token * a.q_st + (int64_t)(h0 + h) * a.q_sh + 8 * c);
    *(bf16x8_t*)(s_q + h * kBwPitch + 16 * c) = v;
  }
  for (int i = tid; i < HB * (kDv / 8); i += 256) {
    const int h = i / (kDv / 8), c = i % (kDv / 8);
    bf16x8_t v = {};
    if (h0 + h < a.num_heads) v = *(const bf16x8_t*)(a.dout + token * a.do_st + (int64_t)(h0 + h) * a.do_sh + 8 * c);
    *(bf16x8_t*)(s_do + h * kBwOPitch + 16 * c) = v;
  }
  // D = dO . O and LSE (log2 units) per head: wave w takes heads HB/4 * w ..
  for (int hh = 0; hh < HB / 4; ++hh) {
    const int h = (HB / 4) * wave + hh;
    float d = 0.f;
    if (h0 + h < a.num_heads) {
      const bf16x8_t o = *(const bf16x8_t*)(a.out + token * a.o_st + (int64_t)(h0 + h) * a.o_sh + 8 * lane);
      const bf16x8_t dd = *(const bf16x8_t*)(a.dout + token * a.do_st + (int64_t)(h0 + h) * a.do_sh + 8 * lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) d += (float)o[e] * (float)dd[e];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) d += __shfl_xor(d, off);
    if (lane == 0) {
      s_D[h] = d;
      // padded heads: +inf, so their P = exp2(score - inf) = 0
      s_lse2[h] = h0 + h < a.num_heads ? a.lse[token * a.lse_st + h0 + h] * 1.4426950408889634f : INFINITY;
    }
  }
  __syncthreads();

  // Q^T (waves 0, 1) or dO^T (waves 2, 3) as the MFMA B operand, head tile ht:
  // lane holds head 16ht + n, columns 32c + 8g .. +7
  const bool s_role = wave < 2;
  const int kb = wave & 1;   // key block of the phase-1 product
  bf16x8_t breg[HT][kDqk / 32];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int c = 0; c < kDqk / 32; ++c)
      breg[ht][c] = s_role ? lds16(s_q + (16 * ht + n) * kBwPitch + 2 * (32 * c + 8 * g))
                           : (c < kDv / 32 ? lds16(s_do + (16 * ht + n) * kBwOPitch + 2 * (32 * c + 8 * g))
                                           : (bf16x8_t){});

  // dq column tiles m = 4k + w (k = 0 .. 8) of head tile ht: lane holds
  // column 16m + n of heads 16ht + 4g .. +3
  float4_t dq_acc[HT][9];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int k = 0; k < 9; ++k) dq_acc[ht][k] = (float4_t){0.f, 0.f, 0.f, 0.f};

  // stage offsets of the lane's reads. Phase 1 (A operand): key kb*16 + n,
  // logical granule 4c + g; latent c = 4i + c' at a_lat[c'] + 256i, rope c = 16 + c' at a_rope[c'].
  uint32_t a_lat[4], a_rope[2];
  {
    const int r = kb * 16 + n;
#pragma unroll
    for (int c = 0; c < 4; ++c) a_lat[c] = (uint32_t)(r * 1024 + 16 * ((4 * c + g) ^ bw_swz(r)));
#pragma unroll
    for (int c = 0; c < 2; ++c) a_rope[c] = (uint32_t)(kBwLat + r * 128 + 16 * ((4 * c + g) ^ bw_swz_r(r)));
  }
  // Phase 3a (K^T operand of column tile m = 4k + w): lane (g, n) points at
  // key 4g + n/4 (and 16 + 4g + n/4), columns 16m + 4(n % 4) ..; latent tile
  // k at t_lat[k % 2] + 256 (k / 2), the rope tile (k = 8) at t_rope.
  uint32_t t_lat[2], t_rope;
  {
    const int r = 4 * g + (n >> 2), hb = (n >> 1) & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      t_lat[i] = (uint32_t)(r * 1024 + 16 * ((2 * (wave + 4 * i) + hb) ^ bw_swz(r)) + 8 * (n & 1));
    t_rope = (uint32_t)(kBwLat + r * 128 + 16 * ((2 * wave + hb) ^ bw_swz_r(r)) + 8 * (n & 1));
  }

  FwdArgs fa = {};   // the forward's index stage, with row ids as the offsets
  fa.idx = a.idx;
  fa.idx_st = a.idx_st;
  fa.num_kv = a.num_kv;
  fa.kv_row_gran = 1;
  fa.topk = a.topk;
  fa.seg_len = kSegment;

  const int nseg = (a.topk + kSegment - 1) / kSegment;
  for (int seg = 0; seg < nseg; ++seg) {
    const int nvalid = build_key_list<false>(fa, token, seg, wave, lane, s_rows, s_cnt, [] {});
    const int ntiles = (nvalid + kTileKeys - 1) / kTileKeys;

    // rows of tile t: thread tid holds granules tid + 256k (row = gi / 72, granule gi % 72)
    bf16x8_t greg[kBwGran];
    // all row ids first, then all loads: one LDS round trip per tile, not one per load
    auto load_tile = [&](int t) {
      uint32_t rid[kBwGran];
#pragma unroll
      for (int k = 0; k < kBwGran; ++k) rid[k] = s_rows[t * kTileKeys + (tid + 256 * k) / (kDqk / 8)];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kBwGran; ++k) {
        const int c = (tid + 256 * k) % (kDqk / 8);
        greg[k] = *(const bf16x8_t*)(a.kv + (int64_t)rid[k] * a.kv_st + 8 * c);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto store_tile = [&](int t) {
      uint8_t* st = s_stage[t & 1];
#pragma unroll
      for (int k = 0; k < kBwGran; ++k) {
        const int gi = tid + 256 * k, row = gi / (kDqk / 8), c = gi % (kDqk / 8);
        uint8_t* d = c < kDv / 8 ? st + row * 1024 + 16 * (c ^ bw_swz(row))
                                 : st + kBwLat + row * 128 + 16 * ((c - kDv / 8) ^ bw_swz_r(row));
        *(bf16x8_t*)d = greg[k];
      }
    };
    if (ntiles > 0) {
      load_tile(0);
      store_tile(0);
    }
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
      if (j + 1 < ntiles) load_tile(j + 1);   // in flight during the three phases
      const uint8_t* st = s_stage[j & 1];

      // ---- phase 1: S^T (waves 0, 1) or dP^T (waves 2, 3) of key block kb, every head tile
      float4_t acc[HT];
      // key kb*16 + n, columns 32c + 8g ..
      auto arow = [&](int c) { return c < 16 ? st + a_lat[c & 3] + 256 * (c >> 2) : st + a_rope[c - 16]; };
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) acc[ht] = (float4_t){0.f, 0.f, 0.f, 0.f};
      if (s_role) {
#pragma unroll
        for (int c = 0; c < kDqk / 32; ++c) {
          const bf16x8_t av = lds16(arow(c));
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
            acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, breg[ht][c], acc[ht], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int c = 0; c < kDv / 32; ++c) {
          const bf16x8_t av = lds16(arow(c));
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
            acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, breg[ht][c], acc[ht], 0, 0, 0);
        }
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) s_dp[kb][ht][lane] = acc[ht];
      }
      __syncthreads();

      // ---- phase 2: P and s*dS (lane: head 16ht + n, keys kb*16 + 4g + e)
      if (s_role) {
        const int lim = nvalid - j * kTileKeys;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          const int h = 16 * ht + n;
          const float4_t dp = s_dp[kb][ht][lane];
          const float Dh = s_D[h], l2 = s_lse2[h];
          float p[4], ds[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool ok = kb * 16 + 4 * g + e < lim;
            p[e] = ok ? __builtin_amdgcn_exp2f(acc[ht][e] * a.scale_log2 - l2) : 0.f;
            ds[e] = p[e] * (dp[e] - Dh) * a.scale;
          }
          const int off = h * 64 + 16 * g + 8 * kb;   // keys kb*16 + 4g .. +3 (k-slot order)
          *(uint2*)(s_pt + off) = (uint2){pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
          *(uint2*)(s_dst + off) = (uint2){pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3])};
        }
      }
      __syncthreads();

      // ---- phase 3a: dq tiles 4k + w += (s dS)[16 heads x 32 keys] K[32 keys x 16 columns],
      //      k slots 8g .. 8g+7 = keys 4g .. 4g+3, 16+4g .. 16+4g+3
      {
        bf16x8_t ads[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) ads[ht] = lds16(s_dst + (16 * ht + n) * 64 + 16 * g);
        // K^T operands read 4 tiles ahead (pinned order: the scheduler would
        // otherwise sink each read next to its products)
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
          for (int ht = 0; ht < HT; ++ht)
            dq_acc[ht][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ads[ht], b, dq_acc[ht][k], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // ---- phase 3b: dkv of key block kb2 = w >> 1, column tiles 18(w & 1) .. +17:
      //   [16 keys x 16 columns] = (s dS)^T Q + P^T dO over the HB heads
      {
        const int kb2 = wave >> 1;
        const int kbase = j * kTileKeys + kb2 * 16 + 4 * g;   // this lane's outputs: keys kbase + e
        uint32_t rid[4];
        bool rok[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          rid[e] = s_rows[kbase + e];
          rok[e] = kbase + e < nvalid;
        }
        if constexpr (HT == 1) {
          // 16x16x16 over heads 4g .. 4g+3: A operands (lane (g, n) points at head
          // 4g + n/4, keys kb2*16 + 4(n % 4)) receive key kb2*16 + n
          const int aoff = (4 * g + (n >> 2)) * 64 + 16 * (n & 3) + 8 * kb2;
          const short4_t ads = lds_read_tr16(s_dst + aoff);
          const short4_t ap = lds_read_tr16(s_pt + aoff);
          const uint8_t* bq = s_q + (4 * g + (n >> 2)) * kBwPitch + 8 * (n & 3);
          const uint8_t* bo = s_do + (4 * g + (n >> 2)) * kBwOPitch + 8 * (n & 3);
#pragma unroll 2
          for (int k = 0; k < 18; ++k) {
            const int d0 = 16 * (18 * (wave & 1) + k);
            float4_t c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ads, lds_read_tr16(bq + 2 * d0),
                                                                   (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            if (d0 < kDv) c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ap, lds_read_tr16(bo + 2 * d0), c, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (rok[e]) unsafeAtomicAdd(a.dkv + (int64_t)rid[e] * a.dkv_st + d0 + n, c[e]);
          }
        } else {
          // 16x16x32 over heads 8g .. 8g+7: two transposed reads per operand
          // (heads 8g + n/4 and 8g + 4 + n/4)
          const int aoff = (8 * g + (n >> 2)) * 64 + 16 * (n & 3) + 8 * kb2;
          const bf16x8_t ads = join4(lds_read_tr16(s_dst + aoff), lds_read_tr16(s_dst + aoff + 4 * 64));
          const bf16x8_t ap = join4(lds_read_tr16(s_pt + aoff), lds_read_tr16(s_pt + aoff + 4 * 64));
          const uint8_t* bq = s_q + (8 * g + (n >> 2)) * kBwPitch + 8 * (n & 3);
          const uint8_t* bo = s_do + (8 * g + (n >> 2)) * kBwOPitch + 8 * (n & 3);
#pragma unroll 2
          for (int k = 0; k < 18; ++k) {
            const int d0 = 16 * (18 * (wave & 1) + k);
            const bf16x8_t b1 = join4(lds_read_tr16(bq + 2 * d0), lds_read_tr16(bq + 4 * kBwPitch + 2 * d0));
            float4_t c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ads, b1, (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            if (d0 < kDv) {
              const bf16x8_t b2 = join4(lds_read_tr16(bo + 2 * d0), lds_read_tr16(bo + 4 * kBwOPitch + 2 * d0));
              c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, b2, c, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (rok[e]) unsafeAtomicAdd(a.dkv + (int64_t)rid[e] * a.dkv_st + d0 + n, c[e]);
          }
        }
      }
      if (j + 1 < ntiles) store_tile(j + 1);   // the other stage: last read before this tile's barrier
      __syncthreads();
    }
  }

  // ---------------------------------------------------------------- dq (fp32)
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      const int d = 16 * (4 * k + wave) + n;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int h = h0 + 16 * ht + 4 * g + e;
        if (h < a.num_heads) a.dq[token * a.dq_st + (int64_t)h * a.dq_sh + d] = dq_acc[ht][k][e];
      }
    }
}

// ==================================================================== kv-major pass
// For few heads (<= 16) and index rows that name a large share of the kv rows
// (causal prefill: token t names most of 0..t), the token-major kernel above
// adds 576 floats to dkv per (token, key): the atomics, not the MFMAs, bound
// it. The kv-major pass turns the loops around. A workgroup owns two blocks
// of 32 kv rows and a chunk of 64 tokens. The chunk's tokens that name rows
// of the blocks are taken in steps: each step runs the three phases of one
// tile of the token-major kernel with the 64 rows as the tile, the named rows
// as its valid keys, and the 16 MFMA columns filled by 16 / hp tokens of hp
// heads each (hp = num_heads rounded up to a power of two). dkv of the rows
// accumulates in registers over the chunk and is added once; dq takes the
// atomics instead, num_heads x 576 per (token, 64 rows). With 8 heads and
// dense causal rows that is ~8x fewer atomic adds.
//
// A prepass per token builds the occupancy masks (bit r % 32 of word r / 32:
// row r named), D = dO . O per head, and zeroes the token's dq. A token whose
// row names some kv row twice is left to the token-major kernel (its masks
// stay 0 and only[t] = 1), so duplicates keep counting once per occurrence.
// For the split schedule it also numbers the token's named rows in row order
// (their rank): the rank of each valid entry, and per 256-row block the
// number of named rows below it.

constexpr int kKvChunk = 64;        // tokens per kv-major workgroup (one wave's ballot)
constexpr int kKvMaxWords = 8192;   // mask words per token row held in LDS (kv rows <= 262144)

struct KvMajorArgs {
  uint32_t* mask;     // u32 [num_words][num_tokens]: word w of token t at mask[w * T + t]
  uint32_t* dup;      // u32 [num_tokens]: 1 = the row names a kv row twice
  float* dbuf;        // fp32 [num_tokens][16]: D = dO . O per head (0 past num_heads); null: not formed
  int64_t d_st;       // heads per token row of dbuf (16)
  int32_t num_words;  // ceil(num_kv / 32)
  int32_t zero_dq;    // 1: the prepass zeroes dq (the kv-major pass adds into it)
  // Split schedule only (null otherwise). A token's named rows, ordered by
  // row id, are numbered 0, 1, ... (their rank); the dq pass stores P and
  // s*dS of each named row at its rank, so that the dkv pass finds the named
  // rows of any 256-row block as one contiguous run.
  int32_t* pre;       // i32 [num_blk][num_tokens]: named rows of token t below row 256b
  int32_t* rank;      // i32 [num_tokens][cap]: rank of the token's c-th valid entry (index-row order)
  uint16_t* pds;      // bf16 [num_tokens][groups][cap][64]: per rank, P of the group's 32 heads, then s*dS
  int64_t cap;        // entries per token in rank and pds (topk)
  int32_t groups;     // head groups of 32: ceil(num_heads / 32)
  int32_t num_blk;    // ceil(num_words / 8): blocks of 256 rows
  uint32_t* queue;    // u32 [8]: the dkv pass's work-queue counters (the prepass clears them)
};

__global__ void __launch_bounds__(256)
sparse_mla_bwd_prep_kernel(const BwdArgs a, const KvMajorArgs m) {
  __shared__ uint32_t s_bm[kKvMaxWords];
  __shared__ int s_wp[kKvMaxWords];   // split schedule: named rows below each word
  __shared__ uint32_t s_dup;
  __shared__ int s_sum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t token = blockIdx.x;
  for (int w = tid; w < m.num_words; w += 256) s_bm[w] = 0u;
  if (tid == 0) s_dup = 0u;
  __syncthreads();
  const int32_t* row = a.idx + token * a.idx_st;
  for (int j = tid; j < a.topk; j += 256) {
    const int32_t v = row[j];
    if (v >= 0 && (int64_t)v < a.num_kv) {
      const uint32_t bit = 1u << (v & 31);
      if (atomicOr(&s_bm[v >> 5], bit) & bit) s_dup = 1u;
    }
  }
  // D per head (wave w: heads w, w + 4, ..; the kv-major pass only: the
  // split schedule's dq pass forms D itself) and, for the kv-major pass, dq = 0
  for (int h = wave; m.dbuf != nullptr && h < m.d_st; h += 4) {
    float d = 0.f;
    if (h < a.num_heads) {
      const bf16x8_t o = *(const bf16x8_t*)(a.out + token * a.o_st + (int64_t)h * a.o_sh + 8 * lane);
      const bf16x8_t dd = *(const bf16x8_t*)(a.dout + token * a.do_st + (int64_t)h * a.do_sh + 8 * lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) d += (float)o[e] * (float)dd[e];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) d += __shfl_xor(d, off);
    if (lane == 0) m.dbuf[token * m.d_st + h] = d;
  }
  if (m.zero_dq)
    for (int i = tid; i < a.num_heads * kDqk; i += 256)
      a.dq[token * a.dq_st + (int64_t)(i / kDqk) * a.dq_sh + i % kDqk] = 0.f;
  __syncthreads();
  const uint32_t dup = s_dup;
  if (tid == 0) m.dup[token] = dup;
  for (int w = tid; w < m.num_words; w += 256) m.mask[(int64_t)w * a.num_tokens + token] = dup ? 0u : s_bm[w];
  if (m.queue != nullptr && token == 0 && tid < 8) m.queue[tid] = 0u;
  if (m.rank == nullptr || dup) return;   // uniform

  // ---- split schedule: ranks. s_wp[w] = named rows below row 32w (an
  // exclusive scan of the words' popcounts; thread i takes a run of words).
  const int per = (m.num_words + 255) / 256;
  const int w0 = min(tid * per, m.num_words), w1 = min(w0 + per, m.num_words);
  int run = 0;
  for (int w = w0; w < w1; ++w) run += __popc(s_bm[w]);
  int incl = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_sum[wave] = incl;
  __syncthreads();
  int base = incl - run;
  for (int i = 0; i < wave; ++i) base += s_sum[i];
  for (int w = w0; w < w1; ++w) {
    s_wp[w] = base;
    base += __popc(s_bm[w]);
  }
  __syncthreads();
  for (int b = tid; b < m.num_blk; b += 256) m.pre[(int64_t)b * a.num_tokens + token] = s_wp[8 * b];
  // the c-th valid entry of the row (the order of the dq pass's key list)
  int cbase = 0;
  int32_t* const rk = m.rank + token * m.cap;
  for (int j0 = 0; j0 < a.topk; j0 += 256) {
    const int j = j0 + tid;
    const int32_t v = j < a.topk ? row[j] : -1;
    const bool ok = v >= 0 && (int64_t)v < a.num_kv;
    const uint64_t bal = __ballot(ok);
    __syncthreads();   // the previous round's reads of s_sum are done
    if (lane == 0) s_sum[wave] = __popcll(bal);
    __syncthreads();
    int before = cbase;
    for (int i = 0; i < wave; ++i) before += s_sum[i];
    if (ok) {
      const int c = before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      rk[c] = s_wp[v >> 5] + __popc(s_bm[v >> 5] & ((1u << (v & 31)) - 1u));
    }
    cbase += s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3];
  }
}

// One workgroup = (two kv blocks bp = rows 64bp .. 64bp+63, token chunk c);
// blockIdx.x = c * ceil(num_words / 2) + bp. A token's dq collects both
// blocks before it is added. One workgroup per CU (155 KB of LDS), so the
// compiler may use the whole register file to keep operand reads in flight.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
sparse_mla_bwd_kv_kernel(const BwdArgs a, const KvMajorArgs m) {
  constexpr int HB = 16;
  constexpr int KR = 2 * kTileKeys;   // kv rows of the workgroup (64)
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[KR * kBwPitch];   // the two blocks' rows
  __shared__ __attribute__((aligned(16))) uint8_t s_q[2][HB * kBwPitch];    // the step's Q columns, double-buffered
  __shared__ __attribute__((aligned(16))) uint8_t s_do[2][HB * kBwOPitch];  // the step's dO columns
  __shared__ __attribute__((aligned(16))) float4_t s_dp[4][64];              // dP^T per 16-key block
  __shared__ __attribute__((aligned(16))) uint8_t s_pt[HB * 2 * KR];          // P, bf16 [column][64 keys]
  __shared__ __attribute__((aligned(16))) uint8_t s_dst[HB * 2 * KR];         // s*dS, bf16 [column][64 keys]
  __shared__ float s_D[2][HB], s_lse2[2][HB];
  __shared__ int s_tok[kKvChunk];
  __shared__ uint64_t s_msk[kKvChunk];
  __shared__ int s_np;
  constexpr int kKP = 2 * KR;   // bytes per column row of s_pt / s_dst

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int nbp = (m.num_words + 1) / 2;
  const int bp = (int)(blockIdx.x % nbp);
  const int64_t t0 = (int64_t)(blockIdx.x / nbp) * kKvChunk;
  const int64_t r0 = (int64_t)bp * KR;

  // the chunk's tokens that name rows of the two blocks, in token order (the
  // token list), with a 64-bit mask of the named rows
  if (wave == 0) {
    const int64_t t = t0 + lane;
    uint64_t w = 0;
    if (t < a.num_tokens) {
      w = m.mask[(int64_t)(2 * bp) * a.num_tokens + t];
      if (2 * bp + 1 < m.num_words) w |= (uint64_t)m.mask[(int64_t)(2 * bp + 1) * a.num_tokens + t] << 32;
    }
    const uint64_t act = __ballot(w != 0u);
    if (w != 0u) {
      const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(act >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)act, 0u));
      s_tok[pos] = (int)lane;
      s_msk[pos] = w;
    }
    if (lane == 0) s_np = __builtin_popcountll(act);
  }
  __syncthreads();
  const int np = s_np;
  if (np == 0) return;
  // The 16 MFMA columns ("heads" of the products) carry tpp tokens of the
  // list at once, hp = 16 / tpp columns each (hp = num_heads rounded up to a
  // power of two): column h is head h % hp of token entry p*tpp + h / hp.
  // The dkv product then sums over those tokens too, and at 8 heads two
  // tokens take the MFMA work that one did.
  const int lhp = a.num_heads <= 1 ? 0 : 32 - __builtin_clz((unsigned)(a.num_heads - 1));
  const int hp = 1 << lhp, tpp = 16 >> lhp;
  const int nsteps = (np + tpp - 1) / tpp;
  // token (or -1) and head of column h in step p
  auto column = [&](int p, int h, int& hh) -> int64_t {
    const int ti = p * tpp + (h >> lhp);
    hh = h & (hp - 1);
    return (ti < np && hh < a.num_heads) ? t0 + s_tok[ti] : (int64_t)-1;
  };

  // the blocks' rows (rows past num_kv are 0; their mask bits are never set)
#pragma unroll 6
  for (int k = 0; k < 2 * kBwGran; ++k) {
    const int gi = tid + 256 * k, row = gi / (kDqk / 8), c = gi % (kDqk / 8);
    bf16x8_t v = {};
    if (r0 + row < a.num_kv) v = *(const bf16x8_t*)(a.kv + (r0 + row) * a.kv_st + 8 * c);
    *(bf16x8_t*)(s_stage + row * kBwPitch + 16 * c) = v;
  }

  // the arguments the step loop uses, as values: the lambdas below capture by
  // reference, and through a reference to the argument block the compiler
  // re-read them from memory in every step
  const uint16_t* const q_ptr = a.q;
  const uint16_t* const do_ptr = a.dout;
  const float* const lse_ptr = a.lse;
  const float* const dbuf = m.dbuf;
  const int64_t d_st = m.d_st;
  float* const dq_ptr = a.dq;
  const int64_t q_st = a.q_st, q_sh = a.q_sh, do_st = a.do_st, do_sh = a.do_sh, lse_st = a.lse_st;
  const int64_t dq_st = a.dq_st, dq_sh = a.dq_sh;
  const int num_heads = a.num_heads;
  const float scale = a.scale, scale_log2 = a.scale_log2;

  // Q (16 columns x 72 granules) and dO (16 x 64) of step p: thread tid holds granules tid + 256k
  constexpr int kPairGran = (HB * (kDqk / 8) + HB * (kDv / 8) + 255) / 256;   // 9
  bf16x8_t preg[kPairGran];
  uint32_t pvalid = 0;   // bit k: granule k holds data (else it is stored as 0)
  float pl2 = 0.f, pD = 0.f;
  bool pok = false;
  // Branch-free: every granule's load is issued, those of empty columns from
  // q's first element, and zeroed when stored. Conditional loads here had
  // split the issue into branches with waits between them.
  auto load_step = [&](int p) {
    pvalid = 0;
#pragma unroll
    for (int k = 0; k < kPairGran; ++k) {
      const int gi = tid + 256 * k;
      const bool isq = gi < HB * (kDqk / 8);
      const int gj = isq ? gi : gi - HB * (kDqk / 8);
      const int h = isq ? gj / (kDqk / 8) : gj / (kDv / 8);
      const int c = isq ? gj % (kDqk / 8) : gj % (kDv / 8);
      const int ti = p * tpp + (h >> lhp), hh = h & (hp - 1);
      const bool ok = gi < HB * (kDqk / 8) + HB * (kDv / 8) && ti < np && hh < num_heads;
      const int64_t t = t0 + s_tok[ti < np ? ti : np - 1];
      const uint16_t* src = isq ? q_ptr + t * q_st + hh * q_sh + 8 * c : do_ptr + t * do_st + hh * do_sh + 8 * c;
      preg[k] = *(const bf16x8_t*)(ok ? src : q_ptr);
      pvalid |= (uint32_t)ok << k;
    }
    {
      const int h = tid & (HB - 1);
      const int ti = p * tpp + (h >> lhp), hh = h & (hp - 1);
      pok = ti < np && hh < num_heads;
      const int64_t t = t0 + s_tok[ti < np ? ti : np - 1];
      pl2 = *(pok ? lse_ptr + t * lse_st + hh : lse_ptr);   // scaled when stored: no wait on the loads here
      pD = *(pok ? dbuf + t * d_st + hh : dbuf);
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int k = 0; k < kPairGran; ++k) {
      const int gi = tid + 256 * k;
      const bf16x8_t v = (pvalid >> k) & 1u ? preg[k] : (bf16x8_t){};
      if (gi < HB * (kDqk / 8)) {
        const int h = gi / (kDqk / 8), c = gi % (kDqk / 8);
        *(bf16x8_t*)(s_q[buf] + h * kBwPitch + 16 * c) = v;
      } else if (gi < HB * (kDqk / 8) + HB * (kDv / 8)) {
        const int gj = gi - HB * (kDqk / 8), h = gj / (kDv / 8), c = gj % (kDv / 8);
        *(bf16x8_t*)(s_do[buf] + h * kBwOPitch + 16 * c) = v;
      }
    }
    if (tid < HB) {
      // empty columns: +inf, so their P = exp2(score - inf) = 0
      s_lse2[buf][tid] = pok ? pl2 * 1.4426950408889634f : INFINITY;
      s_D[buf][tid] = pok ? pD : 0.f;
    }
  };
  load_step(0);
  store_step(0);
  __syncthreads();

  // phase 1 roles: K (waves 0, 1) or V (waves 2, 3) of 16-key blocks
  // kb = w & 1 and kb + 2 as the MFMA A operand (lane: key 16kb + n, columns 32c + 8g ..)
  const bool s_role = wave < 2;
  const int kb = wave & 1;
  const uint8_t* arow0 = s_stage + (kb * 16 + n) * kBwPitch + 16 * g;
  const uint8_t* arow1 = arow0 + 32 * kBwPitch;
  // key block kb's operand stays in registers for the whole chunk (the rows
  // do not change); kb + 2's is read from LDS in each step
  bf16x8_t areg[kDqk / 32];
#pragma unroll
  for (int c = 0; c < kDqk / 32; ++c) areg[c] = (s_role || c < kDv / 32) ? lds16(arow0 + 64 * c) : (bf16x8_t){};

  // dkv of 16-key blocks kb2 = w >> 1 and kb2 + 2, column tiles 18(w & 1) .. +17:
  // lane holds column 16dt + n of keys 16kb + 4g .. +3
  const int kb2 = wave >> 1;
  float4_t dkv_acc[2][18];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int k = 0; k < 18; ++k) dkv_acc[j][k] = (float4_t){0.f, 0.f, 0.f, 0.f};

  for (int p = 0; p < nsteps; ++p) {
    const int buf = p & 1;
    if (p + 1 < nsteps) load_step(p + 1);   // in flight during the three phases
    const uint8_t* sq = s_q[buf];
    const uint8_t* sd = s_do[buf];

    // ---- phase 1: S^T (waves 0, 1) or dP^T (waves 2, 3) of key blocks kb, kb + 2
    float4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    if (s_role) {
#pragma unroll
      for (int c = 0; c < kDqk / 32; ++c) {
        const bf16x8_t bv = lds16(sq + n * kBwPitch + 64 * c + 16 * g);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(areg[c], bv, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds16(arow1 + 64 * c), bv, acc1, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int c = 0; c < kDv / 32; ++c) {
        const bf16x8_t bv = lds16(sd + n * kBwOPitch + 64 * c + 16 * g);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(areg[c], bv, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds16(arow1 + 64 * c), bv, acc1, 0, 0, 0);
      }
      s_dp[kb][lane] = acc0;
      s_dp[kb + 2][lane] = acc1;
    }
    __syncthreads();

    // ---- phase 2: P and s*dS (lane: column n, keys 16kb' + 4g + e), masked by each column's token's rows
    if (s_role) {
      const int ti = p * tpp + (n >> lhp);   // the token entry of this lane's column
      const uint64_t msk = ti < np ? s_msk[ti] : 0u;
      const float Dh = s_D[buf][n], l2 = s_lse2[buf][n];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int kbj = kb + 2 * j;
        const float4_t sc = j ? acc1 : acc0;
        const float4_t dp = s_dp[kbj][lane];
        float pv[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = (msk >> (kbj * 16 + 4 * g + e)) & 1u;
          pv[e] = ok ? __builtin_amdgcn_exp2f(sc[e] * scale_log2 - l2) : 0.f;
          ds[e] = pv[e] * (dp[e] - Dh) * scale;
        }
        const int off = n * kKP + 2 * (kbj * 16 + 4 * g);
        *(uint2*)(s_pt + off) = (uint2){pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
        *(uint2*)(s_dst + off) = (uint2){pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3])};
      }
    }
    __syncthreads();

    // ---- phase 3a: dq tiles 9w .. 9w+8 of the step's tokens += (s dS) K over
    // the 64 keys, added with atomics. Operand reads go ahead of the products.
    {
      const uint8_t* kt = s_stage + (8 * g + (n >> 2)) * kBwPitch + 8 * (n & 3);
      const bf16x8_t ads0 = lds16(s_dst + n * kKP + 16 * g);        // keys 8g ..
      const bf16x8_t ads1 = lds16(s_dst + n * kKP + 64 + 16 * g);   // keys 32 + 8g ..
      float4_t c[9];
#pragma unroll
      for (int k3 = 0; k3 < 9; k3 += 3) {
        bf16x8_t bk0[3], bk1[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          const int d0 = 16 * (9 * wave + k3 + k);
          bk0[k] = join4(lds_read_tr16(kt + 2 * d0), lds_read_tr16(kt + 4 * kBwPitch + 2 * d0));
          bk1[k] = join4(lds_read_tr16(kt + 32 * kBwPitch + 2 * d0), lds_read_tr16(kt + 36 * kBwPitch + 2 * d0));
        }
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          c[k3 + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ads0, bk0[k], (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          c[k3 + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ads1, bk1[k], c[k3 + k], 0, 0, 0);
        }
      }
      // row 4g + e of the tile is column 4g + e of the step; empty columns add nothing
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int hh;
        const int64_t t = column(p, 4 * g + e, hh);
        if (t >= 0) {
          float* dqt = dq_ptr + t * dq_st + hh * dq_sh + n;
#pragma unroll
          for (int k = 0; k < 9; ++k) unsafeAtomicAdd(dqt + 16 * (9 * wave + k), c[k][e]);
        }
      }
    }
    // ---- phase 3b: dkv of key blocks kb2, kb2 + 2 += (s dS)^T Q + P^T dO over
    // the 16 columns (registers); the Q and dO operands serve both key blocks
    {
      short4_t ads[2], ap[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int aoff = (4 * g + (n >> 2)) * kKP + 2 * ((kb2 + 2 * j) * 16 + 4 * (n & 3));
        ads[j] = lds_read_tr16(s_dst + aoff);
        ap[j] = lds_read_tr16(s_pt + aoff);
      }
      const uint8_t* bq = sq + (4 * g + (n >> 2)) * kBwPitch + 8 * (n & 3);
      const uint8_t* bo = sd + (4 * g + (n >> 2)) * kBwOPitch + 8 * (n & 3);
#pragma unroll
      for (int part = 0; part < 3; ++part) {
        short4_t oq[6], oo[6];
#pragma unroll
        for (int k = 0; k < 6; ++k) {
          const int d0 = 16 * (18 * (wave & 1) + 6 * part + k);
          oq[k] = lds_read_tr16(bq + 2 * d0);
          oo[k] = d0 < kDv ? lds_read_tr16(bo + 2 * d0) : (short4_t){};
        }
#pragma unroll
        for (int k = 0; k < 6; ++k) {
          const int d0 = 16 * (18 * (wave & 1) + 6 * part + k);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float4_t& acc2 = dkv_acc[j][6 * part + k];
            acc2 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ads[j], oq[k], acc2, 0, 0, 0);
            if (d0 < kDv) acc2 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ap[j], oo[k], acc2, 0, 0, 0);
          }
        }
      }
    }
    if (p + 1 < nsteps) store_step(buf ^ 1);   // the other buffer: last read before the previous step's barrier
    __syncthreads();
  }

  // ---- the blocks' dkv, once per workgroup (other chunks add to the same rows)
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int k = 0; k < 18; ++k) {
      const int d0 = 16 * (18 * (wave & 1) + k);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t r = r0 + (kb2 + 2 * j) * 16 + 4 * g + e;
        if (r < a.num_kv) unsafeAtomicAdd(a.dkv + r * a.dkv_st + d0 + n, dkv_acc[j][k][e]);
      }
    }
}

// dkv = 0 before the backward accumulates into it: one thread per float4.
__global__ void __launch_bounds__(256)
dkv_zero_kernel(float* dkv, int64_t rows, int64_t row_stride) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_row = kDqk / 4;
  if (i >= rows * per_row) return;
  const int64_t r = i / per_row, c = i % per_row;
  *(float4_t*)(dkv + r * row_stride + 4 * c) = (float4_t){0.f, 0.f, 0.f, 0.f};
}

}  // namespace dsa
