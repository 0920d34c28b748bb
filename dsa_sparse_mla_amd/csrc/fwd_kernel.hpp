// Device kernels of the DSA sparse MLA forward for gfx950 (MI355X).
//
// One workgroup handles one query token (or one segment of its index row when
// the row is split). Steps, all inside the kernel:
//   1. index stage: read the token's index segment, keep the entries that name
//      a KV row (for the paged cache: map logical position -> page -> row),
//      and compact their row offsets, in order, into an LDS list;
//   2. gather: stream the listed 576-wide bf16 rows, 16 keys per block, from
//      HBM straight into LDS (global_load_lds_dwordx4, 16 B per lane) through
//      a two-stage ring, so the next tile is in flight while this one is used;
//   3. S^T = K Q^T on bf16 MFMA (v_mfma_f32_16x16x32_bf16), keys as M and
//      16 heads as N, Q held in registers as the B operand;
//   4. online softmax in fp32 in the base-2 domain (scale folded with log2 e);
//   5. O^T += V^T P^T on bf16 MFMA (v_mfma_f32_16x16x16_bf16): the S^T
//      accumulator layout is already the B-operand layout of P^T, so P never
//      leaves registers; V is the leading 512 columns of the same LDS rows;
//   6. epilogue: merge the key groups of the workgroup, normalise, write bf16
//      O and fp32 LSE -- or fp32 partials that a second kernel merges.
//
// Work split inside a workgroup: HT head tiles (16 heads each) x KG key
// groups, one wave per (head tile, key group). A wave keeps its own running
// max, sum and O^T accumulator for its head tile over the keys of its group,
// so the inner loop needs no exchange between waves; the groups are merged
// once at the end.
//
// Pages: "feat: add XTuner TileLang sparse MLA backend" (lmdeploy PR 4904),
// Summary and Performance > Isolated sparse MLA forward; "[Feature] Add
// optional FlashMLA backend for DSA Sparse MLA" (xtuner PR 2083), Runtime
// constraints.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowGran = 72;      // 16-byte granules in one 576-wide bf16 row
constexpr int kLdsPitch = 73;     // LDS row pitch in granules: odd, so the 16 rows an
                                  // MFMA operand read touches fall in 16 different banks
constexpr int kBlockKeys = 16;    // keys per MFMA block
constexpr int kSegment = 2048;    // index entries one workgroup compacts into LDS
constexpr float kLn2 = 0.693147180559945309f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

struct FwdArgs {
  const uint16_t* q;       // bf16 [T, H, 576]
  int64_t q_st, q_sh;      // strides in elements
  const uint8_t* kv;       // byte base of the rows (flat) or of the pages
  int64_t kv_row_gran;     // row pitch in 16-byte granules
  int64_t num_kv;          // flat: number of rows
  int64_t kv_page_gran;    // paged: page pitch in granules
  int32_t page_shift;      // paged: log2(page_size)
  int32_t page_mask;       // paged: page_size - 1
  const int32_t* page_table;
  int64_t pt_stride;
  int32_t max_pages;
  const int32_t* seq_lens;
  int32_t q_per_seq;
  int64_t num_pages;
  const int32_t* idx;      // int32 [T, topk]
  int64_t idx_st;
  int64_t num_tokens;
  int32_t num_heads;
  int32_t topk;
  float scale_log2;        // sm_scale * log2(e)
  uint16_t* out;           // bf16 [T, H, 512]
  int64_t o_st, o_sh;
  float* lse;              // fp32 [T, H]
  int64_t lse_st;
  int32_t splits;          // workgroups per token
  int32_t seg_len;         // index entries per split
  float* part_o;           // splits > 1: fp32 [T, splits, H, 512], normalised per split
  float* part_ml;          // splits > 1: fp32 [T, splits, H, 2] = (max in log2 units, sum)
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS byte offset of a __shared__ object.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const uint8_t*)(p)));
}

// One wave-wide 16-byte-per-lane copy HBM -> LDS: lane L's 16 bytes from
// `src` land at LDS byte lds_base + 16 * L (lds_base is wave-uniform, in M0).
// Issued through asm so the compiler does not tie every later LDS read to it;
// completion is awaited explicitly with s_waitcnt vmcnt.
__device__ __forceinline__ void dma_row_16b(const void* src, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(lds_base)
      : "memory");  // M0 is reserved by the compiler and not otherwise used by these kernels
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo;  // round to nearest even
  __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int HT, int KG>
struct FwdShape {
  static constexpr int kWaves = HT * KG;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kTileKeys = KG * kBlockKeys;
  static constexpr int kTileGran = kTileKeys * kLdsPitch;
  static constexpr int kDmaPerTile = (kTileGran + 63) / 64;   // 1 KB per wave instruction
  static constexpr int kStageBytes = kDmaPerTile * 1024;
  static constexpr int kChunksPerWave = kSegment / 64 / kWaves;
  // merge scratch (reuses the stage area): m and l per wave, then 8 dv tiles per wave
  static constexpr int kMergeBytes = kWaves * 16 * 2 * 4 + kWaves * 8 * 64 * 16;
  static_assert(kSegment % (64 * kWaves) == 0, "index chunks must divide evenly");
  static_assert(KG == 1 || kMergeBytes <= 2 * kStageBytes, "merge scratch must fit the stages");
};

template <int HT, int KG, bool PAGED>
__global__ void __launch_bounds__(64 * HT * KG)
sparse_mla_fwd_kernel(const FwdArgs a) {
  using S = FwdShape<HT, KG>;
  constexpr int NW = S::kWaves;

  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[2 * S::kStageBytes];
  __shared__ uint32_t s_goff[kSegment];
  __shared__ int s_cnt[kSegment / 64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hcol = lane & 15;   // MFMA column: a head (N) or a key row (M)
  const int kq = lane >> 4;     // MFMA k-group of the lane

  // Tokens in reverse order: in causal prefill the late tokens hold the most
  // keys, and launching the longest rows first balances the tail.
  const int64_t bid = blockIdx.x;
  const int64_t token = a.num_tokens - 1 - bid / a.splits;
  const int split = (int)(bid % a.splits);

  // ---------------------------------------------------------------- 1. index stage
  const int k0 = split * a.seg_len;
  const int n = min(a.topk - k0, a.seg_len);
  const int32_t* irow = a.idx + token * a.idx_st + k0;

  uint32_t goff[S::kChunksPerWave];
  uint64_t vmask[S::kChunksPerWave];
  int32_t seq_len = 0;
  const int32_t* ptab = nullptr;
  if constexpr (PAGED) {
    const int64_t seq = token / a.q_per_seq;
    seq_len = a.seq_lens[seq];
    ptab = a.page_table + seq * a.pt_stride;
  }
#pragma unroll
  for (int c = 0; c < S::kChunksPerWave; ++c) {
    const int e = (c * NW + wave) * 64 + lane;
    bool ok = e < n;
    const int32_t v = ok ? irow[e] : -1;
    uint32_t go = 0;
    if constexpr (!PAGED) {
      ok = ok && v >= 0 && (int64_t)v < a.num_kv;
      go = (uint32_t)((int64_t)v * a.kv_row_gran);
    } else {
      ok = ok && v >= 0 && v < seq_len;
      const int slot = v >> a.page_shift;
      ok = ok && slot < a.max_pages;
      const int32_t pg = ok ? ptab[slot] : -1;
      ok = ok && pg >= 0 && (int64_t)pg < a.num_pages;
      go = (uint32_t)((int64_t)pg * a.kv_page_gran + (int64_t)(v & a.page_mask) * a.kv_row_gran);
    }
    goff[c] = go;
    vmask[c] = __ballot(ok);
    if (lane == 0) s_cnt[c * NW + wave] = __popcll(vmask[c]);
  }
  __syncthreads();
  // exclusive prefix of the 32 chunk counts, computed by every wave (lane c = chunk c)
  const int cnt = lane < kSegment / 64 ? s_cnt[lane] : 0;
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < kSegment / 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  const int nvalid = __shfl(incl, kSegment / 64 - 1);
#pragma unroll
  for (int c = 0; c < S::kChunksPerWave; ++c) {
    const int base = __shfl(incl - cnt, c * NW + wave);
    const uint64_t m = vmask[c];
    if ((m >> lane) & 1ull) {
      const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
      s_goff[pos] = goff[c];
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- per-wave state
  const int ht = wave % HT;        // head tile of this wave
  const int grp = wave / HT;       // key group of this wave
  const int head = ht * 16 + hcol;
  const bool head_ok = head < a.num_heads;

  // Q as the MFMA B operand: lane holds dims 32c + 8kq .. +7 of head `head`
  bf16x8_t qreg[kDqk / 32];
  {
    const uint16_t* qp = a.q + token * a.q_st + (int64_t)(head_ok ? head : 0) * a.q_sh + kq * 8;
#pragma unroll
    for (int c = 0; c < kDqk / 32; ++c) {
      bf16x8_t v = *(const bf16x8_t*)(qp + 32 * c);
      qreg[c] = head_ok ? v : (bf16x8_t){};
    }
    // Use Q once here, so the compiler's wait for these loads sits before the
    // loop; a wait at the first use inside the loop would also wait for the
    // prefetch of the next tile on every iteration.
#pragma unroll
    for (int c = 0; c < kDqk / 32; ++c) asm volatile("" ::"v"(qreg[c]));
  }

  float4_t oacc[kDv / 16];
#pragma unroll
  for (int j = 0; j < kDv / 16; ++j) oacc[j] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of this lane's head, log2 units
  float l_run = 0.f;        // running sum over this lane's 4 keys of each block

  // ---------------------------------------------------------------- 2. gather
  const int ntiles = (nvalid + S::kTileKeys - 1) / S::kTileKeys;
  const uint32_t stage_lds = lds_offset(s_stage);
  auto issue_tile = [&](int j) {
    constexpr int kPer = (S::kDmaPerTile + NW - 1) / NW;   // DMA instructions of this wave
    const uint8_t* src[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = u * NW + wave;
      const int pos = i * 64 + lane;           // LDS granule this lane fills
      const int r = pos / kLdsPitch;           // tile row (key)
      const int col = pos - r * kLdsPitch;     // granule in the row; 72 is pitch padding
      const int key = j * S::kTileKeys + r;
      const bool real = i < S::kDmaPerTile && r < S::kTileKeys && key < nvalid;
      const uint32_t go = s_goff[real ? key : 0];   // padding lanes re-read a valid row
      const int gcol = col < kRowGran ? col : kRowGran - 1;
      src[u] = a.kv + ((uint64_t)go + (uint32_t)gcol) * 16ull;
    }
    const uint32_t base = stage_lds + (j & 1) * S::kStageBytes;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = u * NW + wave;
      if (i < S::kDmaPerTile) dma_row_16b(src[u], __builtin_amdgcn_readfirstlane(base + i * 1024));
    }
  };

  if (ntiles > 0) issue_tile(0);
  for (int j = 0; j < ntiles; ++j) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < ntiles) issue_tile(j + 1);

    const int kb = j * S::kTileKeys + grp * kBlockKeys;   // first key of this wave's block
    if (kb < nvalid) {
      const uint8_t* blk = s_stage + (j & 1) * S::kStageBytes + grp * kBlockKeys * kLdsPitch * 16;

      // ------------------------------------------------------------ 3. S^T = K Q^T
      float4_t s = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* arow = blk + hcol * (kLdsPitch * 16) + kq * 16;
#pragma unroll
      for (int c = 0; c < kDqk / 32; ++c) {
        const bf16x8_t kop = *(const bf16x8_t*)(arow + c * 64);
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qreg[c], s, 0, 0, 0);
      }

      // ------------------------------------------------------------ 4. online softmax
      // s[i] = score of key kb + 4kq + i for head `head`
      float sc[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool kv_ok = kb + kq * 4 + i < nvalid;
        sc[i] = kv_ok ? s[i] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sc[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);     // finite: key kb is valid
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      float p[4];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = fast_exp2(sc[i] - m_new);
        psum += p[i];
      }
      l_run = l_run * alpha + psum;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int jt = 0; jt < kDv / 16; ++jt) oacc[jt] *= alpha;
      }
      short4_t pop;
      {
        const uint32_t lo = pack_bf16x2(p[0], p[1]);
        const uint32_t hi = pack_bf16x2(p[2], p[3]);
        pop[0] = (short)(lo & 0xffff);
        pop[1] = (short)(lo >> 16);
        pop[2] = (short)(hi & 0xffff);
        pop[3] = (short)(hi >> 16);
      }

      // ------------------------------------------------------------ 5. O^T += V^T P^T
      // A operand: lane holds V[key 4kq+i][dv 16jt + hcol], i = 0..3
      const uint8_t* vb = blk + (kq * 4) * (kLdsPitch * 16) + hcol * 2;
#pragma unroll
      for (int jt = 0; jt < kDv / 16; ++jt) {
        short4_t vop;
#pragma unroll
        for (int i = 0; i < 4; ++i) vop[i] = *(const short*)(vb + i * (kLdsPitch * 16) + jt * 32);
        oacc[jt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pop, oacc[jt], 0, 0, 0);
      }
    }
  }

  // ---------------------------------------------------------------- 6. epilogue
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);

  float m_all = m_run;   // merged over the key groups of this head tile
  float l_all = l_tot;
  float wself = 1.f;     // weight of this wave's accumulator in the merge
  float* mbuf = (float*)s_stage;
  float4_t* obuf = (float4_t*)(s_stage + NW * 16 * 2 * 4);
  if constexpr (KG > 1) {
    __syncthreads();  // every wave is done with the stages
    if (kq == 0) {
      mbuf[wave * 16 + hcol] = m_run;
      mbuf[NW * 16 + wave * 16 + hcol] = l_tot;
    }
    __syncthreads();
    m_all = -INFINITY;
#pragma unroll
    for (int g2 = 0; g2 < KG; ++g2) m_all = fmaxf(m_all, mbuf[(g2 * HT + ht) * 16 + hcol]);
    l_all = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < KG; ++g2) {
      const float mg = mbuf[(g2 * HT + ht) * 16 + hcol];
      if (mg != -INFINITY) l_all += fast_exp2(mg - m_all) * mbuf[NW * 16 + (g2 * HT + ht) * 16 + hcol];
    }
    wself = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_all);
  }
  const float inv_l = l_all > 0.f ? 1.f / l_all : 0.f;

  const int64_t ot = token;
  auto store = [&](int jt, float4_t v) {   // v = normalised O^T[16jt + 4kq + i][head]
    if (!head_ok) return;
    if (a.splits == 1) {
      uint16_t* op = a.out + ot * a.o_st + (int64_t)head * a.o_sh + jt * 16 + kq * 4;
      uint2 w;
      w.x = pack_bf16x2(v[0], v[1]);
      w.y = pack_bf16x2(v[2], v[3]);
      *(uint2*)op = w;
    } else {
      float* pp = a.part_o + ((ot * a.splits + split) * a.num_heads + head) * (int64_t)kDv + jt * 16 + kq * 4;
      *(float4_t*)pp = v;
    }
  };

  if constexpr (KG == 1) {
#pragma unroll
    for (int jt = 0; jt < kDv / 16; ++jt) store(jt, oacc[jt] * inv_l);
  } else {
    // merge the KG partial accumulators of each head tile, 8 dv tiles at a time
    const float f = wself;
#pragma unroll
    for (int ch = 0; ch < kDv / 16 / 8; ++ch) {
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) obuf[(wave * 8 + tt) * 64 + lane] = oacc[ch * 8 + tt] * f;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 8 / KG; ++u) {
        const int tt = grp * (8 / KG) + u;
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g2 = 0; g2 < KG; ++g2) acc += obuf[((g2 * HT + ht) * 8 + tt) * 64 + lane];
        store(ch * 8 + tt, acc * inv_l);
      }
      __syncthreads();
    }
  }

  if (grp == 0 && kq == 0 && head_ok) {
    if (a.splits == 1) {
      a.lse[ot * a.lse_st + head] = l_all > 0.f ? (m_all + __log2f(l_all)) * kLn2 : -INFINITY;
    } else {
      float* pm = a.part_ml + ((ot * a.splits + split) * a.num_heads + head) * 2;
      pm[0] = m_all;
      pm[1] = l_all;
    }
  }
}

// Merge of split partials: one wave per (token, head).
//   M = max_s m_s;  w_s = 2^(m_s - M) l_s;  O = sum_s w_s O_s / sum_s w_s;
//   LSE = (M + log2 sum_s w_s) ln 2.  Fixed order over s, so it is deterministic.
__global__ void __launch_bounds__(256)
sparse_mla_combine_kernel(const FwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= a.num_tokens * a.num_heads) return;
  const int64_t token = pair / a.num_heads;
  const int head = (int)(pair % a.num_heads);
  const float* ml = a.part_ml + (token * a.splits * a.num_heads + head) * 2;
  const int64_t sstride = (int64_t)a.num_heads * 2;
  float M = -INFINITY;
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, ml[s * sstride]);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  float W = 0.f;
  if (M != -INFINITY) {
    const float* po = a.part_o + (token * a.splits * a.num_heads + head) * (int64_t)kDv + lane * 8;
    const int64_t ostride = (int64_t)a.num_heads * kDv;
    for (int s = 0; s < a.splits; ++s) W += ml[s * sstride] == -INFINITY ? 0.f : fast_exp2(ml[s * sstride] - M) * ml[s * sstride + 1];
    const float invW = 1.f / W;
    for (int s = 0; s < a.splits; ++s) {
      const float ms = ml[s * sstride];
      if (ms == -INFINITY) continue;
      const float w = fast_exp2(ms - M) * ml[s * sstride + 1] * invW;
      const float4_t x0 = *(const float4_t*)(po + s * ostride);
      const float4_t x1 = *(const float4_t*)(po + s * ostride + 4);
      acc[0] += w * x0[0]; acc[1] += w * x0[1]; acc[2] += w * x0[2]; acc[3] += w * x0[3];
      acc[4] += w * x1[0]; acc[5] += w * x1[1]; acc[6] += w * x1[2]; acc[7] += w * x1[3];
    }
  }
  uint16_t* op = a.out + token * a.o_st + (int64_t)head * a.o_sh + lane * 8;
  uint4 w;
  w.x = pack_bf16x2(acc[0], acc[1]);
  w.y = pack_bf16x2(acc[2], acc[3]);
  w.z = pack_bf16x2(acc[4], acc[5]);
  w.w = pack_bf16x2(acc[6], acc[7]);
  *(uint4*)op = w;
  if (lane == 0) a.lse[token * a.lse_st + head] = W > 0.f ? (M + __log2f(W)) * kLn2 : -INFINITY;
}

}  // namespace dsa
