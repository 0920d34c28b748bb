// Device kernels of the DSA sparse MLA forward for gfx950 (MI355X).
//
// One workgroup of 4 waves handles one query token (or one segment of its
// index row when the row is split) for a block of up to 64 heads. Steps, all
// inside the kernel:
//   1. index stage: read the token's index segment, keep the entries that name
//      a KV row (for the paged cache: map logical position -> page -> row),
//      and compact their row offsets, in order, into an LDS list;
//   2. gather: stream the listed 576-wide bf16 rows, 64 keys per tile, from
//      HBM straight into LDS (global_load_lds_dwordx4, 16 B per lane) through
//      a two-stage ring, so the next tile is in flight while this one is used;
//   3. S^T = K Q^T on bf16 MFMA (v_mfma_f32_16x16x32_bf16): 16 keys as M,
//      16 heads as N, Q held in registers as the B operand;
//   4. online softmax in fp32, base-2 domain (scale folded with log2 e);
//   5. O^T += V^T P^T on bf16 MFMA (v_mfma_f32_16x16x32_bf16, 32 keys per
//      step). The S^T accumulator layout is already the B-operand layout of
//      P^T, so P never leaves registers. V is the leading 512 columns of the
//      same LDS rows, read transposed with ds_read_b64_tr_b16;
//   6. epilogue: normalise, write bf16 O and fp32 LSE -- or fp32 partials
//      that a second kernel merges when the row was split.
//
// Work split: the workgroup's heads form HT tiles of 16. Wave w computes S
// for head tile w % HT over every key of the tile, and PV for that head tile
// over its own slice of 512 * HT / 4 value columns. With HT < 4 the waves of
// one head tile repeat the (small) S product instead of exchanging P, so no
// wave ever waits for another inside the key loop except at the tile barrier.
//
// LDS tile layout (64 keys, 72 KB): a latent region of 64 rows x 1 KB
// (dims 0..511, i.e. V) and a rope region of 64 rows x 128 B (dims 512..575).
// Granule G (16 B) of latent row r sits at position G ^ (r & 15), of rope row
// r at G ^ ((r >> 1) & 7). Both spread the 16 rows of an MFMA operand read,
// and the 16 rows of a transposed V read, over all 64 LDS banks, and both let
// every per-lane LDS address be one of a few lane bases plus an immediate.
// Each gather instruction fills exactly one latent row, or 8 rope rows.
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
constexpr int kRowGran = 72;                          // 16-byte granules per 576-wide bf16 row
constexpr int kTileKeys = 64;                         // keys per tile
constexpr int kTileBytes = kTileKeys * kRowGran * 16;  // 73728
constexpr int kWaves = 4;
constexpr int kRopeOff = kTileKeys * 1024;            // rope region offset inside a tile
constexpr int kDmaPerTile = kTileKeys * kRowGran / 64;  // 72 wave-wide 1 KB copies
constexpr int kDmaPerWave = kDmaPerTile / kWaves;       // 18: 16 latent rows + 2 x 8 rope rows
constexpr int kSegment = 2048;                        // index entries one workgroup compacts into LDS
constexpr int kChunks = kSegment / 64;
constexpr int kChunksPerWave = kChunks / kWaves;
constexpr int kHeadsPerBlock = 64;                    // heads per workgroup at most
constexpr float kLn2 = 0.693147180559945309f;

static_assert(kDmaPerTile % kWaves == 0, "every wave issues the same number of copies");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

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
  int32_t splits;          // workgroups per token along the index row
  int32_t seg_len;         // index entries per split
  int32_t head_blocks;     // workgroups per token along the heads
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
__device__ __forceinline__ void dma_16b(const void* src, uint32_t lds_base) {
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

// Transposed read: with lane j of each 16-lane group pointing at 4 bf16 of
// row R + j/4, columns c + 4(j%4) .. +3, lane i of the group receives column
// c + i of rows R .. R+3.
__device__ __forceinline__ short4_t lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(
      (__attribute__((address_space(3))) uint8_t*)(p)));
}

template <int HT>
struct FwdShape {
  static constexpr int kHeads = 16 * HT;               // heads of the workgroup
  static constexpr int kDvParts = kWaves / HT;         // waves sharing one head tile
  static constexpr int kDvCols = kDv / kDvParts;       // value columns of one wave
  static constexpr int kDvTiles = kDvCols / 16;        // 16-column MFMA tiles of one wave
  static_assert(kWaves % HT == 0, "head tiles must divide the waves");
};

template <int HT, bool PAGED>
__global__ void __launch_bounds__(256)
sparse_mla_fwd_kernel(const FwdArgs a) {
  using S = FwdShape<HT>;

  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[2 * kTileBytes];
  __shared__ uint32_t s_goff[kSegment];
  __shared__ int s_cnt[kChunks];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hcol = lane & 15;   // MFMA row/column index of the lane
  const int kq = lane >> 4;     // MFMA k-group of the lane

  // Tokens in reverse order: in causal prefill the late tokens hold the most
  // keys, and launching the longest rows first balances the tail.
  const int64_t per_token = (int64_t)a.splits * a.head_blocks;
  const int64_t bid = blockIdx.x;
  const int64_t token = a.num_tokens - 1 - bid / per_token;
  const int rem = (int)(bid % per_token);
  const int split = rem / a.head_blocks;
  const int hblock = rem % a.head_blocks;

  // ---------------------------------------------------------------- 1. index stage
  const int k0 = split * a.seg_len;
  const int n = min(a.topk - k0, a.seg_len);
  const int32_t* irow = a.idx + token * a.idx_st + k0;

  int32_t val[kChunksPerWave];
#pragma unroll
  for (int c = 0; c < kChunksPerWave; ++c) {
    const int e = (c * kWaves + wave) * 64 + lane;
    val[c] = e < n ? irow[e] : -1;
  }
  uint32_t goff[kChunksPerWave];
  uint64_t vmask[kChunksPerWave];
  if constexpr (!PAGED) {
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) {
      const int32_t v = val[c];
      const bool ok = v >= 0 && (int64_t)v < a.num_kv;
      goff[c] = (uint32_t)((int64_t)v * a.kv_row_gran);
      vmask[c] = __ballot(ok);
    }
  } else {
    const int64_t seq = token / a.q_per_seq;
    const int32_t seq_len = a.seq_lens[seq];
    const int32_t* ptab = a.page_table + seq * a.pt_stride;
    int32_t pg[kChunksPerWave];
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) {
      const int32_t v = val[c];
      const bool ok = v >= 0 && v < seq_len && (v >> a.page_shift) < a.max_pages;
      pg[c] = ok ? ptab[v >> a.page_shift] : -1;
    }
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) {
      const bool ok = pg[c] >= 0 && (int64_t)pg[c] < a.num_pages;
      goff[c] = (uint32_t)((int64_t)pg[c] * a.kv_page_gran + (int64_t)(val[c] & a.page_mask) * a.kv_row_gran);
      vmask[c] = __ballot(ok);
    }
  }
  if (lane < kChunksPerWave) {
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) cnt = lane == c ? __popcll(vmask[c]) : cnt;
    s_cnt[lane * kWaves + wave] = cnt;
  }
  __syncthreads();
  // exclusive prefix of the chunk counts, computed by every wave (lane c = chunk c)
  const int cnt = lane < kChunks ? s_cnt[lane] : 0;
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < kChunks; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  const int nvalid = __shfl(incl, kChunks - 1);
#pragma unroll
  for (int c = 0; c < kChunksPerWave; ++c) {
    const int base = __shfl(incl - cnt, c * kWaves + wave);
    const uint64_t m = vmask[c];
    if ((m >> lane) & 1ull) s_goff[base + __popcll(m & ((1ull << lane) - 1ull))] = goff[c];
  }
  __syncthreads();

  // ---------------------------------------------------------------- per-wave state
  const int ht = wave % HT;                  // head tile of this wave
  const int dpart = wave / HT;               // value-column slice of this wave
  const int dv0 = dpart * S::kDvCols;
  const int head = hblock * S::kHeads + ht * 16 + hcol;
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

  float4_t oacc[S::kDvTiles];
#pragma unroll
  for (int j = 0; j < S::kDvTiles; ++j) oacc[j] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of this lane's head, log2 units
  float l_run = 0.f;        // running sum over the keys this lane holds

  // ---------------------------------------------------------------- 2. gather
  const int ntiles = (nvalid + kTileKeys - 1) / kTileKeys;
  const uint32_t stage_lds = lds_offset(s_stage);
  // Gather of tile j: wave w copies latent rows 16w .. 16w+15 (one row, 1 KB,
  // per instruction; lane L fetches logical granule L ^ (row & 15)) and rope
  // rows 16w .. 16w+15 (8 rows per instruction; lane L fetches rope granule
  // (L & 7) ^ ((row >> 1) & 7) of row 16w + 8t + L/8). Rows past the list
  // re-read a valid row; nothing reads them back.
  auto issue_tile = [&](int j) {
    const uint32_t base = stage_lds + (j & 1) * kTileBytes;
    uint32_t go[18];   // row offsets first: one LDS wait for the whole burst
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int key = j * kTileKeys + 16 * wave + u;
      go[u] = s_goff[key < nvalid ? key : 0];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = j * kTileKeys + 16 * wave + 8 * t + (lane >> 3);
      go[16 + t] = s_goff[key < nvalid ? key : 0];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int row = 16 * wave + u;
      const uint8_t* src = a.kv + ((uint64_t)go[u] + (uint32_t)(lane ^ u)) * 16ull;  // row & 15 == u
      dma_16b(src, __builtin_amdgcn_readfirstlane(base + row * 1024));
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = 16 * wave + 8 * t + (lane >> 3);
      const int g = (lane & 7) ^ ((row >> 1) & 7);
      const uint8_t* src = a.kv + ((uint64_t)go[16 + t] + 64u + (uint32_t)g) * 16ull;
      dma_16b(src, __builtin_amdgcn_readfirstlane(base + kRopeOff + (2 * wave + t) * 1024));
    }
  };

  // Per-lane LDS bases (inside a tile); every operand address is one of them
  // plus a compile-time offset.
  // S operand, dims 32c + 8kq .. +7 of row 16b + hcol. Latent (c < 16):
  // granule (4c + kq) ^ hcol = 4 * ((c & ~3) + ((c & 3) ^ (hcol >> 2))) + (kq ^ (hcol & 3)).
  int kbase[4];
#pragma unroll
  for (int cl = 0; cl < 4; ++cl)
    kbase[cl] = hcol * 1024 + 16 * (4 * (cl ^ (hcol >> 2)) + (kq ^ (hcol & 3)));
  // rope (c = 16, 17): granule (4(c-16) + kq) ^ ((hcol >> 1) & 7) of a 128 B row
  int rbase[2];
#pragma unroll
  for (int cr = 0; cr < 2; ++cr) rbase[cr] = kRopeOff + hcol * 128 + 16 * ((4 * cr + kq) ^ ((hcol >> 1) & 7));
  // V operand (transposed): row 32s2 + 16h + vr, columns dv0 + 16jt + 4(hcol & 3) .. +3,
  // i.e. granule dv0/8 + 2jt + ((hcol >> 1) & 1) at byte (hcol & 1) * 8; rows have
  // row & 15 == vr, so the stored granule is dv0/8 + 16(jt >> 3) + ((2(jt & 7) + gl) ^ vr).
  const int vr = 4 * kq + (hcol >> 2);
  int vbase[8];
#pragma unroll
  for (int jl = 0; jl < 8; ++jl)
    vbase[jl] = vr * 1024 + 16 * ((2 * jl + ((hcol >> 1) & 1)) ^ vr) + (hcol & 1) * 8 + 2 * dv0;

  if (ntiles > 0) issue_tile(0);
  for (int j = 0; j < ntiles; ++j) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < ntiles) issue_tile(j + 1);
    const uint8_t* tile = s_stage + (j & 1) * kTileBytes;

    // -------------------------------------------------------------- 3. S^T = K Q^T
    // 4 independent accumulators (16-key blocks b); operands for dim chunk c+2
    // are read while chunk c multiplies. The scheduling barriers keep the
    // compiler from hoisting all 72 reads (and 288 registers) to the top.
    float4_t sacc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) sacc[b] = (float4_t){0.f, 0.f, 0.f, 0.f};
    auto kread = [&](int c, int b) {
      const int off = c < 16 ? kbase[c & 3] + 64 * (c & ~3) + b * 16 * 1024 : rbase[c - 16] + b * 16 * 128;
      return *(const bf16x8_t*)(tile + off);
    };
    bf16x8_t kring[2][4];
#pragma unroll
    for (int b = 0; b < 4; ++b) kring[0][b] = kread(0, b);
#pragma unroll
    for (int c = 0; c < kDqk / 32; ++c) {
      if (c + 1 < kDqk / 32) {
#pragma unroll
        for (int b = 0; b < 4; ++b) kring[(c + 1) & 1][b] = kread(c + 1, b);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b)
        sacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kring[c & 1][b], qreg[c], sacc[b], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }

    // -------------------------------------------------------------- 4. online softmax
    // sacc[b][i] = score of key 64j + 16b + 4kq + i for head `head`
    float p[4][4];
    float mx = -INFINITY;
    const int kbase = j * kTileKeys + 4 * kq;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = kbase + 16 * b + i < nvalid;
        p[b][i] = ok ? sacc[b][i] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, p[b][i]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);   // finite: the tile holds a valid key
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[b][i] = fast_exp2(p[b][i] - m_new);
        psum += p[b][i];
      }
    }
    l_run = l_run * alpha + psum;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int jt = 0; jt < S::kDvTiles; ++jt) oacc[jt] *= alpha;
    }
    // P^T as the B operand of a 32-key step: slots 0-3 = block 2s, 4-7 = block 2s+1
    bf16x8_t pk[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      uint4 w;
      w.x = pack_bf16x2(p[2 * s2][0], p[2 * s2][1]);
      w.y = pack_bf16x2(p[2 * s2][2], p[2 * s2][3]);
      w.z = pack_bf16x2(p[2 * s2 + 1][0], p[2 * s2 + 1][1]);
      w.w = pack_bf16x2(p[2 * s2 + 1][2], p[2 * s2 + 1][3]);
      pk[s2] = __builtin_bit_cast(bf16x8_t, w);
    }

    // -------------------------------------------------------------- 5. O^T += V^T P^T
    // A operand of step s2 for value tile jt: column dv0 + 16jt + hcol of the
    // 4 rows 32s2 + 4kq .. +3 (slots 0-3) and of the 4 rows 16 further (4-7),
    // read transposed; operands for tile jt+2 are read while jt multiplies.
    auto vread = [&](int jt, int s2) {
      const uint8_t* p = tile + vbase[jt & 7] + 256 * (jt >> 3) + 32 * s2 * 1024;
      const short4_t lo = lds_read_tr16(p);               // rows 32s2 + vr: slots 0-3
      const short4_t hi = lds_read_tr16(p + 16 * 1024);   // rows 32s2 + 16 + vr: slots 4-7
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8_t vring[3][2];
#pragma unroll
    for (int jt = 0; jt < 2 && jt < S::kDvTiles; ++jt)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) vring[jt][s2] = vread(jt, s2);
#pragma unroll
    for (int jt = 0; jt < S::kDvTiles; ++jt) {
      if (jt + 2 < S::kDvTiles) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) vring[(jt + 2) % 3][s2] = vread(jt + 2, s2);
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        oacc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vring[jt % 3][s2], pk[s2], oacc[jt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---------------------------------------------------------------- 6. epilogue
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;

  if (head_ok) {
    if (a.splits == 1) {
      uint16_t* op = a.out + token * a.o_st + (int64_t)head * a.o_sh + dv0 + kq * 4;
#pragma unroll
      for (int jt = 0; jt < S::kDvTiles; ++jt) {
        const float4_t v = oacc[jt] * inv_l;   // O^T[dv0 + 16jt + 4kq + i][head]
        uint2 w;
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        *(uint2*)(op + 16 * jt) = w;
      }
      if (dpart == 0 && kq == 0)
        a.lse[token * a.lse_st + head] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
      const int64_t prow = (token * a.splits + split) * a.num_heads + head;
      float* pp = a.part_o + prow * kDv + dv0 + kq * 4;
#pragma unroll
      for (int jt = 0; jt < S::kDvTiles; ++jt) *(float4_t*)(pp + 16 * jt) = oacc[jt] * inv_l;
      if (dpart == 0 && kq == 0) {
        a.part_ml[prow * 2] = m_run;
        a.part_ml[prow * 2 + 1] = l_tot;
      }
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
    for (int s = 0; s < a.splits; ++s)
      W += ml[s * sstride] == -INFINITY ? 0.f : fast_exp2(ml[s * sstride] - M) * ml[s * sstride + 1];
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
