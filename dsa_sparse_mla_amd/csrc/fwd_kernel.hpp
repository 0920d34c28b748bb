// Device kernels of the DSA sparse MLA forward for gfx950 (MI355X).
//
// One workgroup of 4 waves handles one query token (or one segment of its
// index row when the row is split) for a block of up to 64 heads. Steps, all
// inside the kernel:
//   1. index stage: read the token's index segment, keep the entries that name
//      a KV row (for the paged cache: map logical position -> page -> row),
//      and compact their row offsets, in order, into an LDS list;
//   2. gather: stream the listed 576-wide bf16 rows, 32 keys per tile, from
//      HBM straight into LDS (global_load_lds_dwordx4, 16 B per lane) through
//      a four-stage ring: two tiles are in flight while two are in use;
//   3. S^T = K Q^T on bf16 MFMA (v_mfma_f32_16x16x32_bf16): 16 keys as M,
//      16 heads as N, Q held in registers as the B operand;
//   4. online softmax in fp32, base-2 domain (scale folded with log2 e),
//      with a lazily moved reference max;
//   5. O^T += V^T P^T on bf16 MFMA (v_mfma_f32_16x16x32_bf16, one 32-key
//      step per tile). The S^T accumulator layout is already the B-operand
//      layout of P^T, so P never leaves registers. V is the leading 512
//      columns of the same LDS rows, read transposed with ds_read_b64_tr_b16;
//   6. epilogue: normalise, write bf16 O and fp32 LSE -- or fp32 partials
//      that a second kernel merges when the row was split.
// Steps 3 and 5 are software-pipelined across tiles: the PV product of tile
// j and the QK^T product of tile j+1 are independent, so one instruction
// stream interleaves their MFMAs and LDS reads, and each hides the other's
// latency.
//
// Work split: the workgroup's heads form HT tiles of 16. With HT = 2, wave w
// computes S for head tile w % 2 over every key of the tile, and PV for that
// head tile over its own half of the 512 value columns: the two waves of a
// head tile repeat the S product instead of exchanging P. With HT = 1, wave
// w scores key block w & 1 of each tile (16 keys) and takes the PV product
// of those keys for value half w >> 1 on 16x16x16 MFMAs; the two waves of a
// value half keep separate softmax state and merge their partial outputs
// once, at the end. Either way no wave waits for another inside the key
// loop except at the tile barrier.
//
// LDS stage layout (32 keys, 36 KB): a latent region of 32 rows x 1 KB
// (dims 0..511, i.e. V) and a rope region of 32 rows x 128 B (dims 512..575).
// Granule G (16 B) of latent row r sits at position G ^ swz(r), with
// swz(r) = (r & 15) ^ ((r & 1) << 3), and granule G of rope row r at
// G ^ ((r >> 1) & 7). That spreads the 16 rows of an MFMA operand read over
// all 64 LDS banks in each 16-lane quarter, and the rows of a transposed V
// read over all banks in each 32-lane half, and it lets every per-lane LDS
// address be one of a few lane bases plus an immediate. Each gather
// instruction fills exactly one latent row, or 8 rope rows.
//
// Pages: "feat: add XTuner TileLang sparse MLA backend" (lmdeploy PR 4904),
// Summary and Performance > Isolated sparse MLA forward; "[Feature] Add
// optional FlashMLA backend for DSA Sparse MLA" (xtuner PR 2083), Runtime
// constraints.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dsa {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kTileKeys = 32;                         // keys per tile
constexpr int kStages = 4;                            // LDS ring depth
constexpr int kRopeOff = kTileKeys * 1024;            // rope region offset inside a stage
constexpr int kStageBytes = kTileKeys * 1152;         // 36864
constexpr int kWaves = 4;
constexpr int kDmaPerWave = kTileKeys / kWaves + 1;   // 8 latent rows + 8 rope rows = 9 copies
constexpr int kSegment = 2048;                        // index entries one workgroup compacts into LDS
constexpr int kChunks = kSegment / 64;
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kRescaleSlack = 8.f;                  // log2 units; p <= 256 between rescales

static_assert(kTileKeys == 8 * kWaves, "each wave copies 8 latent rows and 8 rope rows per tile");

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
  float scale_log2;        // sm_scale * log2(e), >= 0
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

// Latent-row swizzle (see the layout note above).
__host__ __device__ constexpr int swz(int r) { return (r & 15) ^ ((r & 1) << 3); }

// One wave-wide 16-byte-per-lane copy HBM -> LDS: lane L's 16 bytes from
// `src` land at LDS byte lds_base + 16 * L (lds_base is wave-uniform, in M0).
// Issued through asm so the compiler does not tie every later LDS read to it;
// completion is awaited explicitly with s_waitcnt vmcnt.
__device__ __forceinline__ void dma_16b(const void* src, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");  // M0 is reserved by the compiler and not otherwise used by these kernels
}

// The same copy with a wave-uniform 64-bit base (SGPRs) and a per-lane
// 32-bit byte offset.
__device__ __forceinline__ void dma_16b_sbase(uint64_t sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

// Wait until at most N of this wave's vector-memory operations (the gather
// copies) are still outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
// Two floats to bf16 (round to nearest even), lo in the low half: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){lo, hi}, bf16x2_t));
}

// Transposed read: with lane j of each 16-lane group pointing at 4 bf16 of
// row R + j/4, columns c + 4(j%4) .. +3, lane i of the group receives column
// c + i of rows R .. R+3.
__device__ __forceinline__ short4_t lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(
      (__attribute__((address_space(3))) uint8_t*)(p)));
}
// With one head tile (HT = 1) the waves split the keys as well as the value
// columns: wave w scores key block w & 1 of each tile (16 keys) and takes
// the PV product of those keys for value half w >> 1 (16x16x16 MFMAs), so
// each score is computed twice instead of four times; the two waves of a
// value half merge their partial outputs at the end.
template <int HT>
struct FwdShape {
  static constexpr int kHeads = 16 * HT;               // heads of the workgroup
  static constexpr int kKeyBlocks = HT == 1 ? 1 : 2;   // 16-key blocks of a tile per wave
  static constexpr int kDvParts = HT == 1 ? 2 : kWaves / HT;   // value slices of a head tile
  static constexpr int kDvCols = kDv / kDvParts;       // value columns of one wave
  static constexpr int kDvTiles = kDvCols / 16;        // 16-column MFMA tiles of one wave
  static constexpr int kSSteps = kKeyBlocks * (kDqk / 32);   // QK^T MFMAs per tile (blocks x 18 chunks)
  static_assert(kWaves % HT == 0, "head tiles must divide the waves");
};

// Index stage (step 1): keep the entries of this workgroup's segment that
// name a KV row, and compact their row offsets (in 16-byte granules), in
// order, into s_goff. The list is padded with offset 0 to a whole tile. All
// waves of the workgroup call this; it returns the number of valid entries.
// NW waves share the work (chunk c of wave w covers entries (c NW + w) * 64 ..).
// after_issue() runs once the index loads are issued and before their values
// are used: loads issued there overlap the index latency.
template <bool PAGED, int NW = kWaves, typename F>
__device__ __forceinline__ int build_key_list(const FwdArgs& a, int64_t token, int split, int wave, int lane,
                                              uint32_t* s_goff, int* s_cnt, F&& after_issue) {
  constexpr int kChunksPerWave = kChunks / NW;
  static_assert(kChunks % NW == 0, "chunks must divide over the waves");
  const int k0 = split * a.seg_len;
  const int n = min(a.topk - k0, a.seg_len);
  const int32_t* irow = a.idx + token * a.idx_st + k0;

  int32_t val[kChunksPerWave];
#pragma unroll
  for (int c = 0; c < kChunksPerWave; ++c) {
    const int e = (c * NW + wave) * 64 + lane;
    val[c] = e < n ? irow[e] : -1;
  }
  __builtin_amdgcn_sched_barrier(0);
  after_issue();
  __builtin_amdgcn_sched_barrier(0);
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
    s_cnt[lane * NW + wave] = cnt;
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
  const int nvalid = __builtin_amdgcn_readfirstlane(__shfl(incl, kChunks - 1));   // uniform: scalar loop bounds
#pragma unroll
  for (int c = 0; c < kChunksPerWave; ++c) {
    const int base = __shfl(incl - cnt, c * NW + wave);
    const uint64_t m = vmask[c];
    if ((m >> lane) & 1ull) s_goff[base + __popcll(m & ((1ull << lane) - 1ull))] = goff[c];
  }
  // Pad the list to a whole tile with offset 0 (the first row; it exists
  // whenever the list is not empty), so the gather needs no bounds check.
  if (wave == 0 && nvalid + lane < ((nvalid + kTileKeys - 1) & ~(kTileKeys - 1))) s_goff[nvalid + lane] = 0;
  __syncthreads();

  return nvalid;
}

// Gather (step 2) of tile j into LDS stage j % kStages: wave w copies latent
// rows 8w .. 8w+7 (one 1 KB row per instruction; lane i fetches logical
// granule i ^ swz(row)) and rope rows
// 8w .. 8w+7 (one instruction; lane i fetches rope granule
// (i & 7) ^ ((row >> 1) & 7) of row 8w + i/8): kDmaPerWave copies in all.
__device__ __forceinline__ void issue_tile(const FwdArgs& a, const uint32_t* s_goff, uint32_t stage_lds, int j,
                                           int wave, int lane) {
  const uint32_t base = stage_lds + (j % kStages) * kStageBytes;
  const uint4* gl = (const uint4*)(s_goff + j * kTileKeys + 8 * wave);
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
  const uint32_t gr = s_goff[j * kTileKeys + rrow];
  const uint32_t lane16 = (uint32_t)lane * 16u;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = 8 * wave + u;
    const uint64_t sb = (uint64_t)a.kv + (uint64_t)__builtin_amdgcn_readfirstlane(go[u]) * 16ull;
    dma_16b_sbase(sb, lane16 ^ (uint32_t)(swz(row) * 16), base + row * 1024);
  }
  const int g = (lane & 7) ^ ((rrow >> 1) & 7);
  dma_16b(a.kv + ((uint64_t)gr + 64u + (uint32_t)g) * 16ull, base + kRopeOff + wave * 1024);
}

// FP8 MLA cache rows (paged decode over an FP8 cache): 656 bytes per key,
// 512 float8 e4m3 latent values in 4 groups of 128, then 4 fp32 scales (one
// per group), then the 64 rope values in bf16. A tile is brought in by every
// wave for rows 8w .. 8w+7: lane i reads row 8w + i/8, latent granules
// (i & 7) + 8g of group g (16 codes each), the row's 4 scales and rope
// granule i & 7 -- six 16-byte loads into registers, two steps ahead.
constexpr int kFp8Scales = 512;   // byte offset of the scales in a row
constexpr int kFp8Rope = 528;     // byte offset of the rope values
struct Fp8Share {
  uint4 v[6];   // latent granules of groups 0..3, the scales, the rope granule
};

__device__ __forceinline__ void fp8_load(const FwdArgs& a, const uint32_t* s_goff, int t, int wave, int lane,
                                         Fp8Share& b) {
  const int r = 8 * wave + (lane >> 3);
  const uint8_t* row = a.kv + (uint64_t)s_goff[t * kTileKeys + r] * 16ull;
  const int g = lane & 7;
#pragma unroll
  for (int q = 0; q < 4; ++q) b.v[q] = *(const uint4*)(row + 16 * (g + 8 * q));
  b.v[4] = *(const uint4*)(row + kFp8Scales);
  b.v[5] = *(const uint4*)(row + kFp8Rope + 16 * g);
}

// Dequantise this wave's share of a tile into its LDS stage, in the layout
// the bf16 gather produces: e4m3 -> fp32 (v_cvt_pk_f32_fp8, exact), times
// the group's fp32 scale, rounded to bf16; the rope granule as it is.
__device__ __forceinline__ void fp8_store(uint8_t* stage, int wave, int lane, const Fp8Share& b) {
  const int r = 8 * wave + (lane >> 3);
  const int g = lane & 7;
  const float4_t sc = __builtin_bit_cast(float4_t, b.v[4]);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w[4] = {b.v[q].x, b.v[q].y, b.v[q].z, b.v[q].w};
    uint32_t o[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);   // codes 4k, 4k+1
      const float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);    // codes 4k+2, 4k+3
      o[2 * k] = pack_bf16x2(lo[0] * sc[q], lo[1] * sc[q]);
      o[2 * k + 1] = pack_bf16x2(hi[0] * sc[q], hi[1] * sc[q]);
    }
    const int G = 2 * (g + 8 * q);   // logical 16-byte granule of the first 8 values
    *(uint4*)(stage + r * 1024 + 16 * (G ^ swz(r))) = (uint4){o[0], o[1], o[2], o[3]};
    *(uint4*)(stage + r * 1024 + 16 * ((G + 1) ^ swz(r))) = (uint4){o[4], o[5], o[6], o[7]};
  }
  *(uint4*)(stage + kRopeOff + r * 128 + 16 * (g ^ ((r >> 1) & 7))) = b.v[5];
}

template <int HT, bool PAGED, bool FP8 = false>
__global__ void __launch_bounds__(256)
sparse_mla_fwd_kernel(const FwdArgs a) {
  using S = FwdShape<HT>;

  __shared__ __attribute__((aligned(1024))) uint8_t s_stage[kStages * kStageBytes];
  __shared__ __attribute__((aligned(16))) uint32_t s_goff[kSegment];
  __shared__ int s_cnt[kChunks];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: keep it scalar
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
  const int nvalid = build_key_list<PAGED>(a, token, split, wave, lane, s_goff, s_cnt, [] {});

  // ---------------------------------------------------------------- per-wave state
  constexpr int KBW = S::kKeyBlocks;
  const int ht = wave % HT;                  // head tile of this wave
  const int dpart = HT == 1 ? wave >> 1 : wave / HT;   // value-column slice of this wave
  const int kbw = HT == 1 ? wave & 1 : 0;    // first key block of this wave
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
    // gather of later tiles on every iteration.
#pragma unroll
    for (int c = 0; c < kDqk / 32; ++c) asm volatile("" ::"v"(qreg[c]));
  }

  float4_t oacc[S::kDvTiles];
#pragma unroll
  for (int j = 0; j < S::kDvTiles; ++j) {
    oacc[j] = (float4_t){0.f, 0.f, 0.f, 0.f};
    asm volatile("" : "+a"(oacc[j]));   // the accumulator lives in AGPRs throughout
  }
  float m_run = -INFINITY;  // reference max of this lane's head, log2 units
  float l_run = 0.f;        // running sum over the keys this lane holds

  // ---------------------------------------------------------------- 2. gather
  const int ntiles = (nvalid + kTileKeys - 1) / kTileKeys;
  const uint32_t stage_lds = lds_offset(s_stage);
  // Per-lane LDS bases (inside a stage); every operand address is one of them
  // plus a compile-time offset.
  // Key order inside a 16-key block: MFMA row i (lane i & 15 of the K
  // operand) is key kr = 4 sigma(i >> 2) + (i & 3), so S^T row 4q + e and P^T
  // slot e of k-group q hold key 4 sigma(q) + e. A ds_read_b128 serves in one
  // cycle the 16 lanes of a half-wave whose quad index (lane bits 2..4) has
  // one parity; with sigma = (1, 0, 2, 3) and swz those lanes hit 16 distinct
  // slots (with the identity, every latent K read is a 2-way conflict).
  const int ksig = 4 * ((0x3201 >> (4 * kq)) & 15);   // 4 sigma(kq): first key of this lane's k-group
  const int kr = 4 * ((0x3201 >> (4 * (hcol >> 2))) & 15) + (hcol & 3);
  // S operand, dims 32c + 8kq .. +7 of row 16b + kr. Latent (c < 16):
  // granule (4c + kq) ^ fh = 4 * ((c & ~3) + ((c & 3) ^ (fh >> 2))) + (kq ^ (fh & 3)),
  // fh = swz(kr) = swz(16b + kr).
  const int fh = swz(kr);
  int kbase[4];
#pragma unroll
  for (int cl = 0; cl < 4; ++cl)
    kbase[cl] = kr * 1024 + 16 * (4 * (cl ^ (fh >> 2)) + (kq ^ (fh & 3)));
  // rope (c = 16, 17): granule (4(c-16) + kq) ^ ((kr >> 1) & 7) of a 128 B row
  int rbase[2];
#pragma unroll
  for (int cr = 0; cr < 2; ++cr) rbase[cr] = kRopeOff + kr * 128 + 16 * ((4 * cr + kq) ^ ((kr >> 1) & 7));
  // V operand (transposed): rows vr (slots 0-3) and 16 + vr (slots 4-7),
  // columns dv0 + 16jt + 4(hcol & 3) .. +3, i.e. granule
  // dv0/8 + 2jt + ((hcol >> 1) & 1) at byte (hcol & 1) * 8; both rows have
  // swizzle swz(vr), so the stored granule is
  // dv0/8 + 16(jt >> 3) + ((2(jt & 7) + gl) ^ swz(vr)). The 16 lanes of
  // k-group kq read keys ksig .. ksig+3, the keys of their P^T slots.
  const int vr = ksig + (hcol >> 2);
  const int fv = swz(vr);
  int vbase[8];
#pragma unroll
  for (int jl = 0; jl < 8; ++jl)
    vbase[jl] = vr * 1024 + 16 * ((2 * jl + ((hcol >> 1) & 1)) ^ fv) + (hcol & 1) * 8 + 2 * dv0;

  auto kread = [&](const uint8_t* st, int c, int b) {
    const int off = c < 16 ? kbase[c & 3] + 64 * (c & ~3) + b * 16 * 1024 : rbase[c - 16] + b * 16 * 128;
    return *(const bf16x8_t*)(st + off);
  };
  // V^T operand of value tile jt: 8 keys (both blocks) for the 16x16x32
  // MFMA, or with one key block per wave 4 keys of block kbw (16x16x16)
  using VOp = std::conditional_t<KBW == 2, bf16x8_t, short4_t>;
  auto vread = [&](const uint8_t* st, int jt) -> VOp {
    const uint8_t* p = st + vbase[jt & 7] + 256 * (jt >> 3);
    if constexpr (KBW == 2) {
      const short4_t lo = lds_read_tr16(p);               // keys vr      (block 0): slots 0-3
      const short4_t hi = lds_read_tr16(p + 16 * 1024);   // keys 16 + vr (block 1): slots 4-7
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return lds_read_tr16(p + kbw * 16 * 1024);          // keys 16 kbw + vr
    }
  };

  // ---------------------------------------------------------------- 3-5. pipelined steps
  // One step runs, in one instruction stream:
  //   phase A: the 36 QK^T MFMAs of tile jn (into sacc), interleaved 2:1 with
  //            the first half of the PV MFMAs of the previous tile (operand
  //            pk_cur), plus the gather issue of a later tile;
  //   phase B: the rest of the PV MFMAs, each followed by one slice of the
  //            online softmax of tile jn (which needs only sacc), so the VALU
  //            work runs while the MFMA pipe is busy.
  // The softmax writes P^T of tile jn to pk_next; moving the reference max
  // only sets alpha, and the accumulator is rescaled after the step's last PV
  // MFMA (O of the previous tile must be complete first).
  float4_t sacc[KBW];
  VOp pk_cur = {}, pk_next = {};
  float sp[KBW][4];
  float smx = -INFINITY;
  float alpha = 1.f;

  // Slice k of the softmax of tile jn. sacc[b][i] = raw score q . k of key
  // 32jn + 16(kbw + b) + ksig + i for head `head`; the scale (>= 0, folded
  // with log2 e) is applied inside the exponent.
  auto soft_piece = [&](int k, int jn) {
    if (k == 0) {
#pragma unroll
      for (int b = 0; b < KBW; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) sp[b][i] = sacc[b][i];
      if ((jn + 1) * kTileKeys > nvalid) {   // the last tile: mask keys past the list
        const int kb = jn * kTileKeys + 16 * kbw + ksig;
#pragma unroll
        for (int b = 0; b < KBW; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kb + 16 * b + i >= nvalid) sp[b][i] = -INFINITY;
      }
      smx = -INFINITY;
#pragma unroll
      for (int b = 0; b < KBW; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) smx = fmaxf(smx, sp[b][i]);
    } else if (k == 1) {
      smx = fmaxf(smx, __shfl_xor(smx, 16));
    } else if (k == 2) {
      smx = fmaxf(smx, __shfl_xor(smx, 32)) * a.scale_log2;
      // Lazy rescaling: the reference max moves only when the tile max
      // exceeds it by more than kRescaleSlack (log2 units); until then
      // p = 2^(s - m_run) <= 2^kRescaleSlack. alpha = 1 unless it moves.
      // (a tile always holds a valid key, but with one key block per wave
      // the block may not: then smx = -inf and the reference stays)
      const float m_new = smx > m_run + kRescaleSlack ? fmaxf(m_run, smx) : m_run;
      alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
    } else if (k == 3 || (k == 4 && KBW == 2)) {
      const int b = k - 3;
#pragma unroll
      for (int i = 0; i < 4; ++i) sp[b][i] = fast_exp2(__builtin_fmaf(sp[b][i], a.scale_log2, -m_run));
      if ((jn + 1) * kTileKeys > nvalid) {   // last tile: a masked slot has weight 0 (also when the scale is 0)
        const int kb = jn * kTileKeys + ksig + 16 * (kbw + b);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb + i >= nvalid) sp[b][i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) l_run += sp[b][i];
    } else if (k == 5) {
      // P^T as the B operand of the tile's PV step: slots 0-3 = block 0, 4-7
      // = block 1 (32-key step), or the wave's block alone (16-key step)
      if constexpr (KBW == 2) {
        uint4 w;
        w.x = pack_bf16x2(sp[0][0], sp[0][1]);
        w.y = pack_bf16x2(sp[0][2], sp[0][3]);
        w.z = pack_bf16x2(sp[1][0], sp[1][1]);
        w.w = pack_bf16x2(sp[1][2], sp[1][3]);
        pk_next = __builtin_bit_cast(bf16x8_t, w);
      } else {
        const uint2 w = {pack_bf16x2(sp[0][0], sp[0][1]), pack_bf16x2(sp[0][2], sp[0][3])};
        pk_next = __builtin_bit_cast(short4_t, w);
      }
      // anchor the softmax here, beside the PV MFMAs (no sinking past the rescale)
      asm volatile("" : "+v"(pk_next), "+v"(l_run));
    }
  };

  // FP8: the share of the tile that a step dequantises (f8_cur) and the one
  // still in flight (f8_nxt); the caller alternates them
  Fp8Share f8a, f8b;
  // The step's gather: the bf16 path issues the copies of tile issue_j; the
  // FP8 path dequantises tile issue_j (loaded two steps ago) into its stage
  // and loads tile issue_j + 2 into the same registers.
  auto gather = [&](int issue_j, Fp8Share& f8) {
    if constexpr (FP8) {
      fp8_store(s_stage + (issue_j % kStages) * kStageBytes, wave, lane, f8);
      if (issue_j + 2 < ntiles) fp8_load(a, s_goff, issue_j + 2, wave, lane, f8);
    } else {
      issue_tile(a, s_goff, stage_lds, issue_j, wave, lane);
    }
  };
  auto step = [&](const uint8_t* st_s, bool do_s, int jn, const uint8_t* st_pv, bool do_pv, int issue_j,
                  Fp8Share& f8) {
    constexpr int kS = S::kSSteps;        // QK^T MFMAs: (chunk t / KBW, block kbw + t % KBW)
    constexpr int kP = S::kDvTiles;       // PV MFMAs: value tile u
    constexpr int kPA = kP / 2;           // PV MFMAs placed in phase A
    constexpr int kKA = 4, kVA = 3;       // read-ahead (<= 15 LDS operations in flight)
    constexpr int kPieces = 6;
    bf16x8_t kr[kKA + 1];
    VOp vrg[kVA + 1];
    if (do_pv) {
#pragma unroll
      for (int u = 0; u < kVA; ++u) vrg[u] = vread(st_pv, u);
    }
    auto pv_mfma = [&](int u) {
      if (u + kVA < kP) vrg[(u + kVA) % (kVA + 1)] = vread(st_pv, u + kVA);
      if constexpr (KBW == 2)
        oacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vrg[u % (kVA + 1)], pk_cur, oacc[u], 0, 0, 0);
      else
        oacc[u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vrg[u % (kVA + 1)], pk_cur, oacc[u], 0, 0, 0);
    };
    if (do_s) {
#pragma unroll
      for (int b = 0; b < KBW; ++b) sacc[b] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < kKA; ++t) kr[t] = kread(st_s, t / KBW, kbw + t % KBW);
      // phase A
#pragma unroll
      for (int t = 0; t < kS; ++t) {
        if (t + kKA < kS) kr[(t + kKA) % (kKA + 1)] = kread(st_s, (t + kKA) / KBW, kbw + (t + kKA) % KBW);
        sacc[t % KBW] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[t % (kKA + 1)], qreg[t / KBW], sacc[t % KBW], 0, 0, 0);
        if (t >= kS - KBW) asm volatile("" : "+v"(sacc[t % KBW]));   // scores in VGPRs: read by the softmax
        if (do_pv && (t & 1) && (t >> 1) < kPA) pv_mfma(t >> 1);
        if (t == 3 && issue_j >= 0) gather(issue_j, f8);
        __builtin_amdgcn_sched_barrier(0);
      }
      // phase B: remaining PV MFMAs with softmax slices (slot 0 left free so
      // the last QK^T MFMA can finish); slices go to slots 1 .. nB-1
      constexpr int kB = kP - kPA;
#pragma unroll
      for (int s2 = 0; s2 < kB; ++s2) {
        if (do_pv) pv_mfma(kPA + s2);
#pragma unroll
        for (int k = 0; k < kPieces; ++k)
          if (1 + k * (kB - 1) / kPieces == s2 || (kB == 1 && s2 == 0)) soft_piece(k, jn);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if (do_pv) {
#pragma unroll
      for (int u = 0; u < kP; ++u) {
        pv_mfma(u);
        if (u == 1 && issue_j >= 0) gather(issue_j, f8);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // keep the loop-carried accumulator in AGPRs (no copies between tiles)
#pragma unroll
    for (int jt = 0; jt < kP; ++jt) asm volatile("" : "+a"(oacc[jt]));
    if (do_s) {
      if (__ballot(alpha != 1.f)) {   // the reference moved: rescale O (rare)
#pragma unroll
        for (int jt = 0; jt < kP; ++jt) {
          // The accumulator lives in AGPRs (it is only ever an MFMA operand);
          // copy it to VGPRs here, scale, and put it back, so that the copies
          // stay inside this rarely taken branch.
          float4_t t = oacc[jt];
          asm volatile("" : "+v"(t));
          t *= alpha;
          asm volatile("" : "+a"(t));
          oacc[jt] = t;
        }
      }
      pk_cur = pk_next;
    }
  };

  auto stage_ptr = [&](int j) { return (const uint8_t*)s_stage + (j % kStages) * kStageBytes; };

  if (ntiles > 0 && !FP8) {
    // prologue: tiles 0..2 in flight, then QK^T and softmax of tile 0
    issue_tile(a, s_goff, stage_lds, 0, wave, lane);
    if (ntiles > 1) issue_tile(a, s_goff, stage_lds, 1, wave, lane);
    if (ntiles > 2) issue_tile(a, s_goff, stage_lds, 2, wave, lane);
    if (ntiles > 2) wait_vmem<2 * kDmaPerWave>();
    else if (ntiles > 1) wait_vmem<kDmaPerWave>();
    else wait_vmem<0>();
    __syncthreads();
    step(stage_ptr(0), true, 0, stage_ptr(0), false, -1, f8a);
    // steady state: PV of tile j with QK^T and softmax of tile j+1
    for (int j = 0; j + 1 < ntiles; ++j) {
      if (j + 2 < ntiles) wait_vmem<kDmaPerWave>();   // tile j+1 landed; tile j+2 may still fly
      else wait_vmem<0>();
      __syncthreads();   // ... in every wave; and tile j-1's stage is free for tile j+3
      step(stage_ptr(j + 1), true, j + 1, stage_ptr(j), true, j + 3 < ntiles ? j + 3 : -1, f8a);
    }
    // PV of the last tile
    step(stage_ptr(ntiles - 1), false, ntiles - 1, stage_ptr(ntiles - 1), true, -1, f8a);
  }
  if (ntiles > 0 && FP8) {
    // prologue: tiles 0 and 1 dequantised into their stages, tiles 2 and 3
    // in flight (tile t in f8a if t is even, f8b if odd)
    fp8_load(a, s_goff, 0, wave, lane, f8a);
    if (ntiles > 1) fp8_load(a, s_goff, 1, wave, lane, f8b);
    fp8_store(s_stage, wave, lane, f8a);
    if (ntiles > 2) fp8_load(a, s_goff, 2, wave, lane, f8a);
    if (ntiles > 1) fp8_store(s_stage + kStageBytes, wave, lane, f8b);
    if (ntiles > 3) fp8_load(a, s_goff, 3, wave, lane, f8b);
    __syncthreads();
    step(stage_ptr(0), true, 0, stage_ptr(0), false, -1, f8a);
    // steady state: PV of tile j, QK^T and softmax of tile j+1, tile j+2
    // dequantised into the stage tile j-2 left (its loads landed a step ago),
    // tile j+4 loaded; two steps per pass so each share stays in its registers
    int j = 0;
    while (j + 1 < ntiles) {
      __syncthreads();   // tile j+1 stored in every wave; tile j-2's stage is free
      step(stage_ptr(j + 1), true, j + 1, stage_ptr(j), true, j + 2 < ntiles ? j + 2 : -1, f8a);
      if (++j + 1 >= ntiles) break;
      __syncthreads();
      step(stage_ptr(j + 1), true, j + 1, stage_ptr(j), true, j + 2 < ntiles ? j + 2 : -1, f8b);
      ++j;
    }
    step(stage_ptr(ntiles - 1), false, ntiles - 1, stage_ptr(ntiles - 1), true, -1, f8a);
  }

  // ---------------------------------------------------------------- 6. epilogue
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  float m_fin = m_run;
  if constexpr (KBW == 1) {
    // The two waves of a value half merge: the wave of key block 1 hands its
    // unnormalised O, reference max and row sum to the wave of key block 0
    // through the stage memory, idle once every wave has left the loop.
    __syncthreads();
    float* xo = reinterpret_cast<float*>(s_stage) + dpart * (S::kDvTiles * 256 + 128);
    if (kbw == 1) {
#pragma unroll
      for (int jt = 0; jt < S::kDvTiles; ++jt) *(float4_t*)(xo + 4 * (jt * 64 + lane)) = oacc[jt];
      xo[S::kDvTiles * 256 + lane] = m_run;
      xo[S::kDvTiles * 256 + 64 + lane] = l_tot;
    }
    __syncthreads();
    if (kbw == 1) return;   // uniform per wave; no barrier follows
    const float m1 = xo[S::kDvTiles * 256 + lane], l1 = xo[S::kDvTiles * 256 + 64 + lane];
    const float M = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - M);   // a block with no key has weight 0
    const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - M);
#pragma unroll
    for (int jt = 0; jt < S::kDvTiles; ++jt) oacc[jt] = oacc[jt] * a0 + *(const float4_t*)(xo + 4 * (jt * 64 + lane)) * a1;
    l_tot = l_tot * a0 + l1 * a1;
    m_fin = M;
  }
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
        a.lse[token * a.lse_st + head] = l_tot > 0.f ? (m_fin + __log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
      const int64_t prow = (token * a.splits + split) * a.num_heads + head;
      float* pp = a.part_o + prow * kDv + dv0 + kq * 4;
#pragma unroll
      for (int jt = 0; jt < S::kDvTiles; ++jt) *(float4_t*)(pp + 16 * jt) = oacc[jt] * inv_l;
      if (dpart == 0 && kq == 0) {
        a.part_ml[prow * 2] = m_fin;
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
