// C ABI and launch layer of the DSA sparse MLA forward (gfx950 only).
//
// Every argument is checked on the host before any HIP call, so a bad call
// returns a status without touching the device. Then the layer picks the
// head-tile / key-group shape of the workgroup from the head count, picks the
// split of each index row, and enqueues the kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "dsa_sparse_mla.h"
#include "fwd_kernel.hpp"
#include "fwd_kernel_ws.hpp"
#include "bwd_kernel.hpp"
#include "bwd_dq_kernel.hpp"
#include "bwd_dkv_kernel.hpp"
#include "topk_kernel.hpp"

namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
  int cus = 0;
  bool gfx950 = false;
  bool ok = false;
};

DeviceInfo g_dev[kMaxDevices];
std::once_flag g_dev_once[kMaxDevices];

const DeviceInfo* device_info(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
    g_dev[dev].cus = prop.multiProcessorCount;
    g_dev[dev].gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev[dev].ok = true;
  });
  return g_dev[dev].ok ? &g_dev[dev] : nullptr;
}

int current_device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const DeviceInfo* d = device_info(dev);
  return d ? d->cus : 256;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Split choice. Each workgroup gathers at most kSegment entries. With few
// tokens and long rows, more workgroups per token fill the 256 CUs; short
// problems are not split (the merge pass would cost more than it saves).
// Head tiles of 16 per workgroup (HT) and workgroups per token along the heads.
int head_tiles(int32_t H) { return H <= 16 ? 1 : H <= 32 ? 2 : 4; }
int head_blocks(int32_t H) { return (H + 16 * head_tiles(H) - 1) / (16 * head_tiles(H)); }

// Splits of each index row: at least ceil(topk / 2048); for a large enough
// problem, doubled while the grid holds fewer than two workgroups per CU
// (one workgroup fills a CU, and a second hides its start-up and tail),
// while each split keeps at least 128 entries and the count stays <= 64.
int choose_splits(int64_t T, int32_t H, int32_t topk, int32_t requested, int cus) {
  const int smin = (topk + dsa::kSegment - 1) / dsa::kSegment;
  if (requested > 0) return requested;
  int s = smin;
  if (T * (int64_t)topk >= (int64_t)256 * 1024) {
    const int64_t per_split = T * head_blocks(H);
    while (per_split * s < 2LL * cus && (int64_t)s * 2 * 128 <= topk && s * 2 <= 64) s *= 2;
  }
  return s;
}

int check_splits(int64_t T, int32_t H, int32_t topk, int32_t requested, int* splits, int* seg_len,
                 int64_t* ws_bytes) {
  const int smin = (topk + dsa::kSegment - 1) / dsa::kSegment;
  if (requested < 0) return DSA_ERR_INVALID_ARGUMENT;
  if (requested > 0 && (requested < smin || requested > topk)) return DSA_ERR_INVALID_ARGUMENT;
  const int s = choose_splits(T, H, topk, requested, requested > 0 ? 256 : current_device_cus());
  const int seg = (topk + s - 1) / s;  // <= kSegment because s >= smin; a split may own no entry
  *splits = s;
  *seg_len = seg;
  *ws_bytes = s > 1 ? T * (int64_t)s * H * (int64_t)(dsa::kDv + 2) * 4 : 0;
  return DSA_OK;
}

int check_common(const void* q, int64_t q_st, int64_t q_sh, const int32_t* idx, int64_t idx_st,
                 int64_t T, int32_t H, int32_t topk, const void* out, int64_t o_st, int64_t o_sh,
                 const float* lse, int64_t lse_st) {
  if (T < 0) return DSA_ERR_INVALID_ARGUMENT;
  if (H < 1 || H > DSA_MAX_HEADS || topk < 1 || topk > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
  if (T == 0) return DSA_OK;
  if (!q || !idx || !out || !lse) return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(idx, 4) || !aligned(lse, 4))
    return DSA_ERR_INVALID_ARGUMENT;
  if (q_st < 0 || q_sh < 0 || o_st < 0 || o_sh < 0 || idx_st < 0 || lse_st < 0)
    return DSA_ERR_INVALID_ARGUMENT;
  if (q_st % 8 || q_sh % 8 || o_st % 8 || o_sh % 8) return DSA_ERR_INVALID_ARGUMENT;
  if (T > 1 && (q_st == 0 || o_st == 0 || idx_st < topk || lse_st < H)) return DSA_ERR_INVALID_ARGUMENT;
  if (H > 1 && (q_sh < DSA_DQK || o_sh < DSA_DV)) return DSA_ERR_INVALID_ARGUMENT;
  return DSA_OK;
}

// Byte ranges [lo, hi) of strided tensors, for the check that no output
// overlaps an input or another output. An empty tensor has lo == hi.
struct Extent {
  uintptr_t lo = 0, hi = 0;
};
// rows x cols elements of `bytes` each, rows `stride` elements apart
Extent extent2(const void* p, int64_t rows, int64_t stride, int64_t cols, int64_t bytes) {
  Extent e;
  if (!p || rows <= 0 || cols <= 0) return e;
  e.lo = reinterpret_cast<uintptr_t>(p);
  e.hi = e.lo + (uintptr_t)(((rows - 1) * stride + cols) * bytes);
  return e;
}
// [d0, d1, cols] with strides (s0, s1, 1)
Extent extent3(const void* p, int64_t d0, int64_t s0, int64_t d1, int64_t s1, int64_t cols, int64_t bytes) {
  Extent e;
  if (!p || d0 <= 0 || d1 <= 0 || cols <= 0) return e;
  e.lo = reinterpret_cast<uintptr_t>(p);
  e.hi = e.lo + (uintptr_t)(((d0 - 1) * s0 + (d1 - 1) * s1 + cols) * bytes);
  return e;
}
bool overlap(const Extent& a, const Extent& b) {
  return a.hi > a.lo && b.hi > b.lo && a.lo < b.hi && b.lo < a.hi;
}
// DSA_ERR_INVALID_ARGUMENT if an output overlaps an input or another output
int check_overlaps(std::initializer_list<Extent> outs, std::initializer_list<Extent> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    for (const Extent& i : ins)
      if (overlap(*o, i)) return DSA_ERR_INVALID_ARGUMENT;
    for (auto o2 = o + 1; o2 != outs.end(); ++o2)
      if (overlap(*o, *o2)) return DSA_ERR_INVALID_ARGUMENT;
  }
  return DSA_OK;
}

int device_check() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DSA_ERR_HIP;
  const DeviceInfo* d = device_info(dev);
  if (!d) return DSA_ERR_HIP;
  return d->gfx950 ? DSA_OK : DSA_ERR_UNSUPPORTED;
}

// Scratch of dsa_sparse_mla_fwd_paged_noalloc: the split partials live in
// this file-scope device array instead of a caller workspace. Each device
// holds its own copy at its own address; host code uses only the address
// that hipGetSymbolAddress returns for the current device (the array's name
// on the host is a stand-in, not a device pointer).
static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

void* g_scratch_ptr[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// The device address of `scratch` on device `dev` (which must be current),
// looked up once per device; nullptr if the lookup failed.
void* scratch_address(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[dev] = ptr;
    else (void)hipGetLastError();
  });
  return g_scratch_ptr[dev];
}

// Backward schedule and workspace, from the sizes alone.
//
// kv-major when the rows are dense enough: per (token, 64 kv rows) it adds
// H x 576 to dq where the token-major kernel adds 576 per named row, and its
// steps carry every column. The shapes stand in for the density: topk at
// least 3/256 of H x num_kv, i.e. uniform rows name 0.75 H or more of every
// 64 rows. Measured: 2.9x faster on 8192-token causal rows at 8 heads, 1.5x
// at 16, 4.7x on packed documents at 8 heads. Its workspace holds the
// per-token occupancy masks ([word][token] u32), the per-token repeat flags
// and D = dout . out per (token, head); above 1 GiB of it the token-major
// kernel runs instead. The split schedule (more than 16 heads, num_kv at most
// 16 topk) keeps the masks and flags (its dq pass forms D itself) and adds
// the prepass's ranks (per 256-row block and per index entry), the dq pass's
// P and s*dS, 128 bytes per (token, entry, 32-head group): topk x H x 4
// bytes per token, and the dkv pass's 8 work-queue counters. Above 64 GiB of
// it the token-major kernel runs instead.
struct BwdPlan {
  int schedule = DSA_BWD_TOKEN_MAJOR;
  int64_t words = 0, chunks = 0, blk = 0, groups = 0;
  int64_t dup_off = 0, d_off = 0, pre_off = 0, rank_off = 0, pds_off = 0;
  int64_t ws_bytes = 0;
};

void bwd_plan(int64_t T, int32_t H, int64_t N, int32_t topk, BwdPlan* p) {
  *p = BwdPlan();
  if (T <= 0 || N <= 0) return;
  const int64_t words = (N + 31) / 32;
  const bool wide = H > 16;
  const int64_t chunk = wide ? dsa::kDkChunk : dsa::kKvChunk;
  const int64_t chunks = (T + chunk - 1) / chunk;
  const int64_t blk = (words + 7) / 8, groups = (H + 31) / 32;   // split: 256-row blocks
  const int64_t mask_bytes = words * T * 4;
  const int64_t dup_off = round_up(mask_bytes, 256);
  const int64_t d_off = dup_off + round_up(T * 4, 256);
  int64_t bytes = d_off + (wide ? 0 : T * 16 * 4);   // D: kv-major only (the split dq pass forms it)
  int64_t pre_off = 0, rank_off = 0, pds_off = 0;
  if (wide) {
    pre_off = round_up(bytes, 256);
    rank_off = pre_off + round_up(blk * T * 4, 256);
    pds_off = rank_off + round_up(T * topk * 4, 256);
    bytes = pds_off + round_up(T * groups * topk * dsa::kDkEnt, 256) + 256;   // then the 8 queue counters
  }
  // kv-major (H <= 16) and split (H > 16) need rows that name a large share
  // of the kv rows; both keep the prepass bitmap in LDS and the grid in 31 bits
  const bool dense = wide ? N <= 16 * (int64_t)topk : 3 * N * H <= 256 * (int64_t)topk;
  const int64_t wgs = wide ? 2 * blk * chunks : (words + 1) / 2 * chunks;
  const bool fits = words <= dsa::kKvMaxWords && bytes <= ((int64_t)1 << (wide ? 36 : 30)) &&
                    wgs < ((int64_t)1 << 31);
  if (!dense || !fits) return;
  p->schedule = wide ? DSA_BWD_SPLIT : DSA_BWD_KV_MAJOR;
  p->words = words;
  p->chunks = chunks;
  p->blk = blk;
  p->groups = groups;
  p->dup_off = dup_off;
  p->d_off = d_off;
  p->pre_off = pre_off;
  p->rank_off = rank_off;
  p->pds_off = pds_off;
  p->ws_bytes = bytes;
}

// Heads per workgroup: 16, 32 or 64 (HT head tiles of 16); more heads use
// several workgroups per token, one per block of 64. FP8 (paged FP8 cache):
// blocks of up to 32 heads only.
template <bool PAGED, bool FP8 = false>
int launch(dsa::FwdArgs& args, hipStream_t stream) {
  const int H = args.num_heads;
  const int ht = head_tiles(H);
  args.head_blocks = head_blocks(H);
  const dim3 grid((unsigned)(args.num_tokens * args.splits * args.head_blocks));
  const dim3 block(64 * dsa::kWaves);
  if (ht == 1) {
    hipLaunchKernelGGL((dsa::sparse_mla_fwd_kernel<1, PAGED, FP8>), grid, block, 0, stream, args);
  } else if (ht == 2) {
    hipLaunchKernelGGL((dsa::sparse_mla_fwd_kernel<2, PAGED, FP8>), grid, block, 0, stream, args);
  } else if (FP8) {
    return DSA_ERR_UNSUPPORTED;
  } else {
    hipLaunchKernelGGL((dsa::sparse_mla_fwd_ws_kernel<PAGED>), grid, dim3(64 * dsa::kWsWaves), 0, stream, args);
  }
  if (hipGetLastError() != hipSuccess) return DSA_ERR_HIP;
  if (args.splits > 1) {
    const int64_t pairs = args.num_tokens * (int64_t)H;
    hipLaunchKernelGGL(dsa::sparse_mla_combine_kernel, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0,
                       stream, args);
    if (hipGetLastError() != hipSuccess) return DSA_ERR_HIP;
  }
  return DSA_OK;
}

int fill_outputs_and_splits(dsa::FwdArgs& a, const void* q, int64_t q_st, int64_t q_sh,
                            const int32_t* idx, int64_t idx_st, int64_t T, int32_t H, int32_t topk,
                            float sm_scale, void* out, int64_t o_st, int64_t o_sh, float* lse,
                            int64_t lse_st, int32_t num_splits, void* ws, int64_t ws_bytes) {
  if (!std::isfinite(sm_scale) || sm_scale < 0.f) return DSA_ERR_INVALID_ARGUMENT;
  int splits = 1, seg = topk;
  int64_t need = 0;
  int st = check_splits(T, H, topk, num_splits, &splits, &seg, &need);
  if (st != DSA_OK) return st;
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 16))) return DSA_ERR_WORKSPACE;
  a.q = static_cast<const uint16_t*>(q);
  a.q_st = q_st;
  a.q_sh = q_sh;
  a.idx = idx;
  a.idx_st = idx_st;
  a.num_tokens = T;
  a.num_heads = H;
  a.topk = topk;
  a.scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  a.out = static_cast<uint16_t*>(out);
  a.o_st = o_st;
  a.o_sh = o_sh;
  a.lse = lse;
  a.lse_st = lse_st;
  a.splits = splits;
  a.seg_len = seg;
  if (splits > 1) {
    a.part_o = static_cast<float*>(ws);
    a.part_ml = a.part_o + T * (int64_t)splits * H * dsa::kDv;
  }
  return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_sparse_mla_workspace_size(int64_t num_tokens, int32_t num_heads, int32_t topk,
                                  int32_t num_splits, int32_t* splits_out, int64_t* bytes_out) {
  if (!bytes_out) return DSA_ERR_INVALID_ARGUMENT;
  if (num_tokens < 0) return DSA_ERR_INVALID_ARGUMENT;
  if (num_heads < 1 || num_heads > DSA_MAX_HEADS || topk < 1 || topk > DSA_MAX_TOPK)
    return DSA_ERR_UNSUPPORTED;
  int splits = 1, seg = topk;
  int64_t need = 0;
  int st = check_splits(num_tokens, num_heads, topk, num_splits, &splits, &seg, &need);
  if (st != DSA_OK) return st;
  if (splits_out) *splits_out = splits;
  *bytes_out = need;
  return DSA_OK;
}

int dsa_sparse_mla_fwd(const void* q, int64_t q_stride_tok, int64_t q_stride_head, const void* kv,
                       int64_t kv_stride_row, int64_t num_kv, const int32_t* indices,
                       int64_t idx_stride_tok, int64_t num_tokens, int32_t num_heads, int32_t topk,
                       float sm_scale, void* out, int64_t out_stride_tok, int64_t out_stride_head,
                       float* lse, int64_t lse_stride_tok, int32_t num_splits, void* workspace,
                       int64_t workspace_bytes, void* stream) {
  int st = check_common(q, q_stride_tok, q_stride_head, indices, idx_stride_tok, num_tokens, num_heads,
                        topk, out, out_stride_tok, out_stride_head, lse, lse_stride_tok);
  if (st != DSA_OK || num_tokens == 0) return st;
  if (num_kv < 0) return DSA_ERR_INVALID_ARGUMENT;
  if (num_kv > 0) {
    if (!kv || !aligned(kv, 16) || kv_stride_row % 8 || kv_stride_row < (num_kv > 1 ? DSA_DQK : 0))
      return DSA_ERR_INVALID_ARGUMENT;
    // row offsets are kept as 32-bit counts of 16-byte granules
    const int64_t gran = kv_stride_row / 8;
    if (num_kv > ((int64_t)1 << 32) / (gran > 0 ? gran : 1) - 1) return DSA_ERR_UNSUPPORTED;
  }
  dsa::FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  st = fill_outputs_and_splits(a, q, q_stride_tok, q_stride_head, indices, idx_stride_tok, num_tokens,
                               num_heads, topk, sm_scale, out, out_stride_tok, out_stride_head, lse,
                               lse_stride_tok, num_splits, workspace, workspace_bytes);
  if (st != DSA_OK) return st;
  a.kv = static_cast<const uint8_t*>(kv);
  a.kv_row_gran = kv_stride_row / 8;
  a.num_kv = num_kv;
  {
    int64_t ws_need = 0;
    int sp = 0, sl = 0;
    check_splits(num_tokens, num_heads, topk, num_splits, &sp, &sl, &ws_need);
    st = check_overlaps(
        {extent3(out, num_tokens, out_stride_tok, num_heads, out_stride_head, DSA_DV, 2),
         extent2(lse, num_tokens, lse_stride_tok, num_heads, 4), extent2(ws_need > 0 ? workspace : nullptr, 1, 0, ws_need, 1)},
        {extent3(q, num_tokens, q_stride_tok, num_heads, q_stride_head, DSA_DQK, 2),
         extent2(kv, num_kv, kv_stride_row, DSA_DQK, 2), extent2(indices, num_tokens, idx_stride_tok, topk, 4)});
    if (st != DSA_OK) return st;
  }
  st = device_check();
  if (st != DSA_OK) return st;
  return launch<false>(a, static_cast<hipStream_t>(stream));
}

int dsa_sparse_mla_fwd_paged(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                             const void* kv_pages, int64_t kv_stride_page, int64_t kv_stride_row,
                             int64_t num_pages, int32_t page_size, const int32_t* page_table,
                             int64_t page_table_stride, int32_t max_pages_per_seq,
                             const int32_t* seq_lens, const int32_t* indices, int64_t idx_stride_tok,
                             int32_t num_seqs, int32_t q_per_seq, int32_t num_heads, int32_t topk,
                             float sm_scale, void* out, int64_t out_stride_tok, int64_t out_stride_head,
                             float* lse, int64_t lse_stride_tok, int32_t num_splits, void* workspace,
                             int64_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || q_per_seq < 1) return DSA_ERR_INVALID_ARGUMENT;
  const int64_t T = (int64_t)num_seqs * q_per_seq;
  int st = check_common(q, q_stride_tok, q_stride_head, indices, idx_stride_tok, T, num_heads, topk, out,
                        out_stride_tok, out_stride_head, lse, lse_stride_tok);
  if (st != DSA_OK || T == 0) return st;
  if (page_size < 1 || page_size > 4096 || (page_size & (page_size - 1))) return DSA_ERR_UNSUPPORTED;
  if (num_pages < 0 || max_pages_per_seq < 0 || page_table_stride < 0) return DSA_ERR_INVALID_ARGUMENT;
  if (!seq_lens || !aligned(seq_lens, 4)) return DSA_ERR_INVALID_ARGUMENT;
  if (max_pages_per_seq > 0 && (!page_table || !aligned(page_table, 4))) return DSA_ERR_INVALID_ARGUMENT;
  if (num_seqs > 1 && max_pages_per_seq > 0 && page_table_stride < max_pages_per_seq)
    return DSA_ERR_INVALID_ARGUMENT;
  if (num_pages > 0) {
    if (!kv_pages || !aligned(kv_pages, 16) || kv_stride_row % 8 || kv_stride_page % 8)
      return DSA_ERR_INVALID_ARGUMENT;
    if ((page_size > 1 && kv_stride_row < DSA_DQK) ||
        (num_pages > 1 && kv_stride_page < (int64_t)page_size * kv_stride_row))
      return DSA_ERR_INVALID_ARGUMENT;
    const int64_t page_gran = kv_stride_page / 8;
    const int64_t span = (num_pages - 1) * page_gran + (int64_t)page_size * (kv_stride_row / 8);
    if (span >= ((int64_t)1 << 32)) return DSA_ERR_UNSUPPORTED;
  }
  dsa::FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  st = fill_outputs_and_splits(a, q, q_stride_tok, q_stride_head, indices, idx_stride_tok, T, num_heads,
                               topk, sm_scale, out, out_stride_tok, out_stride_head, lse, lse_stride_tok,
                               num_splits, workspace, workspace_bytes);
  if (st != DSA_OK) return st;
  a.kv = static_cast<const uint8_t*>(kv_pages);
  a.kv_row_gran = kv_stride_row / 8;
  a.kv_page_gran = kv_stride_page / 8;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  a.page_shift = shift;
  a.page_mask = page_size - 1;
  a.page_table = page_table;
  a.pt_stride = page_table_stride;
  a.max_pages = max_pages_per_seq;
  a.seq_lens = seq_lens;
  a.q_per_seq = q_per_seq;
  a.num_pages = num_pages;
  {
    int64_t ws_need = 0;
    int sp = 0, sl = 0;
    check_splits(T, num_heads, topk, num_splits, &sp, &sl, &ws_need);
    st = check_overlaps(
        {extent3(out, T, out_stride_tok, num_heads, out_stride_head, DSA_DV, 2),
         extent2(lse, T, lse_stride_tok, num_heads, 4), extent2(ws_need > 0 ? workspace : nullptr, 1, 0, ws_need, 1)},
        {extent3(q, T, q_stride_tok, num_heads, q_stride_head, DSA_DQK, 2),
         extent3(kv_pages, num_pages, kv_stride_page, page_size, kv_stride_row, DSA_DQK, 2),
         extent2(indices, T, idx_stride_tok, topk, 4),
         extent2(page_table, num_seqs, page_table_stride, max_pages_per_seq, 4),
         extent2(seq_lens, 1, 0, num_seqs, 4)});
    if (st != DSA_OK) return st;
  }
  st = device_check();
  if (st != DSA_OK) return st;
  return launch<true>(a, static_cast<hipStream_t>(stream));
}

int dsa_sparse_mla_fwd_paged_fp8(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                                 const void* kv_pages, int64_t kv_stride_page_bytes, int64_t kv_stride_row_bytes,
                                 int64_t num_pages, int32_t page_size, const int32_t* page_table,
                                 int64_t page_table_stride, int32_t max_pages_per_seq, const int32_t* seq_lens,
                                 const int32_t* indices, int64_t idx_stride_tok, int32_t num_seqs,
                                 int32_t q_per_seq, int32_t num_heads, int32_t topk, float sm_scale, void* out,
                                 int64_t out_stride_tok, int64_t out_stride_head, float* lse,
                                 int64_t lse_stride_tok, int32_t num_splits, void* workspace,
                                 int64_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || q_per_seq < 1) return DSA_ERR_INVALID_ARGUMENT;
  const int64_t T = (int64_t)num_seqs * q_per_seq;
  int st = check_common(q, q_stride_tok, q_stride_head, indices, idx_stride_tok, T, num_heads, topk, out,
                        out_stride_tok, out_stride_head, lse, lse_stride_tok);
  if (st != DSA_OK || T == 0) return st;
  if (num_heads > 32) return DSA_ERR_UNSUPPORTED;   // the FP8 path runs blocks of up to 32 heads
  if (page_size < 1 || page_size > 4096 || (page_size & (page_size - 1))) return DSA_ERR_UNSUPPORTED;
  if (num_pages < 0 || max_pages_per_seq < 0 || page_table_stride < 0) return DSA_ERR_INVALID_ARGUMENT;
  if (!seq_lens || !aligned(seq_lens, 4)) return DSA_ERR_INVALID_ARGUMENT;
  if (max_pages_per_seq > 0 && (!page_table || !aligned(page_table, 4))) return DSA_ERR_INVALID_ARGUMENT;
  if (num_seqs > 1 && max_pages_per_seq > 0 && page_table_stride < max_pages_per_seq)
    return DSA_ERR_INVALID_ARGUMENT;
  if (num_pages > 0) {
    if (!kv_pages || !aligned(kv_pages, 16) || kv_stride_row_bytes % 16 || kv_stride_page_bytes % 16)
      return DSA_ERR_INVALID_ARGUMENT;
    if ((page_size > 1 && kv_stride_row_bytes < DSA_FP8_ROW_BYTES) ||
        (num_pages > 1 && kv_stride_page_bytes < (int64_t)page_size * kv_stride_row_bytes))
      return DSA_ERR_INVALID_ARGUMENT;
    const int64_t span = (num_pages - 1) * (kv_stride_page_bytes / 16) + (int64_t)page_size * (kv_stride_row_bytes / 16);
    if (span >= ((int64_t)1 << 32)) return DSA_ERR_UNSUPPORTED;
  }
  dsa::FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  st = fill_outputs_and_splits(a, q, q_stride_tok, q_stride_head, indices, idx_stride_tok, T, num_heads, topk,
                               sm_scale, out, out_stride_tok, out_stride_head, lse, lse_stride_tok, num_splits,
                               workspace, workspace_bytes);
  if (st != DSA_OK) return st;
  a.kv = static_cast<const uint8_t*>(kv_pages);
  a.kv_row_gran = kv_stride_row_bytes / 16;
  a.kv_page_gran = kv_stride_page_bytes / 16;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  a.page_shift = shift;
  a.page_mask = page_size - 1;
  a.page_table = page_table;
  a.pt_stride = page_table_stride;
  a.max_pages = max_pages_per_seq;
  a.seq_lens = seq_lens;
  a.q_per_seq = q_per_seq;
  a.num_pages = num_pages;
  {
    int64_t ws_need = 0;
    int sp = 0, sl = 0;
    check_splits(T, num_heads, topk, num_splits, &sp, &sl, &ws_need);
    const int64_t rows = num_pages > 0 ? ((num_pages - 1) * kv_stride_page_bytes + (int64_t)page_size * kv_stride_row_bytes) : 0;
    st = check_overlaps(
        {extent3(out, T, out_stride_tok, num_heads, out_stride_head, DSA_DV, 2),
         extent2(lse, T, lse_stride_tok, num_heads, 4), extent2(ws_need > 0 ? workspace : nullptr, 1, 0, ws_need, 1)},
        {extent3(q, T, q_stride_tok, num_heads, q_stride_head, DSA_DQK, 2), extent2(kv_pages, 1, 0, rows, 1),
         extent2(indices, T, idx_stride_tok, topk, 4),
         extent2(page_table, num_seqs, page_table_stride, max_pages_per_seq, 4),
         extent2(seq_lens, 1, 0, num_seqs, 4)});
    if (st != DSA_OK) return st;
  }
  st = device_check();
  if (st != DSA_OK) return st;
  return launch<true, true>(a, static_cast<hipStream_t>(stream));
}

int dsa_sparse_mla_fwd_paged_noalloc(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                                     const void* kv_pages, int64_t kv_stride_page, int64_t kv_stride_row,
                                     int64_t num_pages, int32_t page_size, const int32_t* page_table,
                                     int64_t page_table_stride, int32_t max_pages_per_seq,
                                     const int32_t* seq_lens, const int32_t* indices, int64_t idx_stride_tok,
                                     int32_t num_seqs, int32_t q_per_seq, int32_t num_heads, int32_t topk,
                                     float sm_scale, void* out, int64_t out_stride_tok,
                                     int64_t out_stride_head, float* lse, int64_t lse_stride_tok,
                                     int32_t num_splits, void* stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DSA_ERR_HIP;
  void* ws = scratch_address(dev);
  if (!ws) return DSA_ERR_HIP;
  // the paged entry point validates everything and returns DSA_ERR_WORKSPACE
  // when the split partials of this call would not fit the array
  return dsa_sparse_mla_fwd_paged(q, q_stride_tok, q_stride_head, kv_pages, kv_stride_page, kv_stride_row,
                                  num_pages, page_size, page_table, page_table_stride, max_pages_per_seq,
                                  seq_lens, indices, idx_stride_tok, num_seqs, q_per_seq, num_heads, topk,
                                  sm_scale, out, out_stride_tok, out_stride_head, lse, lse_stride_tok,
                                  num_splits, ws, DSA_NOALLOC_SCRATCH_BYTES, stream);
}

int dsa_sparse_mla_bwd(const void* q, int64_t q_stride_tok, int64_t q_stride_head, const void* kv,
                       int64_t kv_stride_row, int64_t num_kv, const int32_t* indices,
                       int64_t idx_stride_tok, int64_t num_tokens, int32_t num_heads, int32_t topk,
                       float sm_scale, const void* out, int64_t out_stride_tok, int64_t out_stride_head,
                       const float* lse, int64_t lse_stride_tok, const void* dout, int64_t dout_stride_tok,
                       int64_t dout_stride_head, float* dq, int64_t dq_stride_tok, int64_t dq_stride_head,
                       float* dkv, int64_t dkv_stride_row, void* workspace, int64_t workspace_bytes,
                       void* stream) {
  // q/out/lse checks are those of the forward (out and dout share its layout rules)
  int st = check_common(q, q_stride_tok, q_stride_head, indices, idx_stride_tok, num_tokens, num_heads, topk,
                        out, out_stride_tok, out_stride_head, lse, lse_stride_tok);
  if (st != DSA_OK) return st;
  if (!std::isfinite(sm_scale) || sm_scale < 0.f) return DSA_ERR_INVALID_ARGUMENT;
  if (num_kv < 0) return DSA_ERR_INVALID_ARGUMENT;
  if (num_kv > 0) {
    if (!kv || !aligned(kv, 16) || kv_stride_row % 8 || kv_stride_row < (num_kv > 1 ? DSA_DQK : 0))
      return DSA_ERR_INVALID_ARGUMENT;
    if (!dkv || !aligned(dkv, 16) || dkv_stride_row % 4 || dkv_stride_row < DSA_DQK)
      return DSA_ERR_INVALID_ARGUMENT;
    if (num_kv > ((int64_t)1 << 32) - 1) return DSA_ERR_UNSUPPORTED;   // row ids are 32-bit
  }
  if (num_tokens > 0) {
    if (!dout || !dq || !aligned(dout, 16) || !aligned(dq, 4)) return DSA_ERR_INVALID_ARGUMENT;
    if (dout_stride_tok < 0 || dout_stride_head < 0 || dout_stride_tok % 8 || dout_stride_head % 8)
      return DSA_ERR_INVALID_ARGUMENT;
    if (dq_stride_tok < 0 || dq_stride_head < 0) return DSA_ERR_INVALID_ARGUMENT;
    if (num_tokens > 1 && (dout_stride_tok == 0 || dq_stride_tok == 0)) return DSA_ERR_INVALID_ARGUMENT;
    if (num_heads > 1 && (dout_stride_head < DSA_DV || dq_stride_head < DSA_DQK)) return DSA_ERR_INVALID_ARGUMENT;
  }
  if (workspace_bytes < 0) return DSA_ERR_INVALID_ARGUMENT;
  BwdPlan plan;
  bwd_plan(num_tokens, num_heads, num_kv, topk, &plan);
  const int64_t ws_used = plan.ws_bytes;
  st = check_overlaps(
      {extent3(dq, num_tokens, dq_stride_tok, num_heads, dq_stride_head, DSA_DQK, 4),
       extent2(dkv, num_kv, dkv_stride_row, DSA_DQK, 4),
       extent2(ws_used > 0 ? workspace : nullptr, 1, 0, ws_used, 1)},
      {extent3(q, num_tokens, q_stride_tok, num_heads, q_stride_head, DSA_DQK, 2),
       extent2(kv, num_kv, kv_stride_row, DSA_DQK, 2), extent2(indices, num_tokens, idx_stride_tok, topk, 4),
       extent3(out, num_tokens, out_stride_tok, num_heads, out_stride_head, DSA_DV, 2),
       extent2(lse, num_tokens, lse_stride_tok, num_heads, 4),
       extent3(dout, num_tokens, dout_stride_tok, num_heads, dout_stride_head, DSA_DV, 2)});
  if (st != DSA_OK) return st;
  // checked before anything is enqueued: a call that fails launches nothing
  if (ws_used > 0 && (!workspace || workspace_bytes < ws_used || !aligned(workspace, 256)))
    return DSA_ERR_WORKSPACE;
  st = device_check();
  if (st != DSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (num_kv > 0) {
    const int64_t n4 = num_kv * (DSA_DQK / 4);
    hipLaunchKernelGGL(dsa::dkv_zero_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, dkv, num_kv,
                       dkv_stride_row);
    if (hipGetLastError() != hipSuccess) return DSA_ERR_HIP;
  }
  if (num_tokens == 0) return DSA_OK;
  dsa::BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(q);
  a.q_st = q_stride_tok;
  a.q_sh = q_stride_head;
  a.kv = static_cast<const uint16_t*>(kv);
  a.kv_st = kv_stride_row;
  a.num_kv = num_kv;
  a.idx = indices;
  a.idx_st = idx_stride_tok;
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.topk = topk;
  a.scale = sm_scale;
  a.scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  a.out = static_cast<const uint16_t*>(out);
  a.o_st = out_stride_tok;
  a.o_sh = out_stride_head;
  a.lse = lse;
  a.lse_st = lse_stride_tok;
  a.dout = static_cast<const uint16_t*>(dout);
  a.do_st = dout_stride_tok;
  a.do_sh = dout_stride_head;
  a.dq = dq;
  a.dq_st = dq_stride_tok;
  a.dq_sh = dq_stride_head;
  a.dkv = dkv;
  a.dkv_st = dkv_stride_row;
  // 16 heads per workgroup up to 16 heads, else 32 (each kv row's gradient is
  // then added once per 32 heads)
  const int hb = num_heads <= 16 ? 16 : 32;
  a.head_blocks = (num_heads + hb - 1) / hb;
  const int64_t wgs = num_tokens * a.head_blocks;
  if (wgs >= ((int64_t)1 << 31)) return DSA_ERR_UNSUPPORTED;

  if (plan.schedule != DSA_BWD_TOKEN_MAJOR) {
    const bool split = plan.schedule == DSA_BWD_SPLIT;
    dsa::KvMajorArgs m;
    m.mask = static_cast<uint32_t*>(workspace);
    m.dup = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + plan.dup_off);
    m.dbuf = split ? nullptr : reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.d_off);
    m.d_st = 16;
    m.num_words = (int32_t)plan.words;
    m.zero_dq = split ? 0 : 1;
    m.pre = nullptr;
    m.rank = nullptr;
    m.pds = nullptr;
    m.cap = topk;
    m.groups = (int32_t)plan.groups;
    m.num_blk = (int32_t)plan.blk;
    m.queue = nullptr;
    if (split) {
      m.pre = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan.pre_off);
      m.rank = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan.rank_off);
      m.pds = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + plan.pds_off);
      m.queue = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + plan.ws_bytes - 256);
    }
    hipLaunchKernelGGL(dsa::sparse_mla_bwd_prep_kernel, dim3((unsigned)num_tokens), dim3(256), 0, s, a, m);
    if (split) {
      // dq of every token whose row repeats no entry (which also stores P and
      // s*dS of its entries), then dkv of those tokens from them; the tokens
      // with a repeated entry take the full token-major kernel (dq, and dkv
      // with atomics)
      a.only = m.dup;
      a.only_nonzero = 0;
      // dq: 64 heads per workgroup above 32 heads, else 32
      if (num_heads > 32) {
        dsa::BwdArgs a64 = a;
        a64.head_blocks = (num_heads + 63) / 64;
        hipLaunchKernelGGL(dsa::sparse_mla_bwd_dq_kernel<4>, dim3((unsigned)(num_tokens * a64.head_blocks)),
                           dim3(64 * dsa::kDqWaves), 0, s, a64, m);
      } else {
        hipLaunchKernelGGL(dsa::sparse_mla_bwd_dq_kernel<2>, dim3((unsigned)wgs), dim3(64 * dsa::kDqWaves), 0, s,
                           a, m);
      }
      // persistent: one workgroup per CU (at most one fits), no more than the items
      const int64_t dkv_wgs = std::min<int64_t>(current_device_cus(), 2 * plan.blk * plan.chunks);
      hipLaunchKernelGGL(dsa::sparse_mla_bwd_dkv_kernel, dim3((unsigned)dkv_wgs), dim3(64 * dsa::kDkWaves), 0, s,
                         a, m);
      a.only_nonzero = 1;
      hipLaunchKernelGGL(dsa::sparse_mla_bwd_kernel<2>, dim3((unsigned)wgs), dim3(256), 0, s, a);
    } else {
      const dim3 kv_grid((unsigned)((plan.words + 1) / 2 * plan.chunks));
      hipLaunchKernelGGL(dsa::sparse_mla_bwd_kv_kernel, kv_grid, dim3(256), 0, s, a, m);
      a.only = m.dup;   // rows with a repeated entry: token-major
      a.only_nonzero = 1;
      hipLaunchKernelGGL(dsa::sparse_mla_bwd_kernel<1>, dim3((unsigned)wgs), dim3(256), 0, s, a);
    }
  } else if (hb == 16) {
    hipLaunchKernelGGL(dsa::sparse_mla_bwd_kernel<1>, dim3((unsigned)wgs), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(dsa::sparse_mla_bwd_kernel<2>, dim3((unsigned)wgs), dim3(256), 0, s, a);
  }
  if (hipGetLastError() != hipSuccess) return DSA_ERR_HIP;
  return DSA_OK;
}

int dsa_sparse_mla_bwd_workspace_size(int64_t num_tokens, int32_t num_heads, int64_t num_kv, int32_t topk,
                                      int32_t* schedule_out, int64_t* bytes_out) {
  if (!bytes_out) return DSA_ERR_INVALID_ARGUMENT;
  if (num_tokens < 0 || num_kv < 0) return DSA_ERR_INVALID_ARGUMENT;
  if (num_heads < 1 || num_heads > DSA_MAX_HEADS || topk < 1 || topk > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
  BwdPlan plan;
  bwd_plan(num_tokens, num_heads, num_kv, topk, &plan);
  if (schedule_out) *schedule_out = plan.schedule;
  *bytes_out = plan.ws_bytes;
  return DSA_OK;
}

int dsa_topk_indices(const float* scores, int64_t score_stride_tok, int64_t num_cols,
                     const int32_t* key_start, const int32_t* key_end, int64_t num_tokens, int32_t topk,
                     int32_t* indices, int64_t idx_stride_tok, void* stream) {
  if (num_tokens < 0 || num_cols < 0 || score_stride_tok < 0 || idx_stride_tok < 0)
    return DSA_ERR_INVALID_ARGUMENT;
  if (topk < 1 || topk > DSA_MAX_TOPK) return DSA_ERR_UNSUPPORTED;
  if (num_cols > INT32_MAX) return DSA_ERR_UNSUPPORTED;   // column ids are int32
  if (num_tokens == 0) return DSA_OK;
  if (num_tokens >= ((int64_t)1 << 31)) return DSA_ERR_UNSUPPORTED;   // one workgroup per row
  if (!key_start || !key_end || !indices) return DSA_ERR_INVALID_ARGUMENT;
  if (!aligned(key_start, 4) || !aligned(key_end, 4) || !aligned(indices, 4)) return DSA_ERR_INVALID_ARGUMENT;
  if (num_tokens > 1 && idx_stride_tok < topk) return DSA_ERR_INVALID_ARGUMENT;
  if (scores) {
    if (!aligned(scores, 4)) return DSA_ERR_INVALID_ARGUMENT;
    if (num_tokens > 1 && score_stride_tok < num_cols) return DSA_ERR_INVALID_ARGUMENT;
  }
  int st = check_overlaps({extent2(indices, num_tokens, idx_stride_tok, topk, 4)},
                          {extent2(scores, num_tokens, score_stride_tok, num_cols, 4),
                           extent2(key_start, 1, 0, num_tokens, 4), extent2(key_end, 1, 0, num_tokens, 4)});
  if (st != DSA_OK) return st;
  st = device_check();
  if (st != DSA_OK) return st;
  dsa::TopkArgs a;
  a.scores = scores;
  a.score_st = score_stride_tok;
  a.num_cols = num_cols;
  a.key_start = key_start;
  a.key_end = key_end;
  a.num_tokens = num_tokens;
  a.topk = topk;
  a.out = indices;
  a.out_st = idx_stride_tok;
  hipLaunchKernelGGL(dsa::topk_select_kernel, dim3((unsigned)num_tokens), dim3(dsa::kTkThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  if (hipGetLastError() != hipSuccess) return DSA_ERR_HIP;
  return DSA_OK;
}

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported device or size";
    case DSA_ERR_HIP: return "HIP runtime error";
    case DSA_ERR_WORKSPACE: return "workspace too small for the chosen split";
    default: return "unknown status";
  }
}

int dsa_device_supported(int device) {
  const DeviceInfo* d = device_info(device);
  return d && d->gfx950 ? 1 : 0;
}

int dsa_version(void) { return 100; }

}  // extern "C"
