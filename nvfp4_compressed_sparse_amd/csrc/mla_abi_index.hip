// C ABI of the sparse-indexer entry points (declared in include/mla_nvfp4.h): host-side argument checks,
// workspace sizing and launches.  Nothing is enqueued unless every check passes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_index_internal.h"
#include "mla_internal.h"
#include "mla_nvfp4.h"

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_device() { return mla::check_device_status(); }

// Index top-k workspace: [histograms n*2^12 int32][counters n*8 int32] (the part kept at zero between
// calls), then [segments n*chunks int2][candidates n*kTopkCap uint2], each region 256-byte aligned.
struct TopkLayout {
  size_t ctrl_off, seg_off, cand_off, total;
};

TopkLayout topk_layout(int64_t n, int64_t ld) {
  TopkLayout l{0, 0, 0, 0};
  if (n < 1 || ld < 1) return l;
  const size_t chunks = (size_t)ceil_div(ld, mla::kTopkChunk);
  l.ctrl_off = round256((size_t)n * ((size_t)1 << mla::kTopkBits1) * sizeof(int32_t));
  l.seg_off = l.ctrl_off + round256((size_t)n * mla::kTopkCtrlInts * sizeof(int32_t));
  l.cand_off = l.seg_off + round256((size_t)n * chunks * 2 * sizeof(int32_t));
  l.total = l.cand_off + round256((size_t)n * mla::kTopkCap * 2 * sizeof(uint32_t));
  return l;
}

}  // namespace

extern "C" {

int mla_index_key_quant(const void* keys, int64_t key_stride, const int64_t* slot_mapping, int64_t n, void* pool,
                        int64_t page_stride_bytes, int64_t num_pages, void* stream) {
  if (n < 0) return MLA_ERR_SHAPE;
  if (n == 0) return MLA_OK;
  if (!keys || !slot_mapping || !pool) return MLA_ERR_NULL;
  if (num_pages < 1) return MLA_ERR_SHAPE;
  if (key_stride < 128 || key_stride % 2) return MLA_ERR_STRIDE_ALIGN;
  if (page_stride_bytes < mla::kIndexPageBytes || page_stride_bytes % 16) return MLA_ERR_STRIDE_ALIGN;
  if (!aligned(keys, 4) || !aligned(slot_mapping, 8) || !aligned(pool, 16)) return MLA_ERR_STRIDE_ALIGN;
  if (n > mla::kMaxWriteTokens) return MLA_ERR_SHAPE;
  int st = check_device();
  if (st != MLA_OK) return st;
  mla::IndexKeyArgs a{(const uint16_t*)keys, key_stride, slot_mapping, n, (uint8_t*)pool, page_stride_bytes, num_pages};
  return mla::launch_index_key_quant(a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_index_logits(const void* q, const float* w, int32_t HI, const void* pool, int64_t page_stride_bytes,
                     int64_t num_pages, const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                     int32_t B, int32_t T, int32_t max_context, int32_t causal, float* logits, int64_t ld,
                     void* stream) {
  if (!q || !w || !pool || !block_table || !context_lens || !logits) return MLA_ERR_NULL;
  if (B < 1 || T < 1 || num_pages < 1 || bt_stride < 1 || max_context < 1) return MLA_ERR_SHAPE;
  if (HI != 16 && HI != 32 && HI != 64) return MLA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return MLA_ERR_SHAPE;
  if (ld < max_context) return MLA_ERR_SHAPE;
  if (page_stride_bytes < mla::kIndexPageBytes || page_stride_bytes % 16) return MLA_ERR_STRIDE_ALIGN;
  if (!aligned(q, 16) || !aligned(w, 16) || !aligned(pool, 16) || !aligned(block_table, 4) ||
      !aligned(context_lens, 4) || !aligned(logits, 4))
    return MLA_ERR_STRIDE_ALIGN;
  const int64_t chunks = ceil_div(ceil_div(max_context, 64), mla::kIdxPagesPerWg);
  if ((int64_t)B * chunks * 256 > mla::kMaxLaunchThreads) return MLA_ERR_SHAPE;  // 256-thread workgroups
  int st = check_device();
  if (st != MLA_OK) return st;
  mla::IndexLogitsArgs a;
  a.q = (const uint16_t*)q;
  a.w = w;
  a.HI = HI;
  a.pool = (const uint8_t*)pool;
  a.page_stride = page_stride_bytes;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.bt_stride = bt_stride;
  a.ctx = context_lens;
  a.B = B;
  a.T = T;
  a.causal = causal;
  a.chunks = (int)chunks;
  a.logits = logits;
  a.ld = ld;
  return mla::launch_index_logits(a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

size_t mla_index_topk_workspace_bytes(int64_t n, int64_t ld) { return topk_layout(n, ld).total; }

int mla_index_topk(const float* logits, int64_t ld, const int32_t* lengths, int64_t n, int32_t k, int32_t* out,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (n < 0 || k < 1 || k > MLA_MAX_TOPK) return MLA_ERR_SHAPE;
  if (ld < 4 || ld % 4) return MLA_ERR_STRIDE_ALIGN;
  if (ld > INT32_MAX) return MLA_ERR_SHAPE;  // positions are int32
  const int64_t chunks = ceil_div(ld, mla::kTopkChunk);
  // one workgroup of kTopkThreads per chunk of every row: the grid, in threads, fits the dispatch limit
  if (n * chunks * mla::kTopkThreads > mla::kMaxLaunchThreads) return MLA_ERR_SHAPE;
  if (n == 0) return MLA_OK;
  if (!logits || !lengths || !out || !workspace) return MLA_ERR_NULL;
  if (!aligned(logits, 16) || !aligned(lengths, 4) || !aligned(out, 4) || !aligned(workspace, 256))
    return MLA_ERR_STRIDE_ALIGN;
  const TopkLayout l = topk_layout(n, ld);
  if (workspace_bytes < l.total) return MLA_ERR_WORKSPACE;
  int st = check_device();
  if (st != MLA_OK) return st;
  mla::TopkArgs a;
  a.logits = logits;
  a.n = n;
  a.ld = ld;
  a.lengths = lengths;
  a.k = k;
  a.chunks = (int)chunks;
  a.out = out;
  char* ws = (char*)workspace;
  a.hist = (int*)ws;
  a.ctrl = (int*)(ws + l.ctrl_off);
  a.seg = (int2*)(ws + l.seg_off);
  a.cand = (uint2*)(ws + l.cand_off);
  return mla::launch_topk(a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
