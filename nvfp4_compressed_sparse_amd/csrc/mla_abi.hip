// C ABI of libmla_nvfp4 (declared in include/mla_nvfp4.h): host-side argument checks, the split
// choice, workspace sizing and launches.  Nothing is enqueued unless every check passes.
#include <algorithm>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "mla_internal.h"
#include "mla_nvfp4.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  int st = g_device_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_DEVICE;
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? MLA_OK : MLA_ERR_DEVICE;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool valid_heads(int32_t H) { return H == 16 || H == 32 || H == 64 || H == 128; }

int head_groups(int32_t H) { return H == 16 ? 1 : H / 32; }

constexpr int kTargetWorkgroups = 256;  // one resident workgroup per compute unit
constexpr int kMaxSplits = 64;
constexpr int kMaxChunk = 2048;  // list entries one workgroup can hold
constexpr int kMinSplitEntries = 256;  // four 64-row steps

// Split count of the 16/32-head-group kernel: as many splits as fit one workgroup per compute unit
// (never more workgroups than units: a second round of workgroups costs a whole split's latency), and at
// least 256 list entries per split (a split of one or two steps is mostly fixed latency, and every
// extra split adds to what the merging workgroup reads).  Measured at 15/20/35 query tokens with 16
// heads, top-2048: 8, 8 and 7 splits against 18, 13 and 8 before, 20-32% faster.
int auto_splits(int64_t units, int64_t entries, int64_t min_splits) {
  int64_t s = kTargetWorkgroups / units;
  int64_t cap = ceil_div(entries, kMinSplitEntries);
  if (s > cap) s = cap;
  if (s < min_splits) s = min_splits;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  return (int)s;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout when S > 1: [split arrival counters: a fixed region of kMaxSplitCounters int32, of
// which B*T*head groups are used][partial outputs: B*T*H*S*512 fp16][partial lse: B*T*H*S fp32], each
// region 256-byte aligned.  The counters must be zero before the first call; every call leaves them
// zero, and since the counter region is the same for every shape, later calls of any shape may reuse
// the workspace.
struct WsLayout {
  size_t cnt_off, o_off, lse_off, total;
};

WsLayout workspace_layout(int64_t B, int64_t T, int64_t H, int S) {
  WsLayout l{0, 0, 0, 0};
  if (S <= 1) return l;
  const size_t rows = (size_t)(B * T * H);
  l.o_off = round256((size_t)mla::kMaxSplitCounters * sizeof(int32_t));
  l.lse_off = l.o_off + round256(rows * (size_t)S * 512 * sizeof(uint16_t));
  l.total = l.lse_off + round256(rows * (size_t)S * sizeof(float));
  return l;
}

// The decode launch for these sizes stays inside the dispatch limits: its grid, in threads, fits 32 bits,
// and a split launch has at most kMaxSplitCounters arrival counters.
bool decode_launch_fits(int64_t B, int64_t T, int32_t H, int S) {
  const int64_t units = B * T * head_groups(H);
  if (units * S * mla::kDecodeThreads > mla::kMaxLaunchThreads) return false;
  if (S > 1 && units > mla::kMaxSplitCounters) return false;
  return true;
}

size_t workspace_for(int64_t B, int64_t T, int64_t H, int S) { return workspace_layout(B, T, H, S).total; }

int check_quant(const void* k_nope, int64_t nope_stride, const void* k_rope, int64_t rope_stride,
                const int64_t* slot_mapping, int64_t n, void* pool, int64_t page_stride, int64_t num_pages,
                int row_bytes) {
  if (n < 0) return MLA_ERR_SHAPE;
  if (n == 0) return MLA_OK;
  if (!k_nope || !k_rope || !slot_mapping || !pool) return MLA_ERR_NULL;
  if (num_pages <= 0 || n > mla::kMaxWriteTokens) return MLA_ERR_SHAPE;
  if (nope_stride < 512 || rope_stride < 64 || nope_stride % 8 || rope_stride % 8) return MLA_ERR_STRIDE_ALIGN;
  if (!aligned(k_nope, 16) || !aligned(k_rope, 16) || !aligned(pool, 16) || !aligned(slot_mapping, 8))
    return MLA_ERR_STRIDE_ALIGN;
  if (page_stride < 64LL * row_bytes || page_stride % 16) return MLA_ERR_STRIDE_ALIGN;
  return MLA_OK;
}

int run_quant(int fmt, const void* k_nope, int64_t nope_stride, const void* k_rope, int64_t rope_stride,
              const int64_t* slot_mapping, int64_t n, void* pool, int64_t page_stride, int64_t num_pages,
              void* stream) {
  int st = check_quant(k_nope, nope_stride, k_rope, rope_stride, slot_mapping, n, pool, page_stride, num_pages,
                       fmt == 0 ? MLA_NVFP4_ROW_BYTES : MLA_FP8_ROW_BYTES);
  if (st != MLA_OK || n == 0) return st;
  if ((st = check_device()) != MLA_OK) return st;
  mla::QuantArgs a{(const uint16_t*)k_nope, nope_stride, (const uint16_t*)k_rope, rope_stride, slot_mapping, n,
                   (uint8_t*)pool, page_stride, num_pages};
  return mla::launch_quant(fmt, a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int check_decode_common(const void* q, const void* pool, int64_t page_stride, int64_t num_pages,
                        const int32_t* block_table, int64_t bt_stride, const int32_t* ctx, int32_t B, int32_t T,
                        int32_t H, float sm_scale, int32_t causal, void* out, int row_bytes) {
  if (!q || !pool || !block_table || !ctx || !out) return MLA_ERR_NULL;
  if (B < 1 || T < 1 || !valid_heads(H) || num_pages < 1 || bt_stride < 1) return MLA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return MLA_ERR_SHAPE;
  // a softmax scale: positive, and finite also in base 2 (times log2 e)
  if (!(sm_scale > 0.0f) || !(sm_scale * 1.4426950408889634f < INFINITY)) return MLA_ERR_SHAPE;
  if ((int64_t)B * T * H * 576 > ((int64_t)1 << 40)) return MLA_ERR_SHAPE;
  if (page_stride < 64LL * row_bytes || page_stride % 16) return MLA_ERR_STRIDE_ALIGN;
  // row addresses travel as 32-bit multiples of 16 bytes
  if ((num_pages * page_stride) / 16 > (int64_t)0xFFFFFFFFLL) return MLA_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(pool, 16) || !aligned(block_table, 4) || !aligned(ctx, 4))
    return MLA_ERR_STRIDE_ALIGN;
  return MLA_OK;
}

// The new rows of mla_sparse_decode_append (bf16, row strides in elements).
struct AppendRows {
  const void* k_nope;
  int64_t nope_stride;
  const void* k_rope;
  int64_t rope_stride;
};

int run_decode(int fmt, const void* q, const void* pool, int64_t page_stride, int64_t num_pages,
               const int32_t* block_table, int64_t bt_stride, const int32_t* ctx, const int32_t* indices, int32_t B,
               int32_t T, int32_t H, int32_t entries, float sm_scale, int32_t causal, int32_t num_splits, void* out,
               float* lse, void* workspace, size_t workspace_bytes, void* stream, const AppendRows* app = nullptr) {
  int S = num_splits;
  int chunk = (int)ceil_div(entries, S);
  // a dense split starts on a page boundary, so that each 64-row step of the decoder is one page
  if (!indices) chunk = (int)ceil_div(chunk, 64) * 64;
  if (chunk > kMaxChunk) return MLA_ERR_SHAPE;
  if (!decode_launch_fits(B, T, H, S)) return MLA_ERR_SHAPE;
  size_t need = workspace_for(B, T, H, S);
  if (need > 0) {
    if (!workspace) return MLA_ERR_NULL;
    if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MLA_ERR_STRIDE_ALIGN;
  }
  if (lse && !aligned(lse, 4)) return MLA_ERR_STRIDE_ALIGN;
  int st = check_device();
  if (st != MLA_OK) return st;
  mla::DecodeArgs a;
  a.q = (const uint16_t*)q;
  a.pool = (const uint8_t*)pool;
  a.page_stride = page_stride;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.bt_stride = bt_stride;
  a.ctx = ctx;
  a.indices = indices;
  a.B = B;
  a.T = T;
  a.H = H;
  a.entries = entries;
  a.chunk = chunk;
  a.splits = S;
  a.causal = causal;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.out = (uint16_t*)out;
  a.lse = lse;
  const WsLayout wl = workspace_layout(B, T, H, S);
  a.part_o = need ? (uint16_t*)((char*)workspace + wl.o_off) : nullptr;
  a.part_lse = need ? (float*)((char*)workspace + wl.lse_off) : nullptr;
  a.counters = need ? (int*)((char*)workspace + wl.cnt_off) : nullptr;
  if (app) {
    a.new_nope = (const uint16_t*)app->k_nope;
    a.new_nope_stride = app->nope_stride;
    a.new_rope = (const uint16_t*)app->k_rope;
    a.new_rope_stride = app->rope_stride;
    a.wpool = (uint8_t*)const_cast<void*>(pool);
  }
  return mla::launch_decode(fmt, a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

// ---- scratch of the entry point that allocates nothing (mla_sparse_decode_noalloc).  The split arrival
// counters and partial results live in this file-scope device array instead of a caller workspace: the
// fixed counter region first (zero at module load; every call returns the counters it used to zero, and
// no call writes anything else there), then the partials.  In host code `scratch` names a host-side
// stand-in, not device memory: the device address is looked up once per device with hipGetSymbolAddress
// and only that address is handed to kernels.
namespace {

constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MLA_OK;
}

}  // namespace

int mla::check_device_status() { return check_device(); }

extern "C" {

int mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(int s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "a size is out of range";
    case MLA_ERR_STRIDE_ALIGN: return "a stride is too small or a pointer/stride is misaligned";
    case MLA_ERR_WORKSPACE: return "workspace too small";
    case MLA_ERR_DEVICE: return "the current device is not a gfx950 GPU";
    case MLA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int mla_kv_quant_nvfp4(const void* k_nope, int64_t nope_stride, const void* k_rope, int64_t rope_stride,
                       const int64_t* slot_mapping, int64_t n, void* pool, int64_t page_stride_bytes,
                       int64_t num_pages, void* stream) {
  return run_quant(0, k_nope, nope_stride, k_rope, rope_stride, slot_mapping, n, pool, page_stride_bytes, num_pages,
                   stream);
}

int mla_kv_quant_fp8(const void* k_nope, int64_t nope_stride, const void* k_rope, int64_t rope_stride,
                     const int64_t* slot_mapping, int64_t n, void* pool, int64_t page_stride_bytes, int64_t num_pages,
                     void* stream) {
  return run_quant(1, k_nope, nope_stride, k_rope, rope_stride, slot_mapping, n, pool, page_stride_bytes, num_pages,
                   stream);
}

int mla_sparse_decode_splits(int32_t B, int32_t T, int32_t H, int32_t topk) {
  if (B < 1 || T < 1 || !valid_heads(H) || topk < 1 || topk > MLA_MAX_TOPK) return 0;
  return auto_splits((int64_t)B * T * head_groups(H), topk, 1);
}

int mla_sparse_decode_fp8_splits(int32_t B, int32_t T, int32_t H, int32_t topk) {
  if (B < 1 || T < 1 || !valid_heads(H) || topk < 1 || topk > MLA_MAX_TOPK) return 0;
  return auto_splits((int64_t)B * T * head_groups(H), topk, 1);
}

int mla_dense_decode_splits(int32_t B, int32_t T, int32_t H, int32_t max_context) {
  if (B < 1 || T < 1 || !valid_heads(H) || max_context < 1) return 0;
  return auto_splits((int64_t)B * T * head_groups(H), max_context, ceil_div(max_context, kMaxChunk));
}

size_t mla_sparse_decode_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t topk, int32_t num_splits) {
  int S = num_splits > 0 ? num_splits : mla_sparse_decode_splits(B, T, H, topk);
  if (S < 1) return 0;
  return workspace_for(B, T, H, S);
}

size_t mla_sparse_decode_fp8_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t topk, int32_t num_splits) {
  int S = num_splits > 0 ? num_splits : mla_sparse_decode_fp8_splits(B, T, H, topk);
  if (S < 1) return 0;
  return workspace_for(B, T, H, S);
}

size_t mla_dense_decode_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t max_context, int32_t num_splits) {
  int S = num_splits > 0 ? num_splits : mla_dense_decode_splits(B, T, H, max_context);
  if (S < 1) return 0;
  return workspace_for(B, T, H, S);
}

int mla_sparse_decode(const void* q, const void* pool, int64_t page_stride_bytes, int64_t num_pages,
                      const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                      const int32_t* indices, int32_t B, int32_t T, int32_t H, int32_t topk, float sm_scale,
                      int32_t causal, int32_t num_splits, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_decode_common(q, pool, page_stride_bytes, num_pages, block_table, bt_stride, context_lens, B, T, H,
                               sm_scale, causal, out, MLA_NVFP4_ROW_BYTES);
  if (st != MLA_OK) return st;
  if (!indices) return MLA_ERR_NULL;
  if (!aligned(indices, 4)) return MLA_ERR_STRIDE_ALIGN;
  if (topk < 1 || topk > MLA_MAX_TOPK) return MLA_ERR_SHAPE;
  if (num_splits < 0 || num_splits > kMaxSplits) return MLA_ERR_SHAPE;
  int S = num_splits ? num_splits : mla_sparse_decode_splits(B, T, H, topk);
  return run_decode(0, q, pool, page_stride_bytes, num_pages, block_table, bt_stride, context_lens, indices, B, T, H,
                    topk, sm_scale, causal, S, out, lse, workspace, workspace_bytes, stream);
}

int mla_sparse_decode_append(const void* q, void* pool, int64_t page_stride_bytes, int64_t num_pages,
                             const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                             const int32_t* indices, const void* k_nope, int64_t nope_stride, const void* k_rope,
                             int64_t rope_stride, int32_t B, int32_t T, int32_t H, int32_t topk, float sm_scale,
                             int32_t causal, int32_t num_splits, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  int st = check_decode_common(q, pool, page_stride_bytes, num_pages, block_table, bt_stride, context_lens, B, T, H,
                               sm_scale, causal, out, MLA_NVFP4_ROW_BYTES);
  if (st != MLA_OK) return st;
  if (!indices || !k_nope || !k_rope) return MLA_ERR_NULL;
  if (!aligned(indices, 4)) return MLA_ERR_STRIDE_ALIGN;
  // the new rows as the writer takes them: 16-byte aligned bf16 rows of at least 512 and 64 values
  if (nope_stride < 512 || rope_stride < 64 || nope_stride % 8 || rope_stride % 8) return MLA_ERR_STRIDE_ALIGN;
  if (!aligned(k_nope, 16) || !aligned(k_rope, 16)) return MLA_ERR_STRIDE_ALIGN;
  if (topk < 1 || topk > MLA_MAX_TOPK) return MLA_ERR_SHAPE;
  if (num_splits < 0 || num_splits > kMaxSplits) return MLA_ERR_SHAPE;
  int S = num_splits ? num_splits : mla_sparse_decode_splits(B, T, H, topk);
  const AppendRows app{k_nope, nope_stride, k_rope, rope_stride};
  return run_decode(0, q, pool, page_stride_bytes, num_pages, block_table, bt_stride, context_lens, indices, B, T, H,
                    topk, sm_scale, causal, S, out, lse, workspace, workspace_bytes, stream, &app);
}

int mla_sparse_decode_fp8(const void* q, const void* pool, int64_t page_stride_bytes, int64_t num_pages,
                          const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                          const int32_t* indices, int32_t B, int32_t T, int32_t H, int32_t topk, float sm_scale,
                          int32_t causal, int32_t num_splits, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int st = check_decode_common(q, pool, page_stride_bytes, num_pages, block_table, bt_stride, context_lens, B, T, H,
                               sm_scale, causal, out, MLA_FP8_ROW_BYTES);
  if (st != MLA_OK) return st;
  if (!indices) return MLA_ERR_NULL;
  if (!aligned(indices, 4)) return MLA_ERR_STRIDE_ALIGN;
  if (topk < 1 || topk > MLA_MAX_TOPK) return MLA_ERR_SHAPE;
  if (num_splits < 0 || num_splits > kMaxSplits) return MLA_ERR_SHAPE;
  int S = num_splits ? num_splits : mla_sparse_decode_fp8_splits(B, T, H, topk);
  return run_decode(1, q, pool, page_stride_bytes, num_pages, block_table, bt_stride, context_lens, indices, B, T, H,
                    topk, sm_scale, causal, S, out, lse, workspace, workspace_bytes, stream);
}

size_t mla_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

int mla_sparse_decode_noalloc(const void* q, const void* pool, int64_t page_stride_bytes, int64_t num_pages,
                              const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                              const int32_t* indices, int32_t B, int32_t T, int32_t H, int32_t topk, float sm_scale,
                              int32_t causal, int32_t num_splits, void* out, float* lse, void* stream) {
  int st = check_decode_common(q, pool, page_stride_bytes, num_pages, block_table, bt_stride, context_lens, B, T, H,
                               sm_scale, causal, out, MLA_NVFP4_ROW_BYTES);
  if (st != MLA_OK) return st;
  if (!indices) return MLA_ERR_NULL;
  if (!aligned(indices, 4)) return MLA_ERR_STRIDE_ALIGN;
  if (topk < 1 || topk > MLA_MAX_TOPK) return MLA_ERR_SHAPE;
  if (num_splits < 0 || num_splits > kMaxSplits) return MLA_ERR_SHAPE;
  const int S = num_splits ? num_splits : mla_sparse_decode_splits(B, T, H, topk);
  const size_t need = workspace_for(B, T, H, S);
  if (need > kNoallocScratchBytes) return MLA_ERR_WORKSPACE;  // more partial results than the scratch holds
  void* ws = nullptr;
  if (need > 0) {
    if ((st = check_device()) != MLA_OK) return st;
    if ((st = scratch_address(&ws)) != MLA_OK) return st;
  }
  return run_decode(0, q, pool, page_stride_bytes, num_pages, block_table, bt_stride, context_lens, indices, B, T, H,
                    topk, sm_scale, causal, S, out, lse, ws, need, stream);
}

int mla_dense_decode_fp8(const void* q, const void* pool, int64_t page_stride_bytes, int64_t num_pages,
                         const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens, int32_t B,
                         int32_t T, int32_t H, int32_t max_context, float sm_scale, int32_t causal, int32_t num_splits,
                         void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_decode_common(q, pool, page_stride_bytes, num_pages, block_table, bt_stride, context_lens, B, T, H,
                               sm_scale, causal, out, MLA_FP8_ROW_BYTES);
  if (st != MLA_OK) return st;
  if (max_context < 1) return MLA_ERR_SHAPE;
  if (num_splits < 0 || num_splits > kMaxSplits) return MLA_ERR_SHAPE;
  int S = num_splits ? num_splits : mla_dense_decode_splits(B, T, H, max_context);
  return run_decode(1, q, pool, page_stride_bytes, num_pages, block_table, bt_stride, context_lens, nullptr, B, T, H,
                    max_context, sm_scale, causal, S, out, lse, workspace, workspace_bytes, stream);
}

int mla_stage_nvfp4_fp8(const void* pool, int64_t page_stride_bytes, int64_t num_pages, const int32_t* block_table,
                        int64_t bt_stride, const int32_t* context_lens, const int32_t* indices, int32_t B, int32_t T,
                        int32_t topk, int32_t causal, void* staged, int32_t* staged_block_table, int32_t* staged_lens,
                        void* stream) {
  if (!pool || !block_table || !context_lens || !indices || !staged || !staged_block_table || !staged_lens)
    return MLA_ERR_NULL;
  if (B < 1 || T < 1 || topk < 1 || topk > MLA_MAX_TOPK || num_pages < 1 || bt_stride < 1) return MLA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return MLA_ERR_SHAPE;
  // staged rows are addressed with 32-bit row counts, and the launch (at most 16 workgroups of 256
  // threads per query token) must fit the dispatch limit
  if ((int64_t)B * T > ((int64_t)1 << 31) / 64 || (int64_t)B * T * 16 * 256 > mla::kMaxLaunchThreads)
    return MLA_ERR_SHAPE;
  if (page_stride_bytes < 64LL * MLA_NVFP4_ROW_BYTES || page_stride_bytes % 16) return MLA_ERR_STRIDE_ALIGN;
  // row addresses travel as 32-bit multiples of 16 bytes
  if ((num_pages * page_stride_bytes) / 16 > (int64_t)0xFFFFFFFFLL) return MLA_ERR_SHAPE;
  if (!aligned(pool, 16) || !aligned(staged, 16) || !aligned(block_table, 4) || !aligned(context_lens, 4) ||
      !aligned(indices, 4) || !aligned(staged_block_table, 4) || !aligned(staged_lens, 4))
    return MLA_ERR_STRIDE_ALIGN;
  int st = check_device();
  if (st != MLA_OK) return st;
  mla::StageArgs a;
  a.pool = (const uint8_t*)pool;
  a.page_stride = page_stride_bytes;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.bt_stride = bt_stride;
  a.ctx = context_lens;
  a.indices = indices;
  a.B = B;
  a.T = T;
  a.topk = topk;
  a.causal = causal;
  a.pages_per_token = (int)ceil_div(topk, 64);
  // enough workgroups to fill the chip a few times over, at most one per 128 list entries
  a.parts = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(topk, 128), ceil_div(1024, (int64_t)B * T)));
  a.staged = (uint8_t*)staged;
  a.staged_block_table = staged_block_table;
  a.staged_lens = staged_lens;
  return mla::launch_stage(a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
