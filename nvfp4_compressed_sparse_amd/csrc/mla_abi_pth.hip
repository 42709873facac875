// C ABI of the per-token-head FP8 layout's entry points (declared in include/mla_nvfp4.h): host-side
// argument checks, the split choice, workspace sizing and launches.  Nothing is enqueued unless every
// check passes.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mla_internal.h"
#include "mla_nvfp4.h"
#include "mla_pth_internal.h"

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Splits: enough workgroups to give every compute unit two (512, the decode kernel's occupancy), at
// least 128 list entries (two 64-row steps) each, and a chunk of at most kPthMaxChunk entries rounded up
// to whole 64-row steps.  A requested count sets the chunk, ceil(topk / requested) rounded up to whole
// steps, so the effective count S = ceil(topk / chunk) may be lower than the request.
void pth_splits(int64_t units, int32_t topk, int32_t requested, int& S, int& chunk) {
  int64_t s = requested > 0 ? requested : ceil_div(512, units);
  const int64_t cap = ceil_div(topk, 128);
  if (requested <= 0 && s > cap) s = cap;
  if (s < 1) s = 1;
  int64_t c = ceil_div(ceil_div(topk, s), 64) * 64;
  if (c > mla::kPthMaxChunk) c = mla::kPthMaxChunk;
  S = (int)ceil_div(topk, c);
  chunk = (int)c;
}

size_t pth_workspace(int64_t rows, int S) {
  if (S <= 1) return 0;
  return round256((size_t)rows * S * 512 * sizeof(float)) + round256((size_t)rows * S * sizeof(float));
}

}  // namespace

extern "C" {

int mla_kv_quant_pth(const void* k_nope, int64_t nope_stride, const void* k_rope, int64_t rope_stride,
                     const int64_t* slot_mapping, int64_t n, void* lat, float* scale, void* rope, int64_t num_slots,
                     void* stream) {
  if (n < 0) return MLA_ERR_SHAPE;
  if (n == 0) return MLA_OK;
  if (!k_nope || !k_rope || !slot_mapping || !lat || !scale || !rope) return MLA_ERR_NULL;
  if (num_slots < 1 || n > mla::kMaxWriteTokens) return MLA_ERR_SHAPE;
  if (nope_stride < 512 || rope_stride < 64 || nope_stride % 8) return MLA_ERR_STRIDE_ALIGN;
  if (!aligned(k_nope, 16) || !aligned(k_rope, 2) || !aligned(slot_mapping, 8) || !aligned(lat, 8) ||
      !aligned(scale, 4) || !aligned(rope, 2))
    return MLA_ERR_STRIDE_ALIGN;
  int st = mla::check_device_status();
  if (st != MLA_OK) return st;
  mla::PthQuantArgs a{(const uint16_t*)k_nope, nope_stride, (const uint16_t*)k_rope, rope_stride, slot_mapping, n,
                      (uint8_t*)lat, scale, (uint16_t*)rope, num_slots};
  return mla::launch_pth_quant(a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

size_t mla_sparse_decode_pth_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t topk, int32_t num_splits) {
  if (B < 1 || T < 1 || H < 16 || H % 16 || topk < 1 || topk > MLA_MAX_TOPK || num_splits < 0) return 0;
  int S, chunk;
  pth_splits((int64_t)B * T * (H / 16), topk, num_splits, S, chunk);
  return pth_workspace((int64_t)B * T * H, S);
}

int mla_sparse_decode_pth(const void* q, const void* lat, const float* scale, const void* rope, int64_t num_slots,
                          const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                          const int32_t* indices, int32_t B, int32_t T, int32_t H, int32_t topk, float sm_scale,
                          int32_t causal, int32_t num_splits, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!q || !lat || !scale || !rope || !block_table || !context_lens || !indices || !out) return MLA_ERR_NULL;
  if (B < 1 || T < 1 || num_slots < 64 || bt_stride < 1) return MLA_ERR_SHAPE;
  if (H != 16 && H != 32 && H != 64 && H != 128) return MLA_ERR_SHAPE;
  if (topk < 1 || topk > MLA_MAX_TOPK || num_splits < 0 || num_splits > 64) return MLA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return MLA_ERR_SHAPE;
  if (!(sm_scale > 0.0f) || !(sm_scale * 1.4426950408889634f < INFINITY)) return MLA_ERR_SHAPE;
  if ((int64_t)B * T * H * 576 > ((int64_t)1 << 40)) return MLA_ERR_SHAPE;
  if (num_slots > ((int64_t)1 << 32)) return MLA_ERR_SHAPE;  // slots travel as 32-bit values
  if (!aligned(q, 16) || !aligned(lat, 16) || !aligned(scale, 4) || !aligned(rope, 16) || !aligned(block_table, 4) ||
      !aligned(context_lens, 4) || !aligned(indices, 4) || !aligned(out, 16) || (lse && !aligned(lse, 4)))
    return MLA_ERR_STRIDE_ALIGN;
  int S, chunk;
  pth_splits((int64_t)B * T * (H / 16), topk, num_splits, S, chunk);
  const int64_t rows = (int64_t)B * T * H;
  // the decode grid (256-thread workgroups) and the merge grid (128 threads per head row) fit the
  // dispatch limit
  if ((int64_t)B * T * (H / 16) * S * 256 > mla::kMaxLaunchThreads || rows * 128 > mla::kMaxLaunchThreads)
    return MLA_ERR_SHAPE;
  const size_t need = pth_workspace(rows, S);
  if (need) {
    if (!workspace) return MLA_ERR_NULL;
    if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MLA_ERR_STRIDE_ALIGN;
  }
  int st = mla::check_device_status();
  if (st != MLA_OK) return st;
  mla::PthDecodeArgs a;
  a.q = (const uint16_t*)q;
  a.lat = (const uint8_t*)lat;
  a.scale = scale;
  a.rope = (const uint16_t*)rope;
  a.num_slots = num_slots;
  a.block_table = block_table;
  a.bt_stride = bt_stride;
  a.ctx = context_lens;
  a.indices = indices;
  a.B = B;
  a.T = T;
  a.H = H;
  a.topk = topk;
  a.causal = causal;
  a.splits = S;
  a.chunk = chunk;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.part_o = need ? (float*)workspace : nullptr;
  a.part_lse = need ? (float*)((char*)workspace + round256((size_t)rows * S * 512 * sizeof(float))) : nullptr;
  return mla::launch_pth_decode(a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
