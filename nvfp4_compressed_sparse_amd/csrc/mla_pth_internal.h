// Internal launch interface of the per-token-head FP8 layout's kernels (mla_pth.hip) and their C ABI
// (mla_abi_pth.hip).  Arguments are already validated when these structs are filled.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kPthMaxChunk = 2048;  // list entries per split workgroup

struct PthQuantArgs {
  const uint16_t* k_nope;     // bf16 [n, 512], row stride nope_stride elements
  int64_t nope_stride;
  const uint16_t* k_rope;     // bf16 [n, 64], row stride rope_stride elements
  int64_t rope_stride;
  const int64_t* slot_mapping;
  int64_t n;
  uint8_t* lat;               // E4M3 [num_slots, 512]
  float* scale;               // [num_slots]
  uint16_t* rope;             // bf16 [num_slots, 64]
  int64_t num_slots;
};

struct PthDecodeArgs {
  const uint16_t* q;          // bf16 [B, T, H, 576]
  const uint8_t* lat;
  const float* scale;
  const uint16_t* rope;
  int64_t num_slots;
  const int32_t* block_table;
  int64_t bt_stride;
  const int32_t* ctx;
  const int32_t* indices;     // [B, T, topk]
  int B, T, H, topk, causal;
  int splits, chunk;          // S workgroups per (query token, head group), chunk list entries each
  float scale_log2;           // sm_scale * log2(e)
  uint16_t* out;              // bf16 [B, T, H, 512]
  float* lse;                 // [B, T, H] or nullptr
  float* part_o;              // [B*T*H, S, 512] when S > 1
  float* part_lse;            // [B*T*H, S]
};

hipError_t launch_pth_quant(const PthQuantArgs& a, hipStream_t stream);
hipError_t launch_pth_decode(const PthDecodeArgs& a, hipStream_t stream);

}  // namespace mla
