// Internal launch interface between the C ABI (mla_abi.hip) and the kernels.  Arguments are already
// validated when these structs are filled.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct QuantArgs {
  const uint16_t* k_nope;
  int64_t nope_stride;
  const uint16_t* k_rope;
  int64_t rope_stride;
  const int64_t* slot_mapping;
  int64_t n;
  uint8_t* pool;
  int64_t page_stride;
  int64_t num_pages;
};

struct DecodeArgs {
  const uint16_t* q;          // [B,T,H,576]
  const uint8_t* pool;
  int64_t page_stride;
  int64_t num_pages;
  const int32_t* block_table;
  int64_t bt_stride;
  const int32_t* ctx;         // [B]
  const int32_t* indices;     // [B,T,topk] (sparse) or nullptr (dense)
  int B, T, H;
  int entries;                // topk (sparse) or max_context (dense): length of the position list
  int chunk;                  // entries per split
  int splits;                 // S
  int causal;
  float scale_log2;           // sm_scale * log2(e)
  uint16_t* out;              // bf16 [B,T,H,512]
  float* lse;                 // [B,T,H] or nullptr
  uint16_t* part_o;           // FP16 [B*T*H, S, 512] when S > 1
  float* part_lse;            // [B*T*H, S]
  int* counters;              // [B*T*head groups] split arrival counters, zero between calls
  // append (mla_sparse_decode_append): the B*T new rows, token t of request b written at position
  // ctx[b] - T + t before any row is read; every workgroup of request b writes all T of them (the same
  // bytes), so each has them in memory before its own gathers.  nullptr otherwise.
  const uint16_t* new_nope = nullptr;  // [B*T rows, new_nope_stride] bf16, 512 used
  int64_t new_nope_stride = 0;
  const uint16_t* new_rope = nullptr;  // [B*T rows, new_rope_stride] bf16, 64 used
  int64_t new_rope_stride = 0;
  uint8_t* wpool = nullptr;            // the pool, writable (the memory of pool)
};

struct StageArgs {
  const uint8_t* pool;        // NVFP4 page pool
  int64_t page_stride;
  int64_t num_pages;
  const int32_t* block_table;
  int64_t bt_stride;
  const int32_t* ctx;         // [B]
  const int32_t* indices;     // [B,T,topk]
  int B, T, topk, causal;
  int pages_per_token;        // P = ceil(topk / 64)
  int parts;                  // workgroups per query token
  uint8_t* staged;            // FP8 pool of B*T*P pages of 64 x 576 bytes
  int32_t* staged_block_table;  // [B*T, P]
  int32_t* staged_lens;       // [B*T]
};

constexpr int kDecodeThreads = 512;  // decode_kernel workgroup size
// A launch's grid, counted in threads, must fit 32 bits (the dispatch packet's grid size).
constexpr int64_t kMaxLaunchThreads = 0xFFFFFFFFLL;
// Split arrival counters live in a fixed region at the start of a split decode's workspace, one int32
// per (query token, head group) up to this many.  No shape ever writes partial results there, and every
// call leaves its counters at zero, so a zero-filled workspace stays valid for later calls of any shape.
constexpr int64_t kMaxSplitCounters = 65536;

// Tokens one writer call may take: the writers run one 64-lane wave per token.
constexpr int64_t kMaxWriteTokens = kMaxLaunchThreads / 64;

hipError_t launch_quant(int fmt, const QuantArgs& a, hipStream_t stream);
hipError_t launch_decode(int fmt, const DecodeArgs& a, hipStream_t stream);
// The staged path's unpack of each query token's selected NVFP4 rows into FP8 rows (mla_stage.hip).
hipError_t launch_stage(const StageArgs& a, hipStream_t stream);

// The current device is a gfx950 GPU: MLA_OK, else the C ABI's error status (mla_abi.hip).
int check_device_status();

}  // namespace mla
