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

// Index top-k (mla_topk.hip).  Workspace per row: a histogram of the top kTopkBits1 key bits and
// kTopkCtrlInts counters (both zero between calls), one segment (slot, count) per kTopkChunk positions,
// and kTopkCap candidate (key, position) pairs.
constexpr int kTopkChunk = 8192;
constexpr int kTopkBits1 = 12;
constexpr int kTopkCap = 8192;
constexpr int kTopkCtrlInts = 8;

struct TopkArgs {
  const float* logits;        // [n, ld]
  int64_t n;
  int64_t ld;
  const int32_t* lengths;     // [n]
  int k;
  int chunks;                 // ceil(ld / kTopkChunk)
  int32_t* out;               // [n, k]
  int* hist;                  // [n, 1 << kTopkBits1]
  int* ctrl;                  // [n, kTopkCtrlInts]: candidate cursor, level-1 bin, count above it,
                              // candidate count, histogram arrival counter
  int2* seg;                  // [n, chunks]: candidate slot, count
  uint2* cand;                // [n, kTopkCap]
};

// Sparse-indexer keys and logits (mla_indexer.hip).  Indexer pool page: 64 rows of 128 E4M3 codes,
// then 64 fp32 scales.
constexpr int kIndexPageBytes = 64 * 128 + 64 * 4;
constexpr int kIdxPagesPerWave = 8;
constexpr int kIdxPagesPerWg = 4 * kIdxPagesPerWave;

struct IndexKeyArgs {
  const uint16_t* keys;       // bf16 [n, 128], row stride key_stride elements
  int64_t key_stride;
  const int64_t* slot_mapping;
  int64_t n;
  uint8_t* pool;
  int64_t page_stride;
  int64_t num_pages;
};

struct IndexLogitsArgs {
  const uint16_t* q;          // bf16 [B, T, HI, 128]
  const float* w;             // [B, T, HI]
  int HI;
  const uint8_t* pool;
  int64_t page_stride;
  int64_t num_pages;
  const int32_t* block_table;
  int64_t bt_stride;
  const int32_t* ctx;         // [B]
  int B, T, causal;
  int chunks;                 // workgroups per request: ceil(pages / kIdxPagesPerWg)
  float* logits;              // [B*T, ld]
  int64_t ld;
};

// Which decode kernel serves a shape: the wide-head kernel for NVFP4 rows with 64 or 128 heads (every
// row dequantized once for all heads), the 16/32-head-group kernel otherwise.
inline bool uses_wide_kernel(int fmt, int H) { return fmt == 0 && (H == 64 || H == 128); }

hipError_t launch_quant(int fmt, const QuantArgs& a, hipStream_t stream);
hipError_t launch_decode(int fmt, const DecodeArgs& a, hipStream_t stream);
// 64 or 128 heads: one workgroup per (query token, split) covers every head (mla_decode_wide.hip).
hipError_t launch_decode_wide(int fmt, const DecodeArgs& a, hipStream_t stream);
// The staged path's unpack of each query token's selected NVFP4 rows into FP8 rows (mla_stage.hip).
hipError_t launch_stage(const StageArgs& a, hipStream_t stream);
hipError_t launch_index_key_quant(const IndexKeyArgs& a, hipStream_t stream);
hipError_t launch_index_logits(const IndexLogitsArgs& a, hipStream_t stream);
// The three launches of the index top-k (mla_topk.hip).
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);

}  // namespace mla
