// Internal launch interface of the sparse-indexer kernels (keys, logits, top-k) between their C ABI
// (mla_abi_index.hip) and the kernels.  Arguments are already validated when these structs are filled.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Index top-k (mla_topk.hip).  Workspace per row: a histogram of the top kTopkBits1 key bits and
// kTopkCtrlInts counters (both zero between calls), one segment (slot, count) per kTopkChunk positions,
// and kTopkCap candidate (key, position) pairs.
constexpr int kTopkChunk = 8192;
constexpr int kTopkThreads = 512;  // workgroup size of the three top-k kernels
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

hipError_t launch_index_key_quant(const IndexKeyArgs& a, hipStream_t stream);
hipError_t launch_index_logits(const IndexLogitsArgs& a, hipStream_t stream);
// The three launches of the index top-k (mla_topk.hip).
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);

}  // namespace mla
