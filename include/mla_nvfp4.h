/*
 * mla_nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 compressed-latent sparse-MLA decode library
 * (libmla_nvfp4.so).
 *
 * The operation (sources: "Prime Inference" launch post, sections "为低延迟解码腾出空间" (making room for
 * low-latency decode) and "原生 NVFP4 稀疏 MLA 解码内核" (native NVFP4 sparse MLA decode kernel); the independent analysis "Prime Inference: serving GLM-5.3
 * to agents is a KV-cache problem", sections "Four bits per latent value: where 352 comes from" and
 * "A kernel that reads four bits directly"):
 *   - every cached token of one layer is one row: a 512-value MLA latent stored as NVFP4 (e2m1
 *     nibbles, one E4M3 scale per 16 values) and a 64-value rope part stored as E4M3: 352 bytes,
 *     against 576 bytes for the all-FP8 row;
 *   - a decode query token attends to at most 2,048 cached positions picked by a sparse top-k
 *     indexer; unused list entries are -1; the kernel loads only the selected compressed rows and
 *     unpacks them on chip; scores and outputs accumulate in FP32.
 *
 * Row byte layout (NVFP4, 352 bytes):   [0,256)   nibbles, byte i holds element 2i in its low nibble
 *                                                 and element 2i+1 in its high nibble
 *                                       [256,288) E4M3 scale of elements 16j..16j+15 at byte 256+j
 *                                       [288,352) rope, one E4M3 byte per value, no scale
 * Row byte layout (FP8, 576 bytes):     [0,512) latent E4M3, [512,576) rope E4M3, no scale.
 * Pool: pages of 64 rows; row `slot` lives at pool + (slot/64)*page_stride_bytes + (slot%64)*row_bytes.
 * Rounding (the pages fix the format, not the rounding): block scale = E4M3 value nearest to
 * amax/6, ties to the even code, saturating at 448; element = e2m1 value nearest to |x|/scale, ties
 * to the even code, saturating at 6 (zero scale -> 0); sign bit copied from the input; rope and
 * FP8 rows: nearest E4M3, ties to even, saturating at +-448.
 *
 * Conventions for every entry point:
 *   - Pointers marked (device) are device memory owned by the caller; the library keeps none of
 *     them after the call returns and allocates nothing.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only enqueues work on it and
 *     returns; outputs are valid once the stream reaches that point.  A write into the pool and a
 *     later decode are ordered only by the caller's stream order.
 *   - Arguments are checked on the host before anything is enqueued.  On an error status nothing
 *     is enqueued and no memory is written.  MLA_ERR_HIP reports a failed launch.
 *   - There is no device-side error reporting: slot entries < 0 or on pages outside
 *     [0, num_pages) are skipped by the writers; index entries < 0, beyond the query token's limit,
 *     or on a page-table entry outside [0, num_pages) are ignored by the decoders, as if absent.
 *   - bf16 arguments are IEEE bfloat16 bit patterns (uint16), non-finite inputs are outside the
 *     contract.  A decode query may hold any finite bf16 values: the matrix operands are FP16, and each
 *     head's query is scaled by a power of two that brings its largest magnitude to [2^15, 2^16) before
 *     the conversion (undone exactly in the score scale), so no element overflows and every element
 *     within a factor 2^29 of the head's largest converts exactly.  The scores
 *     sm_scale * <q, K_i> are accumulated in fp32: they must stay below 2^120 in magnitude, and their
 *     absolute error grows with sm_scale * sum_d |q_d K_id| (about 2^-24 of it per term).
 *   - A launch's grid must fit the dispatch limits: sizes whose grid would exceed 2^32 - 1 threads
 *     return MLA_ERR_SHAPE (each entry point's limit follows from its grid, documented there).
 */
#ifndef MLA_NVFP4_H
#define MLA_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 1
#define MLA_LATENT_DIM 512
#define MLA_ROPE_DIM 64
#define MLA_QK_DIM 576
#define MLA_PAGE_TOKENS 64
#define MLA_NVFP4_ROW_BYTES 352
#define MLA_FP8_ROW_BYTES 576
#define MLA_MAX_TOPK 2048

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,         /* a required pointer is NULL */
  MLA_ERR_SHAPE = 2,        /* a size is out of range (B, T, H, topk, n, num_pages, ...) */
  MLA_ERR_STRIDE_ALIGN = 3, /* a stride is too small or a pointer / stride is misaligned */
  MLA_ERR_WORKSPACE = 4,    /* workspace smaller than the matching *_workspace_bytes() */
  MLA_ERR_DEVICE = 5,       /* the current device is not a gfx950 GPU */
  MLA_ERR_HIP = 6           /* a HIP launch failed */
} mla_status;

/* Version of this ABI (MLA_ABI_VERSION). */
int mla_abi_version(void);

/* Static text for a status code. */
const char* mla_status_string(int status);

/*
 * Quantize-on-write, NVFP4 rows (launch post, making room for low-latency decode; the write API shape follows the
 * TokenSpeed write-up's MLA KV layout section: separate nope/rope inputs plus a slot-index tensor).
 *   k_nope        (device) bf16 [n, 512], row r at k_nope + r*nope_stride elements; 16-byte aligned,
 *                 nope_stride a multiple of 8 and >= 512
 *   k_rope        (device) bf16 [n, 64], row r at k_rope + r*rope_stride elements; 16-byte aligned,
 *                 rope_stride a multiple of 8 and >= 64
 *   slot_mapping  (device) int64 [n]; token r is written to slot slot_mapping[r]; < 0 skips the token
 *   n             number of tokens, 0 <= n < 2^26 (one 64-lane wave per token; 0 enqueues nothing)
 *   pool          (device) page pool, 16-byte aligned; page_stride_bytes >= 64*352, a multiple of 16
 *   num_pages     pages in the pool (> 0); slots on pages >= num_pages are skipped
 * Writes exactly 352 bytes per written token and nothing else.  Two tokens mapped to one slot race.
 */
int mla_kv_quant_nvfp4(const void* k_nope, int64_t nope_stride, const void* k_rope, int64_t rope_stride,
                       const int64_t* slot_mapping, int64_t n, void* pool, int64_t page_stride_bytes,
                       int64_t num_pages, void* stream);

/* Quantize-on-write, 576-byte FP8 rows (the FP8 cache the pages compare against; analysis, row
 * table: no per-row scale).  Same arguments and rules as mla_kv_quant_nvfp4, with
 * page_stride_bytes >= 64*576. */
int mla_kv_quant_fp8(const void* k_nope, int64_t nope_stride, const void* k_rope, int64_t rope_stride,
                     const int64_t* slot_mapping, int64_t n, void* pool, int64_t page_stride_bytes,
                     int64_t num_pages, void* stream);

/* Split count the decoders use for this shape when num_splits = 0 (the batch-adaptive choice: the
 * launch post sizes its cooperating thread-block clusters by batch; here the selected rows of one
 * query token are split across workgroups instead). */
int mla_sparse_decode_splits(int32_t B, int32_t T, int32_t H, int32_t topk);
int mla_sparse_decode_fp8_splits(int32_t B, int32_t T, int32_t H, int32_t topk);
int mla_dense_decode_splits(int32_t B, int32_t T, int32_t H, int32_t max_context);

/* Workspace bytes a decode call with these arguments needs (0 when it runs unsplit): a fixed region of
 * 65,536 int32 split arrival counters (one per query token and head group is used; a split launch with
 * more query tokens x head groups returns MLA_ERR_SHAPE), then the FP16 partial outputs and fp32
 * log-sum-exps of the splits.  The last workgroup of a query token to finish merges its splits in the
 * same launch (the pages merge a cluster's partial results without a second launch either).
 * A workspace must be ZERO-FILLED before its first use.  Every call returns the counters it used to
 * zero, and no call writes partial results into the counter region, so a workspace can then be reused
 * without refilling by later calls of any shape on the same stream.  Two calls that can run
 * concurrently must not share a workspace. */
size_t mla_sparse_decode_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t topk, int32_t num_splits);
size_t mla_sparse_decode_fp8_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t topk, int32_t num_splits);
size_t mla_dense_decode_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t max_context, int32_t num_splits);

/*
 * Sparse MLA decode over NVFP4 rows (launch post, native NVFP4 sparse MLA decode kernel).  For every
 * query token (b, t) and head h, with L = context_lens[b] and limit = causal ? L - T + t : L - 1,
 * the selection J is the multiset of entries i of indices[b][t][:] with 0 <= i <= limit whose page
 * entry block_table[b*bt_stride + i/64] is in [0, num_pages).  Each selected row is dequantized to
 * K[576] (V = K[0..511]); then
 *     z_i = sm_scale * <q[b][t][h][:], K_i>,   out[b][t][h][:] = sum_i softmax(z)_i V_i,
 *     lse[b][t][h] = ln sum_i e^{z_i}  (natural log);  empty J gives out = 0, lse = -inf.
 *   q             (device) bf16 [B, T, H, 576] contiguous, 16-byte aligned (the absorbed query)
 *   pool          (device) NVFP4 page pool as written by mla_kv_quant_nvfp4; page_stride_bytes as there
 *   block_table   (device) int32 [B, bt_stride], request b's logical page p at block_table[b*bt_stride + p];
 *                 all bt_stride entries of each request's row are read (whatever its context length),
 *                 so the whole B*bt_stride table must be readable
 *   context_lens  (device) int32 [B], tokens in each request's cache (the T query tokens included)
 *   indices       (device) int32 [B, T, topk] logical positions, -1 = unused
 *   B, T          >= 1;  H in {16, 32, 64, 128};  1 <= topk <= 2048
 *   sm_scale      > 0, with sm_scale * log2(e) finite in fp32 (the softmax scale, 1/sqrt(192) for the
 *                 pages' model)
 *   causal        0 or 1 (the T query tokens are the last T positions of the request)
 *   num_splits    0 = the library's choice, else 1..64: the selected rows of each query token are split
 *                 into this many parts whose results are merged with their log-sum-exp weights
 *   out           (device) bf16 [B, T, H, 512], 16-byte aligned
 *   lse           (device) fp32 [B, T, H] or NULL
 *   workspace     (device) >= mla_sparse_decode_workspace_bytes(...) bytes, 256-byte aligned, zero-filled
 *                 before its first use (see above); may be NULL when that size is 0
 * The grid is B*T*(H/32, or 1 at H = 16)*S workgroups of 512 threads (at H = 64 or 128 unsplit, with
 * B*T*H/64 >= 256: B*T*H/64 workgroups of 64 heads); it must stay below 2^32 threads.
 */
int mla_sparse_decode(const void* q, const void* pool, int64_t page_stride_bytes, int64_t num_pages,
                      const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                      const int32_t* indices, int32_t B, int32_t T, int32_t H, int32_t topk, float sm_scale,
                      int32_t causal, int32_t num_splits, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * One decode step of a layer in one launch: the quantize-on-write of each query token's own new row, then
 * mla_sparse_decode over the cache with those rows in it (the pages' decode step writes the new token's
 * row into the NVFP4 cache, then attends over the selected rows).  Token t of request b is position
 * p = context_lens[b] - T + t, so its row goes to slot block_table[b*bt_stride + p/64]*64 + p%64; the
 * results (out, lse and the pool's bytes) are those of mla_kv_quant_nvfp4 of the B*T rows at these slots
 * followed by mla_sparse_decode with the same arguments.  A row whose position is negative, beyond the
 * table width, or on a page entry outside [0, num_pages) is not written (the writer skips such slots, and
 * the decode selects nothing there).
 *   k_nope, k_rope  (device) bf16 new rows [B*T, nope_stride] and [B*T, rope_stride] (row b*T + t), 512 and
 *                   64 values used, as for mla_kv_quant_nvfp4: strides >= 512 / >= 64, multiples of 8,
 *                   pointers 16-byte aligned
 *   pool            (device, written) the NVFP4 page pool
 *   other arguments, the workspace, the split choice and errors as for mla_sparse_decode.
 * Every workgroup of request b writes all T rows of the request (the same bytes) and waits for its stores
 * before its first gather, so no workgroup reads a row before it is written; other requests' lists
 * must not select these slots in the same call (they may read the old or the new bytes).
 */
int mla_sparse_decode_append(const void* q, void* pool, int64_t page_stride_bytes, int64_t num_pages,
                             const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                             const int32_t* indices, const void* k_nope, int64_t nope_stride, const void* k_rope,
                             int64_t rope_stride, int32_t B, int32_t T, int32_t H, int32_t topk, float sm_scale,
                             int32_t causal, int32_t num_splits, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * mla_sparse_decode without a workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation.  It runs the same
 * kernels with the same split choice (same results, bit for bit) and allocates nothing: the split
 * counters and partial results live in a 32 MiB device array inside the library, one per GPU the library
 * runs on, held until the process ends (mla_noalloc_scratch_bytes() returns its size).  A call whose
 * splits would need more than that (mla_sparse_decode_workspace_bytes(...) > mla_noalloc_scratch_bytes())
 * returns MLA_ERR_WORKSPACE and enqueues nothing.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents; its split counters start at zero and every call returns them to zero.
 * Calls that can overlap on one GPU (other streams, other threads) race on the array: serialize them.
 * Arguments, other errors and results as for mla_sparse_decode.
 */
size_t mla_noalloc_scratch_bytes(void);
int mla_sparse_decode_noalloc(const void* q, const void* pool, int64_t page_stride_bytes, int64_t num_pages,
                              const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                              const int32_t* indices, int32_t B, int32_t T, int32_t H, int32_t topk, float sm_scale,
                              int32_t causal, int32_t num_splits, void* out, float* lse, void* stream);

/*
 * Sparse MLA decode over 576-byte FP8 rows: the definition of mla_sparse_decode with K = the E4M3 values
 * of the row (analysis page, row table: 512 latent + 64 rope bytes, no per-row scale), over a pool
 * written by mla_kv_quant_fp8 (page_stride_bytes >= 64*576).  This is the third arm of the launch post's
 * comparison (section "原生 NVFP4 稀疏 MLA 解码内核": native NVFP4, staged NVFP4, and FP8 attention over
 * an FP8 cache; analysis page, "A kernel that reads four bits directly").  Arguments, workspace rules and
 * errors as for mla_sparse_decode (its own split choice and workspace size, below); every H runs
 * 512-thread workgroups of 16 or 32 heads, B*T*(H/32 or 1)*S of them.
 */
int mla_sparse_decode_fp8(const void* q, const void* pool, int64_t page_stride_bytes, int64_t num_pages,
                          const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                          const int32_t* indices, int32_t B, int32_t T, int32_t H, int32_t topk, float sm_scale,
                          int32_t causal, int32_t num_splits, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Dense MLA decode over 576-byte FP8 rows: the same definition with J = {0, ..., limit} (every cached
 * position), the comparison path of the launch post ("FP8 attention").  max_context >= every
 * context_lens[b] (it sizes the grid); other arguments as for mla_sparse_decode, with the pool
 * written by mla_kv_quant_fp8 (page_stride_bytes >= 64*576).  Here the entries of block_table that are
 * read are those of the pages below min(bt_stride, ceil(max_context/64)) in each request's row.
 */
int mla_dense_decode_fp8(const void* q, const void* pool, int64_t page_stride_bytes, int64_t num_pages,
                         const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens, int32_t B,
                         int32_t T, int32_t H, int32_t max_context, float sm_scale, int32_t causal,
                         int32_t num_splits, void* out, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * The staged path, for comparison (launch post, native NVFP4 sparse MLA decode section; the analysis
 * page, "A kernel that reads four bits directly": before the native kernel, the selected rows were
 * unpacked into a temporary FP8 buffer that an FP8 attention kernel then read, 352 + 576 + 576 bytes per
 * row).  For every query token id = b*T + t, the rows mla_sparse_decode would select (same rule, list
 * order) are unpacked into 576-byte FP8 rows: latent value = e2m1 x block scale (exact) cast to E4M3
 * (nearest, ties to even, saturating at 448, sign = nibble sign xor scale sign), rope bytes copied.
 * The copy is a paged FP8 cache of B*T*P pages (P = ceil(topk/64)) that mla_dense_decode_fp8 reads with
 * q viewed as [B*T, 1, H, 576], page stride 64*576, num_pages B*T*P, this call's block table (bt_stride
 * P), context_lens = staged_lens, max_context P*64 and causal 0: the causal limit is already applied.
 *   pool, page_stride_bytes, num_pages, block_table, bt_stride, context_lens, indices, B, T, topk, causal:
 *                      as for mla_sparse_decode
 *   staged             (device) B*T*P*64*576 bytes, 16-byte aligned: query token id's j-th selected row
 *                      at byte ((id*P*64) + j) * 576; rows past its count are not written
 *   staged_block_table (device) int32 [B*T, P], written: entry id*P + p
 *   staged_lens        (device) int32 [B*T], written: the number of rows staged for query token id
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE (sizes as for mla_sparse_decode; B*T below 2^20, so that up to 16
 * workgroups of 256 threads per query token fit the dispatch limit), MLA_ERR_STRIDE_ALIGN, MLA_ERR_DEVICE,
 * MLA_ERR_HIP.
 */
int mla_stage_nvfp4_fp8(const void* pool, int64_t page_stride_bytes, int64_t num_pages, const int32_t* block_table,
                        int64_t bt_stride, const int32_t* context_lens, const int32_t* indices, int32_t B, int32_t T,
                        int32_t topk, int32_t causal, void* staged, int32_t* staged_block_table, int32_t* staged_lens,
                        void* stream);

/*
 * TokenSpeed's per-token-head FP8 layout (TokenSpeed write-up, MLA KV layout section), a format variant for
 * comparison: three slot-indexed buffers, the latent as E4M3 codes lat[slot*512 ..], one fp32 scale
 * scale[slot], the rope part as bf16 rope[slot*64 ..].  Written per token, in fp32:
 *     s = max(max_i |latent_i|, 1e-26) / 448,  lat_i = E4M3(latent_i / s) (nearest, ties to even),
 *     rope_i = bf16(rope_in_i / s) (nearest, ties to even; inf past the bf16 range).
 *   k_nope, k_rope    (device) bf16, k_nope 16-byte aligned with nope_stride a multiple of 8 (>= 512),
 *                     rope_stride >= 64 elements
 *   slot_mapping      (device) int64 [n], 0 <= n < 2^26; slots < 0 or >= num_slots are skipped
 *   lat               (device) [num_slots, 512] bytes, 8-byte aligned; scale (device) fp32 [num_slots];
 *   rope              (device) bf16 [num_slots, 64]
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_STRIDE_ALIGN, MLA_ERR_DEVICE, MLA_ERR_HIP.
 */
int mla_kv_quant_pth(const void* k_nope, int64_t nope_stride, const void* k_rope, int64_t rope_stride,
                     const int64_t* slot_mapping, int64_t n, void* lat, float* scale, void* rope, int64_t num_slots,
                     void* stream);

/*
 * Sparse MLA decode over the per-token-head layout: the definition of mla_sparse_decode with position p of
 * request b at slot = block_table[b*bt_stride + p/64]*64 + p%64 (page entries in [0, num_slots/64)), and
 * K = (lat * scale, rope * scale), V = lat * scale (the inverse of the write).  Scores use FP16 latent
 * operands (each head's q scaled by a power of two into FP16's range as for mla_sparse_decode, then
 * rounded to fp16; the codes exact) and bf16 rope operands (q's rope part scaled by the same power of two,
 * exact), accumulated in fp32.
 *   lat, scale, rope, num_slots    as written by mla_kv_quant_pth (lat and rope 16-byte aligned)
 *   q, block_table, bt_stride, context_lens, indices, B, T, topk, sm_scale, causal, out, lse
 *                  as for mla_sparse_decode; H in {16, 32, 64, 128}
 *   num_splits     0 = the library's choice, else 1..64: the list is cut into chunks of ceil(topk / num_splits)
 *                  entries rounded up to whole 64-entry steps, so ceil(topk / chunk) splits run, which may be
 *                  fewer than requested (mla_sparse_decode_pth_workspace_bytes sizes for the same count)
 *   workspace      >= mla_sparse_decode_pth_workspace_bytes(...) bytes, 256-byte aligned (the splits' fp32
 *                  partial results; no zero-fill needed); may be NULL when that size is 0
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_STRIDE_ALIGN, MLA_ERR_WORKSPACE, MLA_ERR_DEVICE, MLA_ERR_HIP.
 */
size_t mla_sparse_decode_pth_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t topk, int32_t num_splits);
int mla_sparse_decode_pth(const void* q, const void* lat, const float* scale, const void* rope, int64_t num_slots,
                          const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                          const int32_t* indices, int32_t B, int32_t T, int32_t H, int32_t topk, float sm_scale,
                          int32_t causal, int32_t num_splits, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Sparse-indexer keys (analysis page, section "Four bits per latent value: where 352 comes from": 128 FP8
 * values plus a scale per token, stored the way DeepSeek's indexer is; the pages give no quantization
 * rule, and this one is the TokenSpeed write-up's per-token FP8 rule from its MLA KV layout section):
 * for each key r, with x = keys[r*key_stride .. +127] (bf16), in fp32:
 *     s = max(max_i |x_i|, 1e-26) / 448,  code_i = E4M3(x_i / s) (nearest, ties to even, saturating,
 *     sign from x_i),
 * written to indexer-pool page slot/64, row slot%64: the 128 codes at page + (slot%64)*128 and s at
 * page + 8192 + (slot%64)*4 (a page is 64 code rows, then 64 fp32 scales: 8448 bytes).
 *   keys               (device) bf16, 4-byte aligned, key_stride >= 128 elements and even
 *   slot_mapping       (device) int64 [n], 8-byte aligned; negative slots and slots on pages outside
 *                      [0, num_pages) are skipped
 *   pool               (device) 16-byte aligned, page p at pool + p*page_stride_bytes
 *   page_stride_bytes  >= 8448, a multiple of 16
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE (n < 0 or n >= 2^26, num_pages < 1), MLA_ERR_STRIDE_ALIGN, MLA_ERR_DEVICE,
 * MLA_ERR_HIP.
 */
int mla_index_key_quant(const void* keys, int64_t key_stride, const int64_t* slot_mapping, int64_t n, void* pool,
                        int64_t page_stride_bytes, int64_t num_pages, void* stream);

/*
 * Sparse-indexer logits.  No page defines them; this is the DeepSeek-style form that the analysis page
 * points to.  For query token id = b*T + t and every position p <= limit (limit as for mla_sparse_decode):
 *     logits[id*ld + p] = s_p * sum_j w[id*HI + j] * max(0, <q[id][j][:], k_p>)
 * k_p = the E4M3 values of position p's key (through the request's page table), s_p its scale; the dot
 * products are exact products accumulated in fp32 (bf16 MFMA), the head sum in fp32.  Positions whose
 * page entry is outside [0, num_pages) get -inf; positions past the limit are not written.
 *   q             (device) bf16 [B, T, HI, 128] contiguous, 16-byte aligned
 *   w             (device) fp32 [B, T, HI], 16-byte aligned (per-head weights, the softmax scale included)
 *   HI            16, 32 or 64 index heads
 *   pool, page_stride_bytes, num_pages   the indexer pool as written by mla_index_key_quant
 *   block_table, bt_stride, context_lens, B, T, causal   as for mla_sparse_decode (shared with the MLA cache)
 *   max_context   >= every context_lens[b] (it sizes the grid)
 *   logits        (device) fp32 [B*T, ld], 4-byte aligned, ld >= max_context; feed it to mla_index_topk with
 *                 lengths limit + 1
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_STRIDE_ALIGN, MLA_ERR_DEVICE, MLA_ERR_HIP.
 */
int mla_index_logits(const void* q, const float* w, int32_t HI, const void* pool, int64_t page_stride_bytes,
                     int64_t num_pages, const int32_t* block_table, int64_t bt_stride, const int32_t* context_lens,
                     int32_t B, int32_t T, int32_t max_context, int32_t causal, float* logits, int64_t ld,
                     void* stream);

/*
 * Index top-k: the sparse indexer's selection step that produces the decoders' index lists (launch post:
 * a query token attends to at most 2,048 cached positions picked by the indexer, unused entries -1; the
 * analysis page, section "Decode: TP4, and the copies it keeps": index_topk 2048).  The pages do not define the
 * indexer's logits; this call takes them as an input.  For each row r < n with m = lengths[r]:
 *   out[r][:] = the positions i < m of the k largest logits[r*ld + i], ties at the k-th largest value
 *               going to the lower positions, in ascending order; when m <= k, out[r] = 0, 1, ..., m-1
 *               followed by k - m entries of -1.
 * Values are compared as numbers (-0 equals +0; -inf and +inf are ordinary values); NaN logits are outside
 * the contract (the output is then still k distinct positions below m, or the short-row list).
 *   logits     (device) fp32, row r at logits + r*ld, 16-byte aligned; only positions below lengths[r] are
 *              read
 *   ld         row stride in elements: a multiple of 4, at least every lengths[r]; lengths[r] outside
 *              [0, ld] are clamped to it
 *   lengths    (device) int32 [n]
 *   n          rows (query tokens), >= 0; n = 0 does nothing
 *   k          1..2048
 *   out        (device) int32 [n, k], 4-byte aligned
 *   workspace  (device) >= mla_index_topk_workspace_bytes(n, ld) bytes, 256-byte aligned, zero-filled
 *              before its first use.  Every call returns its per-row histograms and counters to zero, so the
 *              workspace can be reused without refilling by later calls on the same stream with the same n
 *              and ld (zero-fill it again before a call with another n or ld).  Concurrent calls must not
 *              share a workspace.
 * Errors: MLA_ERR_SHAPE (n < 0, k outside 1..2048, ld above 2^31-1, n * ceil(ld / 8192) workgroups of 512
 * threads past 2^32 - 1 threads), MLA_ERR_STRIDE_ALIGN (ld not a positive multiple of 4, misaligned pointers), MLA_ERR_NULL,
 * MLA_ERR_WORKSPACE, MLA_ERR_DEVICE, MLA_ERR_HIP.
 */
size_t mla_index_topk_workspace_bytes(int64_t n, int64_t ld);
int mla_index_topk(const float* logits, int64_t ld, const int32_t* lengths, int64_t n, int32_t k, int32_t* out,
                   void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_NVFP4_H */
