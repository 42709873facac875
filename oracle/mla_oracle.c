/*
 * mla_oracle.c -- plain FP64 CPU oracle for NVFP4 compressed-latent sparse-MLA decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  It shares no code, header, table or helper with the HIP path
 * under nvfp4_compressed_sparse_amd/, and it includes none of that path's files.
 *
 * What it follows (page titles as in the source pages; no line numbers):
 *  - "Prime Inference" launch post (Chinese translation), section "为低延迟解码腾出空间" (making
 *    room for low-latency decode): the 512-value MLA latent is stored as NVFP4, four bits per value with one
 *    FP8 scale per group of 16 values; the 64-value rope part stays FP8; a row shrinks from 576 to
 *    352 bytes.  Section "原生 NVFP4 稀疏 MLA 解码内核" (native NVFP4 sparse MLA decode kernel): the decode reads only the rows the
 *    sparse indexer selected (at most 2,048 per query token), unpacks them and runs attention with
 *    FP32 accumulation; list entries of -1 are unused slots.
 *  - "Prime Inference: serving GLM-5.3 to agents is a KV-cache problem", section "Four bits per
 *    latent value: where 352 comes from" (row table 256 + 32 + 64 = 352; FP8 row 512 + 64 = 576 with
 *    no per-row scale) and section "A kernel that reads four bits directly".
 *  - TokenSpeed write-up, section on the MLA KV layout: the write path takes separate nope/rope
 *    tensors plus a slot-index tensor; FP8 is torch's float8_e4m3fn with maximum 448.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  - no second-level (per-tensor) scale: the row has no byte for one;
 *  - block scale = E4M3 value nearest to amax/6 (6 = largest e2m1 magnitude), ties to the even
 *    code, saturating at 448; element code = e2m1 value nearest to |x|/scale, ties to the even
 *    code, saturating at 6; a zero scale gives magnitude 0; the sign bit is the input's;
 *  - byte order: nibble bytes first (low nibble = even element), then the 32 scale bytes
 *    (scale j covers elements 16j..16j+15), then the 64 rope bytes (E4M3, no scale);
 *  - indices are logical token positions of the request, mapped through a page table of 64-token
 *    pages; entries < 0, beyond the causal limit, or whose page entry is outside the pool are
 *    ignored (as if absent); an empty selection gives out = 0 and lse = -inf;
 *  - duplicates count once per occurrence (plain multiset softmax).
 *
 * Per-token-head FP8 layout (TokenSpeed write-up, MLA KV layout section): three slot-indexed buffers,
 * latent codes [slots, 512] E4M3, one fp32 scale per slot, rope [slots, 64] in the model dtype (bf16).
 * The write is the write-up's: in fp32, s = max(amax(latent), 1e-26) / 448, codes = E4M3(x / s),
 * rope = bf16(r / s).  Readings: E4M3 and bf16 rounding nearest with ties to even (bf16 overflow gives
 * inf); the read reconstructs K = (code value * s, rope * s), the plain inverse of the write.
 *
 * Sparse indexer (analysis page, section "Four bits per latent value: where 352 comes from": the
 * indexer keeps 128 FP8 values plus a scale per token on the layers that have one, stored the way
 * DeepSeek's indexer is; the launch post and the analysis page: each query token keeps at most 2,048
 * positions).  The pages give the key size, not the quantization or the logits; readings:
 *  - key quantization as in the TokenSpeed write-up's per-token FP8 path (its MLA KV layout section):
 *    in fp32, s = max(amax, 1e-26) / 448, each value E4M3(x / s) nearest with ties to even, saturating;
 *    page layout: 64 rows of 128 code bytes, then 64 fp32 scales;
 *  - logits, PARITY UNPINNED (no page defines them; the DeepSeek-style form the analysis page points
 *    to): logit(p) = s_p * sum_j w_j * max(0, <q_j, e4m3(code_p)>) over the index heads j.
 *
 * Floating point: everything in double.  Encoding decisions are exact: distances between a bf16
 * input and a candidate grid value are computed exactly in double (the bit span of both operands
 * fits in 53 bits inside the guarded range; outside it the nearest value is fixed by saturation or
 * by the zero end of the grid).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define LATENT 512
#define ROPE 64
#define QK (LATENT + ROPE)
#define PAGE 64
#define NVFP4_ROW 352 /* 512/2 nibble bytes + 512/16 scale bytes + 64 rope bytes */
#define FP8_ROW 576   /* 512 + 64 E4M3 bytes */

/* ------------------------------------------------------------------ value definitions */

/* bf16 bit pattern -> exact value (bf16 is the upper half of an IEEE binary32). */
double mlo_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* E4M3FN byte s.eeee.mmm -> value.  Exponent bias 7, no infinities, 0x7F/0xFF are NaN, largest
 * finite 448 (torch.float8_e4m3fn). */
double mlo_e4m3_value(uint32_t code) {
  code &= 0xFF;
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp((double)m, -9)                   /* subnormal: m/8 * 2^-6 */
                      : ldexp(1.0 + (double)m / 8.0, e - 7);   /* normal */
  return s ? -v : v;
}

/* e2m1 nibble s.ee.m -> value.  Exponent bias 1: ee = 0 is subnormal (0 or 0.5), otherwise
 * 2^(ee-1) * (1 + m/2).  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double mlo_e2m1_value(uint32_t code) {
  code &= 0xF;
  int s = code >> 3, e = (code >> 1) & 3, m = code & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* ------------------------------------------------------------------ encoders (nearest value) */

/* Code (0..126) of the non-negative finite E4M3FN value nearest to num/den, ties to the even
 * code.  num >= 0, den > 0, num a bf16 value or a product e2m1 x E4M3 (at most 6 significant bits),
 * den in {1, 6}.  Brute force over every candidate. */
static uint32_t nearest_e4m3_code(double num, double den) {
  if (num >= 448.0 * den) return 0x7E;               /* nothing finite lies above 448 */
  if (num <= ldexp(den, -10)) return 0;              /* at most half the smallest step: 0 (tie -> even 0) */
  uint32_t best = 0;
  double bestd = INFINITY;
  for (uint32_t c = 0; c <= 0x7E; ++c) {
    double d = fabs(num - den * mlo_e4m3_value(c));  /* exact in this range */
    if (d < bestd || (d == bestd && (c & 1) == 0)) { best = c; bestd = d; }
  }
  return best;
}

/* E4M3FN byte for a bf16 input: nearest finite value, ties to even, saturating at +-448, sign bit
 * copied from the input (so -0 and tiny negatives give 0x80). */
uint32_t mlo_e4m3_encode_bf16(uint16_t x) {
  double v = mlo_bf16_value(x);
  uint32_t sign = (x >> 15) & 1;
  return (sign << 7) | nearest_e4m3_code(fabs(v), 1.0);
}

/* Block scale byte for a block whose largest magnitude is amax (a bf16 value): the E4M3 value
 * nearest to amax / 6. */
uint32_t mlo_scale_code(double amax) { return nearest_e4m3_code(amax, 6.0); }

/* e2m1 nibble for a bf16 input under a block scale byte: magnitude = e2m1 grid point nearest to
 * |x| / scale, ties to the even code, saturating at 6; zero scale gives magnitude 0; sign copied. */
uint32_t mlo_e2m1_encode(uint16_t x, uint32_t scale_code) {
  static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  uint32_t sign = (x >> 15) & 1;
  double a = fabs(mlo_bf16_value(x));
  double s = mlo_e4m3_value(scale_code);
  uint32_t best = 0;
  if (s == 0.0 || a <= 0.25 * s) {
    best = 0;
  } else if (a >= 6.0 * s) {
    best = 7;
  } else {
    double bestd = INFINITY;
    for (uint32_t k = 0; k < 8; ++k) {
      double d = fabs(a - s * grid[k]);  /* exact: both sides have few significant bits */
      if (d < bestd || (d == bestd && (k & 1) == 0)) { best = k; bestd = d; }
    }
  }
  return (sign << 3) | best;
}

void mlo_e2m1_encode_bulk(const uint16_t* x, int64_t n, uint32_t scale_code, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)mlo_e2m1_encode(x[i], scale_code);
}
void mlo_e4m3_encode_bulk(const uint16_t* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)mlo_e4m3_encode_bf16(x[i]);
}
void mlo_scale_code_bulk(const uint16_t* amax, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)mlo_scale_code(fabs(mlo_bf16_value(amax[i])));
}

/* ------------------------------------------------------------------ one row */

/* Quantize one token: latent[512] and rope[64] given as bf16 bits -> 352-byte NVFP4 row. */
void mlo_quant_row_nvfp4(const uint16_t* latent, const uint16_t* rope, uint8_t* row) {
  for (int j = 0; j < LATENT / 16; ++j) {
    double amax = 0.0;
    for (int i = 0; i < 16; ++i) {
      double a = fabs(mlo_bf16_value(latent[16 * j + i]));
      if (a > amax) amax = a;
    }
    uint32_t sc = mlo_scale_code(amax);
    row[256 + j] = (uint8_t)sc;
    for (int k = 0; k < 8; ++k) {
      uint32_t lo = mlo_e2m1_encode(latent[16 * j + 2 * k], sc);
      uint32_t hi = mlo_e2m1_encode(latent[16 * j + 2 * k + 1], sc);
      row[8 * j + k] = (uint8_t)(lo | (hi << 4));
    }
  }
  for (int i = 0; i < ROPE; ++i) row[288 + i] = (uint8_t)mlo_e4m3_encode_bf16(rope[i]);
}

/* Quantize one token to the 576-byte FP8 row: every value cast to E4M3, no scale. */
void mlo_quant_row_fp8(const uint16_t* latent, const uint16_t* rope, uint8_t* row) {
  for (int i = 0; i < LATENT; ++i) row[i] = (uint8_t)mlo_e4m3_encode_bf16(latent[i]);
  for (int i = 0; i < ROPE; ++i) row[LATENT + i] = (uint8_t)mlo_e4m3_encode_bf16(rope[i]);
}

/* 352-byte row -> K[576]; V is K[0..511]. */
void mlo_dequant_row_nvfp4(const uint8_t* row, double* K) {
  for (int d = 0; d < LATENT; ++d) {
    uint32_t byte = row[d / 2];
    uint32_t nib = (d & 1) ? (byte >> 4) : (byte & 15);
    K[d] = mlo_e2m1_value(nib) * mlo_e4m3_value(row[256 + d / 16]);
  }
  for (int i = 0; i < ROPE; ++i) K[LATENT + i] = mlo_e4m3_value(row[288 + i]);
}

void mlo_dequant_row_fp8(const uint8_t* row, double* K) {
  for (int d = 0; d < QK; ++d) K[d] = mlo_e4m3_value(row[d]);
}

/* ------------------------------------------------------------------ quantize-on-write */

/* Write n tokens into a paged pool.  Token r goes to slot = slot_mapping[r]: page slot>>6, row
 * slot&63, at pool + page*page_stride + (slot&63)*row_bytes.  Negative slots and slots whose page
 * is outside [0, num_pages) are skipped.  Strides are in elements.  fmt: 0 = NVFP4, 1 = FP8. */
static int64_t quant_pool(int fmt, const uint16_t* k_nope, int64_t nope_stride, const uint16_t* k_rope,
                          int64_t rope_stride, const int64_t* slot_mapping, int64_t n, uint8_t* pool,
                          int64_t page_stride, int64_t num_pages) {
  int64_t written = 0;
  int row_bytes = fmt == 0 ? NVFP4_ROW : FP8_ROW;
  for (int64_t r = 0; r < n; ++r) {
    int64_t slot = slot_mapping[r];
    if (slot < 0) continue;
    int64_t page = slot / PAGE;
    if (page >= num_pages) continue;
    uint8_t* dst = pool + page * page_stride + (slot % PAGE) * row_bytes;
    if (fmt == 0) mlo_quant_row_nvfp4(k_nope + r * nope_stride, k_rope + r * rope_stride, dst);
    else mlo_quant_row_fp8(k_nope + r * nope_stride, k_rope + r * rope_stride, dst);
    ++written;
  }
  return written;
}

int64_t mlo_kv_quant_nvfp4(const uint16_t* k_nope, int64_t nope_stride, const uint16_t* k_rope, int64_t rope_stride,
                           const int64_t* slot_mapping, int64_t n, uint8_t* pool, int64_t page_stride,
                           int64_t num_pages) {
  return quant_pool(0, k_nope, nope_stride, k_rope, rope_stride, slot_mapping, n, pool, page_stride, num_pages);
}

int64_t mlo_kv_quant_fp8(const uint16_t* k_nope, int64_t nope_stride, const uint16_t* k_rope, int64_t rope_stride,
                         const int64_t* slot_mapping, int64_t n, uint8_t* pool, int64_t page_stride,
                         int64_t num_pages) {
  return quant_pool(1, k_nope, nope_stride, k_rope, rope_stride, slot_mapping, n, pool, page_stride, num_pages);
}

/* ------------------------------------------------------------------ attention */

/* Softmax attention of one query token (all H heads) over the rows K[j] (j < nrows, dequantized):
 *   z_j = sm_scale * <q_h, K_j>,  out_h = sum_j e^(z_j - m) V_j / sum_j e^(z_j - m),
 *   lse_h = m + ln sum_j e^(z_j - m),  with m = max_j z_j.  nrows = 0 gives out = 0, lse = -inf. */
static void attend(const uint16_t* q, int H, const double* K, int64_t nrows, double sm_scale, double* out,
                   double* lse, double* z) {
  for (int h = 0; h < H; ++h) {
    double* o = out + (int64_t)h * LATENT;
    for (int d = 0; d < LATENT; ++d) o[d] = 0.0;
    if (nrows == 0) {
      lse[h] = -INFINITY;
      continue;
    }
    const uint16_t* qh = q + (int64_t)h * QK;
    double m = -INFINITY;
    for (int64_t j = 0; j < nrows; ++j) {
      const double* Kj = K + j * QK;
      double acc = 0.0;
      for (int d = 0; d < QK; ++d) acc += mlo_bf16_value(qh[d]) * Kj[d];
      z[j] = sm_scale * acc;
      if (z[j] > m) m = z[j];
    }
    double Z = 0.0;
    for (int64_t j = 0; j < nrows; ++j) {
      double w = exp(z[j] - m);
      Z += w;
      const double* Vj = K + j * QK;
      for (int d = 0; d < LATENT; ++d) o[d] += w * Vj[d];
    }
    for (int d = 0; d < LATENT; ++d) o[d] /= Z;
    lse[h] = m + log(Z);
  }
}

/* Largest position query token t of a request with context length L may see. */
static int64_t position_limit(int64_t L, int T, int t, int causal) { return causal ? L - T + t : L - 1; }

/* Address of the row at logical position pos of request b, or NULL if the position or its page entry
 * is not usable. */
static const uint8_t* row_address(const uint8_t* pool, int64_t page_stride, int64_t num_pages, int row_bytes,
                                  const int32_t* block_table, int64_t bt_stride, int b, int64_t pos,
                                  int64_t lim) {
  if (pos < 0 || pos > lim) return NULL;
  int64_t page = block_table[(int64_t)b * bt_stride + pos / PAGE];
  if (page < 0 || page >= num_pages) return NULL;
  return pool + page * page_stride + (pos % PAGE) * row_bytes;
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  return omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}

/* Sparse decode over one row format (0 = NVFP4 352-byte rows, 1 = FP8 576-byte rows).  q bf16
 * [B,T,H,576]; indices int32 [B,T,topk]; out double [n_units,H,512]; lse double [n_units,H].  units:
 * optional list of query-token ids b*T+t to compute (NULL: all B*T in order).  Returns the number of
 * threads used. */
static int sparse_decode_rows(int fmt, const uint16_t* q, const uint8_t* pool, int64_t page_stride, int64_t num_pages,
                              const int32_t* block_table, int64_t bt_stride, const int32_t* ctx,
                              const int32_t* indices, int B, int T, int H, int topk, double sm_scale, int causal,
                              const int64_t* units, int64_t n_units, double* out, double* lse, int nthreads) {
  int used = set_threads(nthreads);
  int64_t nq = units ? n_units : (int64_t)B * T;
  int row_bytes = fmt == 0 ? NVFP4_ROW : FP8_ROW;
#pragma omp parallel
  {
    double* K = (double*)malloc(sizeof(double) * QK * (topk > 0 ? topk : 1));
    double* z = (double*)malloc(sizeof(double) * (topk > 0 ? topk : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < nq; ++u) {
      int64_t id = units ? units[u] : u;
      int b = (int)(id / T), t = (int)(id % T);
      int64_t lim = position_limit(ctx[b], T, t, causal);
      const int32_t* idx = indices + id * topk;
      int64_t nrows = 0;
      for (int j = 0; j < topk; ++j) {
        const uint8_t* row = row_address(pool, page_stride, num_pages, row_bytes, block_table, bt_stride, b,
                                         idx[j], lim);
        if (!row) continue;
        if (fmt == 0) mlo_dequant_row_nvfp4(row, K + (nrows++) * QK);
        else mlo_dequant_row_fp8(row, K + (nrows++) * QK);
      }
      attend(q + id * H * QK, H, K, nrows, sm_scale, out + u * H * LATENT, lse + u * H, z);
    }
    free(K);
    free(z);
  }
  return used;
}

/* Sparse decode over NVFP4 rows (launch post, native NVFP4 sparse MLA decode kernel). */
int mlo_sparse_decode(const uint16_t* q, const uint8_t* pool, int64_t page_stride, int64_t num_pages,
                      const int32_t* block_table, int64_t bt_stride, const int32_t* ctx, const int32_t* indices,
                      int B, int T, int H, int topk, double sm_scale, int causal, const int64_t* units,
                      int64_t n_units, double* out, double* lse, int nthreads) {
  return sparse_decode_rows(0, q, pool, page_stride, num_pages, block_table, bt_stride, ctx, indices, B, T, H, topk,
                            sm_scale, causal, units, n_units, out, lse, nthreads);
}

/* The same sparse decode over 576-byte FP8 rows: the third arm of the launch post's comparison (native
 * NVFP4 / staged NVFP4 / FP8 attention over an FP8 cache, section "原生 NVFP4 稀疏 MLA 解码内核";
 * analysis page, "A kernel that reads four bits directly").  Same selection rule; K = E4M3 values of the
 * row (analysis page, row table: no per-row scale). */
int mlo_sparse_decode_fp8(const uint16_t* q, const uint8_t* pool, int64_t page_stride, int64_t num_pages,
                          const int32_t* block_table, int64_t bt_stride, const int32_t* ctx, const int32_t* indices,
                          int B, int T, int H, int topk, double sm_scale, int causal, const int64_t* units,
                          int64_t n_units, double* out, double* lse, int nthreads) {
  return sparse_decode_rows(1, q, pool, page_stride, num_pages, block_table, bt_stride, ctx, indices, B, T, H, topk,
                            sm_scale, causal, units, n_units, out, lse, nthreads);
}

/* Dense decode over an FP8 (576-byte row) cache: every position 0..limit is selected. */
int mlo_dense_decode_fp8(const uint16_t* q, const uint8_t* pool, int64_t page_stride, int64_t num_pages,
                         const int32_t* block_table, int64_t bt_stride, const int32_t* ctx, int B, int T, int H,
                         double sm_scale, int causal, const int64_t* units, int64_t n_units, double* out,
                         double* lse, int nthreads) {
  int used = set_threads(nthreads);
  int64_t nq = units ? n_units : (int64_t)B * T;
  int64_t maxL = 1;
  for (int b = 0; b < B; ++b)
    if (ctx[b] > maxL) maxL = ctx[b];
#pragma omp parallel
  {
    double* K = (double*)malloc(sizeof(double) * QK * maxL);
    double* z = (double*)malloc(sizeof(double) * maxL);
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < nq; ++u) {
      int64_t id = units ? units[u] : u;
      int b = (int)(id / T), t = (int)(id % T);
      int64_t lim = position_limit(ctx[b], T, t, causal);
      int64_t nrows = 0;
      for (int64_t pos = 0; pos <= lim; ++pos) {
        const uint8_t* row = row_address(pool, page_stride, num_pages, FP8_ROW, block_table, bt_stride, b, pos, lim);
        if (row) mlo_dequant_row_fp8(row, K + (nrows++) * QK);
      }
      attend(q + id * H * QK, H, K, nrows, sm_scale, out + u * H * LATENT, lse + u * H, z);
    }
    free(K);
    free(z);
  }
  return used;
}

/* ------------------------------------------------------------------ staged path */

/* The staged path the launch post used first (section "原生 NVFP4 稀疏 MLA 解码内核"; analysis
 * page, section "A kernel that reads four bits directly", staged-versus-native figure): the rows a
 * query token selects are unpacked from NVFP4 into 576-byte FP8 rows of a temporary buffer, and an FP8
 * attention kernel reads that copy.  Query token id = b*T + t gets its selected rows (the sparse
 * decode's selection, in list order) at staged rows id*rows_per_token + 0..n-1, and counts[id] = n.
 * Latent value d of a row is the exact product e2m1 x block scale, cast to E4M3 (nearest finite, ties
 * to the even code, saturating at 448; sign = nibble sign xor scale sign); the 64 rope bytes are copied.
 * Staged rows past n are left as they were.  Scale bytes 0x7F/0xFF (NaN) never come from the writer;
 * their output is not defined here. */
void mlo_stage_nvfp4_fp8(const uint8_t* pool, int64_t page_stride, int64_t num_pages, const int32_t* block_table,
                         int64_t bt_stride, const int32_t* ctx, const int32_t* indices, int B, int T, int topk,
                         int causal, int64_t rows_per_token, uint8_t* staged, int32_t* counts) {
  for (int64_t id = 0; id < (int64_t)B * T; ++id) {
    int b = (int)(id / T), t = (int)(id % T);
    int64_t lim = position_limit(ctx[b], T, t, causal);
    const int32_t* idx = indices + id * topk;
    int32_t n = 0;
    for (int j = 0; j < topk; ++j) {
      const uint8_t* row = row_address(pool, page_stride, num_pages, NVFP4_ROW, block_table, bt_stride, b, idx[j], lim);
      if (!row) continue;
      uint8_t* dst = staged + (id * rows_per_token + n) * FP8_ROW;
      for (int d = 0; d < LATENT; ++d) {
        uint32_t byte = row[d / 2];
        uint32_t nib = (d & 1) ? (byte >> 4) : (byte & 15);
        uint32_t sc = row[256 + d / 16];
        double mag = fabs(mlo_e2m1_value(nib)) * fabs(mlo_e4m3_value(sc));
        uint32_t sign = ((nib >> 3) ^ (sc >> 7)) & 1;
        dst[d] = (uint8_t)((sign << 7) | nearest_e4m3_code(mag, 1.0));
      }
      memcpy(dst + LATENT, row + 288, ROPE);
      ++n;
    }
    counts[id] = n;
  }
}

/* ------------------------------------------------------------------ per-token-head FP8 layout */

/* fp32 -> bf16 bits, nearest with ties to even (finite inputs; values past the largest bf16 give inf). */
static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* One token: latent bf16 [512] and rope bf16 [64] -> codes [512], scale, rope bf16 [64] (fp32 steps). */
void mlo_pth_quant_row(const uint16_t* lat, const uint16_t* rope, uint8_t* codes, float* scale, uint16_t* rq) {
  float amax = 0.0f;
  for (int i = 0; i < LATENT; ++i) {
    float v = fabsf((float)mlo_bf16_value(lat[i]));
    if (v > amax) amax = v;
  }
  float s = (amax > 1e-26f ? amax : 1e-26f) / 448.0f;
  for (int i = 0; i < LATENT; ++i) {
    float y = (float)mlo_bf16_value(lat[i]) / s;
    uint32_t sign = (lat[i] >> 15) & 1;
    codes[i] = (uint8_t)((sign << 7) | nearest_e4m3_code(fabs((double)y), 1.0));
  }
  for (int i = 0; i < ROPE; ++i) rq[i] = f32_to_bf16_rne((float)mlo_bf16_value(rope[i]) / s);
  *scale = s;
}

/* Write n tokens; token r goes to slot slot_mapping[r] (negative or >= num_slots: skipped).  Strides in
 * elements. */
int64_t mlo_kv_quant_pth(const uint16_t* k_nope, int64_t nope_stride, const uint16_t* k_rope, int64_t rope_stride,
                         const int64_t* slot_mapping, int64_t n, uint8_t* lat_buf, float* scale_buf,
                         uint16_t* rope_buf, int64_t num_slots) {
  int64_t written = 0;
  for (int64_t r = 0; r < n; ++r) {
    int64_t slot = slot_mapping[r];
    if (slot < 0 || slot >= num_slots) continue;
    mlo_pth_quant_row(k_nope + r * nope_stride, k_rope + r * rope_stride, lat_buf + slot * LATENT, scale_buf + slot,
                      rope_buf + slot * ROPE);
    ++written;
  }
  return written;
}

/* K[576] of one slot: code values times the scale, then the stored rope times the scale. */
void mlo_dequant_row_pth(const uint8_t* codes, float scale, const uint16_t* rq, double* K) {
  for (int i = 0; i < LATENT; ++i) K[i] = mlo_e4m3_value(codes[i]) * (double)scale;
  for (int i = 0; i < ROPE; ++i) K[LATENT + i] = mlo_bf16_value(rq[i]) * (double)scale;
}

/* Sparse decode over the per-token-head layout: the selection rule of mlo_sparse_decode, with slots
 * page*64 + position%64 for page entries in [0, num_slots/64). */
int mlo_sparse_decode_pth(const uint16_t* q, const uint8_t* lat_buf, const float* scale_buf, const uint16_t* rope_buf,
                          int64_t num_slots, const int32_t* block_table, int64_t bt_stride, const int32_t* ctx,
                          const int32_t* indices, int B, int T, int H, int topk, double sm_scale, int causal,
                          const int64_t* units, int64_t n_units, double* out, double* lse, int nthreads) {
  int used = set_threads(nthreads);
  int64_t nq = units ? n_units : (int64_t)B * T;
  int64_t num_pages = num_slots / PAGE;
#pragma omp parallel
  {
    double* K = (double*)malloc(sizeof(double) * QK * (topk > 0 ? topk : 1));
    double* z = (double*)malloc(sizeof(double) * (topk > 0 ? topk : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < nq; ++u) {
      int64_t id = units ? units[u] : u;
      int b = (int)(id / T), t = (int)(id % T);
      int64_t lim = position_limit(ctx[b], T, t, causal);
      const int32_t* idx = indices + id * topk;
      int64_t nrows = 0;
      for (int j = 0; j < topk; ++j) {
        int64_t pos = idx[j];
        if (pos < 0 || pos > lim) continue;
        int64_t page = block_table[(int64_t)b * bt_stride + pos / PAGE];
        if (page < 0 || page >= num_pages) continue;
        int64_t slot = page * PAGE + pos % PAGE;
        mlo_dequant_row_pth(lat_buf + slot * LATENT, scale_buf[slot], rope_buf + slot * ROPE, K + (nrows++) * QK);
      }
      attend(q + id * H * QK, H, K, nrows, sm_scale, out + u * H * LATENT, lse + u * H, z);
    }
    free(K);
    free(z);
  }
  return used;
}

/* ------------------------------------------------------------------ sparse indexer */

#define IDX_DIM 128
#define IDX_PAGE_CODES (PAGE * IDX_DIM) /* scales follow the 64 code rows of a page */

/* One indexer key: 128 bf16 values -> 128 E4M3 codes and an fp32 scale (fp32 arithmetic, as the
 * per-token FP8 path computes it).  The codes are the nearest E4M3 values to the fp32 quotients,
 * with the input's sign. */
void mlo_index_key_quant_row(const uint16_t* x, uint8_t* codes, float* scale) {
  float amax = 0.0f;
  for (int i = 0; i < IDX_DIM; ++i) {
    float v = fabsf((float)mlo_bf16_value(x[i]));
    if (v > amax) amax = v;
  }
  float s = (amax > 1e-26f ? amax : 1e-26f) / 448.0f;
  for (int i = 0; i < IDX_DIM; ++i) {
    float y = (float)mlo_bf16_value(x[i]) / s;
    uint32_t sign = (x[i] >> 15) & 1;
    codes[i] = (uint8_t)((sign << 7) | nearest_e4m3_code(fabs((double)y), 1.0));
  }
  *scale = s;
}

/* Write n indexer keys into a paged pool (page p at pool + p*page_stride: 64 rows of 128 code bytes,
 * then 64 fp32 scales).  Negative slots and slots on pages outside [0, num_pages) are skipped.
 * key_stride in elements. */
int64_t mlo_index_key_quant(const uint16_t* keys, int64_t key_stride, const int64_t* slot_mapping, int64_t n,
                            uint8_t* pool, int64_t page_stride, int64_t num_pages) {
  int64_t written = 0;
  for (int64_t r = 0; r < n; ++r) {
    int64_t slot = slot_mapping[r];
    if (slot < 0 || slot / PAGE >= num_pages) continue;
    uint8_t* page = pool + (slot / PAGE) * page_stride;
    float sc;
    mlo_index_key_quant_row(keys + r * key_stride, page + (slot % PAGE) * IDX_DIM, &sc);
    memcpy(page + IDX_PAGE_CODES + (slot % PAGE) * 4, &sc, 4);
    ++written;
  }
  return written;
}

/* Indexer logits of query token id = b*T + t (parity unpinned: the form is a reading, see the file
 * header) over positions p <= limit: logits[id*ld + p] = s_p * sum_j w[id*HI + j] * max(0, <q_j, k_p>)
 * with k_p the E4M3 values of the key's codes, in double.  q bf16 [B,T,HI,128], w fp32 [B,T,HI].
 * Positions on a page entry outside [0, num_pages) get -inf; positions past the limit are left as
 * they are. */
int mlo_index_logits(const uint16_t* q, const float* w, int HI, const uint8_t* pool, int64_t page_stride,
                     int64_t num_pages, const int32_t* block_table, int64_t bt_stride, const int32_t* ctx, int B,
                     int T, int causal, double* logits, int64_t ld, int nthreads) {
  int used = set_threads(nthreads);
#pragma omp parallel for schedule(dynamic)
  for (int64_t id = 0; id < (int64_t)B * T; ++id) {
    int b = (int)(id / T), t = (int)(id % T);
    int64_t lim = position_limit(ctx[b], T, t, causal);
    double* qd = (double*)malloc(sizeof(double) * HI * IDX_DIM);
    for (int64_t i = 0; i < (int64_t)HI * IDX_DIM; ++i) qd[i] = mlo_bf16_value(q[id * HI * IDX_DIM + i]);
    for (int64_t p = 0; p <= lim && p < ld; ++p) {
      int64_t page = block_table[(int64_t)b * bt_stride + p / PAGE];
      if (page < 0 || page >= num_pages) {
        logits[id * ld + p] = -INFINITY;
        continue;
      }
      const uint8_t* codes = pool + page * page_stride + (p % PAGE) * IDX_DIM;
      float sc;
      memcpy(&sc, pool + page * page_stride + IDX_PAGE_CODES + (p % PAGE) * 4, 4);
      double k[IDX_DIM];
      for (int d = 0; d < IDX_DIM; ++d) k[d] = mlo_e4m3_value(codes[d]);
      double acc = 0.0;
      for (int j = 0; j < HI; ++j) {
        double dot = 0.0;
        for (int d = 0; d < IDX_DIM; ++d) dot += qd[j * IDX_DIM + d] * k[d];
        if (dot > 0.0) acc += (double)w[id * HI + j] * dot;
      }
      logits[id * ld + p] = (double)sc * acc;
    }
    free(qd);
  }
  return used;
}

/* Merge S partial results of one query token computed over disjoint parts of its selection:
 *   M = max_s lse_s,  lse = M + ln sum_s e^(lse_s - M),  out = sum_s e^(lse_s - lse) out_s.
 * o_parts [S,H,512], lse_parts [S,H]; parts with lse = -inf carry no weight; all -inf gives 0/-inf. */
void mlo_merge_partials(const double* o_parts, const double* lse_parts, int S, int H, double* out, double* lse) {
  for (int h = 0; h < H; ++h) {
    double M = -INFINITY;
    for (int s = 0; s < S; ++s)
      if (lse_parts[s * H + h] > M) M = lse_parts[s * H + h];
    double* o = out + (int64_t)h * LATENT;
    for (int d = 0; d < LATENT; ++d) o[d] = 0.0;
    if (M == -INFINITY) {
      lse[h] = -INFINITY;
      continue;
    }
    double Z = 0.0;
    for (int s = 0; s < S; ++s) Z += exp(lse_parts[s * H + h] - M);
    lse[h] = M + log(Z);
    for (int s = 0; s < S; ++s) {
      double w = exp(lse_parts[s * H + h] - lse[h]);
      if (w == 0.0) continue;
      const double* os = o_parts + ((int64_t)s * H + h) * LATENT;
      for (int d = 0; d < LATENT; ++d) o[d] += w * os[d];
    }
  }
}
