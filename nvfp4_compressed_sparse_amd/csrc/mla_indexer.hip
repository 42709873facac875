// The sparse indexer's keys and logits.  The pages give the key size: the analysis page ("Four bits
// per latent value: where 352 comes from") counts 128 FP8 values plus a scale per token, stored the way
// DeepSeek's indexer is, and the launch post lets each query token keep at most 2,048 positions.  The
// key quantization follows the TokenSpeed write-up's per-token FP8 path (its MLA KV layout section) and
// the logits are the DeepSeek-style form; both are readings, and the logits' form is not defined by any
// page:
//   key:    s = max(amax, 1e-26) / 448 in fp32, codes = E4M3(x / s) (nearest, ties to even);
//   logit:  logit(p) = s_p * sum_j w_j * max(0, <q_j, k_p>) over the index heads j, k_p the key's
//           E4M3 values (exact in bf16), q_j bf16, products accumulated in fp32.
//
// Pool page (64 positions): 64 rows of 128 code bytes, then 64 fp32 scales (8448 bytes).
//
// index_key_quant_kernel: one wave per key, lane l holds values 2l and 2l+1; the amax is a wave
// maximum; each lane writes its two code bytes, lane 0 the scale.
//
// index_logits_kernel (used when a request's q does not fit the LDS budget of index_logits_multi_kernel,
// which otherwise serves every T and is described below): each wave takes kIdxPagesPerWave consecutive
// 64-position pages of a request (four
// waves per workgroup).  For each query token of the request the wave loads q once and walks its pages,
// the next two pages' keys in flight while it computes S = Q K^T for all index heads with bf16 MFMA
// 16x16x32:
// A = q (16 heads x 32 dims), B = keys (32 dims x 16 positions).  Lane l holds, for position row l%16
// of a 16-position tile, the 32 contiguous key bytes 32(l/16)..32(l/16)+31 (two 16-byte loads), and in
// k-step ks it feeds bytes 8ks..8ks+7 of them; the q fragment uses the same dimension order (dims
// 32(l/16)+8ks..+7), which leaves every dot product unchanged.  The accumulator lane l holds position
// l%16 and heads 4(l/16)..4(l/16)+3 of a 16-head tile, so the ReLU-weighted head sum is a sum over the
// lane's own values, then over the four lane groups (two xor-shuffles).  Lane l then writes position l
// of the page, scaled by s_p.  Positions past the query token's limit are not written; positions on a
// page-table entry outside the pool get -inf.
#include "mla_device.h"
#include "mla_index_internal.h"

namespace mla {

constexpr int kIdxDim = 128;
constexpr int kIdxCodes = 64 * kIdxDim;  // scales follow the page's code rows
constexpr size_t kIdxMultiMaxLds = 72 * 1024;  // q and w of the request's tokens, for T > 1

__global__ __launch_bounds__(256) void index_key_quant_kernel(IndexKeyArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.n) return;
  const int64_t slot = a.slot_mapping[r];
  if (slot < 0 || slot / 64 >= a.num_pages) return;
  const uint32_t xv = *reinterpret_cast<const uint32_t*>(a.keys + r * a.key_stride + 2 * lane);
  const float x0 = bf16_to_f32(xv & 0xFFFFu), x1 = bf16_to_f32(xv >> 16);
  float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  const float s = fmaxf(amax, 1e-26f) / 448.0f;  // correctly rounded fp32 division
  const uint32_t c0 = f32_to_e4m3(x0 / s), c1 = f32_to_e4m3(x1 / s);
  uint8_t* page = a.pool + (slot / 64) * a.page_stride;
  *reinterpret_cast<uint16_t*>(page + (slot % 64) * kIdxDim + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
  if (lane == 0) *reinterpret_cast<float*>(page + kIdxCodes + (slot % 64) * 4) = s;
}

// 8 E4M3 bytes (two dwords) -> 8 bf16 values in MFMA operand order (exact).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  return as_bf16x8(e4m3x2_to_bf16x2<false>(lo), e4m3x2_to_bf16x2<true>(lo), e4m3x2_to_bf16x2<false>(hi),
                   e4m3x2_to_bf16x2<true>(hi));
}

// A wave's page: the key fragments (tile nt, position row r16, bytes 32g..32g+31) and the scale of
// position 64-page offset `lane`.
struct IndexPage {
  u32x4 k[4][2];
  float sc;
};

__device__ __forceinline__ void load_index_page(const uint8_t* base, int r16, int g, int lane, IndexPage& pg) {
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      pg.k[nt][h] = *reinterpret_cast<const u32x4*>(base + (16 * nt + r16) * kIdxDim + 32 * g + 16 * h);
  pg.sc = *reinterpret_cast<const float*>(base + kIdxCodes + 4 * lane);
}

template <int HI>
__global__ __launch_bounds__(256) void index_logits_kernel(IndexLogitsArgs a) {
  constexpr int MT = HI / 16;  // head tiles
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int b = blockIdx.x / a.chunks;
  const int pg_first = (blockIdx.x % a.chunks) * kIdxPagesPerWg + (threadIdx.x >> 6) * kIdxPagesPerWave;
  const int L = a.ctx[b];
  const int p_end = L < a.ld ? L : (int)a.ld;  // positions this request can write
  if (pg_first * 64 >= p_end) return;
  const int n_pages = min(kIdxPagesPerWave, (p_end - pg_first * 64 + 63) / 64);

  // the wave's page-table entries, loaded once (lane j: page pg_first + j; entry 0 read in place of an
  // entry past the table) so that no page waits for its own table lookup
  const int pj = pg_first + (lane < kIdxPagesPerWave ? lane : 0);
  const int32_t tab = a.block_table[(int64_t)b * a.bt_stride + (pj < a.bt_stride ? pj : 0)];
  const int32_t phys_lane = pj < a.bt_stride ? tab : -1;
  // the keys of the wave's page i, or page 0 of the pool (always readable; its values are discarded)
  // for a page whose table entry is outside the pool or past the wave's pages: the loads stay
  // unconditional, so the compiler can keep pages in flight with exact waits
  auto page_base = [&](int i, bool& ok) -> const uint8_t* {
    const int64_t phys = __builtin_amdgcn_readlane(phys_lane, i);
    ok = phys >= 0 && phys < a.num_pages;
    return a.pool + (ok ? phys : 0) * a.page_stride;
  };

  for (int t = 0; t < a.T; ++t) {
    const int64_t id = (int64_t)b * a.T + t;
    const int lim = a.causal ? L - a.T + t : L - 1;  // last position this query token may see
    // q fragments (head 16mt + r16, dims 32g + 8ks .. +7) and head weights (16mt + 4g .. +3), once per
    // query token for all of the wave's pages
    const uint16_t* qt = a.q + id * HI * kIdxDim;
    bf16x8 qf[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qf[mt][ks] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(qt + (16 * mt + r16) * kIdxDim + 32 * g + 8 * ks));
    f32x4 wv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) wv[mt] = *reinterpret_cast<const f32x4*>(a.w + id * HI + 16 * mt + 4 * g);

    // pages in order, the next two pages' keys in flight while the current one is computed: a ring of
    // three page buffers, the loop unrolled so that the ring is indexed statically (no register copies,
    // which would wait for loads still in flight)
    IndexPage buf[3];
    bool ok[3];
    load_index_page(page_base(0, ok[0]), r16, g, lane, buf[0]);
    load_index_page(page_base(n_pages > 1 ? 1 : 0, ok[1]), r16, g, lane, buf[1]);
#pragma unroll
    for (int i = 0; i < kIdxPagesPerWave; ++i) {
      if (i >= n_pages) break;
      if (i + 2 < kIdxPagesPerWave)
        load_index_page(page_base(i + 2 < n_pages ? i + 2 : i, ok[(i + 2) % 3]), r16, g, lane,
                        buf[(i + 2) % 3]);
      const IndexPage& cur = buf[i % 3];
      float tot[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        // k-step ks uses key bytes 8ks..8ks+7 of the lane's 32: dword pair (2ks, 2ks+1)
        bf16x8 kf[4];
        kf[0] = e4m3x8_to_bf16x8(cur.k[nt][0][0], cur.k[nt][0][1]);
        kf[1] = e4m3x8_to_bf16x8(cur.k[nt][0][2], cur.k[nt][0][3]);
        kf[2] = e4m3x8_to_bf16x8(cur.k[nt][1][0], cur.k[nt][1][1]);
        kf[3] = e4m3x8_to_bf16x8(cur.k[nt][1][2], cur.k[nt][1][3]);
        float part = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) acc = mfma16x16x32(qf[mt][ks], kf[ks], acc);
          // acc[e]: head 16mt + 4g + e, position 16nt + r16
#pragma unroll
          for (int e = 0; e < 4; ++e) part += wv[mt][e] * fmaxf(acc[e], 0.0f);
        }
        part += __shfl_xor(part, 16, 64);
        part += __shfl_xor(part, 32, 64);
        tot[nt] = part;  // every lane group now holds position 16nt + r16's head sum
      }
      // lane l writes position l = 16g + r16 of the page: tile g of its own row
      const float mine = g == 0 ? tot[0] : (g == 1 ? tot[1] : (g == 2 ? tot[2] : tot[3]));
      const int p = (pg_first + i) * 64 + lane;
      if (p <= lim && p < p_end) a.logits[id * a.ld + p] = ok[i % 3] ? mine * cur.sc : -INFINITY;
    }
  }
}

// The kernel used whenever q and w of a request's T tokens fit kIdxMultiMaxLds of LDS (T * HI <= 256):
// each page's keys are read and converted once and used for every token.  q and w sit in LDS (q rows
// padded to 272 bytes so that the 16 rows a load instruction touches spread over the banks); per page the
// wave converts its keys to bf16 once, then for each token and head tile reads the q fragments from LDS.
// One page of keys in flight; 150 VGPRs, three waves per SIMD (the register-q kernel above needs 231 and
// runs two; at one token it is 3% slower).
constexpr int kQRowBytes = kIdxDim * 2 + 16;

template <int HI>
__global__ __launch_bounds__(256) void index_logits_multi_kernel(IndexLogitsArgs a) {
  constexpr int MT = HI / 16;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int b = blockIdx.x / a.chunks;
  const int T = a.T;
  float* wl = reinterpret_cast<float*>(lds + T * HI * kQRowBytes);
  const int pg_first = (blockIdx.x % a.chunks) * kIdxPagesPerWg + (tid >> 6) * kIdxPagesPerWave;
  const int L = a.ctx[b];
  const int p_end = L < a.ld ? L : (int)a.ld;
  // the wave's page-table entries, loaded once (lane j: page pg_first + j), as in index_logits_kernel
  const int pj = pg_first + (lane < kIdxPagesPerWave ? lane : 0);
  const int32_t tab = a.block_table[(int64_t)b * a.bt_stride + (pj < a.bt_stride ? pj : 0)];
  const int32_t phys_lane = pj < a.bt_stride ? tab : -1;
  auto page_base = [&](int i, bool& ok) -> const uint8_t* {
    const int64_t phys = __builtin_amdgcn_readlane(phys_lane, i);
    ok = phys >= 0 && phys < a.num_pages;
    return a.pool + (ok ? phys : 0) * a.page_stride;
  };
  // the first page's keys are requested before q is staged, so that the two loads overlap (a wave with
  // no page reads page 0 or the pool's page 0 and leaves after the barrier)
  IndexPage buf[2];
  bool ok[2];
  load_index_page(page_base(0, ok[0]), r16, g, lane, buf[0]);
  {  // the request's q (T*HI rows of 256 bytes, 16 per thread-load) and w into LDS
    const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q + (int64_t)b * T * HI * kIdxDim);
    for (int c = tid; c < T * HI * 16; c += 256) {
      const int row = c >> 4, off = (c & 15) * 16;
      *reinterpret_cast<u32x4*>(lds + row * kQRowBytes + off) = *reinterpret_cast<const u32x4*>(qsrc + row * 256 + off);
    }
    for (int c = tid; c < T * HI; c += 256) wl[c] = a.w[(int64_t)b * T * HI + c];
  }
  __syncthreads();
  if (pg_first * 64 >= p_end) return;
  const int n_pages = min(kIdxPagesPerWave, (p_end - pg_first * 64 + 63) / 64);
#pragma unroll
  for (int i = 0; i < kIdxPagesPerWave; ++i) {
    if (i >= n_pages) break;
    if (i + 1 < kIdxPagesPerWave)
      load_index_page(page_base(i + 1 < n_pages ? i + 1 : i, ok[(i + 1) % 2]), r16, g, lane,
                      buf[(i + 1) % 2]);
    const IndexPage& cur = buf[i % 2];
    bf16x8 kf[4][4];  // tile nt, k-step ks: key bytes 8ks..8ks+7 of the lane's 32
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      kf[nt][0] = e4m3x8_to_bf16x8(cur.k[nt][0][0], cur.k[nt][0][1]);
      kf[nt][1] = e4m3x8_to_bf16x8(cur.k[nt][0][2], cur.k[nt][0][3]);
      kf[nt][2] = e4m3x8_to_bf16x8(cur.k[nt][1][0], cur.k[nt][1][1]);
      kf[nt][3] = e4m3x8_to_bf16x8(cur.k[nt][1][2], cur.k[nt][1][3]);
    }
    const int p = (pg_first + i) * 64 + lane;
    for (int t = 0; t < T; ++t) {
      float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint8_t* qrow = lds + (t * HI + 16 * mt + r16) * kQRowBytes + 64 * g;
        bf16x8 qf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 16 * ks));
        const f32x4 wv = *reinterpret_cast<const f32x4*>(wl + t * HI + 16 * mt + 4 * g);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) acc = mfma16x16x32(qf[ks], kf[nt][ks], acc);
#pragma unroll
          for (int e = 0; e < 4; ++e) part[nt] += wv[e] * fmaxf(acc[e], 0.0f);
        }
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        part[nt] += __shfl_xor(part[nt], 16, 64);
        part[nt] += __shfl_xor(part[nt], 32, 64);
      }
      const float mine = g == 0 ? part[0] : (g == 1 ? part[1] : (g == 2 ? part[2] : part[3]));
      const int lim = a.causal ? L - T + t : L - 1;
      if (p <= lim && p < p_end)
        a.logits[((int64_t)b * T + t) * a.ld + p] = ok[i % 2] ? mine * cur.sc : -INFINITY;
    }
  }
}

hipError_t launch_index_key_quant(const IndexKeyArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(index_key_quant_kernel, dim3((unsigned)((a.n + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

size_t index_logits_multi_lds(int T, int HI) { return (size_t)T * HI * (kQRowBytes + 4); }

hipError_t launch_index_logits(const IndexLogitsArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.B * a.chunks)), block(256);
  if (index_logits_multi_lds(a.T, a.HI) <= kIdxMultiMaxLds) {
    const size_t lds = index_logits_multi_lds(a.T, a.HI);
    switch (a.HI) {
      case 16: hipLaunchKernelGGL(index_logits_multi_kernel<16>, grid, block, lds, stream, a); break;
      case 32: hipLaunchKernelGGL(index_logits_multi_kernel<32>, grid, block, lds, stream, a); break;
      case 64: hipLaunchKernelGGL(index_logits_multi_kernel<64>, grid, block, lds, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (a.HI) {
    case 16: hipLaunchKernelGGL(index_logits_kernel<16>, grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL(index_logits_kernel<32>, grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL(index_logits_kernel<64>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
