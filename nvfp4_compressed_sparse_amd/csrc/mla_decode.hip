// MLA decode over a paged cache of NVFP4 (352-byte) or FP8 (576-byte) rows, for gfx950.
//
// What it computes ("Prime Inference" launch post, section on the native NVFP4 sparse MLA decode
// kernel; the analysis page, section "A kernel that reads four bits directly"): for each query token
// and head, softmax attention of the 576-wide absorbed query over the selected cached rows, with the
// 512-value latent as V; only the selected compressed rows are loaded and they are unpacked on chip;
// accumulation is FP32.  The pages' kernel runs FP16 operands; these MFMAs take bf16 operands (every
// dequantized K/V value is exact in bf16; P and the output round to bf16).
//
// Work decomposition (one 256-thread workgroup = 4 wavefronts):
//   * workgroup = (query token, head group of 16*HT heads, split s of the token's position list);
//     the pages split one token's rows over a cluster of 3-8 SMs merged through distributed shared
//     memory; here the splits are separate workgroups merged by a small LSE kernel.
//   * prologue: the split's list entries are validated (index < 0, past the causal limit, or on a
//     page-table entry outside the pool -> dropped, which also skips their loads) and compacted into
//     an LDS list of row addresses (order kept, so results are deterministic).
//   * per tile of 64 rows: wave w owns rows 16w..16w+15.  Lane (g = lane/16, m = lane%16) gathers its
//     quarter of row m straight into registers (NVFP4: 64 nibble bytes, 8 scale bytes, 16 rope
//     bytes), one tile ahead of use.  It dequantizes them in registers into the MFMA A operand of
//     S^T = K q^T (M = 16 rows, N = 16 heads, K = 576), and stores the latent part into an LDS V tile
//     that all four waves read for PV.  The 576 dims are permuted consistently between K and q
//     (lane group g takes dims 128g..128g+127 and rope dims 512+16g..+15) so each lane reads
//     contiguous bytes.
//   * online softmax (base 2): per-head tile maxima are combined across the four waves through LDS;
//     P (bf16) goes through LDS in exactly the layout of the PV A operand.
//   * O += P V: wave w owns output columns 128w..128w+127 for all heads.  Lane (g, n) reads, for its
//     8 rows, the nibble dword holding dims 128w+8n..+7 and its block scale, and feeds MFMA c (c<8)
//     with column 128w+8n+c of those 8 rows, so V needs no transpose.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

constexpr int kMaxChunk = 2048;

template <int FMT>
struct RowRegs;

template <>
struct RowRegs<0> {  // NVFP4: lane (g, m) holds nibble bytes [64g,+64), scales [256+8g,+8), rope [288+16g,+16)
  u32x4 nib[4];
  u32x2 sc;
  u32x4 rp;
  __device__ __forceinline__ void load(const uint8_t* row, int g) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row + 64 * g);
#pragma unroll
    for (int k = 0; k < 4; ++k) nib[k] = __builtin_nontemporal_load(p + k);
    sc = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(row + 256 + 8 * g));
    rp = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + 288 + 16 * g));
  }
};

template <>
struct RowRegs<1> {  // FP8: lane (g, m) holds latent bytes [128g,+128), rope [512+16g,+16)
  u32x4 lat[8];
  u32x4 rp;
  __device__ __forceinline__ void load(const uint8_t* row, int g) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row + 128 * g);
#pragma unroll
    for (int k = 0; k < 8; ++k) lat[k] = __builtin_nontemporal_load(p + k);
    rp = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + 512 + 16 * g));
  }
};

template <int HT, int FMT, bool DENSE>
__global__ __launch_bounds__(256, 1) void decode_kernel(DecodeArgs a) {
  constexpr int ROWB = FMT == 0 ? kNvfp4Row : kFp8Row;
  constexpr int VSTRIDE = FMT == 0 ? 304 : 528;  // LDS bytes per V-tile row (padded)
  __shared__ uint32_t rowlist[kMaxChunk];
  __shared__ __attribute__((aligned(16))) uint8_t vtile[2][64 * VSTRIDE];
  __shared__ __attribute__((aligned(16))) u32x2 pbuf[4][HT][64];
  __shared__ float red[4][HT][16];
  __shared__ float alph[HT][16];
  __shared__ int wcount[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, n = lane & 15;  // n doubles as m (row within the wave's M tile)

  const int HG = a.H / (16 * HT);
  const int j = xcd_logical_id(blockIdx.x, gridDim.x);
  const int hg = j % HG;
  const int rest = j / HG;
  const int s = rest % a.splits;
  const int qtok = rest / a.splits;
  const int b = qtok / a.T, t = qtok % a.T;
  const int L = a.ctx[b];
  const int lim = a.causal ? L - a.T + t : L - 1;
  const int e0 = s * a.chunk;
  const int e_end = DENSE ? (lim + 1 < a.entries ? lim + 1 : a.entries) : a.entries;
  const int e1 = (e0 + a.chunk < e_end) ? e0 + a.chunk : e_end;

  // ---- prologue: valid rows of this split -> LDS list of 16-byte row addresses
  uint32_t addr[8];
  uint32_t vmask = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int e = e0 + 8 * tid + k;
    bool ok = e < e1;
    int pos = -1;
    if (ok) pos = DENSE ? e : a.indices[(int64_t)qtok * a.entries + e];
    ok = ok && pos >= 0 && pos <= lim;
    int page = -1;
    if (ok) page = a.block_table[(int64_t)b * a.bt_stride + (pos >> 6)];
    ok = ok && page >= 0 && page < a.num_pages;
    addr[k] = ok ? (uint32_t)(((uint64_t)page * (uint64_t)a.page_stride + (uint64_t)(pos & 63) * ROWB) >> 4) : 0u;
    vmask |= (uint32_t)ok << k;
  }
  const int cnt = __builtin_popcount(vmask);
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wcount[w] = incl;
  __syncthreads();
  int off = incl - cnt;
  for (int ww = 0; ww < w; ++ww) off += wcount[ww];
  const int n_valid = wcount[0] + wcount[1] + wcount[2] + wcount[3];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (vmask & (1u << k)) rowlist[off++] = addr[k];

  // ---- query fragments (B operand of S^T = K q^T): lane (g, n) holds head 16t+n, dims D(g, ks)
  const int h0 = hg * 16 * HT;
  bf16x8 qf[HT][18];
  {
    const uint16_t* qb = a.q + ((int64_t)qtok * a.H + h0) * kQK;
#pragma unroll
    for (int tt = 0; tt < HT; ++tt) {
      const uint16_t* qh = qb + (16 * tt + n) * kQK;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qf[tt][ks] = *reinterpret_cast<const bf16x8*>(qh + 128 * g + 8 * ks);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) qf[tt][16 + ks] = *reinterpret_cast<const bf16x8*>(qh + 512 + 16 * g + 8 * ks);
    }
  }
  __syncthreads();  // row list complete

  f32x4 o[HT][8];
  float mrun[HT], lrun[HT];
#pragma unroll
  for (int tt = 0; tt < HT; ++tt) {
    mrun[tt] = -INFINITY;
    lrun[tt] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[tt][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const int ntiles = (n_valid + 63) >> 6;
  RowRegs<FMT> cur, nxt;
  auto row_ptr = [&](int tile) {
    int r = tile * 64 + 16 * w + n;
    uint32_t a16 = rowlist[r < n_valid ? r : 0];
    return a.pool + (uint64_t)a16 * 16u;
  };
  if (ntiles > 0) cur.load(row_ptr(0), g);

  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) nxt.load(row_ptr(it + 1), g);
    uint8_t* vt = vtile[it & 1];

    // ---- V tile: latent part of my row quarter into LDS
    {
      uint8_t* vrow = vt + (16 * w + n) * VSTRIDE;
      if constexpr (FMT == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4*>(vrow + 64 * g + 16 * k) = cur.nib[k];
        *reinterpret_cast<u32x2*>(vrow + 256 + 8 * g) = cur.sc;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) *reinterpret_cast<u32x4*>(vrow + 128 * g + 16 * k) = cur.lat[k];
      }
    }

    // ---- S^T = K q^T for my 16 rows
    f32x4 acc[HT];
#pragma unroll
    for (int tt = 0; tt < HT; ++tt) acc[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (FMT == 0) {
      float scl[8];
      scl[0] = e4m3_to_f32<0>(cur.sc.x);
      scl[1] = e4m3_to_f32<1>(cur.sc.x);
      scl[2] = e4m3_to_f32<2>(cur.sc.x);
      scl[3] = e4m3_to_f32<3>(cur.sc.x);
      scl[4] = e4m3_to_f32<0>(cur.sc.y);
      scl[5] = e4m3_to_f32<1>(cur.sc.y);
      scl[6] = e4m3_to_f32<2>(cur.sc.y);
      scl[7] = e4m3_to_f32<3>(cur.sc.y);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const uint32_t d = cur.nib[ks >> 2][ks & 3];
        const float sj = scl[ks >> 1];
        f32x2 p0 = fp4x2_to_f32<0>(d), p1 = fp4x2_to_f32<1>(d), p2 = fp4x2_to_f32<2>(d), p3 = fp4x2_to_f32<3>(d);
        bf16x8 A = as_bf16x8(pack_hi16(p0[0] * sj, p0[1] * sj), pack_hi16(p1[0] * sj, p1[1] * sj),
                             pack_hi16(p2[0] * sj, p2[1] * sj), pack_hi16(p3[0] * sj, p3[1] * sj));
#pragma unroll
        for (int tt = 0; tt < HT; ++tt) acc[tt] = mfma16x16x32(A, qf[tt][ks], acc[tt]);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const uint32_t w0 = cur.lat[ks >> 1][2 * (ks & 1)], w1 = cur.lat[ks >> 1][2 * (ks & 1) + 1];
        bf16x8 A = as_bf16x8(e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0), e4m3x2_to_bf16x2<false>(w1),
                             e4m3x2_to_bf16x2<true>(w1));
#pragma unroll
        for (int tt = 0; tt < HT; ++tt) acc[tt] = mfma16x16x32(A, qf[tt][ks], acc[tt]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t w0 = cur.rp[2 * ks], w1 = cur.rp[2 * ks + 1];
      bf16x8 A = as_bf16x8(e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0), e4m3x2_to_bf16x2<false>(w1),
                           e4m3x2_to_bf16x2<true>(w1));
#pragma unroll
      for (int tt = 0; tt < HT; ++tt) acc[tt] = mfma16x16x32(A, qf[tt][16 + ks], acc[tt]);
    }

    // ---- online softmax, part 1: per-head maxima of my 16 rows
    const int rbase = it * 64 + 16 * w + 4 * g;
    float sv[HT][4];
#pragma unroll
    for (int tt = 0; tt < HT; ++tt) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = acc[tt][i] * a.scale_log2;
        sv[tt][i] = (rbase + i < n_valid) ? x : -INFINITY;
        mx = fmaxf(mx, sv[tt][i]);
      }
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      if (g == 0) red[w][tt][n] = mx;
    }
    lds_barrier();  // maxima and the V tile are visible

    // ---- part 2: new running max, P, rescale factor
#pragma unroll
    for (int tt = 0; tt < HT; ++tt) {
      float tmax = fmaxf(fmaxf(red[0][tt][n], red[1][tt][n]), fmaxf(red[2][tt][n], red[3][tt][n]));
      float mnew = fmaxf(mrun[tt], tmax);
      float muse = mnew == -INFINITY ? 0.0f : mnew;
      float alpha = __builtin_amdgcn_exp2f(mrun[tt] - muse);
      float p0 = __builtin_amdgcn_exp2f(sv[tt][0] - muse), p1 = __builtin_amdgcn_exp2f(sv[tt][1] - muse);
      float p2 = __builtin_amdgcn_exp2f(sv[tt][2] - muse), p3 = __builtin_amdgcn_exp2f(sv[tt][3] - muse);
      lrun[tt] = lrun[tt] * alpha + ((p0 + p1) + (p2 + p3));
      mrun[tt] = mnew;
      pbuf[w][tt][lane] = u32x2{pack_bf16_rne(p0, p1), pack_bf16_rne(p2, p3)};
      if (w == 0 && g == 0) alph[tt][n] = alpha;
    }
    lds_barrier();  // P and the rescale factors are visible

    // ---- O = alpha * O + P V over my 128 output columns
#pragma unroll
    for (int tt = 0; tt < HT; ++tt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float al = alph[tt][4 * g + i];
#pragma unroll
        for (int c = 0; c < 8; ++c) o[tt][c][i] *= al;
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 pa[HT];
#pragma unroll
      for (int tt = 0; tt < HT; ++tt) {
        u32x2 lo = pbuf[2 * kk][tt][lane], hi = pbuf[2 * kk + 1][tt][lane];
        pa[tt] = as_bf16x8(lo[0], lo[1], hi[0], hi[1]);
      }
      float vv[8][8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int row = 32 * kk + (jj < 4 ? 4 * g + jj : 12 + 4 * g + jj);
        const uint8_t* vr = vt + row * VSTRIDE;
        if constexpr (FMT == 0) {
          const uint32_t d = *reinterpret_cast<const uint32_t*>(vr + 64 * w + 4 * n);
          const float sc = e4m3_to_f32<0>((uint32_t)vr[256 + 8 * w + (n >> 1)]);
          f32x2 p0 = fp4x2_to_f32<0>(d), p1 = fp4x2_to_f32<1>(d), p2 = fp4x2_to_f32<2>(d), p3 = fp4x2_to_f32<3>(d);
          vv[jj][0] = p0[0] * sc;
          vv[jj][1] = p0[1] * sc;
          vv[jj][2] = p1[0] * sc;
          vv[jj][3] = p1[1] * sc;
          vv[jj][4] = p2[0] * sc;
          vv[jj][5] = p2[1] * sc;
          vv[jj][6] = p3[0] * sc;
          vv[jj][7] = p3[1] * sc;
        } else {
          const u32x2 d = *reinterpret_cast<const u32x2*>(vr + 128 * w + 8 * n);
          f32x2 p0 = e4m3x2_to_f32<false>(d[0]), p1 = e4m3x2_to_f32<true>(d[0]);
          f32x2 p2 = e4m3x2_to_f32<false>(d[1]), p3 = e4m3x2_to_f32<true>(d[1]);
          vv[jj][0] = p0[0];
          vv[jj][1] = p0[1];
          vv[jj][2] = p1[0];
          vv[jj][3] = p1[1];
          vv[jj][4] = p2[0];
          vv[jj][5] = p2[1];
          vv[jj][6] = p3[0];
          vv[jj][7] = p3[1];
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        bf16x8 vb = as_bf16x8(pack_hi16(vv[0][c], vv[1][c]), pack_hi16(vv[2][c], vv[3][c]),
                              pack_hi16(vv[4][c], vv[5][c]), pack_hi16(vv[6][c], vv[7][c]));
#pragma unroll
        for (int tt = 0; tt < HT; ++tt) o[tt][c] = mfma16x16x32(pa[tt], vb, o[tt][c]);
      }
    }
    if (it + 1 < ntiles) cur = nxt;
  }

  // ---- finalize: row sums across lane groups and waves, normalize, write
#pragma unroll
  for (int tt = 0; tt < HT; ++tt) {
    float l = lrun[tt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (g == 0) red[w][tt][n] = l;
  }
  lds_barrier();
  const int S = a.splits;
#pragma unroll
  for (int tt = 0; tt < HT; ++tt) {
    if (w == 0 && g == 0) {
      const float ltot = (red[0][tt][n] + red[1][tt][n]) + (red[2][tt][n] + red[3][tt][n]);
      const float lse = ltot > 0.0f ? (mrun[tt] + __log2f(ltot)) * 0.69314718055994531f : -INFINITY;
      const int64_t hrow = (int64_t)qtok * a.H + h0 + 16 * tt + n;
      if (S == 1) {
        if (a.lse) a.lse[hrow] = lse;
      } else {
        a.part_lse[hrow * S + s] = lse;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hl = 4 * g + i;
      const float li = (red[0][tt][hl] + red[1][tt][hl]) + (red[2][tt][hl] + red[3][tt][hl]);
      const float inv = li > 0.0f ? 1.0f / li : 0.0f;
      const int64_t hrow = (int64_t)qtok * a.H + h0 + 16 * tt + hl;
      const int col = 128 * w + 8 * n;
      if (S == 1) {
        u32x4 v = {pack_bf16_rne(o[tt][0][i] * inv, o[tt][1][i] * inv), pack_bf16_rne(o[tt][2][i] * inv, o[tt][3][i] * inv),
                   pack_bf16_rne(o[tt][4][i] * inv, o[tt][5][i] * inv), pack_bf16_rne(o[tt][6][i] * inv, o[tt][7][i] * inv)};
        *reinterpret_cast<u32x4*>(a.out + hrow * kLatent + col) = v;
      } else {
        float* dst = a.part_o + (hrow * S + s) * kLatent + col;
        *reinterpret_cast<f32x4*>(dst) = f32x4{o[tt][0][i] * inv, o[tt][1][i] * inv, o[tt][2][i] * inv, o[tt][3][i] * inv};
        *reinterpret_cast<f32x4*>(dst + 4) =
            f32x4{o[tt][4][i] * inv, o[tt][5][i] * inv, o[tt][6][i] * inv, o[tt][7][i] * inv};
      }
    }
  }
}

// LSE-weighted merge of S split results: one wavefront per (query token, head), lane l owns columns
// 8l..8l+7.  lse = M + ln sum_s e^{lse_s - M}; out = sum_s e^{lse_s - lse} out_s; all-empty -> 0/-inf.
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                                                    int S, int64_t rows, uint16_t* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* pl = part_lse + row * S;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, pl[s]);
  u32x4* dst = reinterpret_cast<u32x4*>(out + row * kLatent + 8 * lane);
  if (M == -INFINITY) {
    *dst = u32x4{0u, 0u, 0u, 0u};
    if (lse && lane == 0) lse[row] = -INFINITY;
    return;
  }
  float Z = 0.0f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int s = 0; s < S; ++s) {
    const float wgt = __expf(pl[s] - M);
    Z += wgt;
    if (wgt != 0.0f) {
      const f32x4* src = reinterpret_cast<const f32x4*>(part_o + (row * S + s) * kLatent + 8 * lane);
      f32x4 v0 = src[0], v1 = src[1];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[k] += wgt * v0[k];
        acc[4 + k] += wgt * v1[k];
      }
    }
  }
  const float inv = 1.0f / Z;
  *dst = u32x4{pack_bf16_rne(acc[0] * inv, acc[1] * inv), pack_bf16_rne(acc[2] * inv, acc[3] * inv),
               pack_bf16_rne(acc[4] * inv, acc[5] * inv), pack_bf16_rne(acc[6] * inv, acc[7] * inv)};
  if (lse && lane == 0) lse[row] = M + __logf(Z);
}

template <int HT, int FMT, bool DENSE>
static void launch_one(const DecodeArgs& a, hipStream_t stream) {
  const int HG = a.H / (16 * HT);
  const unsigned grid = (unsigned)(a.B * a.T * HG * a.splits);
  hipLaunchKernelGGL((decode_kernel<HT, FMT, DENSE>), dim3(grid), dim3(256), 0, stream, a);
}

hipError_t launch_decode(int fmt, const DecodeArgs& a, hipStream_t stream) {
  const bool dense = a.indices == nullptr;
  if (fmt == 0) {
    if (a.H == 16) launch_one<1, 0, false>(a, stream);
    else launch_one<2, 0, false>(a, stream);
  } else {
    if (!dense) return hipErrorInvalidValue;
    if (a.H == 16) launch_one<1, 1, true>(a, stream);
    else launch_one<2, 1, true>(a, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const int64_t rows = (int64_t)a.B * a.T * a.H;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a.part_o, a.part_lse,
                     a.splits, rows, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace mla
