// MLA decode over a paged cache of NVFP4 (352-byte) or FP8 (576-byte) rows, for gfx950.
//
// What it computes ("Prime Inference" launch post, section on the native NVFP4 sparse MLA decode
// kernel; the analysis page, section "A kernel that reads four bits directly"): for each query token
// and head, softmax attention of the 576-wide absorbed query over the selected cached rows, with the
// 512-value latent as V; only the selected compressed rows are loaded and they are unpacked on chip;
// accumulation is FP32.  As in the pages' kernel the matrix operands are FP16: every dequantized K/V
// value is exact in FP16, a bf16 query element converts exactly when its magnitude is in FP16's normal
// range, and P rounds to FP16.
//
// Work decomposition (one 256-thread workgroup = 4 wavefronts, one workgroup per compute unit):
//   * workgroup = (query token, head group of 16*HT heads, split s of the token's position list);
//     the pages split one token's rows over a cluster of 3-8 SMs merged through distributed shared
//     memory; here the splits are separate workgroups merged by a small LSE kernel.
//   * prologue: the page-table entries the split can touch are staged in LDS; the split's list entries
//     are validated (index < 0, past the causal limit, or on a page-table entry outside the pool ->
//     dropped, which also skips their loads) and compacted into an LDS list of row addresses (order
//     kept, so results are deterministic).  The query fragments are converted to FP16 and stay in
//     registers for the whole split.
//   * rows are consumed in steps of 64; wave w gathers rows 16w..16w+15 of each step by LDS-DMA
//     (16 bytes per lane, no registers) into a ring of raw row slots, up to five steps ahead.
//   * S^T = K q^T for the wave's 16 rows (M = 16 rows, N = 16 heads per head tile, K = 576): lane
//     (g = lane/16, m = lane%16) reads its quarter of row m and dequantizes it in registers into the
//     MFMA A operand (cvt to FP16 + packed multiply by the block scale).  The 576 dims are permuted
//     consistently between K and q (lane group g takes dims 128g..128g+127 and rope dims 512+16g..+15).
//   * online softmax in base 2 with a lazy reference shared by the four waves: the per-wave maxima
//     are exchanged through LDS, and the reference is raised (and the output rescaled) only when a
//     score exceeds it by more than 2^8, so P stays below 256.  P (FP16) goes to LDS.
//   * O^T += V^T P^T: wave w owns output columns 128w..128w+127 for all heads of the group and
//     contracts over all 64 rows of the step.  Lane (g, m) reads, for 8 rows, the nibble dword holding
//     columns 128w+8m..+7 and feeds column 128w+8m+c to MFMA tile c (c < 8); the nibbles of two rows
//     are interleaved with bit operations so that each FP16 pair the converter produces is already
//     (row r, row r+1) of one column.  The output tile stays in registers (16*HT heads x 128 columns).
//   * epilogue: the waves' partial sums are added through LDS; each wave normalizes and writes its own
//     columns directly (bf16 output, or fp32 partials for the split merge).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

constexpr int kMaxChunk = 2048;
constexpr float kLazyRescale = 8.0f;  // log2 headroom of the lazy softmax reference
constexpr int kPStride = 64 * 2 + 16;  // bytes per head of the P tile: 64 FP16 values + padding

// Geometry of the raw-row ring: steps of 64 rows, 16 per wave; lane l of the wave's DMA load u
// fetches 16-byte chunk 64u+l of the wave's 16 rows, laid back to back.
template <int FMT>
struct Geo {
  static constexpr int kRowBytes = FMT == 0 ? kNvfp4Row : kFp8Row;
  static constexpr int kChunks = kRowBytes / 16;               // 22 or 36 per row
  static constexpr int kWaveChunks = 16 * kChunks;             // 352 or 576 per wave per step
  static constexpr int kLoads = (kWaveChunks + 63) / 64;       // 6 or 9 DMA loads per wave per step
  static constexpr int kSlot = 64 * kRowBytes;                 // bytes of one step
  static constexpr int kSlots = FMT == 0 ? 6 : 4;              // ring depth
  static constexpr int kRing = kSlots * kSlot;
};

// LDS-DMA of 16 bytes per lane: lane l's global bytes land at lds + 16*l (lds must be wave-uniform).
// Issued through asm so that the compiler's waitcnt tracking does not drain the gathers still in
// flight; completion is awaited explicitly with vmcnt.  M0 is saved and restored around the load.
__device__ __forceinline__ void dma16(const void* src, const uint8_t* lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(m)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((uint16_t)((N & 15) | ((N >> 4) << 14) | 0x0F70));
}

// Byte interleave of two rows' nibble dwords: byte k of the result holds (lo nibble, hi nibble) =
// (row a, row b) of column 2k (ODD = 0) or 2k+1 (ODD = 1).
template <int ODD>
__device__ __forceinline__ uint32_t nib_pair(uint32_t ra, uint32_t rb) {
  constexpr uint32_t M = 0x0F0F0F0Fu;
  return ODD ? (((ra >> 4) & M) | (rb & ~M)) : ((ra & M) | ((rb << 4) & ~M));
}

template <int HT, int FMT, bool DENSE>
__global__ __launch_bounds__(256, 1) void decode_kernel(DecodeArgs a) {
  using G = Geo<FMT>;
  constexpr int ROWB = G::kRowBytes;
  constexpr int NL = G::kLoads;
  constexpr int NS = G::kSlots;
  constexpr int NH = 16 * HT;
  __shared__ __attribute__((aligned(16))) uint8_t ring[G::kRing];
  __shared__ __attribute__((aligned(16))) uint8_t ptile[HT * 16 * kPStride];
  __shared__ uint32_t rowlist[kMaxChunk];
  __shared__ float smax[4][NH], wsum[4][NH];
  __shared__ int wcount[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, n = lane & 15;

  const int HG = a.H / NH;
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

  // ---- prologue: valid rows of this split -> LDS list of 16-byte row addresses.
  // The page-table entries this split can touch are staged in LDS with coalesced loads while the
  // split's list entries (8 per thread) and the query fragments load at the same time: one memory
  // round trip instead of two dependent gathers.
  const int p0 = DENSE ? (e0 >> 6) : 0;
  const int p1 = DENSE ? ((e1 - 1) >> 6) : (lim >> 6);
  const int npg = (e1 > e0 && p1 >= p0) ? p1 - p0 + 1 : 0;
  constexpr int kBtCap = G::kRing / 4;
  const bool staged = npg <= kBtCap;
  int* btl = reinterpret_cast<int*>(ring);
  const int* btg = a.block_table + (int64_t)b * a.bt_stride + p0;
  constexpr int kBtPer = 12;  // entries per thread loaded before any is stored (contexts up to 196,608)
  const bool bt_regs = npg <= 256 * kBtPer;
  int btv[kBtPer];
  if (bt_regs) {
#pragma unroll
    for (int k = 0; k < kBtPer; ++k) btv[k] = tid + 256 * k < npg ? btg[tid + 256 * k] : 0;
  }

  int pos[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) pos[k] = -1;
  if (e1 > e0) {
    const int ebase = e0 + 8 * tid;
    if (DENSE) {
#pragma unroll
      for (int k = 0; k < 8; ++k) pos[k] = ebase + k < e1 ? ebase + k : -1;
    } else {
      const int* ip = a.indices + (int64_t)qtok * a.entries + ebase;
      if (((uintptr_t)a.indices & 15) == 0 && (((int64_t)qtok * a.entries + e0) & 3) == 0 && ebase + 8 <= e1) {
        const u32x4 x0 = reinterpret_cast<const u32x4*>(ip)[0], x1 = reinterpret_cast<const u32x4*>(ip)[1];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          pos[k] = (int)x0[k];
          pos[4 + k] = (int)x1[k];
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) pos[k] = ebase + k < e1 ? ip[k] : -1;
      }
    }
  }

  // query fragments (B operand of S^T = K q^T), FP16: lane (g, n) holds head 16t+n, dims
  // 128g+8ks..+7 (ks < 16) and 512+16g+8(ks-16)..+7 (ks = 16, 17)
  const int h0 = hg * NH;
  f16x8 qf[HT][18];
  {
    const uint16_t* qb = a.q + ((int64_t)qtok * a.H + h0) * kQK;
    u32x4 raw[HT][18];
#pragma unroll
    for (int tt = 0; tt < HT; ++tt) {
      const uint16_t* qh = qb + (16 * tt + n) * kQK;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const int d = ks < 16 ? 128 * g + 8 * ks : 512 + 16 * g + 8 * (ks - 16);
        raw[tt][ks] = *reinterpret_cast<const u32x4*>(qh + d);
      }
    }
#pragma unroll
    for (int tt = 0; tt < HT; ++tt)
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        f16x2 h[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t d = raw[tt][ks][k];
          h[k] = f16x2{(_Float16)__uint_as_float(d << 16), (_Float16)__uint_as_float(d & 0xFFFF0000u)};
        }
        qf[tt][ks] = as_f16x8(h[0], h[1], h[2], h[3]);
      }
  }
  if (bt_regs) {
#pragma unroll
    for (int k = 0; k < kBtPer; ++k)
      if (tid + 256 * k < npg) btl[tid + 256 * k] = btv[k];
  } else if (staged) {
    for (int i = tid; i < npg; i += 256) btl[i] = btg[i];
  }
  __syncthreads();  // staged page-table entries visible

  uint32_t addr[8];
  uint32_t vmask = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool inr = pos[k] >= 0 && pos[k] <= lim;
    const int pg = (inr ? pos[k] : 0) >> 6;
    int page = -1;
    if (inr) page = staged ? btl[pg - p0] : btg[pg - p0];
    const bool ok = inr && page >= 0 && page < a.num_pages;
    addr[k] = ok ? (uint32_t)(((uint64_t)page * (uint64_t)a.page_stride + (uint64_t)(pos[k] & 63) * ROWB) >> 4) : 0u;
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
  // every load the compiler issued (indices, page table, q) has landed: its waits inside the loop
  // would otherwise also drain the row gathers, which it does not see
  wait_vmem();
  __syncthreads();  // row list complete; the staging area is free again

  // ---- main loop
  f32x4 o[HT][8];  // O^T tile c: O[head 16t+n][column 128w+32g+8i+c] = o[t][c][i]
  float mref[HT], lsum[HT];
#pragma unroll
  for (int tt = 0; tt < HT; ++tt) {
    mref[tt] = -INFINITY;
    lsum[tt] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[tt][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const int nsteps = (n_valid + 63) >> 6;
  auto slot_ptr = [&](int st) { return ring + (st % NS) * G::kSlot; };
  auto issue_step = [&](int st) {
    const int rb = st * 64 + 16 * w;
    const uint8_t* dst = slot_ptr(st) + 16 * w * ROWB;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int e = 64 * u + lane;  // my chunk of the wave's 16 rows
      if (64 * (u + 1) <= G::kWaveChunks || e < G::kWaveChunks) {
        const int row = e / G::kChunks;
        const int r = rb + row;
        const uint32_t a16 = rowlist[r < n_valid ? r : 0];
        dma16(a.pool + (uint64_t)a16 * 16u + 16 * (e - row * G::kChunks), dst + 1024 * u);
      }
    }
  };
  if (nsteps > 0) {
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) issue_step(k < nsteps ? k : nsteps - 1);
  }

  // P tile: P[head][k] for the 64 rows of a step in contraction order k = 32*kk + 8*g' + 2*p + e,
  // which is step row 32*kk + 8*p + 2*g' + e (see the V reads below).  This lane's four scores are
  // step rows 16w+4g+i: two FP16 pairs at k0 and k0 + 8.
  const int kw = 32 * (w >> 1) + 16 * (g & 1) + 2 * (2 * (w & 1) + (g >> 1));
  // V reads: lane (g, m=n) reads columns 128w+8m..+7 of rows 8p+2g+e (p < 4, e < 2) of a k-step
  const int vcol = FMT == 0 ? 64 * w + 4 * n : 128 * w + 8 * n;
  const int vsc = 256 + 8 * w + 4 * (n >> 3);  // dword holding the block scale of those columns
  const uint32_t vsel = (uint32_t)((n >> 1) & 3) | ((uint32_t)(4 + ((n >> 1) & 3)) << 8);

  for (int it = 0; it < nsteps; ++it) {
    wait_vmem_le<(NS - 2) * NL>();  // this step's rows of this wave have landed
    const uint8_t* slot = slot_ptr(it);

    // ---- S^T = K q^T for my 16 rows
    f32x4 acc[HT];
#pragma unroll
    for (int tt = 0; tt < HT; ++tt) acc[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const uint8_t* rr = slot + (16 * w + n) * ROWB;
    if constexpr (FMT == 0) {
      u32x4 nib[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) nib[k] = *reinterpret_cast<const u32x4*>(rr + 64 * g + 16 * k);
      const u32x2 sc = *reinterpret_cast<const u32x2*>(rr + 256 + 8 * g);
      const f16x2 s2[4] = {e4m3x2_to_f16<false>(sc[0]), e4m3x2_to_f16<true>(sc[0]), e4m3x2_to_f16<false>(sc[1]),
                           e4m3x2_to_f16<true>(sc[1])};
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const uint32_t d = nib[ks >> 2][ks & 3];
        const _Float16 sh = ((ks >> 1) & 1) ? s2[ks >> 2].y : s2[ks >> 2].x;
        const f16x2 ss = {sh, sh};
        const f16x8 A = as_f16x8(fp4x2_to_f16<0>(d) * ss, fp4x2_to_f16<1>(d) * ss, fp4x2_to_f16<2>(d) * ss,
                                 fp4x2_to_f16<3>(d) * ss);
#pragma unroll
        for (int tt = 0; tt < HT; ++tt) acc[tt] = mfma16x16x32(A, qf[tt][ks], acc[tt]);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const u32x2 wv = *reinterpret_cast<const u32x2*>(rr + 128 * g + 8 * ks);
        const f16x8 A = as_f16x8(e4m3x2_to_f16<false>(wv[0]), e4m3x2_to_f16<true>(wv[0]),
                                 e4m3x2_to_f16<false>(wv[1]), e4m3x2_to_f16<true>(wv[1]));
#pragma unroll
        for (int tt = 0; tt < HT; ++tt) acc[tt] = mfma16x16x32(A, qf[tt][ks], acc[tt]);
      }
    }
    {
      const u32x4 rp = *reinterpret_cast<const u32x4*>(rr + (FMT == 0 ? 288 : 512) + 16 * g);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint32_t w0 = rp[2 * ks], w1 = rp[2 * ks + 1];
        const f16x8 A = as_f16x8(e4m3x2_to_f16<false>(w0), e4m3x2_to_f16<true>(w0), e4m3x2_to_f16<false>(w1),
                                 e4m3x2_to_f16<true>(w1));
#pragma unroll
        for (int tt = 0; tt < HT; ++tt) acc[tt] = mfma16x16x32(A, qf[tt][16 + ks], acc[tt]);
      }
    }

    // ---- scores (base 2) and this wave's maximum per head
    const int rbase = it * 64 + 16 * w + 4 * g;
    float sv[HT][4];
#pragma unroll
    for (int tt = 0; tt < HT; ++tt) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = acc[tt][i] * a.scale_log2;
        sv[tt][i] = rbase + i < n_valid ? x : -INFINITY;
        mx = fmaxf(mx, sv[tt][i]);
      }
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      if (g == 0) smax[w][16 * tt + n] = mx;
    }
    lds_barrier();  // maxima visible; every wave has finished the previous step's PV
    {
      const int nt = it + NS - 1;
      issue_step(nt < nsteps ? nt : nsteps - 1);  // clamped: the same number of loads in flight every step
    }

    // ---- lazy reference (identical in every wave: same inputs), P -> LDS
#pragma unroll
    for (int tt = 0; tt < HT; ++tt) {
      const int h = 16 * tt + n;
      const float ms = fmaxf(fmaxf(smax[0][h], smax[1][h]), fmaxf(smax[2][h], smax[3][h]));
      const bool raise = ms > mref[tt] + kLazyRescale;
      if (__any(raise)) {  // the same decision in every wave
        const float mnew = raise ? ms : mref[tt];
        const float alpha = mref[tt] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mref[tt] - mnew);
        lsum[tt] *= alpha;
        mref[tt] = mnew;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[tt][c] *= alpha;
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(sv[tt][i] - mref[tt]);
        lsum[tt] += p[i];
      }
      uint8_t* pt = ptile + (16 * tt + n) * kPStride + 2 * kw;
      *reinterpret_cast<f16x2*>(pt) = f16x2{(_Float16)p[0], (_Float16)p[1]};
      *reinterpret_cast<f16x2*>(pt + 16) = f16x2{(_Float16)p[2], (_Float16)p[3]};
    }
    lds_barrier();  // P of all 64 rows visible

    // ---- O^T += V^T P^T over the 64 rows, my 128 columns
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f16x8 pb[HT];
#pragma unroll
      for (int tt = 0; tt < HT; ++tt)
        pb[tt] = *reinterpret_cast<const f16x8*>(ptile + (16 * tt + n) * kPStride + 2 * (32 * kk + 8 * g));
      const uint8_t* vb = slot + (32 * kk + 2 * g) * ROWB;  // row 32kk + 8p + 2g + e at vb + (8p + e)*ROWB
      if constexpr (FMT == 0) {
        uint32_t ev[4][2];
        f16x2 sp[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint8_t* ra = vb + 8 * p * ROWB;
          const uint32_t da = *reinterpret_cast<const uint32_t*>(ra + vcol);
          const uint32_t db = *reinterpret_cast<const uint32_t*>(ra + ROWB + vcol);
          const uint32_t sa = *reinterpret_cast<const uint32_t*>(ra + vsc);
          const uint32_t sb = *reinterpret_cast<const uint32_t*>(ra + ROWB + vsc);
          sp[p] = e4m3x2_to_f16<false>(__builtin_amdgcn_perm(sb, sa, vsel));
          ev[p][0] = nib_pair<0>(da, db);
          ev[p][1] = nib_pair<1>(da, db);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          f16x2 v[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t e = ev[p][c & 1];
            f16x2 x;
            switch (c >> 1) {
              case 0: x = fp4x2_to_f16<0>(e); break;
              case 1: x = fp4x2_to_f16<1>(e); break;
              case 2: x = fp4x2_to_f16<2>(e); break;
              default: x = fp4x2_to_f16<3>(e); break;
            }
            v[p] = x * sp[p];
          }
          const f16x8 A = as_f16x8(v[0], v[1], v[2], v[3]);
#pragma unroll
          for (int tt = 0; tt < HT; ++tt) o[tt][c] = mfma16x16x32(A, pb[tt], o[tt][c]);
        }
      } else {
        // FP8: byte interleave (row a, row b) per column with v_perm, then exact FP8 -> FP16 pairs
        uint32_t x[4][4];  // x[p][q]: columns 2q, 2q+1 of rows (a, b) as bytes a, b, a', b'
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint8_t* ra = vb + 8 * p * ROWB;
          const u32x2 da = *reinterpret_cast<const u32x2*>(ra + vcol);
          const u32x2 db = *reinterpret_cast<const u32x2*>(ra + ROWB + vcol);
          x[p][0] = __builtin_amdgcn_perm(db[0], da[0], 0x05010400u);
          x[p][1] = __builtin_amdgcn_perm(db[0], da[0], 0x07030602u);
          x[p][2] = __builtin_amdgcn_perm(db[1], da[1], 0x05010400u);
          x[p][3] = __builtin_amdgcn_perm(db[1], da[1], 0x07030602u);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          f16x2 v[4];
#pragma unroll
          for (int p = 0; p < 4; ++p)
            v[p] = (c & 1) ? e4m3x2_to_f16<true>(x[p][c >> 1]) : e4m3x2_to_f16<false>(x[p][c >> 1]);
          const f16x8 A = as_f16x8(v[0], v[1], v[2], v[3]);
#pragma unroll
          for (int tt = 0; tt < HT; ++tt) o[tt][c] = mfma16x16x32(A, pb[tt], o[tt][c]);
        }
      }
    }
  }
  wait_vmem();  // the clamped prefetches of the last steps are still landing in the ring

  // ---- epilogue: add the waves' partial sums; each wave normalizes and writes its own columns
#pragma unroll
  for (int tt = 0; tt < HT; ++tt) {
    float l = lsum[tt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (g == 0) wsum[w][16 * tt + n] = l;
  }
  __syncthreads();
  const int S = a.splits;
#pragma unroll
  for (int tt = 0; tt < HT; ++tt) {
    const int h = 16 * tt + n;
    const float Lh = wsum[0][h] + wsum[1][h] + wsum[2][h] + wsum[3][h];
    const float inv = Lh > 0.0f ? 1.0f / Lh : 0.0f;
    const int64_t hrow = (int64_t)qtok * a.H + h0 + h;
    if (w == 0 && g == 0) {
      const float lse = Lh > 0.0f ? (mref[tt] + __log2f(Lh)) * 0.69314718055994531f : -INFINITY;
      if (S == 1) {
        if (a.lse) a.lse[hrow] = lse;
      } else {
        a.part_lse[hrow * S + s] = lse;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = 128 * w + 32 * g + 8 * i;
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = o[tt][c][i] * inv;
      if (S == 1) {
        *reinterpret_cast<u32x4*>(a.out + hrow * kLatent + col) =
            u32x4{pack_bf16_rne(v[0], v[1]), pack_bf16_rne(v[2], v[3]), pack_bf16_rne(v[4], v[5]),
                  pack_bf16_rne(v[6], v[7])};
      } else {
        f32x4* dst = reinterpret_cast<f32x4*>(a.part_o + (hrow * S + s) * kLatent + col);
        dst[0] = f32x4{v[0], v[1], v[2], v[3]};
        dst[1] = f32x4{v[4], v[5], v[6], v[7]};
      }
    }
  }
}

// LSE-weighted merge of S split results (the pages merge a cluster's partial results through
// distributed shared memory; here a second, small launch does it): one wavefront per (query token,
// head), lane l owns columns 8l..8l+7.  lse = M + ln sum_s e^{lse_s - M}; out = sum_s e^{lse_s - lse}
// out_s; a split with no rows has lse_s = -inf and no weight; all-empty -> out = 0, lse = -inf.
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                                                    int S, int64_t rows, uint16_t* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* pl = part_lse + row * S;
  float M = -INFINITY;
  for (int k = 0; k < S; ++k) M = fmaxf(M, pl[k]);
  u32x4* dst = reinterpret_cast<u32x4*>(out + row * kLatent + 8 * lane);
  if (M == -INFINITY) {
    *dst = u32x4{0u, 0u, 0u, 0u};
    if (lse && lane == 0) lse[row] = -INFINITY;
    return;
  }
  float Z = 0.0f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int k = 0; k < S; ++k) {
    const float wgt = __expf(pl[k] - M);
    Z += wgt;
    if (wgt != 0.0f) {
      const f32x4* src = reinterpret_cast<const f32x4*>(part_o + (row * S + k) * kLatent + 8 * lane);
      const f32x4 v0 = src[0], v1 = src[1];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[c] += wgt * v0[c];
        acc[4 + c] += wgt * v1[c];
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
