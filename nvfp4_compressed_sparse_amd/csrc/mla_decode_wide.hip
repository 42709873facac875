// MLA decode for 64 or 128 heads over a paged cache of NVFP4 (352-byte) rows with sparse lists, for
// gfx950: every selected row is gathered and dequantized once for all heads of its query token.  (FP8
// rows and dense decodes at these head counts run the 32-head-group kernel.)
//
// What it computes is the same as the 16/32-head kernel (launch post, section "原生 NVFP4 稀疏 MLA 解码
// 内核" (native NVFP4 sparse MLA decode kernel); the analysis page, section "A kernel that reads four
// bits directly"): softmax attention of each head's 576-wide absorbed query over the selected cached
// rows, with the 512-value latent as V, FP16 matrix operands and FP32 accumulation (each head's query
// scaled by a power of two into FP16's range, undone exactly in the score scale).  With 128 heads
// the work per row is large enough for the matrix cores to be the bound, so the design differs from
// the pages' memory-bound kernel: one row is shared by far more MFMA work than its dequantization.
//
// Work decomposition: one 256-thread workgroup (4 wavefronts, one per SIMD) per compute unit and per
// (query token, split); wave w owns heads 16*HT*w .. 16*HT*w + 16*HT-1 for the whole step.
//   * rows are consumed in steps of 32, gathered raw by LDS-DMA into a ring several steps ahead;
//   * each step is dequantized once, cooperatively, into two FP16 tiles in LDS: K row-major (576 dims
//     per row, the A operand of S^T = K q^T) and V^T column-major (32 rows per latent column, the A
//     operand of O^T = V^T P^T), the V^T tile's rows in the order in which each lane holds P;
//   * each wave keeps its query fragments (B operand of S^T) in registers, runs its heads' online
//     softmax without any cross-wave exchange (it sees every row of the step for its heads), keeps P
//     in registers as the B operand of O^T, and accumulates O^T for its heads and all 512 columns
//     (MFMA accumulators, AGPR-resident);
//   * two phases per step, one barrier each: phase 1 = S^T of step k from the K tile while the V^T
//     tile of step k is written; phase 2 = O^T of step k from the V^T tile while the K tile of step
//     k+1 is written.  So the dequantization VALU work of one tile overlaps the MFMAs on the other.
//   * split results are merged in the same launch by the last workgroup of a query token to finish.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kWThreads = kWideDecodeThreads;
constexpr int kWWaves = kWThreads / 64;
constexpr int kWStep = 32;                       // rows per step
constexpr int kWMaxChunk = 2048;                 // list entries one workgroup holds
constexpr int kWEntriesPerThread = kWMaxChunk / kWThreads;
constexpr float kWLazyRescale = 15.0f;           // a score may exceed the softmax reference by this (log2)
                                                 // before it rises: P < 2^15 stays inside FP16
constexpr float kWRefMargin = 4.0f;              // a risen reference sits this far above the new maximum
constexpr int kKStride = kQK * 2 + 16;           // bytes per row of the FP16 K tile (bank spread)
constexpr int kVStride = kWStep * 2 + 16;        // bytes per column of the FP16 V^T tile (bank spread)

struct WGeo {
  static constexpr int kRowBytes = kNvfp4Row;
  static constexpr int kChunks = kRowBytes / 16;                 // 22 or 36 per row
  static constexpr int kStride = kRowBytes + 16;                 // LDS bytes per raw row
  static constexpr int kWaveRows = kWStep / kWWaves;             // 8 rows per wave per step
  static constexpr int kWaveChunks = kWaveRows * (kChunks + 1);  // 184 or 296 LDS chunks
  static constexpr int kLoads = (kWaveChunks + 63) / 64;         // 3 or 5 DMA loads per wave per step
  static_assert((kLoads - 1) * 64 < kWaveChunks, "only a wave's last gather load is partial");
  static_assert(8 * 64 * 16 <= kWaveRows * kKStride, "rescale staging fits a wave's rows of the K tile");
  static constexpr int kSlot = kWStep * kStride;
  static constexpr int kSlots = 6;                               // ring depth
};

struct WShared {
  uint8_t ring[WGeo::kSlots * WGeo::kSlot];
  uint8_t ktile[kWStep * kKStride];   // FP16 K of the step being scored, row-major
  uint8_t vtile[kLatent * kVStride];  // FP16 V^T of the step being accumulated, column-major
  uint32_t rowlist[kWMaxChunk];       // 16-byte row addresses of the split's valid entries
  int wcount[kWWaves];
  int last;
};

// Row of a step that contraction position 8G + j (j < 8) of O^T += V^T P^T stands for: a lane of
// group G holds, after S^T, the scores of rows 4G..4G+3 of row tile 0 and of row tile 1.
__device__ __forceinline__ int wide_pv_row(int G, int j) { return (j < 4 ? 4 * G + j : 12 + 4 * G + j); }

template <int HT>
__global__ __launch_bounds__(kWThreads, 1) void decode_wide_kernel(DecodeArgs a) {
  using G = WGeo;
  constexpr int ROWB = G::kRowBytes;
  constexpr int RS = G::kStride;
  constexpr int NL = G::kLoads;
  constexpr int NS = G::kSlots;
  constexpr int NHW = 16 * HT;  // heads per wave
  __shared__ __attribute__((aligned(16))) WShared sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;

  const int j = xcd_logical_id(blockIdx.x, gridDim.x);
  const int s = j % a.splits;
  const int qtok = j / a.splits;
  const int b = qtok / a.T, t = qtok % a.T;
  const int hw0 = w * NHW;

  // the wave's query fragments (B operand of S^T): lane (g, n) holds head hw0+16tt+n, dims
  // 32ks+8g..+7; loaded first (raw bf16), converted once the prologue has waited for memory anyway
  u32x4 qraw[HT][18];
  {
    const uint16_t* qb = a.q + ((int64_t)qtok * a.H + hw0 + n) * kQK + 8 * g;
#pragma unroll
    for (int tt = 0; tt < HT; ++tt)
#pragma unroll
      for (int ks = 0; ks < 18; ++ks)
        qraw[tt][ks] = *reinterpret_cast<const u32x4*>(qb + (int64_t)16 * tt * kQK + 32 * ks);
  }

  // append (as in the 16/32-head kernel): wave w quantizes new row w of the request while the page table
  // is in flight and writes it once the table is staged; rows w + 4i, when T > 4, are loaded and
  // quantized where they are written
  const bool append = a.new_nope != nullptr;
  u32x4 nraw = u32x4{0u, 0u, 0u, 0u};
  uint32_t nrope = 0;
  if (append && w < a.T) {
    const int64_t nr = (int64_t)b * a.T + w;
    nraw = *reinterpret_cast<const u32x4*>(a.new_nope + nr * a.new_nope_stride + 8 * lane);
    nrope = a.new_rope[nr * a.new_rope_stride + lane];
  }

  // ---- prologue: valid rows of this split -> LDS list of 16-byte row addresses (as in the 16/32-head
  // kernel: page-table entries staged in LDS in the same memory round trip as the list entries,
  // invalid entries dropped, order kept)
  const int e0 = s * a.chunk;
  const int npg = (int)a.bt_stride;
  constexpr int kBtCap = NS * G::kSlot / 4;
  const bool staged = npg <= kBtCap;
  int* btl = reinterpret_cast<int*>(sh.ring);
  const int* btg = a.block_table + (int64_t)b * a.bt_stride;
  constexpr int kBtPer = 12;  // entries per thread loaded before any is stored (tables up to 3,072 pages)
  const bool bt_regs = npg <= kWThreads * kBtPer;
  int btv[kBtPer];
  if (bt_regs) {
#pragma unroll
    for (int k = 0; k < kBtPer; ++k) btv[k] = tid + kWThreads * k < npg ? btg[tid + kWThreads * k] : 0;
  }
  const int L = a.ctx[b];
  const int lim = a.causal ? L - a.T + t : L - 1;
  const int e1 = (e0 + a.chunk < a.entries) ? e0 + a.chunk : a.entries;

  constexpr int EPT = kWEntriesPerThread;
  int pos[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) pos[k] = -1;
  if (e1 > e0) {
    const int ebase = e0 + EPT * tid;
    const int* ip = a.indices + (int64_t)qtok * a.entries + ebase;
    if (((uintptr_t)a.indices & 15) == 0 && (((int64_t)qtok * a.entries + e0) & 3) == 0 && ebase + EPT <= e1) {
#pragma unroll
      for (int h = 0; h < EPT / 4; ++h) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(ip + 4 * h);
#pragma unroll
        for (int k = 0; k < 4; ++k) pos[4 * h + k] = (int)x[k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < EPT; ++k) pos[k] = ebase + k < e1 ? ip[k] : -1;
    }
  }
  RowWords nw{0u, 0u, 0u};
  if (append && w < a.T) {
    nw = quant_row_words<0>(nraw, nrope, lane);
    asm volatile("" : "+v"(nw.lat0), "+v"(nw.lat1), "+v"(nw.rope));  // keep the quantization here
  }
  if (bt_regs) {
#pragma unroll
    for (int k = 0; k < kBtPer; ++k)
      if (tid + kWThreads * k < npg) btl[tid + kWThreads * k] = btv[k];
  } else if (staged) {
    for (int i = tid; i < npg; i += kWThreads) btl[i] = btg[i];
  }
  __syncthreads();  // staged page-table entries visible

  if (append) {
    // the request's new rows at positions L - T + r, written by one wave each (skipped where the writer
    // would skip the slot); complete before any gather (the wait before the row list's barrier)
    for (int r = w; r < a.T; r += kWWaves) {
      RowWords rw = nw;
      if (r >= kWWaves) {
        const int64_t nr = (int64_t)b * a.T + r;
        const u32x4 raw = *reinterpret_cast<const u32x4*>(a.new_nope + nr * a.new_nope_stride + 8 * lane);
        rw = quant_row_words<0>(raw, a.new_rope[nr * a.new_rope_stride + lane], lane);
      }
      const int p = L - a.T + r;
      if (p < 0 || (p >> 6) >= npg) continue;
      const int page = staged ? btl[p >> 6] : btg[p >> 6];
      if (page < 0 || page >= a.num_pages) continue;
      store_row_words<0>(rw, a.wpool + (uint64_t)page * (uint64_t)a.page_stride + (uint64_t)(p & 63) * ROWB, lane);
    }
  }

  uint32_t addr[EPT];
  uint32_t vmask = 0;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int pg = (pos[k] >= 0 ? pos[k] : 0) >> 6;
    const bool inr = pos[k] >= 0 && pos[k] <= lim && pg < npg;
    int page = -1;
    if (inr) page = staged ? btl[pg] : btg[pg];
    const bool ok = inr && page >= 0 && page < a.num_pages;
    addr[k] = ok ? (uint32_t)(((uint64_t)page * (uint64_t)a.page_stride + (uint64_t)(pos[k] & 63) * ROWB) >> 4) : 0u;
    vmask |= (uint32_t)ok << k;
  }
  int off = 0, wave_total = 0;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const uint64_t bal = __ballot((vmask >> k) & 1u);
    off += __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    wave_total += __builtin_popcountll(bal);
  }
  if (lane == 0) sh.wcount[w] = wave_total;
  __syncthreads();
  int n_valid = 0;
#pragma unroll
  for (int ww = 0; ww < kWWaves; ++ww) {
    off += ww < w ? sh.wcount[ww] : 0;
    n_valid += sh.wcount[ww];
  }
#pragma unroll
  for (int k = 0; k < EPT; ++k)
    if (vmask & (1u << k)) sh.rowlist[off++] = addr[k];
  wait_vmem();
  __syncthreads();  // row list complete; the page-table staging area (the ring) is free again

  const int nsteps = (n_valid + kWStep - 1) / kWStep;
  auto slot_ptr = [&](int st) { return sh.ring + (st % NS) * G::kSlot; };
  // gather of one step: wave w fills rows 8w..8w+7; lane l of load u fills LDS chunk e = 64u + l of
  // the wave's rows, chunk c of row e / (kChunks + 1); the chunk after a row's last one is padding and
  // receives the row's first chunk again, so only the lanes past the wave's last row are masked
  auto issue_step = [&](int st) {
    const int rb = st * kWStep + G::kWaveRows * w;
    const uint8_t* dst = slot_ptr(st) + G::kWaveRows * w * RS;
    uint32_t a16[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int r = rb + (64 * u + lane) / (G::kChunks + 1);
      a16[u] = sh.rowlist[r < n_valid ? r : 0];
    }
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int e = 64 * u + lane;
      const int c = e % (G::kChunks + 1);
      // chunk offset folded into the 16-byte row address before the 64-bit add: no per-lane 64-bit
      // pointers stay live across the loop
      const uint8_t* src = a.pool + (uint64_t)(a16[u] + (uint32_t)(c < G::kChunks ? c : 0)) * 16u;
      if (u < NL - 1 || e < G::kWaveChunks) dma16<true>(src, dst + 1024 * u);
    }
  };

  // K tile of one step, in pieces that the MFMA loop of phase 2 interleaves: thread tid dequantizes
  // row tid/8, 16-byte chunks c8 + 8i (piece i < 8) of the latent and, as piece 8, the rope dims
  // 512 + 8*c8 .. +7.  kin holds the raw words: the latent's nibble dwords, the scale dwords, the rope.
  const int kr_row = tid >> 3, c8 = tid & 7;
  uint8_t* const krow = sh.ktile + kr_row * kKStride;
  auto k_load = [&](int st, uint32_t (&kin)[18]) {
    const uint8_t* rr = slot_ptr(st) + kr_row * RS;
#pragma unroll
    for (int i = 0; i < 8; ++i) kin[i] = *reinterpret_cast<const uint32_t*>(rr + 4 * (c8 + 8 * i));
    const u32x4 sc0 = *reinterpret_cast<const u32x4*>(rr + 256);
    const u32x4 sc1 = *reinterpret_cast<const u32x4*>(rr + 272);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kin[8 + i] = sc0[i];
      kin[12 + i] = sc1[i];
    }
    const u32x2 rp = *reinterpret_cast<const u32x2*>(rr + 288 + 8 * c8);
    kin[16] = rp[0];
    kin[17] = rp[1];
  };
  auto k_piece = [&](int i, const uint32_t (&kin)[18]) {
    if (i == 8) {
      *reinterpret_cast<f16x8*>(krow + 2 * kLatent + 16 * c8) =
          as_f16x8(e4m3x2_to_f16<false>(kin[16]), e4m3x2_to_f16<true>(kin[16]), e4m3x2_to_f16<false>(kin[17]),
                   e4m3x2_to_f16<true>(kin[17]));
      return;
    }
    f16x8 v;
    // block of chunk c8 + 8i is (c8 >> 1) + 4i: byte c8 >> 1 of scale dword i, broadcast to a pair
    const uint32_t sd = kin[8 + i];
    const f16x2 ss = e4m3x2_to_f16<false>(__builtin_amdgcn_perm(sd, sd, (uint32_t)(c8 >> 1) * 0x0101u));
    v = as_f16x8(fp4x2_to_f16<0>(kin[i]) * ss, fp4x2_to_f16<1>(kin[i]) * ss, fp4x2_to_f16<2>(kin[i]) * ss,
                 fp4x2_to_f16<3>(kin[i]) * ss);

    *reinterpret_cast<f16x8*>(krow + 16 * (c8 + 8 * i)) = v;
  };

  // V^T tile of one step, in pieces that the MFMA loop of phase 1 interleaves: thread tid = 4*co + G
  // dequantizes latent columns 8co..8co+7 of the rows wide_pv_row(G, 0..7) (pairs of neighbouring
  // rows) and writes, per column (piece c < 8), the 8 contraction positions 8G..8G+7 as one 16-byte
  // store.  v_load fetches the raw words, v_prep pairs the rows up (vpr), v_piece converts a column.
  const int Gq = tid & 3, co = tid >> 2;
  auto v_load = [&](int st, uint32_t (&vin)[16]) {
    const uint8_t* slot = slot_ptr(st);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint8_t* ra = slot + wide_pv_row(Gq, 2 * p) * RS;
      vin[4 * p + 0] = *reinterpret_cast<const uint32_t*>(ra + 4 * co);
      vin[4 * p + 1] = *reinterpret_cast<const uint32_t*>(ra + RS + 4 * co);
      vin[4 * p + 2] = *reinterpret_cast<const uint32_t*>(ra + 256 + 4 * (co >> 3));
      vin[4 * p + 3] = *reinterpret_cast<const uint32_t*>(ra + RS + 256 + 4 * (co >> 3));
    }
  };
  // vpr[p][0..2]: the two nibble interleaves (even, odd columns) of rows (a, b) and their scale pair
  auto v_prep = [&](const uint32_t (&vin)[16], uint32_t (&vpr)[4][3]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t bsel = (uint32_t)((co >> 1) & 3);
      const uint32_t da = vin[4 * p], db = vin[4 * p + 1], sa = vin[4 * p + 2], sb = vin[4 * p + 3];
      vpr[p][0] = nib_pair<0>(da, db);
      vpr[p][1] = nib_pair<1>(da, db);
      // block scales of rows a and b as an FP16 pair
      vpr[p][2] = __builtin_bit_cast(uint32_t, e4m3x2_to_f16<false>(__builtin_amdgcn_perm(sb, sa, bsel | ((4 + bsel) << 8))));
    }
  };
  auto v_piece = [&](int c, const uint32_t (&vpr)[4][3]) {
    f16x2 v[4];  // FP16 pairs (row a, row b) of column c
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t e = vpr[p][c & 1];
      const f16x2 sp = __builtin_bit_cast(f16x2, vpr[p][2]);
      f16x2 x;
      switch (c >> 1) {
        case 0: x = fp4x2_to_f16<0>(e); break;
        case 1: x = fp4x2_to_f16<1>(e); break;
        case 2: x = fp4x2_to_f16<2>(e); break;
        default: x = fp4x2_to_f16<3>(e); break;
      }
      v[p] = x * sp;
    }
    *reinterpret_cast<f16x8*>(sh.vtile + (8 * co + c) * kVStride + 16 * Gq) = as_f16x8(v[0], v[1], v[2], v[3]);
  };

  // FP16 query fragments: each head scaled by its power of two 2^kq (largest magnitude to [2^15, 2^16),
  // the four lane groups together hold the head's 576 values), its score scale by 2^-kq
  f16x8 qf[HT][18];
  float sl2h[HT];  // softmax scale * log2(e) * 2^-kq of head hw0+16tt+n
#pragma unroll
  for (int tt = 0; tt < HT; ++tt) {
    uint32_t mq = 0;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const uint32_t m = bf16x8_max_mag(qraw[tt][ks]);
      mq = mq > m ? mq : m;
    }
    const int kq = q_shift(group4_max_u32(mq));
    sl2h[tt] = __builtin_ldexpf(a.scale_log2, -kq);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const u32x4 raw = qraw[tt][ks];
      qf[tt][ks] = as_f16x8(bf16x2_pow2_to_f16x2(raw[0], kq), bf16x2_pow2_to_f16x2(raw[1], kq),
                            bf16x2_pow2_to_f16x2(raw[2], kq), bf16x2_pow2_to_f16x2(raw[3], kq));
    }
  }

  float ref[HT], lsum[HT];  // softmax reference (base 2) and this lane's partial sum, per head 16tt+n
  f32x4 o[HT][32];          // O^T tile ct: O[head hw0+16tt+n][column 16ct+4g+i] = o[tt][ct][i]
#pragma unroll
  for (int tt = 0; tt < HT; ++tt) {
    ref[tt] = -INFINITY;
    lsum[tt] = 0.0f;
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) o[tt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  int last_issued = -1;
#pragma unroll
  for (int st = 0; st < NS; ++st)
    if (st < nsteps) {
      issue_step(st);
      last_issued = st;
    }
  if (nsteps > 0) {
    wait_steps<NL>(last_issued);
    lds_barrier();  // step 0's rows visible
    uint32_t kin[18];
    k_load(0, kin);
#pragma unroll
    for (int i = 0; i < 9; ++i) k_piece(i, kin);
    lds_barrier();  // K tile of step 0 complete
  }

  for (int k = 0; k < nsteps; ++k) {
    // ---- phase 1: S^T of step k from the K tile, interleaved with the V^T tile of step k (the A
    // operands are read two k-steps ahead)
    f32x4 sacc[2][HT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int tt = 0; tt < HT; ++tt) sacc[rt][tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    {
      uint32_t vin[16];
      uint32_t vpr[4][3];
      v_load(k, vin);
      auto ka = [&](int ks, int rt) {
        return *reinterpret_cast<const f16x8*>(sh.ktile + (16 * rt + n) * kKStride + 2 * (32 * ks + 8 * g));
      };
      constexpr int QD = 4;  // k-steps of A operands in flight
      f16x8 A[QD][2];
#pragma unroll
      for (int c = 0; c < QD - 1; ++c) {
        A[c][0] = ka(c, 0);
        A[c][1] = ka(c, 1);
      }
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        if (ks + QD - 1 < 18) {
          A[(ks + QD - 1) % QD][0] = ka(ks + QD - 1, 0);
          A[(ks + QD - 1) % QD][1] = ka(ks + QD - 1, 1);
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int tt = 0; tt < HT; ++tt) sacc[rt][tt] = mfma16x16x32(A[ks % QD][rt], qf[tt][ks], sacc[rt][tt]);
        if (ks == 1) v_prep(vin, vpr);
        if (ks >= 2 && ks < 10) v_piece(ks - 2, vpr);
      }
    }

    // online softmax of the wave's heads over the step's 32 rows: lane (g, n) holds rows 16rt+4g+i
    f16x8 pb[HT];
    float alpha[HT];
    bool resc[HT];  // wave-uniform: head tile tt's accumulators need alpha[tt]
    const int rbase = k * kWStep;
#pragma unroll
    for (int tt = 0; tt < HT; ++tt) {
      float sv[2][4];
      float m = -INFINITY;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rbase + 16 * rt + 4 * g + i;
          // one rounding of the scaled score (no fused multiply-add into P below): the maximum, the
          // reference and P all see the same value
          sv[rt][i] = row < n_valid ? __fmul_rn(sacc[rt][tt][i], sl2h[tt]) : -INFINITY;
          m = fmaxf(m, sv[rt][i]);
        }
      m = group4_max(m);
      // a difference, not m > ref + 15: a large reference would absorb the 15 and let P overflow FP16
      const bool raise = m - ref[tt] > kWLazyRescale;
      alpha[tt] = 1.0f;
      resc[tt] = false;
      if (__any(raise)) {  // the reference rises; O is rescaled in phase 2 (rare after the first step)
        // The new reference sits kWRefMargin above the maximum, so that a later rise needs a score
        // kWLazyRescale + kWRefMargin above it.  P stays below 2^15, and P of a row below 2^-14 (an
        // FP16 subnormal) weighs less than 2^-10 of the maximum row: its coarser rounding is
        // negligible.
        const float rold = ref[tt];
        const float rnew = raise ? m + kWRefMargin : rold;
        alpha[tt] = rold == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(rold - rnew);
        lsum[tt] *= alpha[tt];
        ref[tt] = rnew;
        resc[tt] = __any(raise && rold != -INFINITY);  // O is still zero on the first rise
      }
      const float mr = ref[tt] == -INFINITY ? 0.0f : ref[tt];
      float p[2][4];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[rt][i] = __builtin_amdgcn_exp2f(sv[rt][i] - mr);
      lsum[tt] += ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
      pb[tt] = as_f16x8(f16x2{(_Float16)p[0][0], (_Float16)p[0][1]}, f16x2{(_Float16)p[0][2], (_Float16)p[0][3]},
                        f16x2{(_Float16)p[1][0], (_Float16)p[1][1]}, f16x2{(_Float16)p[1][2], (_Float16)p[1][3]});
    }

    if (k + 1 < nsteps) wait_steps<NL>(last_issued - (k + 1));  // this wave's rows of step k+1 landed
    lds_barrier();  // V^T tile of step k complete, K tile consumed, raw slot of step k free
    if (k + NS < nsteps) {
      issue_step(k + NS);
      last_issued = k + NS;
    }

    // ---- phase 2: O^T += V^T P^T for step k, interleaved with the K tile of step k+1 (the A operands
    // are read two column tiles ahead)
    // O *= alpha before this step's products, through this wave's rows of the K tile (every wave is
    // past its S^T, and this wave writes those rows again only below), 8 tiles at a time: stored from
    // the accumulator registers, reloaded, multiplied and moved back.  A multiply on the accumulators
    // in place would make the compiler keep all of them in VGPRs, far beyond the register file.
#pragma unroll
    for (int tt = 0; tt < HT; ++tt) {
      if (!resc[tt]) continue;
      f32x4* stage = reinterpret_cast<f32x4*>(sh.ktile + w * G::kWaveRows * kKStride) + lane;
#pragma unroll
      for (int c0 = 0; c0 < 32; c0 += 8) {
#pragma unroll
        for (int c = 0; c < 8; ++c) stage[64 * c] = o[tt][c0 + c];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int c = 0; c < 8; ++c) stage[64 * c] = stage[64 * c] * alpha[tt];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int c = 0; c < 8; ++c) o[tt][c0 + c] = stage[64 * c];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
    }
    {
      // (after the last step this dequantizes a stale ring slot into the K tile, which is never read
      // again: cheaper than a branch in the loop)
      uint32_t kin[18];
      k_load(k + 1, kin);
      auto va = [&](int ct) {
        return *reinterpret_cast<const f16x8*>(sh.vtile + (16 * ct + n) * kVStride + 16 * g);
      };
      constexpr int PD = 4;  // A operands in flight
      f16x8 A[PD];
#pragma unroll
      for (int c = 0; c < PD - 1; ++c) A[c] = va(c);
#pragma unroll
      for (int ct = 0; ct < 32; ++ct) {
        if (ct + PD - 1 < 32) A[(ct + PD - 1) % PD] = va(ct + PD - 1);
#pragma unroll
        for (int tt = 0; tt < HT; ++tt) o[tt][ct] = mfma16x16x32(A[ct % PD], pb[tt], o[tt][ct]);
        if (ct >= 2 && ct < 11) k_piece(ct - 2, kin);
      }
    }
    lds_barrier();  // K tile of step k+1 complete, V^T tile consumed
  }

  // ---- epilogue: per head, the sum over the four lane groups; normalize (o is only read from here
  // on, tile by tile)
  const int S = a.splits;
  float lse[HT], inv[HT];
#pragma unroll
  for (int tt = 0; tt < HT; ++tt) {
    const float Lh = group4_sum(lsum[tt]);
    inv[tt] = Lh > 0.0f ? 1.0f / Lh : 0.0f;
    lse[tt] = Lh > 0.0f ? (ref[tt] + __log2f(Lh)) * 0.69314718055994531f : -INFINITY;
  }
  if (S == 1) {
#pragma unroll
    for (int tt = 0; tt < HT; ++tt) {
      const int64_t hrow = (int64_t)qtok * a.H + hw0 + 16 * tt + n;
      if (g == 0 && a.lse) a.lse[hrow] = lse[tt];
      u32x2* dst = reinterpret_cast<u32x2*>(a.out + hrow * kLatent + 4 * g);
#pragma unroll
      for (int ct = 0; ct < 32; ++ct) {
        const f32x4 v = o[tt][ct] * inv[tt];
        dst[4 * ct] = u32x2{pack_bf16_rne(v[0], v[1]), pack_bf16_rne(v[2], v[3])};
      }
    }
    return;
  }

  // ---- split merge, as in the 16/32-head kernel: every workgroup stores its normalized result (FP16)
  // and lse with agent-coherent relaxed stores, waits for their completion, then moves the query
  // token's arrival counter; the workgroup that moves it to S merges, reading with coherent loads.
#pragma unroll
  for (int tt = 0; tt < HT; ++tt) {
    const int64_t hrow = (int64_t)qtok * a.H + hw0 + 16 * tt + n;
    uint64_t* dst = reinterpret_cast<uint64_t*>(a.part_o + (hrow * S + s) * kLatent + 4 * g);
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) store_coherent_h4(dst + 4 * ct, o[tt][ct] * inv[tt]);
    if (g == 0) __hip_atomic_store(a.part_lse + hrow * S + s, lse[tt], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's split results are complete
  __syncthreads();
  int* counter = a.counters + qtok;
  if (tid == 0) sh.last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
  __syncthreads();
  if (!sh.last) return;
  // weights e^{lse_k - M} of every split, per head, in LDS (the ring is free): [wave][tt][head][split].
  // The splits are added in their order, this workgroup's own result rounded to FP16 as the stored ones
  // are, so the merged bits do not depend on which split's workgroup merges.
  float* wts = reinterpret_cast<float*>(sh.ring);
  static_assert(kWWaves * 2 * 16 * 64 * 4 <= WGeo::kSlots * WGeo::kSlot, "merge weights fit the ring");
#pragma unroll
  for (int tt = 0; tt < HT; ++tt) {
    const int64_t hrow = (int64_t)qtok * a.H + hw0 + 16 * tt + n;
    float* wh = wts + ((w * 2 + tt) * 16 + n) * 64;
    float M = -INFINITY;
    for (int k = g; k < S; k += 4) {  // the four lane groups share the loads
      const float lk = k == s ? lse[tt] : load_coherent(a.part_lse + hrow * S + k);
      wh[k] = lk;
      M = fmaxf(M, lk);
    }
    M = group4_max(M);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's weight writes are done
    float Z = 0.0f;
    for (int k = 0; k < S; ++k) {
      const float lk = wh[k];
      Z += M == -INFINITY ? 0.0f : __expf(lk - M);
    }
    const float zinv = Z > 0.0f ? 1.0f / Z : 0.0f;
    u32x2* dst = reinterpret_cast<u32x2*>(a.out + hrow * kLatent + 4 * g);
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int k = 0; k < S; ++k) {
        if (M == -INFINITY) continue;
        const float wk = __expf(wh[k] - M);
        uint64_t x;
        if (k == s) {
          x = pack_h4(o[tt][ct] * inv[tt]);
        } else {
          const uint64_t* src = reinterpret_cast<const uint64_t*>(a.part_o + (hrow * S + k) * kLatent + 4 * g);
          x = __hip_atomic_load(const_cast<uint64_t*>(src + 4 * ct), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        acc += wk * h4_to_f32x4(x);
      }
      acc *= zinv;
      dst[4 * ct] = u32x2{pack_bf16_rne(acc[0], acc[1]), pack_bf16_rne(acc[2], acc[3])};
    }
    if (g == 0 && a.lse) a.lse[hrow] = Z > 0.0f ? M + __logf(Z) : -INFINITY;
  }
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int HT>
void launch_wide_one(const DecodeArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)(a.B * a.T * a.splits);
  hipLaunchKernelGGL((decode_wide_kernel<HT>), dim3(grid), dim3(kWThreads), 0, stream, a);
}

}  // namespace

hipError_t launch_decode_wide(int fmt, const DecodeArgs& a, hipStream_t stream) {
  // NVFP4 rows and sparse lists only (uses_wide_kernel); other formats run the 32-head-group kernel
  if (fmt != 0 || a.indices == nullptr || (a.H != 64 && a.H != 128)) return hipErrorInvalidValue;
  if (a.H == 64) launch_wide_one<1>(a, stream);
  else launch_wide_one<2>(a, stream);
  return hipGetLastError();
}

}  // namespace mla
