// MLA decode over a paged cache of NVFP4 (352-byte) or FP8 (576-byte) rows, for gfx950.
//
// What it computes (launch post, section "原生 NVFP4 稀疏 MLA 解码内核" (native NVFP4 sparse MLA decode
// kernel); the analysis page, section "A kernel that reads four bits directly"): for each query token
// and head, softmax attention of the 576-wide absorbed query over the selected cached rows, with the
// 512-value latent as V; only the selected compressed rows are loaded and they are unpacked on chip;
// accumulation is FP32.  As in the pages' kernel the matrix operands are FP16: every dequantized K/V
// value is exact in FP16; each head's bf16 query is first scaled by a power of two that brings its
// largest magnitude to [2^15, 2^16) (undone, exactly, in the score scale), so any finite bf16 query
// converts without overflow; P rounds to FP16.
//
// Work decomposition: one 512-thread workgroup (8 wavefronts, two per SIMD) per compute unit.
//   * workgroup = (query token, head group of 16*HT heads, split s of the token's position list); 64
//     and 128 heads are 2 or 4 groups of 32 heads, or, unsplit with enough query tokens, 1 or 2 groups
//     of 64 (HT = 4: each K and V fragment dequantized once for twice the heads); the pages split one
//     token's rows over a cluster of 3-8 SMs
//     merged through distributed shared memory; here the splits are separate workgroups merged by
//     their log-sum-exp weights.
//   * prologue: the page-table entries the split can touch are staged in LDS; the split's list entries
//     are validated (index < 0, past the causal limit, or on a page-table entry outside the pool ->
//     dropped, which also skips their loads) and compacted into an LDS list of row addresses (order
//     kept, so results are deterministic).  In the fused step (mla_sparse_decode_append) the prologue
//     also quantizes and stores the request's new rows, complete before the first gather.
//   * rows are consumed in steps of 64; one role's waves gather them by LDS-DMA (16 bytes per lane, no
//     registers) into a ring of raw row slots, several steps ahead.
//   * the waves specialise, as the pages' warp groups do: waves 0-3 score, waves 4-7 accumulate, one of
//     each per SIMD, so each SIMD interleaves a scoring and an accumulating wave.  The two roles work one
//     step apart and meet at one workgroup barrier per step.
//   * score wave rt computes S^T = K q^T for rows 16rt..16rt+15 of step k (M = 16 rows, N = 16 heads,
//     K = 576 dims, FP16 query fragments resident in registers).  Lane (g, m) reads its quarter of row
//     m and dequantizes it in registers into the MFMA A operand (cvt to FP16 + packed multiply by the
//     block scale).  It then forms P = 2^(s - ref) (base-2 scores) with the current softmax reference
//     and writes it to LDS as FP16.
//   * lazy, speculative softmax reference: ref (per head) is shared by all waves and changes only when
//     a score exceeds it by more than 15 in base 2 (so P stays below 2^15, inside FP16's range; a rise
//     costs a second barrier and rewrites of P and O, so it should be rare).  A score wave that sees such a score
//     raises a flag and publishes its per-head maxima; after the barrier every wave reads the flag and,
//     in that rare case, all of them derive the new reference from the published maxima, the
//     accumulators are rescaled and the score waves rewrite P before one extra barrier.
//   * accumulate wave cq computes O^T += V^T P^T for step k-1 over output columns 128cq..128cq+127 and
//     all heads.  Lane (g, m) reads, for 8 rows, the nibble dword holding columns 128cq+8m..+7 and feeds
//     column 128cq+8m+c to MFMA tile c (c < 8); the nibbles of two rows are interleaved with bit
//     operations so that each FP16 pair the converter produces is already (row r, row r+1) of one
//     column.
//   * epilogue: the score waves' softmax sums go through LDS; the accumulate waves normalize and write
//     (bf16 output, or FP16 partials and the split's lse for the merge by the last split to finish).
#include <cstddef>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

constexpr int kThreads = kDecodeThreads;
constexpr int kWaves = kThreads / 64;
constexpr int kStepRows = 64;
constexpr int kMaxChunk = 2048;        // list entries one workgroup holds
constexpr int kEntriesPerThread = kMaxChunk / kThreads;
constexpr float kLazyRescale = 15.0f;  // log2 headroom of the lazy softmax reference (P < 2^15 in FP16)
constexpr int kPStride = kStepRows * 2 + 16;  // bytes per head of a P tile: 64 FP16 values + padding
constexpr int kTileStride = kLatent + 4;       // floats per head of a split's result tile in LDS (padded)
constexpr int kPrologueSteps = 3;              // steps gathered before step 0 is awaited
constexpr int kHeadStart = 2;                  // of those, steps gathered before the query fragments

// Phase timeline, compiled only into the instrumented library (MLA_TIMELINE defined; the decode library
// has none of it): wave 0 of each workgroup keeps s_memrealtime stamps (a 100 MHz device clock) in
// scalar registers and writes them once, at its end, so no store or wait is added on the way.
// Slots: 0 start, 1 prologue loads issued, 2 page table staged, 3 row list complete, 4 step 0 visible,
// 5 last step done, 6 split result tile complete, 7 arrival counter taken, 8 end; 11 the launch's
// workgroups, 12 XCC id, 13 merged (1 for the workgroup that merged, or for an unsplit one), 14 logical
// workgroup index, 15 steps.
#ifdef MLA_TIMELINE
constexpr int kTimelineSlots = 16;
constexpr int kTimelineWGs = 4096;
__device__ uint64_t g_timeline[kTimelineWGs * kTimelineSlots];
#define MLA_STAMP(i) (stamp[(i)] = __builtin_amdgcn_s_memrealtime())
#else
#define MLA_STAMP(i) ((void)0)
#endif

// Geometry of the raw-row ring: steps of 64 rows; each of the four score waves gathers 16 rows of each
// step (see the kernel for why the score waves).  In LDS a row
// takes one 16-byte chunk more than it holds (368 or 592 bytes), so that the rows read by the 16 lanes
// of a lane group start on 16 different 4-bank groups (the stride is 28 or 20 dwords mod 64).  Lane l
// of a wave's DMA load u fills LDS chunk 64u+l of the wave's 16 rows; the padding chunks are not
// loaded.  A step's slot is reused NS steps later; step k is issued during step k-(NS-2).  Sparse FP8
// lists keep three slots: with the row list beside it, a fourth 37 KB slot would not fit in LDS; a
// 64-head workgroup keeps five NVFP4 slots beside its larger P tiles.
template <int FMT, bool DENSE, int NH>
struct Geo {
  static constexpr int kRowBytes = FMT == 0 ? kNvfp4Row : kFp8Row;
  static constexpr int kChunks = kRowBytes / 16;                 // 22 or 36 per row
  static constexpr int kStride = kRowBytes + 16;                 // LDS bytes per row
  static constexpr int kWaveRows = kStepRows / 4;               // 16 rows per gathering wave
  static constexpr int kWaveChunks = kWaveRows * (kChunks + 1);  // 368 or 592 LDS chunks per wave per step
  static constexpr int kLoads = (kWaveChunks + 63) / 64;         // 6 or 10 DMA loads per wave per step
  static_assert((kLoads - 1) * 64 < kWaveChunks, "only a wave's last gather load is partial");
  static constexpr int kSlot = kStepRows * kStride;              // bytes of one step
  static constexpr int kSlots = FMT == 0 ? (NH > 32 ? 5 : 6) : (DENSE ? 4 : 3);  // ring depth
  static constexpr int kRing = kSlots * kSlot;
};

// Row of a step that lane group g feeds to k-step kk of O^T += V^T P^T as its j-th contraction element
// (j < 8): the four lane groups read rows 4 apart, which start 16 banks apart (28*4 or 20*4 = 48 or 16
// dwords mod 64), and (j, j+1) = (2p, 2p+1) are neighbouring rows.  P is stored in the same order.
__device__ __forceinline__ int pv_row(int kk, int g, int j) { return 16 * (j >> 1) + 4 * g + 2 * kk + (j & 1); }

// P (FP16) of rows 16rt+4g+i (i < 4) of one head into its P-tile row, in the contraction order of
// pv_row: row 16a+4g+2kk+e sits at position 32kk+8g+2a+e.
__device__ __forceinline__ void write_p(uint8_t* prow, int rt, int g, const float (&p)[4]) {
  const f16x2 p01 = {(_Float16)p[0], (_Float16)p[1]}, p23 = {(_Float16)p[2], (_Float16)p[3]};
  *reinterpret_cast<f16x2*>(prow + 2 * (8 * g + 2 * rt)) = p01;
  *reinterpret_cast<f16x2*>(prow + 2 * (32 + 8 * g + 2 * rt)) = p23;
}

// LDS state shared by the roles.  A sparse list keeps the 16-byte addresses of its valid rows; a dense
// split (64-aligned, so that each step is one page) keeps its page-table entries instead.
template <int FMT, int NH, bool DENSE>
struct Shared {
  uint8_t ring[Geo<FMT, DENSE, NH>::kRing];
  uint8_t ptile[2][NH * kPStride];             // P of steps k (even/odd): [head][row], FP16
  uint32_t rowlist[DENSE ? 1 : kMaxChunk];     // sparse: row addresses of the split's valid entries
  int pages[DENSE ? kMaxChunk / kStepRows : 1];  // dense: page of each step, -1 = not in the pool
  int fb_page;                                   // dense: page holding the row masked rows read
  float smax[2][NH][4];             // per-score-wave maxima of step k, per head
  float wsum[NH][4];                // per-score-wave softmax sums
  int flag[2];                      // step k raised the softmax reference
  int wcount[kWaves];
  int last;                         // this workgroup merges the splits
  float tile_lse[NH];               // lse of this workgroup's split, per head
  int qshift[NH];                   // each head's query is scaled by 2^qshift[h] (q_shift of its largest |q|)
};

// The new reference of every head after a raise, from the score waves' maxima of the step (identical
// in every wave: same inputs).  Returns the factor that rescales sums taken against the old one.
// The wave holds head tiles tb..tb+HT-1.
template <int HT, int NH>
__device__ __forceinline__ void raise_reference(const float (&smax)[NH][4], int n, int tb, float (&ref)[HT],
                                                float (&alpha)[HT]) {
#pragma unroll
  for (int tt = 0; tt < HT; ++tt) {
    const int h = 16 * (tb + tt) + n;
    const float ms = fmaxf(fmaxf(smax[h][0], smax[h][1]), fmaxf(smax[h][2], smax[h][3]));
    const float rnew = ms - ref[tt] > kLazyRescale ? ms : ref[tt];
    alpha[tt] = ref[tt] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ref[tt] - rnew);
    ref[tt] = rnew;
  }
}

template <int HT, int FMT, bool DENSE>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(DecodeArgs a) {
  using G = Geo<FMT, DENSE, 16 * HT>;
  constexpr int ROWB = G::kRowBytes;
  constexpr int RS = G::kStride;
  constexpr int NL = G::kLoads;
  constexpr int NS = G::kSlots;
  constexpr int NH = 16 * HT;
  __shared__ __attribute__((aligned(16))) Shared<FMT, NH, DENSE> sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) role indices
  const int g = lane >> 4, n = lane & 15;
  const bool scorer = w < 4;
  const int r4 = w & 3;  // score waves: row tile; accumulate waves: column quarter
  // Score-wave tiles: at 16 and 32 heads a score wave takes one 16-row tile of each step for every head;
  // at 64 heads (HT = 4) two row tiles for half of the heads, so that each K fragment it dequantizes
  // feeds two head tiles, as at 32 heads, and its query fragments stay at 32 heads' worth of registers.
  constexpr int SRT = HT > 2 ? 2 : 1;   // row tiles per score wave
  constexpr int SHT = HT > 2 ? 2 : HT;  // head tiles per score wave
  const int rt0 = HT > 2 ? 2 * (r4 & 1) : r4;   // its first row tile
  const int ht0 = HT > 2 ? 2 * (r4 >> 1) : 0;   // its first head tile
#ifdef MLA_TIMELINE
  uint64_t stamp[kTimelineSlots] = {};
  MLA_STAMP(0);
#endif

  const int HG = a.H / NH;
  const int j = xcd_logical_id(blockIdx.x, gridDim.x);
  const int hg = j % HG;
  const int rest = j / HG;
  const int s = rest % a.splits;
  const int qtok = rest / a.splits;
  const int b = qtok / a.T, t = qtok % a.T;
  const int h0 = hg * NH;
  // The request's context length.  Dense: read here, before any memory operation the compiler cannot
  // see through (the DMA below), so that it is a scalar load, needed at once.  Sparse: loaded after the
  // list and page-table loads, since it is first needed once the table is staged; read here, its
  // dependent round trip was waited for before those loads went out (scalar loads return out of
  // order, so the wait for any kernel argument loaded after it waited for it too).
  int L = DENSE ? a.ctx[b] : 0;

  // The head group's queries (NH x 576 bf16, contiguous) are staged in LDS by DMA, issued first since
  // they depend on nothing else; the accumulate waves convert them in place and the score waves take
  // their fragments from there.  The staging area is the part of LDS the first gathers leave alone: ring
  // slots kQSlot.. (the last two at 16/32 heads; at 64 heads, whose 73.7 KB tile is read once per
  // workgroup instead of once per score wave, the last three and the P tiles after them, with two steps
  // gathered before step 0 is awaited).
  constexpr int kQSlot = HT > 2 ? 2 : NS - 2;
  constexpr int kQBytes = NH * kQK * 2;
  using SharedT = Shared<FMT, NH, DENSE>;
  static_assert(offsetof(SharedT, ptile) == G::kRing, "the P tiles follow the ring");
  static_assert(kQSlot * G::kSlot + kQBytes <= (HT > 2 ? G::kRing + 2 * NH * kPStride : G::kRing),
                "query staging must fit in the slots the first gathers leave alone");
  uint8_t* qstage = sh.ring + kQSlot * G::kSlot;
  {
    const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q + ((int64_t)qtok * a.H + h0) * kQK);
#pragma unroll
    for (int u = 0; u < (kQBytes / 1024 + kWaves - 1) / kWaves; ++u) {
      const int blk = w + kWaves * u;  // 1 KB block of the query tile
      if (blk < kQBytes / 1024) dma16(qsrc + 1024 * blk + 16 * lane, qstage + 1024 * blk);
    }
  }
  // The fused step (new rows given): wave w quantizes new row w of the request (the bf16 input, loaded
  // with the prologue's loads) while the page table and the list entries are in flight, and stores it
  // once the table is staged; rows w + 8i, when T > 8, are loaded and quantized there.  The stores are
  // complete before any gather (the wait before the row list's barrier).
  constexpr bool kAppend = FMT == 0 && !DENSE;
  const bool append = kAppend && a.new_nope != nullptr;
  u32x4 nraw = u32x4{0u, 0u, 0u, 0u};
  uint32_t nrope = 0;
  if (append && w < a.T) {
    const int64_t nr = (int64_t)b * a.T + w;
    nraw = *reinterpret_cast<const u32x4*>(a.new_nope + nr * a.new_nope_stride + 8 * lane);
    nrope = a.new_rope[nr * a.new_rope_stride + lane];
  }

  const int e0 = s * a.chunk;
  const int* btg = a.block_table + (int64_t)b * a.bt_stride;
  int lim = a.causal ? L - a.T + t : L - 1;  // (sparse: set again below, once L is loaded)
  if (tid < 2) sh.flag[tid] = 0;
  // published maxima start at -inf: a raise takes the largest published value, and only waves that
  // raise publish (every score a wave saw before stays within 2^15 of the reference it left behind)
  if (tid < 2 * NH * 4) (&sh.smax[0][0][0])[tid] = -INFINITY;
  int n_valid;
  if constexpr (DENSE) {
    // ---- prologue, dense: the split covers positions [e0, e1), e0 a multiple of 64 (the chunk is), so
    // step k is the request's logical page (e0 >> 6) + k; its table entry is staged, -1 when it is not
    // in the pool or lies beyond the table width (those rows select nothing: their scores are masked)
    const int e_end = lim + 1 < a.entries ? lim + 1 : a.entries;
    const int e1 = (e0 + a.chunk < e_end) ? e0 + a.chunk : e_end;
    n_valid = e1 > e0 ? e1 - e0 : 0;
    int pgv = -1;
    if (tid < a.chunk / kStepRows) {
      const int p = (e0 >> 6) + tid;
      const int pg = p < a.bt_stride ? btg[p] : -1;
      pgv = pg >= 0 && pg < a.num_pages && tid * kStepRows < n_valid ? pg : -1;
      sh.pages[tid] = pgv;
    }
    // masked rows are never read from unwritten memory (bytes 0x7F/0xFF decode to NaN, and a zero
    // weight times NaN is NaN): they are redirected to the first row of the split's first step whose
    // page is in the pool; a split without one selects nothing
    const uint64_t okb = __ballot(pgv >= 0);  // wave 0 holds every step (at most 32)
    const int fbv = __shfl(pgv, okb ? (int)__builtin_ctzll(okb) : 0, 64);
    if (tid == 0) sh.fb_page = okb ? fbv : -1;
    wait_vmem();      // the query DMA has landed
    __syncthreads();  // staged pages and queries visible
    if (sh.fb_page < 0) n_valid = 0;
  } else {
  // ---- prologue, sparse: valid rows of this split -> LDS list of 16-byte row addresses.
  // The request's whole page-table row (it does not depend on the context length) is staged in LDS
  // with coalesced loads while the context length and the split's list entries load at the same
  // time: one memory round trip instead of two or three dependent ones.
  const int npg = (int)a.bt_stride;
  constexpr int kBtCap = kQSlot * G::kSlot / 4;  // below the query staging area
  const bool staged = npg <= kBtCap;
  int* btl = reinterpret_cast<int*>(sh.ring);
  constexpr int kBtPer = 6;  // entries per thread loaded before any is stored (tables up to 3,072 pages)
  const bool bt_regs = npg <= kThreads * kBtPer;
  int btv[kBtPer];
  if (bt_regs) {
#pragma unroll
    for (int k = 0; k < kBtPer; ++k) btv[k] = tid + kThreads * k < npg ? btg[tid + kThreads * k] : 0;
  }
  const int e1 = (e0 + a.chunk < a.entries) ? e0 + a.chunk : a.entries;

  constexpr int EPT = kEntriesPerThread;
  int pos[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) pos[k] = -1;
  if (e1 > e0) {
    const int ebase = e0 + EPT * tid;
    const int* ip = a.indices + (int64_t)qtok * a.entries + ebase;
    if (((uintptr_t)a.indices & 15) == 0 && (((int64_t)qtok * a.entries + e0) & 3) == 0 && ebase + EPT <= e1) {
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(ip);
#pragma unroll
      for (int k = 0; k < 4; ++k) pos[k] = (int)x0[k];
    } else {
#pragma unroll
      for (int k = 0; k < EPT; ++k) pos[k] = ebase + k < e1 ? ip[k] : -1;
    }
  }
  MLA_STAMP(1);
  int ctx_v = a.ctx[b];  // a vector load (it follows the DMA), awaited after the page-table barrier
  RowWords nw{0u, 0u, 0u};
  if (append && w < a.T) {
    nw = quant_row_words<FMT>(nraw, nrope, lane);
    // keep the quantization here, ahead of the table's arrival, rather than next to its store
    asm volatile("" : "+v"(nw.lat0), "+v"(nw.lat1), "+v"(nw.rope));
  }
  if (bt_regs) {
#pragma unroll
    for (int k = 0; k < kBtPer; ++k)
      if (tid + kThreads * k < npg) btl[tid + kThreads * k] = btv[k];
  } else if (staged) {
    for (int i = tid; i < npg; i += kThreads) btl[i] = btg[i];
  }
  __syncthreads();  // staged page-table entries visible
  MLA_STAMP(2);
  asm("" : "+v"(ctx_v));  // used from here on, as a vector value: no wait for it before this point
  L = ctx_v;
  lim = a.causal ? L - a.T + t : L - 1;

  // the request's new rows at positions L - T + r, one wave each (a position before the start of the
  // context, beyond the table width or on a page outside the pool is not written, as the writer skips
  // such slots)
  if (append) {
    for (int r = w; r < a.T; r += kWaves) {
      RowWords rw = nw;
      if (r >= kWaves) {
        const int64_t nr = (int64_t)b * a.T + r;
        const u32x4 raw = *reinterpret_cast<const u32x4*>(a.new_nope + nr * a.new_nope_stride + 8 * lane);
        rw = quant_row_words<FMT>(raw, a.new_rope[nr * a.new_rope_stride + lane], lane);
      }
      const int p = L - a.T + r;
      if (p < 0 || (p >> 6) >= npg) continue;
      const int page = staged ? btl[p >> 6] : btg[p >> 6];
      if (page < 0 || page >= a.num_pages) continue;
      store_row_words<FMT>(rw, a.wpool + (uint64_t)page * (uint64_t)a.page_stride + (uint64_t)(p & 63) * ROWB,
                           lane);
    }
  }

  // a position past the limit, or on a page beyond the table width (only with a context longer than
  // the table allows), selects nothing; every table read of the lane is issued before any is used
  // (LDS reads from the staged table; a table too wide to stage is read from memory)
  bool inr[EPT];
  int pgc[EPT], page[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int pg = (pos[k] >= 0 ? pos[k] : 0) >> 6;
    inr[k] = pos[k] >= 0 && pos[k] <= lim && pg < npg;
    pgc[k] = inr[k] ? pg : 0;
  }
  if (staged) {
#pragma unroll
    for (int k = 0; k < EPT; ++k) page[k] = btl[pgc[k]];
  } else {
#pragma unroll
    for (int k = 0; k < EPT; ++k) page[k] = inr[k] ? btg[pgc[k]] : -1;
  }
  uint32_t addr[EPT];
  uint32_t vmask = 0;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const bool ok = inr[k] && page[k] >= 0 && page[k] < a.num_pages;
    addr[k] = ok ? (uint32_t)(((uint64_t)page[k] * (uint64_t)a.page_stride + (uint64_t)(pos[k] & 63) * ROWB) >> 4)
                 : 0u;
    vmask |= (uint32_t)ok << k;
  }
  // order-keeping compaction (entries ordered by thread, then k): this lane's offset in the wave is
  // the number of valid entries of lower lanes (ballots) plus its own earlier ones; waves follow each
  // other through LDS
  int off = 0, wave_total = 0;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const uint64_t bal = __ballot((vmask >> k) & 1u);
    off += __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    wave_total += __builtin_popcountll(bal);
  }
  if (lane == 0) sh.wcount[w] = wave_total;
  __syncthreads();
  n_valid = 0;
#pragma unroll
  for (int ww = 0; ww < kWaves; ++ww) {
    off += ww < w ? sh.wcount[ww] : 0;
    n_valid += sh.wcount[ww];
  }
#pragma unroll
  for (int k = 0; k < EPT; ++k)
    if (vmask & (1u << k)) sh.rowlist[off++] = addr[k];
  // every load issued so far (indices, page table, the query DMA) has landed before the gathers start
  wait_vmem();
  __syncthreads();  // row list and staged queries complete; the page-table staging area is free again
  MLA_STAMP(3);
  }

  const int nsteps = (n_valid + kStepRows - 1) / kStepRows;
  auto slot_ptr = [&](int st) { return sh.ring + (st % NS) * G::kSlot; };
  // lane l of gather load u fills LDS chunk e = 64u + l of the wave's rows: chunk c of row e / (kChunks
  // + 1).  The chunk after a row's last one is the row's padding: it receives the row's first chunk
  // again, so that only the lanes past the wave's last row (in its last load) are masked.  Per lane and
  // load: the row within the wave's rows and the byte offset of the chunk.
  // (dense: the byte offset within the step's page of that row and chunk)
  int g_row[NL];
  uint32_t g_off[NL];
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int e = (64 * u + lane) < G::kWaveChunks ? 64 * u + lane : G::kWaveChunks - 1;
    const int c = e % (G::kChunks + 1);
    g_row[u] = e / (G::kChunks + 1);
    g_off[u] = c < G::kChunks ? 16u * c : 0u;
    if (DENSE) g_off[u] += (uint32_t)((G::kWaveRows * r4 + g_row[u]) * ROWB);
  }
  // sparse: the 16-byte row addresses of this wave's loads of step st, from the LDS row list; rows past
  // the list (last step only) read its first row (their scores are masked)
  auto step_addrs = [&](int st, uint32_t (&a16)[NL]) {
    const uint32_t* rl = sh.rowlist + st * kStepRows + G::kWaveRows * r4;
    if ((st + 1) * kStepRows <= n_valid) {
#pragma unroll
      for (int u = 0; u < NL; ++u) a16[u] = rl[g_row[u]];
    } else {
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int r = st * kStepRows + G::kWaveRows * r4 + g_row[u];
        a16[u] = sh.rowlist[r < n_valid ? r : 0];
      }
    }
  };
  // sparse: load u of this wave's share of step st (row chunks read once: streaming loads)
  auto issue_load = [&](int st, int u, uint32_t a16) {
    const uint8_t* dst = slot_ptr(st) + G::kWaveRows * r4 * RS;
    const uint8_t* src = a.pool + ((uint64_t)a16 * 16u + g_off[u]);
    if (u < NL - 1 || 64 * u + lane < G::kWaveChunks) dma16<true>(src, dst + 1024 * u);
  };
  auto issue_step = [&](int st) {  // the gathering role only
    const uint8_t* dst = slot_ptr(st) + G::kWaveRows * r4 * RS;
    if constexpr (DENSE) {
      // one page per step; the rows of a masked step, or past the context in the last step, read the
      // split's fallback row instead (their scores are masked)
      const int pg = __builtin_amdgcn_readfirstlane(sh.pages[st]);
      if (pg >= 0 && (st + 1) * kStepRows <= n_valid) {
        const uint8_t* base = a.pool + (uint64_t)pg * (uint64_t)a.page_stride;
#pragma unroll
        for (int u = 0; u < NL; ++u)
          if (u < NL - 1 || 64 * u + lane < G::kWaveChunks) dma16(base + g_off[u], dst + 1024 * u);
      } else {
        const uint8_t* base = a.pool + (uint64_t)(pg >= 0 ? pg : 0) * (uint64_t)a.page_stride;
        const uint8_t* fb = a.pool + (uint64_t)sh.fb_page * (uint64_t)a.page_stride;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
          const int rin = G::kWaveRows * r4 + g_row[u];
          const bool live = pg >= 0 && st * kStepRows + rin < n_valid;
          const uint8_t* src = live ? base + g_off[u] : fb + (g_off[u] - (uint32_t)(rin * ROWB));
          if (u < NL - 1 || 64 * u + lane < G::kWaveChunks) dma16(src, dst + 1024 * u);
        }
      }
    } else {
      // every row address is read first (one LDS round trip), then the loads go out
      uint32_t a16[NL];
      step_addrs(st, a16);
#pragma unroll
      for (int u = 0; u < NL; ++u) issue_load(st, u, a16[u]);
    }
  };
  // The score waves gather.  Issuing a step's LDS-DMA loads stalls the issuing wave for a while (the
  // vector memory path takes them at a limited rate); issuing them from the accumulate waves instead
  // (which then also await them before publishing each step), or from all eight waves, measured slower
  // for both row formats.
  constexpr int kFirst = kPrologueSteps < kQSlot ? kPrologueSteps : kQSlot;
  constexpr int kEarly = kHeadStart < kFirst ? kHeadStart : kFirst;
  // steps gathered so far (score waves; wave-uniform)
  int issued = 0;
  // gather every step up to `upto` not yet issued
  auto issue_upto = [&](int upto) {
    upto = upto < nsteps - 1 ? upto : nsteps - 1;
    for (; issued <= upto; ++issued) issue_step(issued);
  };
  // wait until this wave's rows of step k are in LDS (steps after k may still be in flight)
  auto wait_for_step = [&](int k) {
    const int ahead = issued - 1 - k;
    if (ahead == NS - 3) {  // the steady state: every step up to k + NS - 3 issued
      wait_steps<NL>(NS - 3);
    } else {
      wait_steps<NL>(ahead < 0 ? 0 : ahead);
    }
  };

  // a split's normalized result tile, [NH][kTileStride] fp32, reuses the ring after the main loop
  float* tile = reinterpret_cast<float*>(sh.ring);
  // (64-head workgroups run unsplit only: the host launches them with S = 1, and they have no tile)
  static_assert(HT > 2 || NH * kTileStride * 4 <= G::kRing, "result tile must fit in the ring");
  float ref[HT];  // softmax reference per head 16tt+n (base 2), identical in every wave
#pragma unroll
  for (int tt = 0; tt < HT; ++tt) ref[tt] = -INFINITY;
  const int S = HT > 2 ? 1 : a.splits;

  if (scorer) {
    // ================= score waves: S^T = K q^T, P = 2^(s - ref) for their rows of step k: row tiles
    // rt0..rt0+SRT-1 (16 rows each), head tiles ht0..ht0+SHT-1
    // The first kPrologueSteps steps (at most kQSlot) are gathered before step 0 is awaited, kHeadStart of
    // them before the query fragments are formed and the rest after; the remainder of the prefetch
    // window follows once step 0 has landed.  With every workgroup of the launch gathering at once, a
    // deeper first window makes the memory system interleave the steps, so that step 0 completes only
    // when nearly all of them have; the staggered issue lets the first steps' requests queue first.
    // The query staging area (slots kQSlot..) is not touched before every score wave holds its fragments.
    issue_upto(kEarly - 1);
    lds_barrier();  // the FP16 query tile and the heads' shifts are in LDS (matches the accumulate waves' barrier)
    // query fragments (B operand), FP16: lane (g, n) holds head 16(ht0+tt)+n, latent dims 128g+8ks..+7
    // (ks < 16) and rope dims 512+16g+8(ks-16)..+7 (ks = 16, 17), each head scaled by its power of two
    // 2^kq (the head's score scale is scaled by 2^-kq): read from the tile the accumulate waves
    // converted.
    f16x8 qf[SHT][18];
    float sl2h[SHT];  // softmax scale * log2(e) * 2^-kq of head 16(ht0+tt)+n
#pragma unroll
    for (int tt = 0; tt < SHT; ++tt) {
      const int hq = 16 * (ht0 + tt) + n;
      sl2h[tt] = __builtin_ldexpf(a.scale_log2, -sh.qshift[hq]);
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const int d = ks < 16 ? 128 * g + 8 * ks : 512 + 16 * g + 8 * (ks - 16);
        qf[tt][ks] = *reinterpret_cast<const f16x8*>(qstage + 2 * (hq * kQK + d));
      }
    }
    issue_upto(kFirst - 1);
    wait_for_step(0);
    lds_barrier();  // step 0 visible (matches the accumulate waves' first barrier); q staging is free
    MLA_STAMP(4);
    float sref[SHT];  // this wave's copy of the reference of its heads (the same in every wave)
    float lsum[SRT][SHT];
#pragma unroll
    for (int tt = 0; tt < SHT; ++tt) {
      sref[tt] = -INFINITY;
#pragma unroll
      for (int ri = 0; ri < SRT; ++ri) lsum[ri][tt] = 0.0f;
    }

    for (int k = 0; k <= nsteps; ++k) {
      issue_upto(k + NS - 2);  // up to the slot of step k-2 (fully consumed)
      float sv[SRT][SHT][4];  // scores times the head's scale (base 2); masked rows -inf
      float psum[SRT][SHT];   // sum of this lane's speculative P per row tile and head tile
      if (k < nsteps) {
        // (dense: a step whose page is not in the pool selects nothing)
        const bool page_ok = !DENSE || sh.pages[DENSE ? k : 0] >= 0;
        const bool full = (k + 1) * kStepRows <= n_valid && page_ok;
        bool raise = false;
        float mxs[SRT][SHT];
#pragma unroll
        for (int ri = 0; ri < SRT; ++ri) {
          const int rt = rt0 + ri;
          const uint8_t* rr = slot_ptr(k) + (16 * rt + n) * RS;
          f32x4 acc[SHT];
#pragma unroll
          for (int tt = 0; tt < SHT; ++tt) acc[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          if constexpr (FMT == 0) {
            u32x4 nib[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) nib[q] = *reinterpret_cast<const u32x4*>(rr + 64 * g + 16 * q);
            const u32x2 sc = *reinterpret_cast<const u32x2*>(rr + 256 + 8 * g);
            const f16x2 s2[4] = {e4m3x2_to_f16<false>(sc[0]), e4m3x2_to_f16<true>(sc[0]),
                                 e4m3x2_to_f16<false>(sc[1]), e4m3x2_to_f16<true>(sc[1])};
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) {
              const uint32_t d = nib[ks >> 2][ks & 3];
              const _Float16 shv = ((ks >> 1) & 1) ? s2[ks >> 2].y : s2[ks >> 2].x;
              const f16x2 ss = {shv, shv};
              const f16x8 A = as_f16x8(fp4x2_to_f16<0>(d) * ss, fp4x2_to_f16<1>(d) * ss, fp4x2_to_f16<2>(d) * ss,
                                       fp4x2_to_f16<3>(d) * ss);
#pragma unroll
              for (int tt = 0; tt < SHT; ++tt) acc[tt] = mfma16x16x32(A, qf[tt][ks], acc[tt]);
            }
          } else {
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) {
              const u32x2 wv = *reinterpret_cast<const u32x2*>(rr + 128 * g + 8 * ks);
              const f16x8 A = as_f16x8(e4m3x2_to_f16<false>(wv[0]), e4m3x2_to_f16<true>(wv[0]),
                                       e4m3x2_to_f16<false>(wv[1]), e4m3x2_to_f16<true>(wv[1]));
#pragma unroll
              for (int tt = 0; tt < SHT; ++tt) acc[tt] = mfma16x16x32(A, qf[tt][ks], acc[tt]);
            }
          }
          {
            const u32x4 rp = *reinterpret_cast<const u32x4*>(rr + (FMT == 0 ? 288 : 512) + 16 * g);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              const uint32_t w0 = rp[2 * ks], w1 = rp[2 * ks + 1];
              const f16x8 A = as_f16x8(e4m3x2_to_f16<false>(w0), e4m3x2_to_f16<true>(w0),
                                       e4m3x2_to_f16<false>(w1), e4m3x2_to_f16<true>(w1));
#pragma unroll
              for (int tt = 0; tt < SHT; ++tt) acc[tt] = mfma16x16x32(A, qf[tt][16 + ks], acc[tt]);
            }
          }
          // scores of rows 16rt+4g+i, heads 16(ht0+tt)+n; base-2 maxima; speculative P = 2^(scale*s - ref)
          // with the current ref.  Only the last step can hold rows past the list (its padding): masked
          // -inf.  The scaled score is rounded once (no fused multiply-add) and both the maxima and P use
          // that rounded value, and the reference test compares a difference: so P <= 2^15 holds exactly
          // even where scores are large enough for an added 8 to round away.
          const int rbase = k * kStepRows + 16 * rt + 4 * g;
#pragma unroll
          for (int tt = 0; tt < SHT; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[ri][tt][i] = __fmul_rn(acc[tt][i], sl2h[tt]);
          if (!full) {
#pragma unroll
            for (int tt = 0; tt < SHT; ++tt)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (rbase + i >= n_valid || !page_ok) sv[ri][tt][i] = -INFINITY;
          }
#pragma unroll
          for (int tt = 0; tt < SHT; ++tt) {
            mxs[ri][tt] = max4(sv[ri][tt][0], sv[ri][tt][1], sv[ri][tt][2], sv[ri][tt][3]);
            raise |= mxs[ri][tt] - sref[tt] > kLazyRescale;
            const float mr = sref[tt] == -INFINITY ? 0.0f : sref[tt];
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sv[ri][tt][i] - mr);
            psum[ri][tt] = (p[0] + p[1]) + (p[2] + p[3]);
            write_p(sh.ptile[k & 1] + (16 * (ht0 + tt) + n) * kPStride, rt, g, p);
          }
        }
        if (__any(raise)) {  // rare: publish this wave's per-head maxima and raise the flag
#pragma unroll
          for (int ri = 0; ri < SRT; ++ri)
#pragma unroll
            for (int tt = 0; tt < SHT; ++tt) {
              const float mx = group4_max(mxs[ri][tt]);
              if (g == 0) sh.smax[k & 1][16 * (ht0 + tt) + n][rt0 + ri] = mx;
            }
          if (lane == 0) sh.flag[k & 1] = 1;
        }
      }
      wait_for_step(k + 1);  // this wave's rows of step k+1 have landed
      lds_barrier();  // step k's P, flag and maxima, step k+1's rows visible
      if (k < nsteps) {
        if (sh.flag[k & 1]) {  // rare: the reference rises; every wave takes this branch
          float alpha[SHT];
          raise_reference<SHT, NH>(sh.smax[k & 1], n, ht0, sref, alpha);
#pragma unroll
          for (int tt = 0; tt < SHT; ++tt) {
            const float mr = sref[tt] == -INFINITY ? 0.0f : sref[tt];
#pragma unroll
            for (int ri = 0; ri < SRT; ++ri) {
              lsum[ri][tt] *= alpha[tt];
              float p[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sv[ri][tt][i] - mr);
              psum[ri][tt] = (p[0] + p[1]) + (p[2] + p[3]);
              write_p(sh.ptile[k & 1] + (16 * (ht0 + tt) + n) * kPStride, rt0 + ri, g, p);
            }
          }
          lds_barrier();  // rewritten P visible; every wave has read the flag and the maxima
          // the maxima buffer of this parity starts over at -inf for its next use (step k+2)
          if (tid == 0) sh.flag[k & 1] = 0;
#pragma unroll
          for (int ri = 0; ri < SRT; ++ri)
#pragma unroll
            for (int tt = 0; tt < SHT; ++tt)
              if (g == 0) sh.smax[k & 1][16 * (ht0 + tt) + n][rt0 + ri] = -INFINITY;
        }
#pragma unroll
        for (int ri = 0; ri < SRT; ++ri)
#pragma unroll
          for (int tt = 0; tt < SHT; ++tt) lsum[ri][tt] += psum[ri][tt];
      }
    }
    // softmax sums per head over this wave's rows
#pragma unroll
    for (int ri = 0; ri < SRT; ++ri)
#pragma unroll
      for (int tt = 0; tt < SHT; ++tt) {
        const float l = group4_sum(lsum[ri][tt]);
        if (g == 0) sh.wsum[16 * (ht0 + tt) + n][rt0 + ri] = l;
      }
    wait_vmem();
    MLA_STAMP(5);
    __syncthreads();  // sums visible (matches the accumulate waves' barrier below)
  } else {
  // ================= accumulate waves: O^T += V^T P^T for step k-1, columns 128cq..128cq+127
  {
    // The query tile converted to FP16 in place, each head scaled by its power-of-two shift (from the
    // largest magnitude of its 576 values), here while the score waves issue their first gathers: the 256
    // lanes of the four accumulate waves split the heads, 256 / NH lanes per head, each lane taking every
    // (256/NH)-th 16-byte word of the head's 72 (it reads, then rewrites, only its own words).
    constexpr int LPH = 256 / NH;                          // lanes per head: 4, 8 or 16
    constexpr int CPL = (kQK / 8 + LPH - 1) / LPH;         // words per lane: 18, 9, or 5 (the last partial)
    const int la = (w - 4) * 64 + lane;
    const int hq = la / LPH, part = la % LPH;
    uint8_t* qh = qstage + 2 * hq * kQK;
    u32x4 qc[CPL];
    uint32_t mq = 0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = part + LPH * i;
      if (c < kQK / 8) {
        qc[i] = *reinterpret_cast<const u32x4*>(qh + 16 * c);
        const uint32_t m = bf16x8_max_mag(qc[i]);
        mq = mq > m ? mq : m;
      }
    }
#pragma unroll
    for (int d = 1; d < LPH; d <<= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)mq, d, 64);
      mq = mq > o ? mq : o;
    }
    const int kq = q_shift(mq);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = part + LPH * i;
      if (c < kQK / 8)
        *reinterpret_cast<f16x8*>(qh + 16 * c) =
            as_f16x8(bf16x2_pow2_to_f16x2(qc[i][0], kq), bf16x2_pow2_to_f16x2(qc[i][1], kq),
                     bf16x2_pow2_to_f16x2(qc[i][2], kq), bf16x2_pow2_to_f16x2(qc[i][3], kq));
    }
    if (part == 0) sh.qshift[hq] = kq;
  }
  lds_barrier();  // the FP16 query tile and the shifts are in LDS (matches the score waves' barrier)
  lds_barrier();  // step 0 visible; the score waves hold their query fragments
  const int cq = r4;
  f32x4 o[HT][8];  // O^T tile c: O[head 16t+n][column 128cq+32g+8i+c] = o[t][c][i]
#pragma unroll
  for (int tt = 0; tt < HT; ++tt)
#pragma unroll
    for (int c = 0; c < 8; ++c) o[tt][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // V reads: lane (g, m=n) reads columns 128cq+8m..+7 of rows 32kk+8g+2p+e (p < 4, e < 2) of a step
  const int vcol = FMT == 0 ? 64 * cq + 4 * n : 128 * cq + 8 * n;
  const int vsc = 256 + 8 * cq + 4 * (n >> 3);  // dword holding the block scale of those columns
  const uint32_t vsel = (uint32_t)((n >> 1) & 3) | ((uint32_t)(4 + ((n >> 1) & 3)) << 8);

  for (int k = 0; k <= nsteps; ++k) {
    if (k >= 1) {
      const uint8_t* slot = slot_ptr(k - 1);
      const uint8_t* pt = sh.ptile[(k - 1) & 1];
      // every LDS read of the step first (P of both contraction halves, V words of the 16 rows this
      // lane feeds), then the conversions and products
      f16x8 pb[2][HT];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int tt = 0; tt < HT; ++tt)
          pb[kk][tt] = *reinterpret_cast<const f16x8*>(pt + (16 * tt + n) * kPStride + 2 * (32 * kk + 8 * g));
      // rows pv_row(kk, g, 2p) and the next one feed contraction elements 8g + 2p, 8g + 2p + 1
      if constexpr (FMT == 0) {
        uint32_t da[2][4], db[2][4], sa[2][4], sb[2][4];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint8_t* ra = slot + pv_row(kk, g, 2 * p) * RS;
            da[kk][p] = *reinterpret_cast<const uint32_t*>(ra + vcol);
            sa[kk][p] = *reinterpret_cast<const uint32_t*>(ra + vsc);
            db[kk][p] = *reinterpret_cast<const uint32_t*>(ra + RS + vcol);
            sb[kk][p] = *reinterpret_cast<const uint32_t*>(ra + RS + vsc);
          }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          uint32_t ev[4][2];
          f16x2 sp[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            sp[p] = e4m3x2_to_f16<false>(__builtin_amdgcn_perm(sb[kk][p], sa[kk][p], vsel));
            ev[p][0] = nib_pair<0>(da[kk][p], db[kk][p]);
            ev[p][1] = nib_pair<1>(da[kk][p], db[kk][p]);
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
            for (int tt = 0; tt < HT; ++tt) o[tt][c] = mfma16x16x32(A, pb[kk][tt], o[tt][c]);
          }
        }
      } else {
        // FP8: byte interleave (row a, row b) per column with v_perm, then exact FP8 -> FP16 pairs
        u32x2 da[2][4], db[2][4];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint8_t* ra = slot + pv_row(kk, g, 2 * p) * RS;
            da[kk][p] = *reinterpret_cast<const u32x2*>(ra + vcol);
            db[kk][p] = *reinterpret_cast<const u32x2*>(ra + RS + vcol);
          }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          uint32_t x[4][4];  // x[p][q]: columns 2q, 2q+1 of rows (a, b) as bytes a, b, a', b'
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            x[p][0] = __builtin_amdgcn_perm(db[kk][p][0], da[kk][p][0], 0x05010400u);
            x[p][1] = __builtin_amdgcn_perm(db[kk][p][0], da[kk][p][0], 0x07030602u);
            x[p][2] = __builtin_amdgcn_perm(db[kk][p][1], da[kk][p][1], 0x05010400u);
            x[p][3] = __builtin_amdgcn_perm(db[kk][p][1], da[kk][p][1], 0x07030602u);
          }
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            f16x2 v[4];
#pragma unroll
            for (int p = 0; p < 4; ++p)
              v[p] = (c & 1) ? e4m3x2_to_f16<true>(x[p][c >> 1]) : e4m3x2_to_f16<false>(x[p][c >> 1]);
            const f16x8 A = as_f16x8(v[0], v[1], v[2], v[3]);
#pragma unroll
            for (int tt = 0; tt < HT; ++tt) o[tt][c] = mfma16x16x32(A, pb[kk][tt], o[tt][c]);
          }
        }
      }
    }
    lds_barrier();  // matches the score waves' barrier of step k
    if (k < nsteps && sh.flag[k & 1]) {
      float alpha[HT];
      raise_reference<HT, NH>(sh.smax[k & 1], n, 0, ref, alpha);
#pragma unroll
      for (int tt = 0; tt < HT; ++tt)
#pragma unroll
        for (int c = 0; c < 8; ++c) o[tt][c] *= alpha[tt];
      lds_barrier();  // matches the score waves' second barrier
    }
  }
  wait_vmem();
  __syncthreads();  // the score waves' sums are visible

  // ---- epilogue: normalize; unsplit -> bf16 output directly, split -> the workgroup's result tile in LDS
  // (the ring is free: every gather has landed and every wave is past its last read)
#pragma unroll
  for (int tt = 0; tt < HT; ++tt) {
    const int h = 16 * tt + n;
    const float Lh = (sh.wsum[h][0] + sh.wsum[h][1]) + (sh.wsum[h][2] + sh.wsum[h][3]);
    const float inv = Lh > 0.0f ? 1.0f / Lh : 0.0f;
    const int64_t hrow = (int64_t)qtok * a.H + h0 + h;
    if (cq == 0 && g == 0) {
      const float lse = Lh > 0.0f ? (ref[tt] + __log2f(Lh)) * 0.69314718055994531f : -INFINITY;
      if (S == 1) {
        if (a.lse) a.lse[hrow] = lse;
      } else {
        sh.tile_lse[h] = lse;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = 128 * cq + 32 * g + 8 * i;
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = o[tt][c][i] * inv;
      if (S == 1) {
        *reinterpret_cast<u32x4*>(a.out + hrow * kLatent + col) =
            u32x4{pack_bf16_rne(v[0], v[1]), pack_bf16_rne(v[2], v[3]), pack_bf16_rne(v[4], v[5]),
                  pack_bf16_rne(v[6], v[7])};
      } else {
        f32x4* dst = reinterpret_cast<f32x4*>(tile + h * kTileStride + col);
        dst[0] = f32x4{v[0], v[1], v[2], v[3]};
        dst[1] = f32x4{v[4], v[5], v[6], v[7]};
      }
    }
  }
  }  // accumulate waves

  // ---- split merge (the pages merge a cluster's partial results through distributed shared memory in
  // the same launch; here the last workgroup of a query token to finish merges them): lse = M + ln
  // sum_s e^{lse_s - M}, out = sum_s e^{lse_s - lse} out_s; a split with no rows has lse_s = -inf and no
  // weight; all splits empty -> out = 0, lse = -inf.  The arrival counter returns to zero.
  // Each workgroup stores its normalized result (FP16, far below the bf16 output's rounding) and lse
  // with agent-coherent (L2-bypassing) relaxed stores, waits until they are complete (vmcnt 0) and only
  // then moves the arrival counter; the workgroup that moves it to S merges, reading with coherent
  // loads.  No device-scope fence (which writes back and invalidates the whole L2) is needed.  Thread
  // tid owns head h = tid / TPH and the column quads 4*(tid % TPH) + 4*TPH*j, so each load or store
  // instruction covers whole cache lines.
  if (S > 1) {
    constexpr int TPH = kThreads / NH;        // threads per head: 16 or 32
    constexpr int NQ = kLatent / (4 * TPH);   // column quads per thread: 8 or 4
    const int h = tid / TPH;
    const int c4 = 4 * (tid % TPH);
    const int64_t hrow = (int64_t)qtok * a.H + h0 + h;
    const float* own = tile + h * kTileStride + c4;
    __syncthreads();  // the result tile and its lse are complete
    MLA_STAMP(6);
    {
      uint64_t* dst = reinterpret_cast<uint64_t*>(a.part_o + (hrow * S + s) * kLatent + c4);
#pragma unroll
      for (int jj = 0; jj < NQ; ++jj)
        store_coherent_h4(dst + TPH * jj, *reinterpret_cast<const f32x4*>(own + 4 * TPH * jj));
      if (tid % TPH == 0) __hip_atomic_store(a.part_lse + hrow * S + s, sh.tile_lse[h], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's split results are complete
    __syncthreads();
    int* counter = a.counters + ((int64_t)qtok * HG + hg);
    if (tid == 0) sh.last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
    __syncthreads();
    MLA_STAMP(7);
    if (sh.last) {
      // running merge over the splits in their order, four per round with every load of a round (results
      // and lse) issued together; this workgroup's own split comes from LDS, rounded to FP16 as the
      // stored ones are, so the merged bits do not depend on which split's workgroup merges
      float M = -INFINITY;
      float Z = 0.0f;
      f32x4 acc[NQ];
#pragma unroll
      for (int jj = 0; jj < NQ; ++jj) acc[jj] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      const float* pl = a.part_lse + hrow * S;
      for (int k0 = 0; k0 < S; k0 += 4) {
        float lk[4];
        uint64_t raw[4][NQ];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k = k0 + u;
          lk[u] = -INFINITY;
          if (k >= S) continue;
          if (k == s) {
            lk[u] = sh.tile_lse[h];
#pragma unroll
            for (int jj = 0; jj < NQ; ++jj) raw[u][jj] = pack_h4(*reinterpret_cast<const f32x4*>(own + 4 * TPH * jj));
            continue;
          }
          lk[u] = load_coherent(pl + k);
          const uint64_t* src = reinterpret_cast<const uint64_t*>(a.part_o + (hrow * S + k) * kLatent + c4);
#pragma unroll
          for (int jj = 0; jj < NQ; ++jj)
            raw[u][jj] = __hip_atomic_load(const_cast<uint64_t*>(src + TPH * jj), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        }
        const float mnew = fmaxf(fmaxf(M, fmaxf(lk[0], lk[1])), fmaxf(lk[2], lk[3]));
        if (mnew == -INFINITY) continue;
        const float r = __expf(M - mnew);  // 0 while M = -inf
        Z *= r;
#pragma unroll
        for (int jj = 0; jj < NQ; ++jj) acc[jj] *= r;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (lk[u] == -INFINITY) continue;
          const float wk = __expf(lk[u] - mnew);
          Z += wk;
#pragma unroll
          for (int jj = 0; jj < NQ; ++jj) acc[jj] += wk * h4_to_f32x4(raw[u][jj]);
        }
        M = mnew;
      }
      const float inv = Z > 0.0f ? 1.0f / Z : 0.0f;
      u32x2* dst = reinterpret_cast<u32x2*>(a.out + hrow * kLatent + c4);
#pragma unroll
      for (int jj = 0; jj < NQ; ++jj) {
        const f32x4 v = acc[jj] * inv;
        dst[TPH * jj] = u32x2{pack_bf16_rne(v[0], v[1]), pack_bf16_rne(v[2], v[3])};
      }
      if (tid % TPH == 0 && a.lse) a.lse[hrow] = Z > 0.0f ? M + __logf(Z) : -INFINITY;
      if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
#ifdef MLA_TIMELINE
  MLA_STAMP(8);
  stamp[11] = (uint64_t)gridDim.x;
  stamp[12] = (uint64_t)__builtin_amdgcn_s_getreg(20 | (3 << 11));  // HW_REG_XCC_ID, bits 3:0
  stamp[13] = S == 1 ? 1u : (uint64_t)sh.last;
  stamp[14] = (uint64_t)j;
  stamp[15] = (uint64_t)nsteps;
  if (tid == 0 && blockIdx.x < (unsigned)kTimelineWGs) {
#pragma unroll
    for (int i = 0; i < kTimelineSlots; ++i) g_timeline[blockIdx.x * kTimelineSlots + i] = stamp[i];
  }
#endif
}

template <int HT, int FMT, bool DENSE>
static void launch_one(const DecodeArgs& a, hipStream_t stream) {
  const int HG = a.H / (16 * HT);
  const unsigned grid = (unsigned)(a.B * a.T * HG * a.splits);
  hipLaunchKernelGGL((decode_kernel<HT, FMT, DENSE>), dim3(grid), dim3(kThreads), 0, stream, a);
}

#ifdef MLA_TIMELINE
// The instrumented library's stamps of the last decode launch, workgroups [0, n) (n <= 4096), 16 per
// workgroup; returns 0 on success.
extern "C" int mla_debug_timeline(uint64_t* host, int64_t n) {
  if (!host || n < 1 || n > kTimelineWGs) return 1;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_timeline), (size_t)n * kTimelineSlots * 8, 0,
                             hipMemcpyDeviceToHost) == hipSuccess ? 0 : 1;
}
#endif

hipError_t launch_decode(int fmt, const DecodeArgs& a, hipStream_t stream) {
  const bool dense = a.indices == nullptr;
  if (fmt == 0) {
    if (dense) return hipErrorInvalidValue;
    // 64 or 128 heads, unsplit, with at least one workgroup per compute unit at 64 heads per workgroup:
    // 64-head groups (each K and V fragment dequantized once for twice the heads); otherwise 32
    if (a.H >= 64 && a.splits == 1 && (int64_t)a.B * a.T * (a.H / 64) >= 256) launch_one<4, 0, false>(a, stream);
    else if (a.H == 16) launch_one<1, 0, false>(a, stream);
    else launch_one<2, 0, false>(a, stream);
  } else if (dense) {
    if (a.H == 16) launch_one<1, 1, true>(a, stream);
    else launch_one<2, 1, true>(a, stream);
  } else {
    if (a.H == 16) launch_one<1, 1, false>(a, stream);
    else launch_one<2, 1, false>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace mla
