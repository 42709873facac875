// The sparse indexer's selection step ("Prime Inference" launch post: each query token attends to at most
// 2,048 cached positions picked by the indexer, unused list entries -1; the analysis page, section
// "Decode: TP4, and the copies it keeps": index_topk 2048):
// for each row of fp32 logits, the positions of the k largest values, ties at the k-th value going to the
// lower positions, listed in ascending position order and padded with -1.
//
// An exact radix select on order-preserving 32-bit keys, in three launches per call (the launch
// boundaries publish each step's workspace writes to every XCD's L2; a fence per workgroup instead
// would write back and invalidate an L2 for each of them):
//   * histogram: one 512-thread workgroup per 8192-position chunk of a row counts the top 11 key bits
//     into an LDS histogram and adds its non-zero bins to the row's histogram in the workspace;
//   * collect: the same workgroups find, from the row's histogram, the bin b1 holding the k-th largest
//     key.  When the elements in bins >= b1 fit the row's candidate buffer (the usual case: fewer than
//     k elements lie above b1, plus one bin), each workgroup copies its chunk's candidates (key,
//     position) there in position order, at a segment taken from the row's cursor, and records the
//     segment;
//   * finish: one workgroup per row resolves the remaining 21 key bits over the candidates alone (two
//     more LDS histograms), then walks the segments in chunk order and writes every position whose key
//     is above the threshold, plus the first ties by position, a block scan giving each its output
//     slot.  When the candidates do not fit (very many equal or near-equal logits), it runs the same
//     steps over the whole row instead.  It also returns the row's histogram and cursor to zero for the
//     next call.
#include "mla_internal.h"

namespace mla {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkTile = 4 * kTkThreads;             // positions per load pass of a workgroup
constexpr int kTkChunk = 4 * kTkTile;               // positions per workgroup
static_assert(kTkChunk == kTopkChunk, "chunk size shared with the workspace layout");
constexpr int kTkBins1 = 1 << kTopkBits1;           // key bits 31..21
constexpr int kTkBins2 = 2048;                      // key bits 20..10
constexpr int kTkBins3 = 1024;                      // key bits 9..0
// The candidate path keeps a table of one entry per chunk in LDS: rows of up to this many chunks
// (8.4M positions) use it, longer ones the whole-row path.
constexpr int kTkMaxChunks = 1024;

// Larger float -> larger unsigned key; -0 is mapped to +0 so that the two rank as equal.
__device__ inline uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline int row_length(const TopkArgs& a, int64_t row) {
  const int m = a.lengths[row];
  return m < 0 ? 0 : (m > a.ld ? (int)a.ld : m);
}

__device__ inline int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// Exclusive prefix of v over the workgroup in thread order; `total` receives the sum.  Two barriers.
__device__ inline int block_excl_scan(int v, int* sw, int& total) {
  const int inc = wave_incl_scan(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) sw[w] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kTkWaves; ++i) {
    const int s = sw[i];
    before += i < w ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

// Descending search of an LDS histogram of NB bins: the bin holding the need-th largest element
// (1 <= need <= the histogram's total) goes to res[0], the count in higher bins to res[1].  The
// histogram must be complete (barrier) on entry, and res not read since the last barrier; ends with a
// barrier.
template <int NB>
__device__ inline void find_bin(const int* h, int need, int* sw, int* res) {
  constexpr int per = NB / kTkThreads;
  const int tid = threadIdx.x;
  int s = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) s += h[NB - 1 - (tid * per + i)];
  if (tid == 0) res[0] = res[1] = 0;  // stays in range should the counts be inconsistent
  int tot;
  const int before = block_excl_scan(s, sw, tot);
  if (before < need && need <= before + s) {
    int acc = before;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int b = NB - 1 - (tid * per + i);
      const int c = h[b];
      if (acc < need && acc + c >= need) {
        res[0] = b;
        res[1] = acc;
      }
      acc += c;
    }
  }
  __syncthreads();
}

// Loads the row's positions base + 4*tid .. +3 (those below m) as keys; the rest get key 0, valid 0.
__device__ inline void load_keys4(const float* src, int base, int m, uint32_t key[4], int& valid) {
  const int idx = base + 4 * threadIdx.x;
  valid = 0;
  key[0] = key[1] = key[2] = key[3] = 0u;
  if (idx < m) {
    // idx is a multiple of 4 below m <= ld, and ld is a multiple of 4: the whole float4 is in the row
    const float4 v = *reinterpret_cast<const float4*>(src + idx);
    key[0] = order_key(v.x);
    key[1] = order_key(v.y);
    key[2] = order_key(v.z);
    key[3] = order_key(v.w);
    valid = m - idx < 4 ? m - idx : 4;
  }
}

__global__ __launch_bounds__(kTkThreads) void topk_hist_kernel(TopkArgs a) {
  __shared__ int h[kTkBins1];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x / a.chunks;
  const int chunk = blockIdx.x % a.chunks;
  const int m = row_length(a, row);
  const int start = chunk * kTkChunk;
  if (m <= a.k || start >= m) return;
  const float* src = a.logits + row * a.ld;
  uint32_t key[4][4];
  int valid[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) load_keys4(src, start + j * kTkTile, m, key[j], valid[j]);
  for (int i = tid; i < kTkBins1; i += kTkThreads) h[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < valid[j]) atomicAdd(&h[key[j][e] >> (32 - kTopkBits1)], 1);
  __syncthreads();
  int* gh = a.hist + row * kTkBins1;
  for (int i = tid; i < kTkBins1; i += kTkThreads) {
    const int c = h[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// The level-1 bin b1 of the row's k-th largest key (res[0]) and the count above it (res[1]), from the
// row's histogram in the workspace; ends with a barrier, h holding the histogram.
__device__ inline void level1(const int* gh, int k, int* h, int* sw, int* res) {
  for (int i = threadIdx.x; i < kTkBins1; i += kTkThreads) h[i] = gh[i];
  __syncthreads();
  find_bin<kTkBins1>(h, k, sw, res);
}

__global__ __launch_bounds__(kTkThreads) void topk_collect_kernel(TopkArgs a) {
  __shared__ int h[kTkBins1];
  __shared__ int sw[4 * kTkWaves];
  __shared__ int res[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int64_t row = blockIdx.x / a.chunks;
  const int chunk = blockIdx.x % a.chunks;
  const int m = row_length(a, row);
  const int start = chunk * kTkChunk;
  if (m <= a.k || start >= m) return;
  const float* src = a.logits + row * a.ld;
  int* ctrl = a.ctrl + row * kTopkCtrlInts;
  uint2* cand = a.cand + row * kTopkCap;

  // this chunk's keys, issued before the histogram search so that the loads overlap it
  uint32_t key[4][4];
  int valid[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) load_keys4(src, start + j * kTkTile, m, key[j], valid[j]);

  level1(a.hist + row * kTkBins1, a.k, h, sw, res);
  const uint32_t b1 = (uint32_t)res[0];
  const int n_cand = res[1] + h[b1];
  if (chunk == 0 && tid == 0) {  // for the finishing workgroup
    ctrl[1] = (int)b1;
    ctrl[2] = res[1];
    ctrl[3] = n_cand;
  }
  const int nchunks = (m + kTkChunk - 1) / kTkChunk;
  if (n_cand > kTopkCap || nchunks > kTkMaxChunks) return;  // the finisher scans the whole row

  // candidates: keys whose top bits are >= b1, in position order (tile j, then thread, then element)
  int cnt[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    cnt[j] = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) cnt[j] += (e < valid[j] && (key[j][e] >> (32 - kTopkBits1)) >= b1) ? 1 : 0;
  }
  int excl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int inc = wave_incl_scan(cnt[j]);
    excl[j] = inc - cnt[j];
    if (lane == 63) sw[j * kTkWaves + w] = inc;
  }
  __syncthreads();
  // slots in (tile, wave, lane) order: tiles before j, then waves before w within tile j
  int total = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < kTkWaves; ++i) {
      const int s = sw[j * kTkWaves + i];
      excl[j] += (i < w) ? s : 0;
#pragma unroll
      for (int jj = j + 1; jj < 4; ++jj) excl[jj] += s;
      total += s;
    }
  if (tid == 0) {
    const int base = total ? atomicAdd(&ctrl[0], total) : 0;
    a.seg[row * a.chunks + chunk] = int2{base, total};
    res[2] = base;
  }
  __syncthreads();
  const int base = res[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int o = base + excl[j];
    const int pos0 = start + j * kTkTile + 4 * tid;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < valid[j] && (key[j][e] >> (32 - kTopkBits1)) >= b1) {
        // o stays below kTopkCap whenever the workspace started zeroed
        if ((unsigned)o < (unsigned)kTopkCap) cand[o] = uint2{key[j][e], (uint32_t)(pos0 + e)};
        ++o;
      }
  }
}

// One workgroup per row: the candidates are gathered into LDS in position order (one round of
// independent loads, each placed through its chunk's offset), key bits 20..10 and then 9..0 are resolved
// over them (or over the whole row), then the list is written; finally the row's histogram and counters
// go back to zero.
__global__ __launch_bounds__(kTkThreads) void topk_finish_kernel(TopkArgs a) {
  __shared__ int h[kTkBins2];
  __shared__ uint32_t ckey[kTopkCap];  // candidates in position order
  __shared__ int cpos[kTopkCap];
  __shared__ int cdelta[kTkMaxChunks];  // position-order slot minus cursor slot, per chunk
  __shared__ int sw[4 * kTkWaves];
  __shared__ int res[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int m = row_length(a, row);
  const int k = a.k;
  int32_t* out = a.out + row * k;
  if (m <= k) {  // every position is chosen
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < m ? i : -1;
    return;
  }
  const int nchunks = (m + kTkChunk - 1) / kTkChunk;
  const float* src = a.logits + row * a.ld;
  int* gh = a.hist + row * kTkBins1;
  int* ctrl = a.ctrl + row * kTopkCtrlInts;
  const uint2* cand = a.cand + row * kTopkCap;
  const int2* seg = a.seg + row * a.chunks;

  const uint32_t b1 = (uint32_t)ctrl[1] & (kTkBins1 - 1);
  const int above1 = ctrl[2];
  const int n_cand = ctrl[3];
  const bool fast = n_cand <= kTopkCap && nchunks <= kTkMaxChunks;  // the collecting workgroups' test

  if (fast) {
    // position-order start of each chunk's segment: an exclusive scan of the counts in chunk order
    constexpr int per = kTkMaxChunks / kTkThreads;
    int2 sg[per];
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int c = per * tid + i;
      sg[i] = c < nchunks ? seg[c] : int2{0, 0};
      cnt += sg[i].y;
    }
    int tot;
    int p = block_excl_scan(cnt, sw, tot);
#pragma unroll
    for (int i = 0; i < per; ++i) {
      cdelta[per * tid + i] = p - sg[i].x;
      p += sg[i].y;
    }
    __syncthreads();
    constexpr int kLoads = kTopkCap / kTkThreads;
    uint2 cd[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int g = tid + i * kTkThreads;
      cd[i] = g < n_cand ? cand[g] : uint2{0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int g = tid + i * kTkThreads;
      if (g < n_cand) {
        const int dst = g + cdelta[(cd[i].y / kTkChunk) % kTkMaxChunks];
        if ((unsigned)dst < (unsigned)kTopkCap) {  // always, with a zeroed workspace
          ckey[dst] = cd[i].x;
          cpos[dst] = (int)cd[i].y;
        }
      }
    }
    __syncthreads();
  }

  auto histogram = [&](uint32_t prefix, int pshift, int shift, uint32_t dmask) {
    for (int i = tid; i < kTkBins2; i += kTkThreads) h[i] = 0;
    __syncthreads();
    if (fast) {
      for (int i = tid; i < n_cand; i += kTkThreads) {
        const uint32_t kk = ckey[i];
        if ((kk >> pshift) == prefix) atomicAdd(&h[(kk >> shift) & dmask], 1);
      }
    } else {
      for (int b = 0; b < m; b += kTkTile) {
        uint32_t kk[4];
        int v;
        load_keys4(src, b, m, kk, v);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < v && (kk[e] >> pshift) == prefix) atomicAdd(&h[(kk[e] >> shift) & dmask], 1);
      }
    }
    __syncthreads();
  };
  int need = k - above1;  // elements still to take from bin b1, >= 1
  histogram(b1, 21, 10, kTkBins2 - 1);
  find_bin<kTkBins2>(h, need, sw, res);
  const uint32_t b2 = (uint32_t)res[0];
  need -= res[1];
  __syncthreads();
  histogram((b1 << 11) | b2, 10, 0, kTkBins3 - 1);
  find_bin<kTkBins3>(h, need, sw, res);
  const uint32_t thr = (b1 << 21) | (b2 << 10) | (uint32_t)res[0];
  const int need_ties = need - res[1];  // keys equal to thr to take, lowest positions first, >= 1
  __syncthreads();

  // ---- output in position order: a key above thr goes to slot (keys above thr before it) +
  // min(ties before it, need_ties); a tie is taken while fewer than need_ties ties precede it
  int run_gt = 0, run_eq = 0;
  auto emit = [&](const uint32_t kk[4], const int pp[4], int v) {
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gt += (e < v && kk[e] > thr) ? 1 : 0;
      eq += (e < v && kk[e] == thr) ? 1 : 0;
    }
    int tot;
    const int ex = block_excl_scan((eq << 16) | gt, sw, tot);  // a tile holds at most 2048 elements
    int g = run_gt + (ex & 0xFFFF), q = run_eq + (ex >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (e >= v) continue;
      // the slots are below k whenever the workspace started zeroed; the checks keep a misused one in bounds
      if (kk[e] > thr) {
        const int slot = g + (q < need_ties ? q : need_ties);
        if (slot < k) out[slot] = pp[e];
        ++g;
      } else if (kk[e] == thr) {
        if (q < need_ties && g + q < k) out[g + q] = pp[e];
        ++q;
      }
    }
    run_gt += tot & 0xFFFF;
    run_eq += tot >> 16;
  };
  if (fast) {
    for (int t0 = 0; t0 < n_cand; t0 += kTkTile) {
      uint32_t kk[4];
      int pp[4];
      const int idx = t0 + 4 * tid;
      const int v = idx < n_cand ? (n_cand - idx < 4 ? n_cand - idx : 4) : 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kk[e] = e < v ? ckey[idx + e] : 0u;
        pp[e] = e < v ? cpos[idx + e] : 0;
      }
      emit(kk, pp, v);
    }
  } else {
    for (int b = 0; b < m; b += kTkTile) {
      uint32_t kk[4];
      int v;
      load_keys4(src, b, m, kk, v);
      const int pp[4] = {b + 4 * tid, b + 4 * tid + 1, b + 4 * tid + 2, b + 4 * tid + 3};
      emit(kk, pp, v);
    }
  }

  // ---- leave the row's histogram and counters at zero for the next call
  for (int i = tid; i < kTkBins1; i += kTkThreads) gh[i] = 0;
  if (tid < kTopkCtrlInts) ctrl[tid] = 0;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)(a.n * a.chunks);
  hipLaunchKernelGGL(topk_hist_kernel, dim3(grid), dim3(kTkThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_collect_kernel, dim3(grid), dim3(kTkThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)a.n), dim3(kTkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
