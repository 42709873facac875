// The sparse indexer's selection step ("Prime Inference" launch post: each query token attends to at most
// 2,048 cached positions picked by the indexer, unused list entries -1; the analysis page, section
// "Decode: TP4, and the copies it keeps": index_topk 2048):
// for each row of fp32 logits, the positions of the k largest values, ties at the k-th value going to the
// lower positions, listed in ascending position order and padded with -1.
//
// An exact radix select on order-preserving 32-bit keys, in three launches per call:
//   * histogram: one 512-thread workgroup per 8192-position chunk of a row counts the top 12 key bits
//     into an LDS histogram and adds its non-zero bins to the row's histogram in the workspace; the
//     row's last workgroup to finish finds the bin b1 holding the row's k-th largest key;
//   * collect: when the elements in bins >= b1 fit the row's candidate buffer (the usual case: fewer
//     than k elements lie above b1, plus one bin), each chunk's workgroup copies its candidates (key,
//     position) there in position order, at a segment taken from the row's cursor, and records the
//     segment;
//   * finish: one workgroup per row gathers the candidates into LDS in position order (one round of
//     independent loads, each placed through its chunk's offset), resolves the remaining 20 key bits
//     over them (two more LDS histograms), and writes every position whose key is above the threshold,
//     plus the first ties by position, a block scan giving each its output slot.  When the candidates
//     do not fit (very many equal or near-equal logits), it runs the same steps over the whole row.  It
//     also returns the row's histogram and counters to zero for the next call.
#include "mla_index_internal.h"

namespace mla {

constexpr int kTkThreads = kTopkThreads;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkTile = 4 * kTkThreads;             // positions per load pass of a workgroup
constexpr int kTkChunk = kTopkChunk;                // positions per workgroup
constexpr int kTkTPC = kTkChunk / kTkTile;          // tiles per chunk
static_assert(kTkChunk % kTkTile == 0, "whole tiles per chunk");
constexpr int kTkBins1 = 1 << kTopkBits1;           // key bits 31..20
constexpr int kTkBins2 = 1024;                      // key bits 19..10
constexpr int kTkBins3 = 1024;                      // key bits 9..0
static_assert(kTopkBits1 == 12, "the lower levels resolve 10 + 10 bits");
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

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS traffic): shifts by 1, 2, 4
// and 8 lanes within each row of 16, then row 0's total into row 1 and row 2's into row 3 (row_bcast:15),
// then the total of rows 0-1 into rows 2 and 3 (row_bcast:31).  Lanes without a source add the 0 passed
// as the old value.
__device__ inline int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
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

// The bin of the row's k-th largest key (1 <= k < the row's length), the count in higher bins and the
// bin's own count, found by wave 0 (threadIdx.x < 64) in a complete LDS copy of the row's histogram:
// lane l sums bins 64l..64l+63, a DPP prefix over the lanes locates the lane range holding the k-th
// largest, and a second prefix over that range's 64 bins, one per lane from the top, locates the bin.
// The lane that finds it writes res[0..2].
__device__ inline void level1_search(const int* hist, int k, int* res) {
  const int lane = threadIdx.x & 63;
  constexpr int kPerLane = kTkBins1 / 64;
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kPerLane / 4; ++i) {
    const int4 q = reinterpret_cast<const int4*>(hist)[lane * (kPerLane / 4) + i];
    sum += q.x + q.y + q.z + q.w;
  }
  int incl = wave_incl_scan(sum);
  const int total = __shfl(incl, 63, 64);
  int above = total - incl;  // keys in bins above lane l's range
  const uint64_t hit = __ballot(above < k && k <= above + sum);
  const int L = (int)__builtin_ctzll(hit);
  above = __shfl(above, L, 64);
  const int b = L * kPerLane + (kPerLane - 1 - lane);  // lane i takes the range's i-th bin from the top
  const int c = hist[b];
  incl = wave_incl_scan(c);
  if (above + incl - c < k && k <= above + incl) {
    res[0] = b;
    res[1] = above + incl - c;
    res[2] = c;
  }
}

__global__ __launch_bounds__(kTkThreads) void topk_hist_kernel(TopkArgs a) {
  __shared__ __align__(16) int h[kTkBins1];
  __shared__ int res[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x / a.chunks;
  const int chunk = blockIdx.x % a.chunks;
  const int m = row_length(a, row);
  const int start = chunk * kTkChunk;
  if (m <= a.k || start >= m) return;
  const float* src = a.logits + row * a.ld;
  uint32_t key[kTkTPC][4];
  int valid[kTkTPC];
#pragma unroll
  for (int j = 0; j < kTkTPC; ++j) load_keys4(src, start + j * kTkTile, m, key[j], valid[j]);
  for (int i = tid; i < kTkBins1; i += kTkThreads) h[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kTkTPC; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < valid[j]) atomicAdd(&h[key[j][e] >> (32 - kTopkBits1)], 1);
  __syncthreads();
  int* gh = a.hist + row * kTkBins1;
  for (int i = tid; i < kTkBins1; i += kTkThreads) {
    const int c = h[i];
    if (c) __hip_atomic_fetch_add(&gh[i], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // The row's last workgroup to finish finds the bin of the k-th largest key once for the row.  Each
  // workgroup waits until its agent-scope adds are performed (vmcnt 0) before it moves the row's arrival
  // counter, and the last one reads the histogram with agent-coherent loads: no device-scope fence (an
  // L2 write-back and invalidate per workgroup) is needed.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int* ctrl = a.ctrl + row * kTopkCtrlInts;
  const int nchunks = (m + kTkChunk - 1) / kTkChunk;
  if (tid == 0) res[3] = __hip_atomic_fetch_add(&ctrl[4], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nchunks - 1;
  __syncthreads();
  if (!res[3]) return;
  for (int i = tid; i < kTkBins1; i += kTkThreads)
    h[i] = __hip_atomic_load(&gh[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (tid < 64) level1_search(h, a.k, res);
  __syncthreads();
  if (tid == 0) {  // read by the next two launches
    ctrl[1] = res[0];
    ctrl[2] = res[1];
    ctrl[3] = res[1] + res[2];
  }
}

__global__ __launch_bounds__(kTkThreads) void topk_collect_kernel(TopkArgs a) {
  __shared__ int sw[kTkTPC * kTkWaves];
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

  uint32_t key[kTkTPC][4];
  int valid[kTkTPC];
#pragma unroll
  for (int j = 0; j < kTkTPC; ++j) load_keys4(src, start + j * kTkTile, m, key[j], valid[j]);
  const uint32_t b1 = (uint32_t)ctrl[1] & (kTkBins1 - 1);  // the row's level-1 bin and candidate count
  const int n_cand = ctrl[3];
  const int nchunks = (m + kTkChunk - 1) / kTkChunk;
  if (n_cand > kTopkCap || nchunks > kTkMaxChunks) return;  // the finisher scans the whole row

  // candidates: keys whose top bits are >= b1, in position order (tile j, then thread, then element)
  int cnt[kTkTPC];
#pragma unroll
  for (int j = 0; j < kTkTPC; ++j) {
    cnt[j] = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) cnt[j] += (e < valid[j] && (key[j][e] >> (32 - kTopkBits1)) >= b1) ? 1 : 0;
  }
  int excl[kTkTPC];
#pragma unroll
  for (int j = 0; j < kTkTPC; ++j) {
    const int inc = wave_incl_scan(cnt[j]);
    excl[j] = inc - cnt[j];
    if (lane == 63) sw[j * kTkWaves + w] = inc;
  }
  __syncthreads();
  // slots in (tile, wave, lane) order: tiles before j, then waves before w within tile j
  int total = 0;
#pragma unroll
  for (int j = 0; j < kTkTPC; ++j)
#pragma unroll
    for (int i = 0; i < kTkWaves; ++i) {
      const int s = sw[j * kTkWaves + i];
      excl[j] += (i < w) ? s : 0;
#pragma unroll
      for (int jj = j + 1; jj < kTkTPC; ++jj) excl[jj] += s;
      total += s;
    }
  if (tid == 0) {
    const int base = total ? atomicAdd(&ctrl[0], total) : 0;
    a.seg[row * a.chunks + chunk] = int2{base, total};
    res[3] = base;
  }
  __syncthreads();
  const int base = res[3];
#pragma unroll
  for (int j = 0; j < kTkTPC; ++j) {
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

// Position-order slots for a group of up to kTkTPC tiles: flags[j] packs (ties << 16 | above) of this
// thread's elements of tile j; on return excl[j] holds the packed count of the group's elements before
// them (tile, then thread order) and the group's packed total is returned.  One barrier pair.
__device__ inline int group_scan(const int flags[kTkTPC], int excl[kTkTPC], int* sw) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < kTkTPC; ++j) {
    const int inc = wave_incl_scan(flags[j]);
    excl[j] = inc - flags[j];
    if (lane == 63) sw[j * kTkWaves + w] = inc;
  }
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int j = 0; j < kTkTPC; ++j)
#pragma unroll
    for (int i = 0; i < kTkWaves; ++i) {
      const int s = sw[j * kTkWaves + i];
      excl[j] += (i < w) ? s : 0;
#pragma unroll
      for (int jj = j + 1; jj < kTkTPC; ++jj) excl[jj] += s;
      total += s;
    }
  __syncthreads();
  return total;
}

// One workgroup per row: the candidates are gathered into LDS in position order, key bits 20..10 and
// then 9..0 are resolved over them (or over the whole row), then the list is written; finally the row's
// histogram and counters go back to zero.
__global__ __launch_bounds__(kTkThreads) void topk_finish_kernel(TopkArgs a) {
  __shared__ int h[kTkBins2];
  __shared__ __align__(16) uint32_t ckey[kTopkCap];  // candidates in position order
  __shared__ __align__(16) int cpos[kTopkCap];
  __shared__ int cdelta[kTkMaxChunks];  // position-order slot minus cursor slot, per chunk
  __shared__ int sw[kTkTPC * kTkWaves];
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

  // one round of independent loads: the counters, the segment table and every candidate slot (slots
  // past the count are read but not used)
  constexpr int per = kTkMaxChunks / kTkThreads;
  constexpr int kLoads = kTopkCap / kTkThreads;
  const uint32_t b1 = (uint32_t)ctrl[1] & (kTkBins1 - 1);
  const int above1 = ctrl[2];
  const int n_cand = ctrl[3];
  int2 sg[per];
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int c = per * tid + i;
    sg[i] = c < nchunks ? seg[c] : int2{0, 0};
  }
  uint2 cd[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) cd[i] = cand[tid + i * kTkThreads];
  const bool fast = n_cand <= kTopkCap && nchunks <= kTkMaxChunks;  // the collecting workgroups' test

  if (fast) {
    // position-order start of each chunk's segment: an exclusive scan of the counts in chunk order
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) cnt += sg[i].y;
    int tot;
    int p = block_excl_scan(cnt, sw, tot);
#pragma unroll
    for (int i = 0; i < per; ++i) {
      cdelta[per * tid + i] = p - sg[i].x;
      p += sg[i].y;
    }
    __syncthreads();
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

  // key bits below the top 12: a histogram of bits [shift, shift + 10) of the keys whose higher bits
  // equal `prefix`, over the candidates or over the whole row (a group of tiles in flight while the
  // previous one is counted)
  auto histogram = [&](uint32_t prefix, int pshift, int shift, uint32_t dmask) {
    for (int i = tid; i < kTkBins2; i += kTkThreads) h[i] = 0;
    __syncthreads();
    if (fast) {
#pragma unroll 4
      for (int i = tid; i < n_cand; i += kTkThreads) {
        const uint32_t kk = ckey[i];
        if ((kk >> pshift) == prefix) atomicAdd(&h[(kk >> shift) & dmask], 1);
      }
    } else {
      uint32_t kk[kTkTPC][4];
      int v[kTkTPC];
#pragma unroll
      for (int j = 0; j < kTkTPC; ++j) load_keys4(src, j * kTkTile, m, kk[j], v[j]);
      for (int b = 0; b < m; b += kTkChunk) {
        uint32_t nk[kTkTPC][4];
        int nv[kTkTPC];
#pragma unroll
        for (int j = 0; j < kTkTPC; ++j) load_keys4(src, b + kTkChunk + j * kTkTile, m, nk[j], nv[j]);
#pragma unroll
        for (int j = 0; j < kTkTPC; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (e < v[j] && (kk[j][e] >> pshift) == prefix) atomicAdd(&h[(kk[j][e] >> shift) & dmask], 1);
#pragma unroll
        for (int j = 0; j < kTkTPC; ++j) {
          v[j] = nv[j];
#pragma unroll
          for (int e = 0; e < 4; ++e) kk[j][e] = nk[j][e];
        }
      }
    }
    __syncthreads();
  };
  int need = k - above1;  // elements still to take from bin b1, >= 1
  histogram(b1, 20, 10, kTkBins2 - 1);
  find_bin<kTkBins2>(h, need, sw, res);
  const uint32_t b2 = (uint32_t)res[0];
  need -= res[1];
  __syncthreads();
  histogram((b1 << 10) | b2, 10, 0, kTkBins3 - 1);
  find_bin<kTkBins3>(h, need, sw, res);
  const uint32_t thr = (b1 << 20) | (b2 << 10) | (uint32_t)res[0];
  const int need_ties = need - res[1];  // keys equal to thr to take, lowest positions first, >= 1
  __syncthreads();

  // ---- output in position order: a key above thr goes to slot (keys above thr before it) +
  // min(ties before it, need_ties); a tie is taken while fewer than need_ties ties precede it.
  int run_gt = 0, run_eq = 0;  // keys above thr, and ties, before the current tile or group
  auto place = [&](uint32_t kk, int pos, int& g, int& q) {
    // the slots are below k whenever the workspace started zeroed; the checks keep a misused one in bounds
    if (kk > thr) {
      const int slot = g + (q < need_ties ? q : need_ties);
      if (slot < k) out[slot] = pos;
      ++g;
    } else if (kk == thr) {
      if (q < need_ties && g + q < k) out[g + q] = pos;
      ++q;
    }
  };
  if (fast) {  // tiles of kTkTile candidates from LDS, 4 consecutive per thread
    for (int t0 = 0; t0 < n_cand; t0 += kTkTile) {
      const int idx = t0 + 4 * tid;
      const int v = idx < n_cand ? (n_cand - idx < 4 ? n_cand - idx : 4) : 0;
      const uint4 kv = reinterpret_cast<const uint4*>(ckey)[idx / 4];
      const int4 pv = reinterpret_cast<const int4*>(cpos)[idx / 4];
      const uint32_t kk[4] = {kv.x, kv.y, kv.z, kv.w};
      const int pp[4] = {pv.x, pv.y, pv.z, pv.w};
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
      for (int e = 0; e < 4; ++e)
        if (e < v) place(kk[e], pp[e], g, q);
      run_gt += tot & 0xFFFF;
      run_eq += tot >> 16;
    }
  } else {  // groups of kTkTPC tiles of the row, the next group's loads in flight
    uint32_t kk[kTkTPC][4];
    int v[kTkTPC];
#pragma unroll
    for (int j = 0; j < kTkTPC; ++j) load_keys4(src, j * kTkTile, m, kk[j], v[j]);
    for (int b = 0; b < m; b += kTkChunk) {
      uint32_t nk[kTkTPC][4];
      int nv[kTkTPC];
#pragma unroll
      for (int j = 0; j < kTkTPC; ++j) load_keys4(src, b + kTkChunk + j * kTkTile, m, nk[j], nv[j]);
      int flags[kTkTPC], excl[kTkTPC];
#pragma unroll
      for (int j = 0; j < kTkTPC; ++j) {
        flags[j] = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          flags[j] += e < v[j] ? (kk[j][e] > thr ? 1 : (kk[j][e] == thr ? 0x10000 : 0)) : 0;
      }
      const int gtot = group_scan(flags, excl, sw);  // a group holds at most 8192 elements
#pragma unroll
      for (int j = 0; j < kTkTPC; ++j) {
        int g = run_gt + (excl[j] & 0xFFFF), q = run_eq + (excl[j] >> 16);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < v[j]) place(kk[j][e], b + j * kTkTile + 4 * tid + e, g, q);
      }
      run_gt += gtot & 0xFFFF;
      run_eq += gtot >> 16;
#pragma unroll
      for (int j = 0; j < kTkTPC; ++j) {
        v[j] = nv[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) kk[j][e] = nk[j][e];
      }
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
