// The staged path ("Prime Inference" launch post, section "原生 NVFP4 稀疏 MLA 解码内核"; the analysis
// page, section "A kernel that reads four bits directly", staged-versus-native figure): before the
// native kernel, the rows a query token selects were unpacked from NVFP4 into 576-byte FP8 rows of a
// temporary buffer and an FP8 attention kernel read that copy, moving 352 + 576 + 576 bytes per selected
// row through memory instead of 352.  This kernel is that unpack step, for comparing the two paths on
// this chip; the FP8 decoder then reads the copy as a paged cache.
//
// A query token id = b*T + t is served by `parts` 256-thread workgroups (enough to fill the chip: a
// single workgroup per token left the unpack waiting on memory with too few rows in flight):
//   * selection, as in the sparse decode, repeated by every part (the list and its page-table entries
//     are a few KB, read from L2 after the first part): the token's list entries that are >= 0, within
//     the causal limit, and on a page whose table entry is in the pool, kept in list order (ballot
//     compaction into an LDS list of row addresses);
//   * unpack: part p takes selected rows p*R .. p*R+R-1 (R = ceil(topk/parts)); each wave takes every
//     fourth of those, eight rows in flight; lane l converts latent values 8l..8l+7 (one
//     nibble dword, block l/2's scale) to fp32 exactly (e2m1 x E4M3 has at most 6 significant bits),
//     clamps to +-448 and packs them with the FP8 conversion (nearest, ties to even), and lanes 0-15
//     copy the 64 rope bytes;
//   * the token's row count and its page-table row over the copy (pages id*P .. id*P+P-1).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

constexpr int kStageThreads = 256;
constexpr int kStageMaxEntries = 2048;
constexpr int kStageEPT = kStageMaxEntries / kStageThreads;  // list entries per thread

__global__ __launch_bounds__(kStageThreads) void stage_rows_kernel(StageArgs a) {
  __shared__ uint32_t rowlist[kStageMaxEntries];  // 16-byte addresses of the selected rows, in list order
  __shared__ int wcount[kStageThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int64_t id = blockIdx.x / a.parts;
  const int part = blockIdx.x % a.parts;
  const int b = (int)(id / a.T), t = (int)(id % a.T);
  const int L = a.ctx[b];
  const int lim = a.causal ? L - a.T + t : L - 1;
  const int32_t* btr = a.block_table + (int64_t)b * a.bt_stride;

  // ---- selection: entries EPT*tid .. EPT*tid+EPT-1
  int pos[kStageEPT];
#pragma unroll
  for (int k = 0; k < kStageEPT; ++k) {
    const int e = kStageEPT * tid + k;
    pos[k] = e < a.topk ? a.indices[id * a.topk + e] : -1;
  }
  uint32_t addr[kStageEPT];
  uint32_t vmask = 0;
#pragma unroll
  for (int k = 0; k < kStageEPT; ++k) {
    const int pg = (pos[k] >= 0 ? pos[k] : 0) >> 6;
    const bool inr = pos[k] >= 0 && pos[k] <= lim && pg < a.bt_stride;
    const int page = inr ? btr[pg] : -1;
    const bool ok = inr && page >= 0 && page < a.num_pages;
    addr[k] = ok ? (uint32_t)(((uint64_t)page * (uint64_t)a.page_stride + (uint64_t)(pos[k] & 63) * kNvfp4Row) >> 4)
                 : 0u;
    vmask |= (uint32_t)ok << k;
  }
  int off = 0, wave_total = 0;
#pragma unroll
  for (int k = 0; k < kStageEPT; ++k) {
    const uint64_t bal = __ballot((vmask >> k) & 1u);
    off += __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    wave_total += __builtin_popcountll(bal);
  }
  if (lane == 0) wcount[w] = wave_total;
  __syncthreads();
  int n = 0;
#pragma unroll
  for (int ww = 0; ww < kStageThreads / 64; ++ww) {
    off += ww < w ? wcount[ww] : 0;
    n += wcount[ww];
  }
#pragma unroll
  for (int k = 0; k < kStageEPT; ++k)
    if (vmask & (1u << k)) rowlist[off++] = addr[k];
  __syncthreads();

  // ---- the token's row count and page-table row over the copy
  const int P = a.pages_per_token;
  if (part == 0) {
    if (tid == 0) a.staged_lens[id] = n;
    for (int p = tid; p < P; p += kStageThreads) a.staged_block_table[id * P + p] = (int32_t)(id * P + p);
  }

  // ---- unpack this part's rows, eight per wave in flight
  constexpr int U = 8;
  const int per = (a.topk + a.parts - 1) / a.parts;
  const int r_begin = part * per;
  const int r_end = r_begin + per < n ? r_begin + per : n;
  uint8_t* base = a.staged + id * (int64_t)P * kPage * kFp8Row;
  for (int r0 = r_begin + w; r0 < r_end; r0 += U * (kStageThreads / 64)) {
    uint32_t nib[U], scw[U], rope[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * (kStageThreads / 64);
      nib[u] = scw[u] = rope[u] = 0;
      if (r < r_end) {
        const uint8_t* src = a.pool + (uint64_t)rowlist[r] * 16u;
        nib[u] = *reinterpret_cast<const uint32_t*>(src + 4 * lane);
        scw[u] = *reinterpret_cast<const uint32_t*>(src + 256 + 4 * (lane >> 3));
        if (lane < 16) rope[u] = *reinterpret_cast<const uint32_t*>(src + 288 + 4 * lane);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * (kStageThreads / 64);
      if (r >= r_end) continue;
      // block l/2's scale: byte (l >> 1) & 3 of the dword holding blocks 4(l>>3) .. 4(l>>3)+3
      const float s = e4m3x2_to_f32<false>(scw[u] >> (8 * ((lane >> 1) & 3)))[0];
      f32x2 v[4] = {fp4x2_to_f32<0>(nib[u]), fp4x2_to_f32<1>(nib[u]), fp4x2_to_f32<2>(nib[u]), fp4x2_to_f32<3>(nib[u])};
      uint32_t packed[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        short2_t acc = {0, 0};
        const f32x2 x = v[2 * h], y = v[2 * h + 1];
        const float x0 = __builtin_amdgcn_fmed3f(x[0] * s, -448.0f, 448.0f);
        const float x1 = __builtin_amdgcn_fmed3f(x[1] * s, -448.0f, 448.0f);
        const float y0 = __builtin_amdgcn_fmed3f(y[0] * s, -448.0f, 448.0f);
        const float y1 = __builtin_amdgcn_fmed3f(y[1] * s, -448.0f, 448.0f);
        acc = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(acc, x0, x1, 1.0f, false);
        acc = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(acc, y0, y1, 1.0f, true);
        packed[h] = __builtin_bit_cast(uint32_t, acc);
      }
      uint8_t* dst = base + (int64_t)r * kFp8Row;
      *reinterpret_cast<u32x2*>(dst + 8 * lane) = u32x2{packed[0], packed[1]};
      if (lane < 16) *reinterpret_cast<uint32_t*>(dst + kLatent + 4 * lane) = rope[u];
    }
  }
}

hipError_t launch_stage(const StageArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(stage_rows_kernel, dim3((unsigned)((int64_t)a.B * a.T * a.parts)), dim3(kStageThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace mla
