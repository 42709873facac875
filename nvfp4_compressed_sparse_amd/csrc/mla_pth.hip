// TokenSpeed's per-token-head FP8 MLA cache (its MLA KV layout section): three slot-indexed buffers,
// the latent as 512 E4M3 codes, one fp32 scale per slot, and the rope part in bf16 divided by the same
// scale.  Write, in fp32: s = max(amax(latent), 1e-26) / 448, codes = E4M3(x / s) (nearest, ties to even),
// rope = bf16(r / s) (nearest, ties to even).  Read: K = (code value * s, rope * s), V = code value * s.
//
// pth_quant_kernel: one wave per token; lane l holds latent values 8l..8l+7 and rope value l.
//
// pth_decode_kernel: one 256-thread workgroup per (query token, group of 16 heads, split).  The split's
// list entries are resolved to slots (order kept) in LDS; then, per step of 64 rows, wave w scores rows
// 16w..16w+15 of the step for the 16 heads with MFMA 16x16x32: the latent part in f16 (q rounded to f16,
// the codes exact), the rope part in bf16 (both exact), one accumulator.  Lane l holds, for row l%16, the
// latent bytes 128(l/16)..+127 and rope dims 16(l/16)..+15, and in latent k-step ks feeds bytes 8ks..+7
// of them (q's fragments use the same dimension order).  The row's scale multiplies the scores; each
// wave keeps its own online softmax (heads 4(l/16)+i of the accumulator lane), folds the row scale into
// P, and accumulates O += P V with MFMA 16x16x16 f16: P goes through LDS to the A layout (head l%16, rows
// 4(l/16)..+3); V is the wave's rows staged in LDS, lane (c, g) reading rows 4g..4g+3 at columns
// 64cq+4c..+3 and transposing the 4x4 bytes with byte permutes, so that its tile 4cq+e covers column
// 64cq+4c+e.  The four waves' states merge elementwise through LDS; with several splits the normalized
// result and its log-sum-exp go to the workspace and pth_merge_kernel combines them.
#include "mla_device.h"
#include "mla_pth_internal.h"

namespace mla {

constexpr int kPthThreads = 256;
constexpr int kPthEPT = kPthMaxChunk / kPthThreads;  // list entries per thread

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__global__ __launch_bounds__(256) void pth_quant_kernel(PthQuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.n) return;
  const int64_t slot = a.slot_mapping[r];
  if (slot < 0 || slot >= a.num_slots) return;
  const u32x4 xv = *reinterpret_cast<const u32x4*>(a.k_nope + r * a.nope_stride + 8 * lane);
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_to_f32(xv[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_to_f32(xv[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  const float s = fmaxf(amax, 1e-26f) / 448.0f;  // correctly rounded fp32 division
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = f32_to_e4m3(x[i] / s);
  *reinterpret_cast<u32x2*>(a.lat + slot * 512 + 8 * lane) =
      u32x2{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
  const float rv = bf16_to_f32(a.k_rope[r * a.rope_stride + lane]);
  a.rope[slot * 64 + lane] = f32_to_bf16_rne(rv / s);
  if (lane == 0) a.scale[slot] = s;
}

struct PthShared {
  uint32_t slots[kPthMaxChunk];
  int wcount[4];
  uint8_t stage[4][16][528];      // a wave's 16 latent rows (512 bytes + 16 padding)
  _Float16 pt[4][16][24];         // a wave's P^T: head, row (16 + 8 padding)
  float mo[2][128][64];           // merge: O values, [value][lane]
  float ml[2][8][64];             // merge: m[4], l[4] per lane
};

// 4 E4M3 bytes -> f16x4 (exact)
__device__ __forceinline__ f16x4 e4m3x4_to_f16x4(uint32_t w) {
  const f16x2 lo = e4m3x2_to_f16<false>(w), hi = e4m3x2_to_f16<true>(w);
  return f16x4{lo[0], lo[1], hi[0], hi[1]};
}

__global__ __launch_bounds__(kPthThreads) void pth_decode_kernel(PthDecodeArgs a) {
  __shared__ __attribute__((aligned(16))) PthShared sh;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int S = a.splits, HG = a.H / 16;
  const int s_idx = blockIdx.x % S;
  const int hg = (blockIdx.x / S) % HG;
  const int64_t id = blockIdx.x / (S * HG);
  const int b = (int)(id / a.T), t = (int)(id % a.T);
  const int L = a.ctx[b];
  const int lim = a.causal ? L - a.T + t : L - 1;
  const int64_t num_pages = a.num_slots / 64;

  // ---- this split's list entries -> slots, in list order
  const int e0 = s_idx * a.chunk;
  uint32_t slot_k[kPthEPT];
  uint32_t vmask = 0;
#pragma unroll
  for (int k = 0; k < kPthEPT; ++k) {
    const int e = e0 + kPthEPT * tid + k;
    const int pos = (kPthEPT * tid + k < a.chunk && e < a.topk) ? a.indices[id * a.topk + e] : -1;
    const int pg = (pos >= 0 ? pos : 0) >> 6;
    const bool inr = pos >= 0 && pos <= lim && pg < a.bt_stride;
    const int64_t page = inr ? a.block_table[(int64_t)b * a.bt_stride + pg] : -1;
    const bool ok = inr && page >= 0 && page < num_pages;
    slot_k[k] = ok ? (uint32_t)(page * 64 + (pos & 63)) : 0u;
    vmask |= (uint32_t)ok << k;
  }
  int off = 0, wave_total = 0;
#pragma unroll
  for (int k = 0; k < kPthEPT; ++k) {
    const uint64_t bal = __ballot((vmask >> k) & 1u);
    off += __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    wave_total += __builtin_popcountll(bal);
  }
  if (lane == 0) sh.wcount[w] = wave_total;
  __syncthreads();
  int n = 0;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    off += ww < w ? sh.wcount[ww] : 0;
    n += sh.wcount[ww];
  }
#pragma unroll
  for (int k = 0; k < kPthEPT; ++k)
    if (vmask & (1u << k)) sh.slots[off++] = slot_k[k];
  __syncthreads();

  // ---- q fragments of head 16hg + r16: latent dims 128g + 8ks .. +7 as f16, rope dims 16g + 8kr .. +7
  const uint16_t* qh = a.q + (id * a.H + 16 * hg + r16) * 576;
  f16x8 qa[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(qh + 128 * g + 8 * j);
    f16x8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = (_Float16)bf16_to_f32(v[i] & 0xFFFFu);
      f[2 * i + 1] = (_Float16)bf16_to_f32(v[i] >> 16);
    }
    qa[j] = f;
  }
  bf16x8 qr[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    qr[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + 512 + 16 * g + 8 * j));

  // ---- the wave's online softmax over its rows: heads 4g + i of this lane group
  float m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.0f;
  }
  f32x4 o[32];  // tile 4cq + e: column 64cq + 4(l%16) + e, heads 4g + i
#pragma unroll
  for (int j = 0; j < 32; ++j) o[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int nsteps = (n + 63) / 64;
  for (int st = 0; st < nsteps; ++st) {
    const int row = st * 64 + 16 * w + r16;
    const bool valid = row < n;
    const uint32_t slot = sh.slots[valid ? row : 0];
    const uint8_t* lp = a.lat + (uint64_t)slot * 512 + 128 * g;
    u32x4 kl[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kl[j] = *reinterpret_cast<const u32x4*>(lp + 16 * j);
    const uint16_t* rp = a.rope + (uint64_t)slot * 64 + 16 * g;
    const u32x4 kr0 = *reinterpret_cast<const u32x4*>(rp);
    const u32x4 kr1 = *reinterpret_cast<const u32x4*>(rp + 8);
    const float sc = a.scale[slot];

    // scores: C[head 4g + i][row r16]
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const uint32_t d0 = kl[ks >> 1][(ks & 1) * 2], d1 = kl[ks >> 1][(ks & 1) * 2 + 1];
      const f16x8 kb = as_f16x8(e4m3x2_to_f16<false>(d0), e4m3x2_to_f16<true>(d0), e4m3x2_to_f16<false>(d1),
                                e4m3x2_to_f16<true>(d1));
      acc = mfma16x16x32(qa[ks], kb, acc);
    }
    acc = mfma16x16x32(qr[0], __builtin_bit_cast(bf16x8, kr0), acc);
    acc = mfma16x16x32(qr[1], __builtin_bit_cast(bf16x8, kr1), acc);

    // stage the latent rows for P V (the wave's own region; no other wave reads it)
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(&sh.stage[w][r16][128 * g + 16 * j]) = kl[j];

    float p[4], alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float z = valid ? acc[i] * sc * a.scale_log2 : -INFINITY;
      float mx = z;
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 16));
      const float mn = fmaxf(m[i], mx);
      const bool live = mn != -INFINITY;  // some row of this head seen so far
      alpha[i] = live ? exp2f(m[i] - mn) : 1.0f;
      p[i] = live ? exp2f(z - mn) : 0.0f;
      float ps = p[i];
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) ps += __shfl_xor(ps, d, 16);
      l[i] = l[i] * alpha[i] + ps;
      m[i] = mn;
      sh.pt[w][4 * g + i][r16] = (_Float16)(p[i] * sc);  // V's row scale folded into P
    }
#pragma unroll
    for (int j = 0; j < 32; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[j][i] *= alpha[i];
    // the stage and P^T writes of this wave are visible to its own later reads after lgkmcnt(0)
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();

    // P^T as the A operand: head l%16, rows 4g..4g+3
    const f16x4 pa = *reinterpret_cast<const f16x4*>(&sh.pt[w][r16][4 * g]);
#pragma unroll
    for (int cq = 0; cq < 8; ++cq) {
      uint32_t d[4];  // rows 4g + i, columns 64cq + 4r16 .. +3
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = *reinterpret_cast<const uint32_t*>(&sh.stage[w][4 * g + i][64 * cq + 4 * r16]);
      const uint32_t p01a = __builtin_amdgcn_perm(d[1], d[0], 0x05010400u);  // d0[0] d1[0] d0[1] d1[1]
      const uint32_t p23a = __builtin_amdgcn_perm(d[3], d[2], 0x05010400u);
      const uint32_t p01b = __builtin_amdgcn_perm(d[1], d[0], 0x07030602u);  // d0[2] d1[2] d0[3] d1[3]
      const uint32_t p23b = __builtin_amdgcn_perm(d[3], d[2], 0x07030602u);
      const uint32_t col[4] = {__builtin_amdgcn_perm(p23a, p01a, 0x05040100u),
                               __builtin_amdgcn_perm(p23a, p01a, 0x07060302u),
                               __builtin_amdgcn_perm(p23b, p01b, 0x05040100u),
                               __builtin_amdgcn_perm(p23b, p01b, 0x07060302u)};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[4 * cq + e] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, e4m3x4_to_f16x4(col[e]), o[4 * cq + e], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();  // the next step's stage writes follow this step's reads
  }

  // ---- merge the four waves' states: 2,3 into 0,1, then 1 into 0
  auto merge_from = [&](int buf) {
    float mb[4], lb[4], f_self[4], f_other[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mb[i] = sh.ml[buf][i][lane];
      lb[i] = sh.ml[buf][4 + i][lane];
      const float mn = fmaxf(m[i], mb[i]);
      f_self[i] = mn == -INFINITY ? 0.0f : exp2f(m[i] - mn);
      f_other[i] = mn == -INFINITY ? 0.0f : exp2f(mb[i] - mn);
      l[i] = l[i] * f_self[i] + lb[i] * f_other[i];
      m[i] = mn;
    }
#pragma unroll
    for (int j = 0; j < 32; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[j][i] = o[j][i] * f_self[i] + sh.mo[buf][4 * j + i][lane] * f_other[i];
  };
  auto store_to = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sh.ml[buf][i][lane] = m[i];
      sh.ml[buf][4 + i][lane] = l[i];
    }
#pragma unroll
    for (int j = 0; j < 32; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sh.mo[buf][4 * j + i][lane] = o[j][i];
  };
  if (w >= 2) store_to(w - 2);
  __syncthreads();
  if (w < 2) merge_from(w);
  __syncthreads();
  if (w == 1) store_to(0);
  __syncthreads();
  if (w != 0) return;
  merge_from(0);

  // ---- wave 0: normalized result (heads 4g + i, columns 64cq + 4r16 + e) and its log-sum-exp
  float inv[4], lse[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    inv[i] = l[i] > 0.0f ? 1.0f / l[i] : 0.0f;
    lse[i] = l[i] > 0.0f ? (m[i] + __log2f(l[i])) * 0.6931471805599453f : -INFINITY;
  }
  const int64_t hrow0 = id * a.H + 16 * hg + 4 * g;
  if (S == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t* dst = a.out + (hrow0 + i) * 512 + 4 * r16;
#pragma unroll
      for (int cq = 0; cq < 8; ++cq)
        *reinterpret_cast<u32x2*>(dst + 64 * cq) =
            u32x2{pack_bf16_rne(o[4 * cq][i] * inv[i], o[4 * cq + 1][i] * inv[i]),
                  pack_bf16_rne(o[4 * cq + 2][i] * inv[i], o[4 * cq + 3][i] * inv[i])};
      if (a.lse && r16 == 0) a.lse[hrow0 + i] = lse[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* dst = a.part_o + ((hrow0 + i) * S + s_idx) * 512 + 4 * r16;
#pragma unroll
      for (int cq = 0; cq < 8; ++cq)
        *reinterpret_cast<f32x4*>(dst + 64 * cq) =
            f32x4{o[4 * cq][i] * inv[i], o[4 * cq + 1][i] * inv[i], o[4 * cq + 2][i] * inv[i], o[4 * cq + 3][i] * inv[i]};
      if (r16 == 0) a.part_lse[(hrow0 + i) * S + s_idx] = lse[i];
    }
  }
}

// One 128-thread workgroup per (query token, head): out = sum_s e^(lse_s - lse) out_s, lse = ln sum_s e^lse_s.
__global__ __launch_bounds__(128) void pth_merge_kernel(PthDecodeArgs a) {
  const int64_t hrow = blockIdx.x;
  const int S = a.splits;
  const float* pl = a.part_lse + hrow * S;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, pl[s]);
  float Z = 0.0f;
  if (M != -INFINITY)
    for (int s = 0; s < S; ++s) Z += __expf(pl[s] - M);
  const float lse = M == -INFINITY ? -INFINITY : M + __logf(Z);
  const int c = 4 * threadIdx.x;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (M != -INFINITY)
    for (int s = 0; s < S; ++s) {
      const float wgt = __expf(pl[s] - lse);
      const f32x4 v = *reinterpret_cast<const f32x4*>(a.part_o + (hrow * S + s) * 512 + c);
      acc += wgt * v;
    }
  *reinterpret_cast<u32x2*>(a.out + hrow * 512 + c) = u32x2{pack_bf16_rne(acc[0], acc[1]), pack_bf16_rne(acc[2], acc[3])};
  if (a.lse && threadIdx.x == 0) a.lse[hrow] = lse;
}

hipError_t launch_pth_quant(const PthQuantArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(pth_quant_kernel, dim3((unsigned)((a.n + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_pth_decode(const PthDecodeArgs& a, hipStream_t stream) {
  const int64_t units = (int64_t)a.B * a.T * (a.H / 16);
  hipLaunchKernelGGL(pth_decode_kernel, dim3((unsigned)(units * a.splits)), dim3(kPthThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL(pth_merge_kernel, dim3((unsigned)((int64_t)a.B * a.T * a.H)), dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
