// TokenSpeed's per-token-head FP8 MLA cache (its MLA KV layout section): three slot-indexed buffers,
// the latent as 512 E4M3 codes, one fp32 scale per slot, and the rope part in bf16 divided by the same
// scale.  Write, in fp32: s = max(amax(latent), 1e-26) / 448, codes = E4M3(x / s) (nearest, ties to even),
// rope = bf16(r / s) (nearest, ties to even).  Read: K = (code value * s, rope * s), V = code value * s.
//
// pth_quant_kernel: one wave per token; lane l holds latent values 8l..8l+7 and rope value l.
//
// pth_decode_kernel: one 256-thread workgroup per (query token, group of 16 heads, split), two per
// compute unit.  The split's list entries are resolved to slots (order kept) in LDS, and the heads'
// latent q goes to LDS as f16; then, per step of 64 rows:
//   * wave w scores rows 16w..16w+15 of the step for the 16 heads with MFMA 16x16x32: the latent part in
//     f16 (each head's q scaled by a power of two into f16's range, then rounded to f16; the codes exact),
//     the rope part in bf16 (both exact), one accumulator, the power of two undone in the score.  Lane
//     l holds, for row l%16, the latent bytes 128(l/16)..+127 and rope dims 16(l/16)..+15, and in latent
//     k-step ks feeds bytes 8ks..+7 of them (q's fragments use the same dimension order).  The scores
//     (times the row's scale) and the scales go to LDS, then, past the step's first barrier, the latent
//     rows; the next step's rows are already loading into a second register buffer;
//   * 16 threads per head take the step's softmax: the running max, P' = p * row scale (V's scale folded
//     into P) as f16 in LDS, the running sum, the rescale factor;
//   * wave w accumulates O += P' V for its 128 output columns over the step's 64 rows with MFMA
//     16x16x16 f16: lane (c, g) reads rows 4g..4g+3 of a 16-row k-step at columns 64cq+4c..+3 from the
//     staged rows and transposes the 4x4 bytes with byte permutes, so that its tile 4cq+e covers column
//     64cq+4c+e.
// Each wave writes its own columns at the end; with several splits the normalized result and its
// log-sum-exp go to the workspace and pth_merge_kernel combines them.
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
  uint8_t stage[64][528];         // the step's 64 latent rows (512 bytes + 16 padding)
  _Float16 qs[16][520];           // the 16 heads' latent q as f16 (512 values + 8 padding)
  float sz[64][17];               // the step's scores z[row][head] (log2 units), row 16w + lane%16 by wave w
  float ss[64];                   // the step's row scales
  _Float16 pp[16][72];            // P'[head][row] = p * row scale (f16), rows padded by 8
  float salpha[16];               // the step's rescale factor per head
  float sl[16], sm[16];           // the final l and m per head
  int qk[16];                     // per head: q is scaled by 2^qk[h] (its largest magnitude to [2^15, 2^16))
};

// 4 E4M3 bytes -> f16x4 (exact)
__device__ __forceinline__ f16x4 e4m3x4_to_f16x4(uint32_t w) {
  const f16x2 lo = e4m3x2_to_f16<false>(w), hi = e4m3x2_to_f16<true>(w);
  return f16x4{lo[0], lo[1], hi[0], hi[1]};
}

__global__ __launch_bounds__(kPthThreads, 2) void pth_decode_kernel(PthDecodeArgs a) {
  __shared__ __attribute__((aligned(16))) PthShared sh;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int S = a.splits, HG = a.H / 16;
  // the head groups of one (token, split) read the same rows: they take consecutive logical ids, which
  // run on one XCD and so share its L2
  const int j = xcd_logical_id(blockIdx.x, gridDim.x);
  const int hg = j % HG;
  const int s_idx = (j / HG) % S;
  const int64_t id = j / (HG * S);
  const int b = (int)(id / a.T), t = (int)(id % a.T);
  const int L = a.ctx[b];
  const int lim = a.causal ? L - a.T + t : L - 1;
  const int64_t num_pages = a.num_slots / 64;

  // the 16 heads' latent q, requested first so that it arrives during the list and page-table lookups:
  // thread tid takes head tid / 16, dims 32 (tid % 16) .. +31
  // (and rope dims 512 + 4 (tid % 16) .. +3, for the head's largest magnitude)
  u32x4 qv[4];
  u32x2 qrm;
  {
    const uint16_t* qsrc = a.q + (id * a.H + 16 * hg + (tid >> 4)) * 576;
#pragma unroll
    for (int j = 0; j < 4; ++j) qv[j] = *reinterpret_cast<const u32x4*>(qsrc + 32 * (tid & 15) + 8 * j);
    qrm = *reinterpret_cast<const u32x2*>(qsrc + 512 + 4 * (tid & 15));
  }

  // ---- this split's list entries -> slots, in list order
  const int e0 = s_idx * a.chunk;
  uint32_t slot_k[kPthEPT];
  uint32_t vmask = 0;
  // every load is issued (an entry past the list reads entry 0, a position outside the table reads
  // page-table entry 0) and its result discarded afterwards: the loads of all entries fly together
  int pos_k[kPthEPT];
#pragma unroll
  for (int k = 0; k < kPthEPT; ++k) {
    const int e = e0 + kPthEPT * tid + k;
    const bool in_list = kPthEPT * tid + k < a.chunk && e < a.topk;
    const int v = a.indices[id * a.topk + (in_list ? e : 0)];
    pos_k[k] = in_list ? v : -1;
  }
  int32_t page_k[kPthEPT];
#pragma unroll
  for (int k = 0; k < kPthEPT; ++k) {
    const int pos = pos_k[k];
    const int pg = (pos >= 0 ? pos : 0) >> 6;
    const bool inr = pos >= 0 && pos <= lim && pg < a.bt_stride;
    page_k[k] = a.block_table[(int64_t)b * a.bt_stride + (inr ? pg : 0)];
    pos_k[k] = inr ? pos : -1;
  }
#pragma unroll
  for (int k = 0; k < kPthEPT; ++k) {
    const int pos = pos_k[k];
    const int64_t page = page_k[k];
    const bool ok = pos >= 0 && page >= 0 && page < num_pages;
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
  // the latent q to LDS as f16, each head scaled by its power of two 2^kq (largest magnitude over all 576
  // dims to [2^15, 2^16)); the 16 threads of a head reduce its largest magnitude
  uint32_t mq = bf16x8_max_mag(u32x4{qrm[0], qrm[1], 0u, 0u});
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t m = bf16x8_max_mag(qv[j]);
    mq = mq > m ? mq : m;
  }
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)mq, d, 16);
    mq = mq > o ? mq : o;
  }
  const int kq = q_shift(mq);
  if ((tid & 15) == 0) sh.qk[tid >> 4] = kq;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 v = qv[j];
    *reinterpret_cast<f16x8*>(&sh.qs[tid >> 4][32 * (tid & 15) + 8 * j]) =
        as_f16x8(bf16x2_pow2_to_f16x2(v[0], kq), bf16x2_pow2_to_f16x2(v[1], kq), bf16x2_pow2_to_f16x2(v[2], kq),
                 bf16x2_pow2_to_f16x2(v[3], kq));
  }
  __syncthreads();

  // ---- q fragments of head 16hg + r16: latent dims 128g + 8ks .. +7 from LDS in each step, rope dims
  // 16g + 8kr .. +7 in registers
  // (the rope part times 2^kq of head r16 stays exact in bf16: it only moves the exponent, and the
  // scaled values stay below 2^16; the score of head 4g+i is scaled back by 2^-kq with the softmax scale)
  const uint16_t* qh = a.q + (id * a.H + 16 * hg + r16) * 576;
  bf16x8 qr[2];
  {
    const int kr = sh.qk[r16];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(qh + 512 + 16 * g + 8 * j);
      u32x4 sc;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc[i] = pack_hi16(__builtin_ldexpf(__uint_as_float(raw[i] << 16), kr),
                          __builtin_ldexpf(__uint_as_float(raw[i] & 0xFFFF0000u), kr));
      qr[j] = __builtin_bit_cast(bf16x8, sc);
    }
  }
  float sl2h[4];  // softmax scale * log2(e) * 2^-kq of heads 4g + i
#pragma unroll
  for (int i = 0; i < 4; ++i) sl2h[i] = __builtin_ldexpf(a.scale_log2, -sh.qk[4 * g + i]);

  // softmax role: thread tid serves head sh_h = tid / 16 over rows 4 * (tid % 16) .. +3 of a step
  const int sh_h = tid >> 4, sh_r = 4 * (tid & 15);
  float m_h = -INFINITY, l_h = 0.0f;
  // accumulate role: wave w owns columns 128w .. 128w + 127 as column quads cq = 2w, 2w + 1; tile
  // 4c + e (c < 2) covers column 64(2w + c) + 4(lane%16) + e, heads 4g + i
  f32x4 o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // a step's rows for this lane: latent bytes 128g..+127, rope dims 16g..+15 and the scale of row
  // 16w + r16 of the step
  struct StepRows {
    u32x4 kl[8];
    u32x4 kr[2];
    float sc;
    bool valid;
  };
  auto load_step = [&](int st, StepRows& sr) {
    const int row = st * 64 + 16 * w + r16;
    sr.valid = row < n;
    const uint32_t listed = sh.slots[sr.valid ? row : 0];  // slots[0] may be unset when n = 0
    const uint32_t slot = sr.valid ? listed : 0u;
    const uint8_t* lp = a.lat + (uint64_t)slot * 512 + 128 * g;
#pragma unroll
    for (int j = 0; j < 8; ++j) sr.kl[j] = *reinterpret_cast<const u32x4*>(lp + 16 * j);
    const uint16_t* rp = a.rope + (uint64_t)slot * 64 + 16 * g;
    sr.kr[0] = *reinterpret_cast<const u32x4*>(rp);
    sr.kr[1] = *reinterpret_cast<const u32x4*>(rp + 8);
    sr.sc = a.scale[slot];
  };
  auto compute_step = [&](const StepRows& sr) {
    // ---- scores of the wave's 16 rows: C[head 4g + i][row r16]
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const uint32_t d0 = sr.kl[ks >> 1][(ks & 1) * 2], d1 = sr.kl[ks >> 1][(ks & 1) * 2 + 1];
      const f16x8 kb = as_f16x8(e4m3x2_to_f16<false>(d0), e4m3x2_to_f16<true>(d0), e4m3x2_to_f16<false>(d1),
                                e4m3x2_to_f16<true>(d1));
      acc = mfma16x16x32(*reinterpret_cast<const f16x8*>(&sh.qs[r16][128 * g + 8 * ks]), kb, acc);
    }
    acc = mfma16x16x32(qr[0], __builtin_bit_cast(bf16x8, sr.kr[0]), acc);
    acc = mfma16x16x32(qr[1], __builtin_bit_cast(bf16x8, sr.kr[1]), acc);
    const int row = 16 * w + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) sh.sz[row][4 * g + i] = sr.valid ? acc[i] * sr.sc * sl2h[i] : -INFINITY;
    // a row past the list gets scale 0 and stages zeros, so that whatever slot 0 holds (it is read in
    // its place) cannot reach O through 0 * NaN
    if (g == 0) sh.ss[row] = sr.valid ? sr.sc : 0.0f;
    lds_barrier();  // (A) scores and scales complete, every wave done with the last step's rows; the
                    // next rows stay in flight

    // ---- stage the rows for P V (one buffer: the last step's readers have all passed (A))
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(&sh.stage[row][128 * g + 16 * j]) = sr.valid ? sr.kl[j] : zero4;

    // ---- softmax over the step's 64 rows, head sh_h: the running max, P' = p * row scale, the sum
    float z[4], mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = sh.sz[sh_r + r][sh_h];
      mx = fmaxf(mx, z[r]);
    }
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 16));
    const float mn = fmaxf(m_h, mx);
    const bool live = mn != -INFINITY;  // some row of this head seen so far
    const float alpha = live ? exp2f(m_h - mn) : 1.0f;
    float ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = live ? exp2f(z[r] - mn) : 0.0f;
      ps += p;
      sh.pp[sh_h][sh_r + r] = (_Float16)(p * sh.ss[sh_r + r]);  // V's row scale folded into P
    }
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) ps += __shfl_xor(ps, d, 16);
    l_h = l_h * alpha + ps;
    m_h = mn;
    if ((tid & 15) == 0) sh.salpha[sh_h] = alpha;
    lds_barrier();  // (B) P', the rescale factors and the staged rows complete

    // ---- O[heads][the wave's columns] = alpha O + P' V over the step's 64 rows (4 k-steps of 16)
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) al[i] = sh.salpha[4 * g + i];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[j][i] *= al[i];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const f16x4 pa = *reinterpret_cast<const f16x4*>(&sh.pp[r16][16 * kk + 4 * g]);  // head lane%16
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int cq = 2 * w + c;
        uint32_t d[4];  // rows 16kk + 4g + i, columns 64cq + 4r16 .. +3
#pragma unroll
        for (int i = 0; i < 4; ++i)
          d[i] = *reinterpret_cast<const uint32_t*>(&sh.stage[16 * kk + 4 * g + i][64 * cq + 4 * r16]);
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
          o[4 * c + e] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, e4m3x4_to_f16x4(col[e]), o[4 * c + e], 0, 0, 0);
      }
    }
  };
  // two register buffers named statically (a copy between them would wait for loads in flight): step
  // st + 1's rows load while step st computes.  The loads are unconditional (a step past the end reads
  // slot 0 and is never used) so that the compiler's counter waits stay exact.  Barriers (A) and (B)
  // order the LDS traffic.
  const int nsteps = (n + 63) / 64;
  StepRows ra, rb;
  load_step(0, ra);
  // The scheduling barriers keep the compiler from hoisting a step's first conversions above the next
  // step's loads, which would make them wait for the loads just issued.
  for (int st = 0; st < nsteps; st += 2) {
    load_step(st + 1, rb);
    __builtin_amdgcn_sched_barrier(0);
    compute_step(ra);
    if (st + 1 >= nsteps) break;
    load_step(st + 2, ra);
    __builtin_amdgcn_sched_barrier(0);
    compute_step(rb);
  }

  // ---- the normalized result of the wave's columns and the log-sum-exp
  if ((tid & 15) == 0) {
    sh.sl[sh_h] = l_h;
    sh.sm[sh_h] = m_h;
  }
  __syncthreads();
  float inv[4], lse[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lv = sh.sl[4 * g + i], mv = sh.sm[4 * g + i];
    inv[i] = lv > 0.0f ? 1.0f / lv : 0.0f;
    lse[i] = lv > 0.0f ? (mv + __log2f(lv)) * 0.6931471805599453f : -INFINITY;
  }
  const int64_t hrow0 = id * a.H + 16 * hg + 4 * g;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int col0 = 64 * (2 * w + c) + 4 * r16;
      const f32x4 v = {o[4 * c][i] * inv[i], o[4 * c + 1][i] * inv[i], o[4 * c + 2][i] * inv[i], o[4 * c + 3][i] * inv[i]};
      if (S == 1)
        *reinterpret_cast<u32x2*>(a.out + (hrow0 + i) * 512 + col0) = u32x2{pack_bf16_rne(v[0], v[1]), pack_bf16_rne(v[2], v[3])};
      else
        *reinterpret_cast<f32x4*>(a.part_o + ((hrow0 + i) * S + s_idx) * 512 + col0) = v;
    }
    if (w == 0 && r16 == 0) {
      if (S == 1) {
        if (a.lse) a.lse[hrow0 + i] = lse[i];
      } else {
        a.part_lse[(hrow0 + i) * S + s_idx] = lse[i];
      }
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
