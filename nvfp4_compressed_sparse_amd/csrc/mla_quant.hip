// Quantize-on-write kernels: bf16 latent[512] + rope[64] per token -> one cache row in a paged pool.
//
// Row formats ("Prime Inference" launch post, section "为低延迟解码腾出空间"; the analysis page's
// row table): NVFP4 row = 256 nibble bytes | 32 E4M3 block scales | 64 E4M3 rope bytes (352 B);
// FP8 row = 512 E4M3 latent bytes | 64 E4M3 rope bytes (576 B).  Rounding: scale = E4M3 nearest to
// amax/6, element = e2m1 nearest to |x|/scale, rope and FP8 = E4M3 nearest; ties to the even code,
// saturating; all decisions are exact comparisons in fp32.
//
// One wavefront per token: lane l owns latent elements 8l..8l+7 (a 16-byte load) and rope element l.
// An NVFP4 block of 16 values is two neighbouring lanes; the row is written as 88 (or 144) coalesced
// dwords.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

template <int FMT>
__global__ __launch_bounds__(256) void quant_rows_kernel(QuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.n) return;
  const int64_t slot = a.slot_mapping[r];
  if (slot < 0) return;
  const int64_t page = slot >> 6;
  if (page >= a.num_pages) return;
  constexpr int kRowBytes = FMT == 0 ? kNvfp4Row : kFp8Row;
  uint8_t* dst = a.pool + page * a.page_stride + (slot & 63) * kRowBytes;

  const u32x4 raw = *reinterpret_cast<const u32x4*>(a.k_nope + r * a.nope_stride + 8 * lane);
  const uint32_t rope_bits = a.k_rope[r * a.rope_stride + lane];
  const uint32_t rope_code = f32_to_e4m3(bf16_to_f32(rope_bits));

  uint32_t h[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    h[2 * k] = raw[k] & 0xFFFFu;
    h[2 * k + 1] = raw[k] >> 16;
  }

  if (FMT == 0) {
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(bf16_to_f32(h[k])));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    const int sc = e4m3_scale_code_div6(amax);
    const float s = e4m3_code_value(sc);
    uint32_t nib = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t mag = sc == 0 ? 0u : e2m1_mag_code(fabsf(bf16_to_f32(h[k])), s);
      uint32_t code = ((h[k] >> 12) & 8u) | mag;
      nib |= code << (4 * k);
    }
    *reinterpret_cast<uint32_t*>(dst + 4 * lane) = nib;
    // scale bytes: block j lives in lanes 2j and 2j+1; dword q holds blocks 4q..4q+3
    const int src = 8 * (lane & 7);
    uint32_t s0 = __shfl(sc, src, 64), s1 = __shfl(sc, src + 2, 64);
    uint32_t s2 = __shfl(sc, src + 4, 64), s3 = __shfl(sc, src + 6, 64);
    if (lane < 8) *reinterpret_cast<uint32_t*>(dst + 256 + 4 * lane) = s0 | (s1 << 8) | (s2 << 16) | (s3 << 24);
  } else {
    uint32_t c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = f32_to_e4m3(bf16_to_f32(h[k]));
    u32x2 v = {c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
    *reinterpret_cast<u32x2*>(dst + 8 * lane) = v;
  }
  // rope bytes: dword q holds rope values 4q..4q+3 (lanes 4q..4q+3)
  const int src = 4 * (lane & 15);
  uint32_t r0 = __shfl(rope_code, src, 64), r1 = __shfl(rope_code, src + 1, 64);
  uint32_t r2 = __shfl(rope_code, src + 2, 64), r3 = __shfl(rope_code, src + 3, 64);
  constexpr int kRopeOff = FMT == 0 ? 288 : 512;
  if (lane < 16) *reinterpret_cast<uint32_t*>(dst + kRopeOff + 4 * lane) = r0 | (r1 << 8) | (r2 << 16) | (r3 << 24);
}

hipError_t launch_quant(int fmt, const QuantArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)((a.n + 3) / 4);
  if (fmt == 0) hipLaunchKernelGGL(quant_rows_kernel<0>, dim3(grid), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(quant_rows_kernel<1>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
