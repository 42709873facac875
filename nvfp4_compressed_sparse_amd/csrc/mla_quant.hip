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
  quant_row_wave<FMT>(raw, rope_bits, dst, lane);
}

hipError_t launch_quant(int fmt, const QuantArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)((a.n + 3) / 4);
  if (fmt == 0) hipLaunchKernelGGL(quant_rows_kernel<0>, dim3(grid), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(quant_rows_kernel<1>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
