// Measurement probes for gfx950 (libmla_probe.so): the rates this chip actually reaches for the three kinds
// of work the decode path is bound by, measured in the same run as the decode so that its roofline fraction
// can be read against both the vendor peak and the achievable one.  Not part of the decode path.
//   - mla_probe_stream_read: a streaming read of a large buffer (HBM read rate);
//   - mla_probe_row_gather: a gather of 16-byte-aligned rows at given addresses (the decode's access
//     pattern: rows of 352 bytes at random slots of a paged pool);
//   - mla_probe_mfma: a chain of independent 16x16x32 FP16 or bf16 MFMAs with no memory traffic (the
//     matrix cores' rate).
#include <hip/hip_runtime.h>
#include <stdint.h>


#include "mla_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;

// Every thread reads 16-byte words with a grid-stride loop, four loads in flight per iteration, and folds
// them into one word it writes at the end (so that no load can be dropped).
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = src[i];
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = x;
}

// Row r is the 16-byte chunks [addr16[r], addr16[r] + chunks) of pool (chunks = row_bytes / 16); chunk c of
// the gather (all rows' chunks in order) is read by thread c mod the grid, CPT chunks per thread in flight.
template <int CPT>
__global__ __launch_bounds__(kThreads) void row_gather_kernel(const uint8_t* __restrict__ pool,
                                                              const uint32_t* __restrict__ addr16, int64_t n_chunks,
                                                              int chunks, uint32_t* __restrict__ sink) {
  const int64_t nth = (int64_t)gridDim.x * kThreads;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 v[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int64_t c = t + k * nth;
    if (c < n_chunks) {
      const int64_t r = c / chunks, j = c - r * chunks;
      v[k] = *reinterpret_cast<const u32x4*>(pool + ((uint64_t)addr16[r] + (uint64_t)j) * 16u);
    } else {
      v[k] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  uint32_t x = 0;
#pragma unroll
  for (int k = 0; k < CPT; ++k) x ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  sink[t] = x;
}

// Each wave runs `iters` rounds of kChains independent MFMAs (enough to keep the matrix pipeline full) on
// register operands, then writes its accumulators (so that none of the work can be dropped).  The round is
// written in assembly: compiled from builtins, the compiler moved the accumulators between register files
// inside the loop, and those moves, not the matrix pipeline, set the rate.
constexpr int kChains = 8;

template <bool BF16>
__global__ __launch_bounds__(kThreads) void mfma_kernel(int iters, float* __restrict__ out) {
  const float s = 1.0f + 1e-3f * (float)(threadIdx.x & 7);
  f16x8 a, b;  // FP16 bit patterns; read as bf16 by the bf16 instruction (any finite values will do)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(s * (float)e);
    b[e] = (_Float16)(s - 0.01f * (float)e);
  }
  f32x4 c[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) c[k] = f32x4{s * k, 0.0f, 0.0f, 0.0f};
  for (int it = 0; it < iters; ++it) {
    if constexpr (BF16) {
      asm volatile(
          "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
          "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
          "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
          "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
          "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
          "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
          "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
          "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7"
          : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]), "+v"(c[4]), "+v"(c[5]), "+v"(c[6]), "+v"(c[7])
          : "v"(a), "v"(b));
    } else {
      asm volatile(
          "v_mfma_f32_16x16x32_f16 %0, %8, %9, %0\n\t"
          "v_mfma_f32_16x16x32_f16 %1, %8, %9, %1\n\t"
          "v_mfma_f32_16x16x32_f16 %2, %8, %9, %2\n\t"
          "v_mfma_f32_16x16x32_f16 %3, %8, %9, %3\n\t"
          "v_mfma_f32_16x16x32_f16 %4, %8, %9, %4\n\t"
          "v_mfma_f32_16x16x32_f16 %5, %8, %9, %5\n\t"
          "v_mfma_f32_16x16x32_f16 %6, %8, %9, %6\n\t"
          "v_mfma_f32_16x16x32_f16 %7, %8, %9, %7"
          : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]), "+v"(c[4]), "+v"(c[5]), "+v"(c[6]), "+v"(c[7])
          : "v"(a), "v"(b));
    }
  }
  // the hazard between an MFMA writing a register and a VALU reading it is left to the wait below
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  f32x4 t = c[0];
#pragma unroll
  for (int k = 1; k < kChains; ++k) t += c[k];
  reinterpret_cast<f32x4*>(out)[(int64_t)blockIdx.x * kThreads + threadIdx.x] = t;
}

}  // namespace

extern "C" {

int mla_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t workgroups, void* stream) {
  if (!src || !sink || bytes < 16 || bytes % 16 || workgroups < 1) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4*)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

int mla_probe_row_gather(const void* pool, const uint32_t* addr16, int64_t rows, int32_t row_bytes, uint32_t* sink,
                         int32_t workgroups, void* stream) {
  if (!pool || !addr16 || !sink || rows < 1 || row_bytes < 16 || row_bytes % 16 || workgroups < 1) return 1;
  const int chunks = row_bytes / 16;
  const int64_t n_chunks = rows * chunks;
  constexpr int CPT = 6;
  // every chunk is covered: the grid's threads times CPT reach the chunk count
  if ((int64_t)workgroups * kThreads * CPT < n_chunks) return 2;
  hipLaunchKernelGGL((row_gather_kernel<CPT>), dim3((unsigned)workgroups), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint8_t*)pool, addr16, n_chunks, chunks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

int mla_probe_mfma(int32_t bf16, int32_t iters, float* out, int32_t workgroups, void* stream) {
  if (!out || iters < 1 || workgroups < 1) return 1;
  if (bf16)
    hipLaunchKernelGGL(mfma_kernel<true>, dim3((unsigned)workgroups), dim3(kThreads), 0, (hipStream_t)stream, iters, out);
  else
    hipLaunchKernelGGL(mfma_kernel<false>, dim3((unsigned)workgroups), dim3(kThreads), 0, (hipStream_t)stream, iters,
                       out);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

int64_t mla_probe_mfma_flops(int32_t iters, int32_t workgroups) {
  // per wave: iters x kChains MFMAs of 16 x 16 x 32 multiply-adds (2 flops each)
  return (int64_t)workgroups * (kThreads / 64) * iters * kChains * (16 * 16 * 32 * 2);
}

}  // extern "C"
