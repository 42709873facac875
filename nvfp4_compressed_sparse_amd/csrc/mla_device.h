// Device-side helpers shared by the gfx950 kernels of libmla_nvfp4: vector types, exact number-format
// conversions, MFMA wrapper, cross-lane helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kQK = 576;
constexpr int kPage = 64;
constexpr int kNvfp4Row = 352;
constexpr int kFp8Row = 576;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short short2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Upper halves of two fp32 values packed as bf16x2 (lo in bits 0..15).  Exact for values that are
// representable in bf16, which every dequantized NVFP4 / FP8 product is.
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Round-to-nearest-even fp32 -> bf16x2 (hardware conversion).
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Two e2m1 nibbles of byte `sel` of `src` -> fp32 (low nibble in .x).  The hardware scale operand
// only contributes its exponent, so it is left at 1.0 and the E4M3 block scale is applied by a
// separate fp32 multiply (exact: at most 6 significant bits).
template <int SEL>
__device__ __forceinline__ f32x2 fp4x2_to_f32(uint32_t src) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(src, 1.0f, SEL);
}

// Two e2m1 nibbles of byte `SEL` of `src` -> fp16x2 (low nibble in .x), exact.  As above the hardware
// scale is left at 1.0; the block scale is applied with a packed fp16 multiply, which is exact too:
// e2m1 * E4M3 needs at most 6 significant bits and lies in [2^-10, 2688], inside fp16's normal range.
template <int SEL>
__device__ __forceinline__ f16x2 fp4x2_to_f16(uint32_t src) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(src, 1.0f, SEL);
}

// Two E4M3FN bytes (bytes 2*HI, 2*HI+1 of src) -> fp16x2 (exact: every E4M3 value is an fp16 normal).
template <bool HI>
__device__ __forceinline__ f16x2 e4m3x2_to_f16(uint32_t src) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src, 1.0f, HI);
}

// E4M3FN byte `SEL` of `src` -> fp32 (exact).
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t src) {
  return __builtin_amdgcn_cvt_f32_fp8((int)src, SEL);
}

// Two E4M3FN bytes (bytes 2*HI, 2*HI+1 of src) -> bf16x2 (exact at scale 1.0).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t src) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 1.0f, HI));
}

// Two E4M3FN bytes (bytes 2*HI, 2*HI+1 of src) -> fp32 pair (exact).
template <bool HI>
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t src) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(src, 1.0f, HI);
}

// Exact value of a non-negative E4M3FN code c (0..126) as fp32, from the format's definition.
__device__ __forceinline__ float e4m3_code_value(int c) {
  int e = c >> 3, m = c & 7;
  float sub = (float)m * 0x1p-9f;
  float nrm = __uint_as_float((uint32_t)((e + 120) << 23) | ((uint32_t)m << 20));
  return e == 0 ? sub : nrm;
}

// Nearest E4M3FN byte to a finite fp32 value, ties to even, saturating at +-448.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  u &= 0x7FFFFFFFu;
  uint32_t code;
  if (u >= 0x43E00000u) {  // |x| >= 448
    code = 0x7E;
  } else if (u < 0x3C800000u) {  // |x| < 2^-6: multiples of 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(u) * 512.0f);
  } else {
    uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  }
  return sign | code;
}

// Nearest E4M3FN code (0..126) to amax / 6, ties to the even code, saturating at 448.  The code of the
// rounded quotient amax * (1/6) is at most one code away (its relative error is below 2^-23, and two
// exact quotients can only round to different codes across a midpoint); it is then corrected against
// the exact midpoints 6 * (v(k) + v(k+1)) / 2 = 3 * (v(k) + v(k+1)), which fp32 holds exactly.
__device__ __forceinline__ int e4m3_scale_code_div6(float amax) {
  auto rounds_up = [amax](int k) {  // amax / 6 lies past the midpoint between codes k and k+1
    const float thr = 3.0f * (e4m3_code_value(k) + e4m3_code_value(k + 1));
    return (amax > thr) || (amax == thr && ((k + 1) & 1) == 0);
  };
  int c = (int)(f32_to_e4m3(amax * (1.0f / 6.0f)) & 0x7Fu);
  if (c <= 125 && rounds_up(c)) ++c;
  else if (c >= 1 && !rounds_up(c - 1)) --c;
  return c;
}

// e2m1 magnitude code (0..7) of a / s, nearest grid point of {0,.5,1,1.5,2,3,4,6}, ties to the even
// code, saturating at 6.  Thresholds s * {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5} are exact in fp32.
__device__ __forceinline__ uint32_t e2m1_mag_code(float a, float s) {
  uint32_t c = 0;
  c += (a > 0.25f * s);
  c += (a >= 0.75f * s);
  c += (a > 1.25f * s);
  c += (a >= 1.75f * s);
  c += (a > 2.5f * s);
  c += (a >= 3.5f * s);
  c += (a > 5.0f * s);
  return c;
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 as_f16x8(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  u32x4 v = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
             __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(f16x8, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

// Max / sum over the four lanes l, l^16, l^32, l^48 (the four 16-lane groups), with the gfx950 lane
// swaps (VALU, no LDS round trip): swap(x, x) yields the pair {x[l], x[l^32]} (resp. x[l^16]).
// Largest of four floats (no NaN among the inputs: matrix-core results or -inf), as two v_max3_f32
// without the quieting steps the compiler adds to fmaxf on values it cannot prove canonical.
__device__ __forceinline__ float max4(float a, float b, float c, float d) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3\n\tv_max_f32 %0, %0, %4" : "=&v"(r) : "v"(a), "v"(b), "v"(c), "v"(d));
  return r;
}

__device__ __forceinline__ float group4_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Largest of the four values of lanes l, l^16, l^32, l^48 (unsigned), as group4_max.
__device__ __forceinline__ uint32_t group4_max_u32(uint32_t v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = r[0] > r[1] ? r[0] : r[1];
  auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return q[0] > q[1] ? q[0] : q[1];
}

// ---- exact power-of-two normalisation of one head's query for FP16 matrix operands.
// Every dequantized K / V value is exact in FP16, but FP16 spans only 2^-24 .. 65504 while a bf16 query
// spans 2^-133 .. 3.4e38.  Each head's query is scaled by 2^k, with k chosen from the head's largest
// magnitude so that this one lands in [2^15, 2^16): then no element overflows, every element within 2^29
// of the largest converts exactly, and smaller ones round with an absolute error below 2^-25 of the
// scaled largest, about 2^16 times below what the fp32 accumulation of the 576 products may already
// lose.  The score is scaled back by 2^-k together with the softmax scale (exact: a power of two), so
// a query and the same query times any power of two (with the softmax scale divided by it) give
// bit-identical results.

// Largest bf16 magnitude (bit pattern & 0x7FFF) among the 8 values of a 16-byte word.
__device__ __forceinline__ uint32_t bf16x8_max_mag(u32x4 raw) {
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = raw[k] & 0x7FFFu, hi = (raw[k] >> 16) & 0x7FFFu;
    m = m > lo ? m : lo;
    m = m > hi ? m : hi;
  }
  return m;
}

// The shift k for a head whose largest magnitude has bf16 bits m (0: an all-zero head, k = 0).  For a
// biased exponent e >= 1 the largest value lies in [2^(e-127), 2^(e-126)), so 2^(142-e) takes it to
// [2^15, 2^16) (at most 65280 < 65504); a subnormal largest value (e = 0) is below 2^-126 and takes
// k = 141.  k lies in [-112, 141].
__device__ __forceinline__ int q_shift(uint32_t m) {
  const int e = (int)(m >> 7);
  return m == 0 ? 0 : 142 - (e > 0 ? e : 1);
}

// bf16 bits (16 bits of `bits` at position SHIFT*16) times 2^k, as FP16 (v_ldexp_f32: exact unless the
// product leaves fp32's range, which |q| * 2^k < 2^16 rules out; then one rounding to FP16).
__device__ __forceinline__ _Float16 bf16_pow2_to_f16(uint32_t bits16, int k) {
  return (_Float16)__builtin_ldexpf(__uint_as_float(bits16 << 16), k);
}

// Two bf16 values of a dword (lo in .x) times 2^k, as FP16.
__device__ __forceinline__ f16x2 bf16x2_pow2_to_f16x2(uint32_t d, int k) {
  return f16x2{bf16_pow2_to_f16(d & 0xFFFFu, k), bf16_pow2_to_f16(d >> 16, k)};
}

// Workgroup barrier ordering LDS accesses only: this wave's LDS operations complete (lgkmcnt(0)),
// then s_barrier.  Vector-memory loads still in flight (the next tiles' row gathers into other LDS
// slots) are not waited for; the "memory" clobber keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until every vector memory load of this wave has landed (vmcnt(0)).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Map the hardware workgroup id to a logical id so that logically consecutive workgroups run on the
// same XCD (workgroups are dealt to the 8 XCDs round-robin; each XCD has its own L2).
__device__ __forceinline__ int xcd_logical_id(int hw, int n) {
  const int nx = 8;
  int q = n / nx, r = n % nx;
  int x = hw % nx, k = hw / nx;
  return x * q + (x < r ? x : r) + k;
}

// LDS-DMA of 16 bytes per lane: lane l's global bytes land at lds + 16*l (lds must be wave-uniform).
// Issued through asm so that the compiler's waitcnt tracking does not drain the gathers still in
// flight; completion is awaited explicitly with vmcnt.  M0 is saved and restored around the load.
// STREAM marks data read once (the cache rows): a non-temporal load, so that the stream does not push
// the data that is reused (queries, tables, split results, the kernel's code) out of the L2.
template <bool STREAM = false>
__device__ __forceinline__ void dma16(const void* src, const uint8_t* lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  uint32_t saved;
  if constexpr (STREAM) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(m)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(m)
        : "memory");
  }
}

template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((uint16_t)((N & 15) | ((N >> 4) << 14) | 0x0F70));
}

// Wait until at most k steps of this wave's gathers (NL loads each) are still in flight, 0 <= k <= 7
// (larger k waits as for 7; a count the 6-bit vmcnt cannot hold waits for as many steps as it can).
template <int NL, int K>
__device__ __forceinline__ void wait_steps_le() {
  constexpr int kMaxSteps = 63 / NL;
  wait_vmem_le<(K < kMaxSteps ? K : kMaxSteps) * NL>();
}
template <int NL>
__device__ __forceinline__ void wait_steps(int k) {
  switch (k <= 0 ? 0 : k) {
    case 0: wait_steps_le<NL, 0>(); break;
    case 1: wait_steps_le<NL, 1>(); break;
    case 2: wait_steps_le<NL, 2>(); break;
    case 3: wait_steps_le<NL, 3>(); break;
    case 4: wait_steps_le<NL, 4>(); break;
    case 5: wait_steps_le<NL, 5>(); break;
    case 6: wait_steps_le<NL, 6>(); break;
    default: wait_steps_le<NL, 7>(); break;
  }
}

// Byte interleave of two rows' nibble dwords: byte k of the result holds (lo nibble, hi nibble) =
// (row a, row b) of column 2k (ODD = 0) or 2k+1 (ODD = 1).
template <int ODD>
__device__ __forceinline__ uint32_t nib_pair(uint32_t ra, uint32_t rb) {
  constexpr uint32_t M = 0x0F0F0F0Fu;
  return ODD ? (((ra >> 4) & M) | (rb & ~M)) : ((ra & M) | ((rb << 4) & ~M));
}

// Agent-coherent relaxed accesses for the split results exchanged between workgroups.
// Four floats as FP16 (round to nearest even) packed in 8 bytes, stored with one agent-coherent store, and
// back to floats.  The merging workgroup rounds its own result the same way, so that a merge gives the
// same bits whichever split's workgroup performs it.
__device__ __forceinline__ uint64_t pack_h4(f32x4 v) {
  const f16x2 lo = {(_Float16)v[0], (_Float16)v[1]}, hi = {(_Float16)v[2], (_Float16)v[3]};
  return (uint64_t)__builtin_bit_cast(uint32_t, lo) | ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32);
}
__device__ __forceinline__ void store_coherent_h4(uint64_t* p, f32x4 v) {
  __hip_atomic_store(p, pack_h4(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 h4_to_f32x4(uint64_t x) {
  const f16x2 lo = __builtin_bit_cast(f16x2, (uint32_t)x), hi = __builtin_bit_cast(f16x2, (uint32_t)(x >> 32));
  return f32x4{(float)lo.x, (float)lo.y, (float)hi.x, (float)hi.y};
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Quantize-on-write of one token by one wavefront (row formats and rounding as in mla_quant.hip): lane l
// holds latent elements 8l..8l+7 (raw, the 16-byte load of the bf16 values) and rope element l
// (rope_bits, bf16).  quant_row_words computes the lane's dwords of the row in registers, store_row_words
// writes the 352- or 576-byte row at dst (88 or 144 coalesced dwords), so that a caller can quantize
// before it knows where the row goes.
struct RowWords {
  uint32_t lat0;  // NVFP4: the lane's 8 nibbles (bytes 4l..4l+3); FP8: codes of elements 8l..8l+3
  uint32_t lat1;  // NVFP4: scale bytes 4l..4l+3 (lanes 0-7); FP8: codes of elements 8l+4..8l+7
  uint32_t rope;  // rope codes 4l..4l+3 (lanes 0-15)
};

template <int FMT>
__device__ __forceinline__ RowWords quant_row_words(u32x4 raw, uint32_t rope_bits, int lane) {
  RowWords o;
  const uint32_t rope_code = f32_to_e4m3(bf16_to_f32(rope_bits));
  uint32_t h[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    h[2 * k] = raw[k] & 0xFFFFu;
    h[2 * k + 1] = raw[k] >> 16;
  }
  if constexpr (FMT == 0) {
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
    o.lat0 = nib;
    // scale bytes: block j lives in lanes 2j and 2j+1; dword q holds blocks 4q..4q+3
    const int src = 8 * (lane & 7);
    uint32_t s0 = __shfl(sc, src, 64), s1 = __shfl(sc, src + 2, 64);
    uint32_t s2 = __shfl(sc, src + 4, 64), s3 = __shfl(sc, src + 6, 64);
    o.lat1 = s0 | (s1 << 8) | (s2 << 16) | (s3 << 24);
  } else {
    uint32_t c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = f32_to_e4m3(bf16_to_f32(h[k]));
    o.lat0 = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    o.lat1 = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
  }
  // rope bytes: dword q holds rope values 4q..4q+3 (lanes 4q..4q+3)
  const int src = 4 * (lane & 15);
  uint32_t r0 = __shfl(rope_code, src, 64), r1 = __shfl(rope_code, src + 1, 64);
  uint32_t r2 = __shfl(rope_code, src + 2, 64), r3 = __shfl(rope_code, src + 3, 64);
  o.rope = r0 | (r1 << 8) | (r2 << 16) | (r3 << 24);
  return o;
}

template <int FMT>
__device__ __forceinline__ void store_row_words(const RowWords& o, uint8_t* dst, int lane) {
  if constexpr (FMT == 0) {
    *reinterpret_cast<uint32_t*>(dst + 4 * lane) = o.lat0;
    if (lane < 8) *reinterpret_cast<uint32_t*>(dst + 256 + 4 * lane) = o.lat1;
  } else {
    *reinterpret_cast<u32x2*>(dst + 8 * lane) = u32x2{o.lat0, o.lat1};
  }
  constexpr int kRopeOff = FMT == 0 ? 288 : 512;
  if (lane < 16) *reinterpret_cast<uint32_t*>(dst + kRopeOff + 4 * lane) = o.rope;
}

template <int FMT>
__device__ __forceinline__ void quant_row_wave(u32x4 raw, uint32_t rope_bits, uint8_t* dst, int lane) {
  store_row_words<FMT>(quant_row_words<FMT>(raw, rope_bits, lane), dst, lane);
}

}  // namespace mla
