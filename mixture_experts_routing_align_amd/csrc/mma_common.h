// Matrix-core building blocks shared by the gfx950 projection kernels.
//
// One v_mfma_f32_16x16x32_bf16 multiplies a 16x32 A tile by a 32x16 B tile.
// Lane l feeds A row l%16 and B column l%16 with 8 consecutive k of quad l/16,
// and receives the 4 results D[4*(l/16) + i][l%16], i = 0..3.  FP8 e4m3 weight
// codes become bf16 exactly in registers (v_cvt_scalef32_pk_bf16_fp8 with
// scale 1), and so do MXFP4 codes with their power-of-two block scale
// (v_cvt_scalef32_pk_bf16_fp4), so a weight's only rounding is the float32
// accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace mma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kKC = 128;        // depth of one chunk (= one FP8 scale block)
constexpr int kPad = 8;         // bf16 elements of padding per staged LDS row (16 B)
constexpr int kWaveCols = 16;   // output columns per wave: one MFMA tile edge

__host__ __device__ constexpr int round_up(int v, int m) { return (v + m - 1) / m * m; }

__device__ __forceinline__ uint16_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// float32 -> bf16 bits, round to nearest even; a NaN stays a quiet NaN (the
// layer's output rounding)
__device__ __forceinline__ uint32_t bf16_rne_out(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// float32 multiply and add that the compiler may not fuse with a neighbouring
// operation into a fused multiply-add (HIP contracts across statements unless a
// pragma says otherwise).  Wherever two kernels must give the same bits for one
// value, its arithmetic goes through these.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ float add_rn(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}

// silu(g) * u = g / (1 + exp(-g)) * u, the product rounded on its own: the
// value is the same float32 whether it is stored or split into bf16 hi + lo in
// registers.
__device__ __forceinline__ float silu_mul(float g, float u) { return mul_rn(g / (1.0f + expf(-g)), u); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// 8 FP8 e4m3 codes (two dwords, lowest byte first) -> 8 bf16, exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t d0, uint32_t d1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// The E8M0 scale byte at bit `pos` of `w` as a float32 scale: the bits
// e << 23, which are 2^(e - 127) exactly for bytes 1..254 (byte 0 gives 0 and
// byte 255, E8M0's NaN, gives infinity; the library specifies bytes 2..252).
// Two instructions: a bit-field extract and a shift.
__device__ __forceinline__ float e8m0_at(uint32_t w, int pos) {
  return __uint_as_float(__builtin_amdgcn_ubfe(w, pos, 8) << 23);
}

// 8 E2M1 codes (one dword, lowest nibble first) times `scale` -> 8 bf16
// (v_cvt_scalef32_pk_bf16_fp4: each byte's two codes, scaled).  With a
// power-of-two scale the products are exact in bf16 for every scale the
// weights carry (their exponents stay far inside bf16's range).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t d, float scale) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 0);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 1);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 2);
  const bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 3);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Element offset, inside a 128-deep chunk, of the 8 consecutive k a lane of
// quad q feeds to MFMA step s.  The A and B operands use the same map, so the
// k order inside one MFMA is a permutation the product does not see.
//  Byte-coded weights (FP8, MXFP4): steps 2h and 2h + 1 take the lane's 16
//  consecutive k 64h + 16q .. +15 (16 FP8 codes = one 16-byte load; 16 E2M1
//  codes = 8 bytes, all in one 32-deep E8M0 block), so each 64-deep half of
//  the chunk is steps 2h and 2h + 1 alone.
//  BF16: one 16-byte load holds 8 elements = one step.
template <bool BYTES>
__device__ __forceinline__ int k_of_step(int s, int q) {
  return BYTES ? ((s >> 1) * 64 + q * 16 + (s & 1) * 8) : (s * 32 + q * 8);
}

// Gate of the shared expert for one token, sigmoid(x . g), computed by the
// first 256 threads of the workgroup (every thread gets it): thread j sums
// h = j, j + 256, ... with float32 fused multiply-adds in ascending h, and the
// 256 partial sums meet in a fixed tree through `red` (256 floats of LDS).
// Every blend kernel calls it, so a token's gate has the same bits on every
// path.  Contains barriers: every thread of the workgroup (at least 256) calls it.
__device__ inline float shared_gate256(const uint16_t* __restrict__ x, const uint16_t* __restrict__ g, int H,
                                       float* red) {
  const int j = threadIdx.x;
  if (j < 256) {
    float s = 0.f;
    for (int h = j; h < H; h += 256) s = fmaf(bf16_bits_to_f32(x[h]), bf16_bits_to_f32(g[h]), s);
    red[j] = s;
  }
  __syncthreads();
  for (int d = 128; d > 0; d >>= 1) {
    if (j < d) red[j] = add_rn(red[j], red[j + d]);
    __syncthreads();
  }
  const float dot = red[0];
  __syncthreads();  // red is free again
  return 1.f / (1.f + expf(-dot));
}

}  // namespace mma
}  // namespace moe
