// Device side of the synthetic-input generator: fills large tensors (hash
// tables, hidden states, projection weights) with the same counter-based
// normal draws that synth/rng.py produces on the host, bit for bit.
//
//   draw(seed, i)  = SplitMix64 output for counter i + 1 (Steele, Lea, Flood,
//                    OOPSLA 2014; mixer constants as published by Vigna)
//   normal(i)      = float32(2 * (sum of the draw's four 16-bit lanes) - 262140)
//                    * scale, one IEEE multiply; bf16 storage rounds to
//                    nearest-even.
//
// This library is input generation only: it holds no part of the N-gram
// method and is not linked into the method's library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float irwin_hall_normal(uint64_t d, float scale) {
  uint32_t s = (uint32_t)(d & 0xFFFFull) + (uint32_t)((d >> 16) & 0xFFFFull) +
               (uint32_t)((d >> 32) & 0xFFFFull) + (uint32_t)(d >> 48);
  float centred = (float)((int32_t)(2u * s) - 262140);
  return __fmul_rn(centred, scale);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t b = __float_as_uint(x);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// 8 consecutive elements per thread per iteration (one 16-byte bf16 store or
// two 16-byte fp32 stores); a scalar tail handles n % 8.
__global__ void fill_normal_bf16(uint16_t* __restrict__ dst, int64_t n, uint64_t seed,
                                 int64_t offset, float scale) {
  const int64_t n8 = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n8; v += stride) {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint64_t i0 = (uint64_t)(offset + v * 8 + 2 * p);
      uint32_t lo = f32_to_bf16_rne(irwin_hall_normal(splitmix64_at(seed, i0), scale));
      uint32_t hi = f32_to_bf16_rne(irwin_hall_normal(splitmix64_at(seed, i0 + 1), scale));
      w[p] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(dst + v * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  for (int64_t i = n8 * 8 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = f32_to_bf16_rne(irwin_hall_normal(splitmix64_at(seed, (uint64_t)(offset + i)), scale));
}

__global__ void fill_normal_f32(float* __restrict__ dst, int64_t n, uint64_t seed,
                                int64_t offset, float scale) {
  const int64_t n4 = n / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n4; v += stride) {
    float4 o;
    uint64_t i0 = (uint64_t)(offset + v * 4);
    o.x = irwin_hall_normal(splitmix64_at(seed, i0 + 0), scale);
    o.y = irwin_hall_normal(splitmix64_at(seed, i0 + 1), scale);
    o.z = irwin_hall_normal(splitmix64_at(seed, i0 + 2), scale);
    o.w = irwin_hall_normal(splitmix64_at(seed, i0 + 3), scale);
    *reinterpret_cast<float4*>(dst + v * 4) = o;
  }
  for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = irwin_hall_normal(splitmix64_at(seed, (uint64_t)(offset + i)), scale);
}

// fp32 -> OCP FP8 E4M3 code, round to nearest, ties to even (finite inputs
// within +-448; larger magnitudes saturate to +-448).
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a < 0x1p-6f)  // subnormals: multiples of 2^-9 (a * 512 is exact)
    return sign | (uint32_t)rintf(a * 512.0f);  // 8 -> code 8 = 2^-6, the first normal
  const uint32_t ab = __float_as_uint(a);
  int e = (int)(ab >> 23) - 127;
  const uint32_t man = ab & 0x7FFFFFu;
  uint32_t keep = man >> 20;
  const uint32_t rest = man & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) {
    keep = 0;
    ++e;
  }
  if (e > 8 || (e == 8 && keep == 7u)) return sign | 0x7Eu;
  return sign | ((uint32_t)(e + 7) << 3) | keep;
}

// 16 consecutive codes per thread per iteration (one 16-byte store): code of
// normal(i) * inv_scale (one fp32 multiply after the normal's own).
__global__ void fill_normal_fp8(uint8_t* __restrict__ dst, int64_t n, uint64_t seed,
                                int64_t offset, float scale, float inv_scale) {
  const int64_t n16 = n / 16;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n16; v += stride) {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint64_t i = (uint64_t)(offset + v * 16 + 4 * p + b);
        const float x = __fmul_rn(irwin_hall_normal(splitmix64_at(seed, i), scale), inv_scale);
        word |= f32_to_e4m3_rne(x) << (8 * b);
      }
      w[p] = word;
    }
    *reinterpret_cast<uint4*>(dst + v * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  for (int64_t i = n16 * 16 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = (uint8_t)f32_to_e4m3_rne(
        __fmul_rn(irwin_hall_normal(splitmix64_at(seed, (uint64_t)(offset + i)), scale), inv_scale));
}

}  // namespace

// FP8 E4M3 codes of normal draws times inv_scale; dst 16-byte aligned.
extern "C" int synth_fill_normal_fp8(void* dst, int64_t n, uint64_t seed, int64_t offset,
                                     float scale, float inv_scale, void* stream) {
  if (n < 0 || (n > 0 && dst == nullptr) || (reinterpret_cast<uintptr_t>(dst) & 15u)) return -1;
  if (n == 0) return 0;
  const int threads = 256;
  int64_t blocks = (n / 16 + threads - 1) / threads;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  fill_normal_fp8<<<dim3((unsigned)blocks), dim3(threads), 0, reinterpret_cast<hipStream_t>(stream)>>>(
      static_cast<uint8_t*>(dst), n, seed, offset, scale, inv_scale);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// dtype: 0 = fp32, 1 = bf16.  dst must be 16-byte aligned.  Returns 0 on
// success, -1 on bad arguments, -2 when the launch fails.
extern "C" int synth_fill_normal(void* dst, int32_t dtype, int64_t n, uint64_t seed,
                                 int64_t offset, float scale, void* stream) {
  if (n < 0 || (n > 0 && dst == nullptr) || (reinterpret_cast<uintptr_t>(dst) & 15u)) return -1;
  if (n == 0) return 0;
  const int threads = 256;
  int64_t per = (dtype == 1) ? 8 : 4;
  int64_t blocks = (n / per + threads - 1) / threads;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == 1)
    fill_normal_bf16<<<dim3((unsigned)blocks), dim3(threads), 0, s>>>(
        static_cast<uint16_t*>(dst), n, seed, offset, scale);
  else if (dtype == 0)
    fill_normal_f32<<<dim3((unsigned)blocks), dim3(threads), 0, s>>>(
        static_cast<float*>(dst), n, seed, offset, scale);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
