// MXFP8 activations for the FP4 x FP8 expert GEMMs: the DeepSeek-V4
// infrastructure walkthrough (section 6.2) feeds FP4 (E2M1) expert weights to
// an FP8 GEMM; how activations become FP8 is this library's reading of the OCP
// Microscaling (MX) format: E4M3 elements with one E8M0 scale per 32
// consecutive values along K.
//   X = floor(log2(amax)) - 8, byte X + 127 clamped to [0, 254] (amax = 0,
//   or no finite value: byte 0); element = E4M3 nearest to v / 2^X, ties to
//   the even code, magnitudes past 448 clamped to 448 (sign kept), NaN -> 0x7F.
// E4M3 is OCP FP8 E4M3: bias 7, subnormals m/8 * 2^-6, no infinities.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// v / 2^X of a bf16 value is exact in fp32 for every value that can round to
// a nonzero E4M3 code, so the rounding below is done on fp32 bits.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                    // NaN
  const float f = __uint_as_float(a);
  uint32_t code;
  if (f < 0.015625f) {                                  // below 2^-6: m/8 * 2^-6 = m * 2^-9
    code = (uint32_t)__builtin_rintf(f * 512.0f);       // 0..8 (8 is the smallest normal)
  } else {
    // round the 23-bit mantissa to 3 bits, ties to even; a carry moves into the exponent
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    const int e = (int)(r >> 23) - 127;                 // >= -6
    code = e > 8 ? 0x7fu : (uint32_t)(((e + 7) << 3) | ((r >> 20) & 7u));
  }
  return sign | (code > 0x7eu ? 0x7eu : code);          // saturate at 448
}

// One wave handles 16 blocks of 32 per pass: lane l covers 8 values
// (16 bytes) of block l / 4; the block's amax comes from its 4 lanes.
__global__ __launch_bounds__(256) void k_mx_e4m3_quantize(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ row_index,
                                                          int64_t R, int K,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int64_t nblk = R * (K / 32);
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 8-value group
  const int64_t blk = g / 4;
  const bool live = blk < nblk;
  const int64_t b = live ? blk : nblk - 1;
  const int64_t r = b / (K / 32);
  const int kb = (int)(b % (K / 32));
  const int64_t src = row_index ? (int64_t)row_index[r] : r;
  const uint4 q = *reinterpret_cast<const uint4*>(x + src * K + kb * 32 + (g % 4) * 8);
  float v[8];
  v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
  v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
  v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
  v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = fabsf(v[i]);
    if (a <= 3.402823466e38f && a > amax) amax = a;  // finite values only
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  int byte = 0;
  if (amax > 0.f) {
    int e;
    frexpf(amax, &e);  // amax = f * 2^e, f in [0.5, 1): floor(log2(amax)) = e - 1
    byte = min(254, max(0, e - 1 - 8 + 127));
  }
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = e4m3_code(ldexpf(v[i], 127 - byte));
  if (!live) return;
  const uint2 packed = make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                                  c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
  *reinterpret_cast<uint2*>(codes + r * K + kb * 32 + (g % 4) * 8) = packed;
  if (g % 4 == 0) scales[r * (K / 32) + kb] = (uint8_t)byte;
}

hipError_t launch_mx_e4m3_quantize(const void* x, const int32_t* row_index, int64_t R, int K,
                                   uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (R == 0) return hipSuccess;
  const int64_t groups = R * (K / 8);
  hipLaunchKernelGGL(k_mx_e4m3_quantize, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), row_index, R, K, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
