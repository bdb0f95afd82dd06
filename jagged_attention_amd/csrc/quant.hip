// MXFP8 quantiser: bf16 -> E4M3 codes with one E8M0 scale per 32 consecutive elements.
//
// Source for the use: "Meta Enhances GEM Training Efficiency with Advanced LLM-Scale
// Innovations", section "Leveraging Compute Efficiency through Customized Kernels" (MXFP8
// attention), and "Meta GEM Training Efficiency ...", section "Bottleneck move 2" (scale-factor
// generation and casting must not eat the low-precision gain).  The format is the public OCP
// Microscaling (MX) v1.0 one: shared exponent e = floor(log2 amax) - 8 (8 = largest E4M3
// exponent), clamped to [-127, 127] and stored as e + 127; elements x * 2^-e rounded to the
// nearest E4M3 value, ties to even, saturating at 448; an all-zero block stores 127.
//
// Four lanes own one 32-element block (16 bytes each): a two-step shuffle gives the block max,
// every lane scales its 8 elements by 2^-e, encodes them with the hardware's pack conversion
// and stores 8 code bytes.
#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa {
namespace {

// floor(log2(a)) for a finite a > 0 (normal or subnormal float).
__device__ __forceinline__ int ilog2f(float a) {
  const uint32_t u = __float_as_uint(a);
  const int ef = (int)(u >> 23);
  if (ef > 0) return ef - 127;
  return (31 - __clz(u & 0x7fffffu)) - 149;
}

// E4M3 codes of two scaled values y0, y1 (|y| < 512 by the choice of e): clamped to +-448
// (saturation), then gfx950's pack conversion to OCP E4M3 with round-to-nearest-even, subnormals
// included.  The clamp makes every value in [448, 512) encode as 448 (0x7E / 0xFE).  Returns the
// two codes in bits [16 W, 16 W + 16) of `old`.
template <bool W>
__device__ __forceinline__ int e4m3_pair(float y0, float y1, int old) {
  y0 = fminf(fmaxf(y0, -448.0f), 448.0f);
  y1 = fminf(fmaxf(y1, -448.0f), 448.0f);
  return __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, old, W);
}

__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const __bf16* __restrict__ x,
                                                          int64_t nblocks, uint8_t* codes,
                                                          uint8_t* scales) {
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = tid >> 2;
  const int sub = (int)(tid & 3);
  const bool ok = blk < nblocks;
  u32x4 raw = {0, 0, 0, 0};
  if (ok) raw = *(const u32x4*)(x + blk * 32 + sub * 8);
  float v[8];
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(raw[e] << 16);
    v[2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
    amax = fmaxf(amax, fmaxf(fabsf(v[2 * e]), fabsf(v[2 * e + 1])));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  if (!ok) return;
  uint32_t sc = 127;
  u32x2 out = {0, 0};
  if (amax > 0.f) {
    int e = ilog2f(amax) - 8;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    sc = (uint32_t)(e + 127);
    // x * 2^-e is exact (a power-of-two scaling of a bf16 value within the float range)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int word = e4m3_pair<false>(ldexpf(v[4 * h], -e), ldexpf(v[4 * h + 1], -e), 0);
      word = e4m3_pair<true>(ldexpf(v[4 * h + 2], -e), ldexpf(v[4 * h + 3], -e), word);
      out[h] = (uint32_t)word;
    }
  }
  *(u32x2*)(codes + blk * 32 + sub * 8) = out;
  if (sub == 0) scales[blk] = (uint8_t)sc;
}

}  // namespace

hipError_t launch_quantize_mxfp8(const void* x, int64_t rows, int32_t d, uint8_t* codes,
                                 uint8_t* scales, hipStream_t s) {
  const int64_t nblocks = rows * (d / 32);
  if (nblocks == 0) return hipSuccess;
  const int64_t threads = nblocks * 4;
  timing_begin("jfa_quant_mxfp8", s);
  hipLaunchKernelGGL(quant_mxfp8_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     (const __bf16*)x, nblocks, codes, scales);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace jfa
