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
#include <algorithm>

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

// Thread tid's quarter (8 elements) of block tid / 4; the block's four lanes are consecutive.
__device__ __forceinline__ void quant_block(const __bf16* __restrict__ x, int64_t nblocks,
                                            uint8_t* codes, uint8_t* scales, int64_t tid) {
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

__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const __bf16* __restrict__ x,
                                                          int64_t nblocks, uint8_t* codes,
                                                          uint8_t* scales) {
  quant_block(x, nblocks, codes, scales, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

// Up to four tensors in one launch: blockIdx.y picks the tensor, and each thread takes one
// quarter-block exactly as quant_mxfp8_kernel does.
constexpr int QB_MAX = 4;
struct QuantBatch {
  const __bf16* x[QB_MAX];
  uint8_t* codes[QB_MAX];
  uint8_t* scales[QB_MAX];
  int64_t nblocks[QB_MAX];
};

__global__ __launch_bounds__(256) void quant_mxfp8_batch_kernel(QuantBatch b) {
  const int t = blockIdx.y;
  if ((int64_t)blockIdx.x * 64 >= b.nblocks[t]) return;    // this tensor ends before the block
  quant_block(b.x[t], b.nblocks[t], b.codes[t], b.scales[t],
              (int64_t)blockIdx.x * 256 + threadIdx.x);
}

// RMS normalisation fused with the MXFP8 quantiser: quantisation folded into the normalisation
// that produces the attention inputs ("Meta GEM Training Efficiency: ...", section "Bottleneck
// move 2": activation quantisation fused into the upstream normalisation, so that scale
// generation and casting add no pass over memory).  Each group of n = 8 LPG consecutive elements
// (a head's d values, or a token's H d) becomes y = x / sqrt(mean(x^2) + eps) * w, and y is
// quantised as above.  LPG lanes own a group (8 elements each); the sum of squares is a fixed
// in-lane order then an xor butterfly, which gives every lane the same fp32 value.
template <int LPG>
__global__ __launch_bounds__(256) void rmsnorm_quant_mxfp8_kernel(
    const __bf16* __restrict__ x, const float* __restrict__ w, float eps, int64_t groups,
    uint8_t* codes, uint8_t* scales) {
  constexpr int N = 8 * LPG;
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t grp = tid / LPG;
  const int sub = (int)(tid % LPG);
  const bool ok = grp < groups;
  u32x4 raw = {0, 0, 0, 0};
  if (ok) raw = *(const u32x4*)(x + grp * N + sub * 8);
  // this lane's 8 gains, issued with the data load (two 16-byte loads; w is 16-byte aligned)
  u32x4 wa = {0x3f800000u, 0x3f800000u, 0x3f800000u, 0x3f800000u}, wb = wa;
  if (w) {
    wa = *(const u32x4*)(w + sub * 8);
    wb = *(const u32x4*)(w + sub * 8 + 4);
  }
  float v[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(raw[e] << 16);
    v[2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
#pragma unroll
  for (int off = 1; off < LPG; off <<= 1) ss += __shfl_xor(ss, off);
  const float rstd = 1.0f / sqrtf(ss * (1.0f / N) + eps);
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float we = __uint_as_float(e < 4 ? wa[e & 3] : wb[e & 3]);
    v[e] = v[e] * rstd * we;
    amax = fmaxf(amax, fabsf(v[e]));
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
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int word = e4m3_pair<false>(ldexpf(v[4 * h], -e), ldexpf(v[4 * h + 1], -e), 0);
      word = e4m3_pair<true>(ldexpf(v[4 * h + 2], -e), ldexpf(v[4 * h + 3], -e), word);
      out[h] = (uint32_t)word;
    }
  }
  const int64_t el = grp * N + sub * 8;
  *(u32x2*)(codes + el) = out;
  if ((sub & 3) == 0) scales[el / 32] = (uint8_t)sc;
}

}  // namespace

hipError_t launch_rmsnorm_quantize_mxfp8(const void* x, const float* w, int64_t groups, int32_t n,
                                         float eps, uint8_t* codes, uint8_t* scales,
                                         hipStream_t s) {
  if (groups == 0) return hipSuccess;
  const int64_t threads = groups * (n / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  timing_begin("jfa_norm_quant_mxfp8", s);
  switch (n) {
    case 32: hipLaunchKernelGGL(rmsnorm_quant_mxfp8_kernel<4>, grid, dim3(256), 0, s, (const __bf16*)x, w, eps, groups, codes, scales); break;
    case 64: hipLaunchKernelGGL(rmsnorm_quant_mxfp8_kernel<8>, grid, dim3(256), 0, s, (const __bf16*)x, w, eps, groups, codes, scales); break;
    case 128: hipLaunchKernelGGL(rmsnorm_quant_mxfp8_kernel<16>, grid, dim3(256), 0, s, (const __bf16*)x, w, eps, groups, codes, scales); break;
    case 256: hipLaunchKernelGGL(rmsnorm_quant_mxfp8_kernel<32>, grid, dim3(256), 0, s, (const __bf16*)x, w, eps, groups, codes, scales); break;
    case 512: hipLaunchKernelGGL(rmsnorm_quant_mxfp8_kernel<64>, grid, dim3(256), 0, s, (const __bf16*)x, w, eps, groups, codes, scales); break;
    default: timing_end(s); return hipErrorInvalidValue;
  }
  timing_end(s);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp8_batch(int32_t count, const void* const* xs,
                                       const int64_t* rows, int32_t d, uint8_t* const* codes,
                                       uint8_t* const* scales, int cu_count, hipStream_t s) {
  if (count < 1 || count > QB_MAX) return hipErrorInvalidValue;
  QuantBatch b{};
  int64_t most = 0;
  for (int t = 0; t < count; ++t) {
    b.x[t] = (const __bf16*)xs[t];
    b.codes[t] = codes[t];
    b.scales[t] = scales[t];
    b.nblocks[t] = rows[t] * (d / 32);
    most = std::max(most, b.nblocks[t]);
  }
  if (most == 0) return hipSuccess;
  (void)cu_count;
  const int64_t need = (most * 4 + 255) / 256;        // one thread per quarter-block
  timing_begin("jfa_quant_mxfp8", s);
  hipLaunchKernelGGL(quant_mxfp8_batch_kernel, dim3((unsigned)need, (unsigned)count), dim3(256),
                     0, s, b);
  timing_end(s);
  return hipGetLastError();
}

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
