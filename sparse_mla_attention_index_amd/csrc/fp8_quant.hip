// Per-row FP8 quantisation (gfx950).
//
// Activations are quantised on the fly with one scale per vector of 128
// elements (DeepSeek multi-node page, "Quantification"); for the indexer a
// head's q_I row is such a vector, and a key row carries its 4-byte scale
// beside 128 FP8 values (GLM-5.3 part 2, footnote 3).  Per row:
//   scale = amax / 448, code = e4m3fn(clamp(x / scale, -448, 448)),
// both divisions correctly rounded in fp32, the convert rounding to nearest
// even (the hardware convert in the default round mode).  A row of zeros
// gets scale 0 and zero codes.
//
// The row is spread over D/8 lanes (one 16-byte load of eight bf16 each);
// the row's amax is a butterfly over those lanes.  HBM-bound: 2 bytes in,
// 1 + 4/D bytes out per element.
#include "sma_device.h"
#include "sma_launch.h"

namespace sma {

template <int D>
__global__ __launch_bounds__(256) void quant_fp8_rows_kernel(const uint16_t* __restrict__ x, int64_t n_rows,
                                                             uint8_t* __restrict__ codes,
                                                             float* __restrict__ scale) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPB = 256 / LPR;      // rows per workgroup
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int sub = tid % LPR;
  // a row's lanes are contiguous and aligned, so they leave together and the
  // butterfly below never reads a lane that has left
  if (row >= n_rows) return;
  const u32x4 v = *reinterpret_cast<const u32x4*>(x + row * D + 8 * sub);
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, LPR));
  const float s = __fdiv_rn(m, 448.f);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = s > 0.f ? fminf(fmaxf(__fdiv_rn(f[i], s), -448.f), 448.f) : 0.f;
  u32x2 out;
  out[0] = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  out[0] = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], out[0], true);
  out[1] = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  out[1] = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], out[1], true);
  *reinterpret_cast<u32x2*>(codes + row * D + 8 * sub) = out;
  if (sub == 0) scale[row] = s;
}

hipError_t launch_quantize_fp8_rows(const uint16_t* x, int64_t n_rows, int d, uint8_t* codes, float* scale,
                                    hipStream_t st) {
  if (n_rows <= 0) return hipSuccess;
  const int rpb = 256 / (d / 8);
  const int64_t grid = (n_rows + rpb - 1) / rpb;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  if (d == 128)
    hipLaunchKernelGGL(quant_fp8_rows_kernel<128>, dim3((unsigned)grid), dim3(256), 0, st, x, n_rows, codes, scale);
  else if (d == 64)
    hipLaunchKernelGGL(quant_fp8_rows_kernel<64>, dim3((unsigned)grid), dim3(256), 0, st, x, n_rows, codes, scale);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sma
