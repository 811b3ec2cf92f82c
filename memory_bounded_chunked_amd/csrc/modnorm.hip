// K1: fused adaLN-modulated LayerNorm, one wavefront per token row.
//
//   out[r][c] = (x[r][c] - mean_r) / sqrt(var_r + eps) * (1 + scale[c]) + shift[c]
//
// The block's normalisation and modulation, applied per token ("LayerStream:
// H3 Chunking", section "How the slicing works"). Statistics are fp32 and
// two-pass (mean, then the mean of squared deviations) over values held in
// registers; the row is read from HBM once and written once. Loads are 16 B
// per lane in 8-element groups, so a wave reads 1 KiB (bf16) or 2 KiB (fp32)
// of one row per instruction, fully coalesced.
#include "common.hpp"
#include "kernels.hpp"

namespace dit {

template <typename Tin, typename Tout, int G>  // G = 8-element groups per lane (d <= 512*G)
__global__ __launch_bounds__(256) void modnorm_kernel(const Tin* __restrict__ x, int64_t ldx,
                                                      const float* __restrict__ shift,
                                                      const float* __restrict__ scale,
                                                      Tout* __restrict__ out, int64_t ldo,
                                                      int64_t rows, int d, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int ngroups = d >> 3;
  const Tin* xr = x + row * ldx;
  // Lanes whose group index passes the row end load the last group again
  // and leave it out of the sums and the stores: no load sits under a
  // branch, so all of them are in flight together (a load under a branch
  // makes the compiler wait for it, and for every store before it, at once).
  float v[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int idx = g * 64 + lane < ngroups ? g * 64 + lane : ngroups - 1;
    if constexpr (sizeof(Tin) == 2) {
      const u32x4 p = *reinterpret_cast<const u32x4*>(xr + idx * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[g][2 * j] = __uint_as_float(p[j] << 16);
        v[g][2 * j + 1] = __uint_as_float(p[j] & 0xffff0000u);
      }
    } else {
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(xr + idx * 8);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(xr + idx * 8 + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[g][j] = p0[j];
        v[g][4 + j] = p1[j];
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const bool ok = g * 64 + lane < ngroups;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += ok ? v[g][j] : 0.f;
  }
  const float inv_d = 1.0f / (float)d;
  const float mu = wave_sum(s) * inv_d;
  float s2 = 0.f;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const bool ok = g * 64 + lane < ngroups;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float t = v[g][j] - mu;
      s2 = ok ? __builtin_fmaf(t, t, s2) : s2;
    }
  }
  const float var = wave_sum(s2) * inv_d;
  const float rstd = 1.0f / sqrtf(var + eps);
  Tout* orow = out + row * ldo;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const bool ok = g * 64 + lane < ngroups;
    const int idx = ok ? g * 64 + lane : ngroups - 1;
    const f32x4 sc0 = *reinterpret_cast<const f32x4*>(scale + idx * 8);
    const f32x4 sc1 = *reinterpret_cast<const f32x4*>(scale + idx * 8 + 4);
    const f32x4 sh0 = *reinterpret_cast<const f32x4*>(shift + idx * 8);
    const f32x4 sh1 = *reinterpret_cast<const f32x4*>(shift + idx * 8 + 4);
    float o[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // n = ((x - mu) * rstd) * (1 + scale) + shift, the last step fused
      o[j] = __builtin_fmaf((v[g][j] - mu) * rstd, 1.0f + sc0[j], sh0[j]);
      o[4 + j] = __builtin_fmaf((v[g][4 + j] - mu) * rstd, 1.0f + sc1[j], sh1[j]);
    }
    if (!ok) continue;
    if constexpr (sizeof(Tout) == 2) {
      u32x4 p;
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = pack_bf16x2(o[2 * j], o[2 * j + 1]);
      *reinterpret_cast<u32x4*>(orow + idx * 8) = p;
    } else {
      *reinterpret_cast<f32x4*>(orow + idx * 8) = f32x4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<f32x4*>(orow + idx * 8 + 4) = f32x4{o[4], o[5], o[6], o[7]};
    }
  }
}

template <typename Tin, typename Tout>
static hipError_t launch_modnorm_t(const void* x, int64_t ldx, const float* shift, const float* scale,
                                   void* out, int64_t ldo, int64_t rows, int d, float eps,
                                   hipStream_t st) {
  const int groups_per_lane = (int)ceil_div(d / 8, 64);
  dim3 grid((unsigned)ceil_div(rows, 4)), block(256);
  const Tin* xi = static_cast<const Tin*>(x);
  Tout* oo = static_cast<Tout*>(out);
#define DIT_MODNORM_CASE(G)                                                                  \
  case G:                                                                                    \
    hipLaunchKernelGGL((modnorm_kernel<Tin, Tout, G>), grid, block, 0, st, xi, ldx, shift,  \
                       scale, oo, ldo, rows, d, eps);                                        \
    break;
  switch (groups_per_lane) {
    DIT_MODNORM_CASE(1)
    DIT_MODNORM_CASE(2)
    DIT_MODNORM_CASE(3)
    DIT_MODNORM_CASE(4)
    DIT_MODNORM_CASE(5)
    DIT_MODNORM_CASE(6)
    DIT_MODNORM_CASE(7)
    DIT_MODNORM_CASE(8)
    DIT_MODNORM_CASE(9)
    DIT_MODNORM_CASE(10)
    DIT_MODNORM_CASE(11)
    DIT_MODNORM_CASE(12)
    DIT_MODNORM_CASE(13)
    DIT_MODNORM_CASE(14)
    DIT_MODNORM_CASE(15)
    DIT_MODNORM_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef DIT_MODNORM_CASE
  return hipGetLastError();
}

hipError_t launch_modnorm(int in_f32, int out_f32, const void* x, int64_t ldx, const float* shift,
                          const float* scale, void* out, int64_t ldo, int64_t rows, int d, float eps,
                          hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (in_f32 && out_f32)
    return launch_modnorm_t<float, float>(x, ldx, shift, scale, out, ldo, rows, d, eps, st);
  if (in_f32)
    return launch_modnorm_t<float, uint16_t>(x, ldx, shift, scale, out, ldo, rows, d, eps, st);
  if (out_f32)
    return launch_modnorm_t<uint16_t, float>(x, ldx, shift, scale, out, ldo, rows, d, eps, st);
  return launch_modnorm_t<uint16_t, uint16_t>(x, ldx, shift, scale, out, ldo, rows, d, eps, st);
}

}  // namespace dit
