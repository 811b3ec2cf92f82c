// Optional QK normalization and rotary positional transform, applied in place
// to each bounded Q slab and to the K rows of each pass-1 slab ("Proposal:
// Generic memory-aware streaming execution for transformer models", section
// "Attention requires a stronger contract": project one bounded Q region and
// apply the model's Q normalization/positional transform before attention).
//
// Per token row and head (dh = 64 or 128):
//   RMSNorm: t <- t / sqrt(mean(t^2) + eps) * w          (w: [dh] fp32)
//   RoPE:    (t[2j], t[2j+1]) <- (a c - b s, a s + b c)  (c, s: [row][dh/2] fp32)
// One wavefront per row. A lane holds 8 consecutive elements of a head, so a
// head spans dh/8 consecutive lanes: its mean square is reduced with dh/8-lane
// xor shuffles and every rotated pair lies inside one lane. Statistics and
// rotation are fp32; the result is rounded once to the storage type.
#include "common.hpp"
#include "kernels.hpp"

namespace dit {

template <typename T, int DH, int G>
__global__ __launch_bounds__(256) void qk_transform_kernel(T* __restrict__ x, int64_t ldx, int64_t rows, int d,
                                                           const float* __restrict__ w,
                                                           const float* __restrict__ cs,
                                                           const float* __restrict__ sn, int64_t ld_rope,
                                                           float eps) {
  constexpr int LPH = DH / 8;  // lanes per head
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int ngroups = d >> 3;
  const int hg = lane % LPH;  // this lane's 8-element group within its head
  T* xr = x + row * ldx;
  // Every load is issued before any store and none sits under a per-lane
  // branch: lanes past the row end re-read the last group (whole heads are
  // valid or invalid together, so the per-head sums never mix the two) and
  // store nothing. The norm weights and the angles depend only on the lane's
  // place in its head, so they are read once.
  float v[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int idx = g * 64 + lane < ngroups ? g * 64 + lane : ngroups - 1;
    if constexpr (sizeof(T) == 2) {
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
  f32x4 w0 = f32x4{1.f, 1.f, 1.f, 1.f}, w1 = w0, c = w0, sv = f32x4{0.f, 0.f, 0.f, 0.f};
  if (w) {
    w0 = *reinterpret_cast<const f32x4*>(w + hg * 8);
    w1 = *reinterpret_cast<const f32x4*>(w + hg * 8 + 4);
  }
  if (cs) {
    c = *reinterpret_cast<const f32x4*>(cs + row * ld_rope + hg * 4);
    sv = *reinterpret_cast<const f32x4*>(sn + row * ld_rope + hg * 4);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int idx = g * 64 + lane;
    if (w) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += v[g][j] * v[g][j];
#pragma unroll
      for (int off = 1; off < LPH; off <<= 1) ss += __shfl_xor(ss, off, 64);
      const float r = 1.0f / sqrtf(ss * (1.0f / DH) + eps);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[g][j] = v[g][j] * r * w0[j];
        v[g][4 + j] = v[g][4 + j] * r * w1[j];
      }
    }
    if (idx >= ngroups) continue;
    if (cs) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = v[g][2 * j], b = v[g][2 * j + 1];
        v[g][2 * j] = a * c[j] - b * sv[j];
        v[g][2 * j + 1] = a * sv[j] + b * c[j];
      }
    }
    if constexpr (sizeof(T) == 2) {
      u32x4 p;
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = pack_bf16x2(v[g][2 * j], v[g][2 * j + 1]);
      *reinterpret_cast<u32x4*>(xr + idx * 8) = p;
    } else {
      *reinterpret_cast<f32x4*>(xr + idx * 8) = f32x4{v[g][0], v[g][1], v[g][2], v[g][3]};
      *reinterpret_cast<f32x4*>(xr + idx * 8 + 4) = f32x4{v[g][4], v[g][5], v[g][6], v[g][7]};
    }
  }
}

template <typename T, int DH>
static hipError_t launch_qk_t(void* x, int64_t ldx, int64_t rows, int d, const float* w, const float* cs,
                              const float* sn, int64_t ld_rope, float eps, hipStream_t st) {
  const int g = (int)ceil_div(d / 8, 64);
  dim3 grid((unsigned)ceil_div(rows, 4)), block(256);
  T* xx = static_cast<T*>(x);
#define DIT_QK_CASE(G)                                                                                 \
  case G:                                                                                              \
    hipLaunchKernelGGL((qk_transform_kernel<T, DH, G>), grid, block, 0, st, xx, ldx, rows, d, w, cs, sn, \
                       ld_rope, eps);                                                                  \
    break;
  switch (g) {
    DIT_QK_CASE(1)
    DIT_QK_CASE(2)
    DIT_QK_CASE(3)
    DIT_QK_CASE(4)
    DIT_QK_CASE(5)
    DIT_QK_CASE(6)
    DIT_QK_CASE(7)
    DIT_QK_CASE(8)
    DIT_QK_CASE(9)
    DIT_QK_CASE(10)
    DIT_QK_CASE(11)
    DIT_QK_CASE(12)
    DIT_QK_CASE(13)
    DIT_QK_CASE(14)
    DIT_QK_CASE(15)
    DIT_QK_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef DIT_QK_CASE
  return hipGetLastError();
}

hipError_t launch_qk_transform(int f32, void* x, int64_t ldx, int64_t rows, int d, int head_dim, const float* w,
                               const float* cs, const float* sn, int64_t ld_rope, float eps, hipStream_t st) {
  if (rows <= 0 || (!w && !cs)) return hipSuccess;
  if (f32) {
    if (head_dim == 64) return launch_qk_t<float, 64>(x, ldx, rows, d, w, cs, sn, ld_rope, eps, st);
    if (head_dim == 128) return launch_qk_t<float, 128>(x, ldx, rows, d, w, cs, sn, ld_rope, eps, st);
  } else {
    if (head_dim == 64) return launch_qk_t<uint16_t, 64>(x, ldx, rows, d, w, cs, sn, ld_rope, eps, st);
    if (head_dim == 128) return launch_qk_t<uint16_t, 128>(x, ldx, rows, d, w, cs, sn, ld_rope, eps, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dit
