// Output head after the last block: adaLN-modulated LayerNorm of each token
// row followed by an fp32 projection to the output width, fused into one
// kernel so that the normalised rows never reach HBM ("LayerStream: H3
// Chunking", "How the slicing works": the fp32 output head; streaming
// proposal, section "Summary": the final projection/modulation is bounded like
// the block).
//
//   out[t][j] = sum_c (LN(x[t])[c] * (1 + scale[c]) + shift[c]) * w[j][c]
//
// A workgroup owns 32 token rows (one 32x32 MFMA row tile) and every output
// column (out_dim <= 128, i.e. up to 4 column tiles of 32).
//   phase 1  each wave computes mean and 1/sqrt(var + eps) of 8 rows, two-pass
//            over the row held in registers (fp32), into LDS;
//   phase 2  wave w contracts columns [w*d/4, (w+1)*d/4) of d: each lane loads
//            8 consecutive x values of its row and normalises/modulates them in
//            registers; those are the A operands of eight 32x32x2 fp32 MFMAs,
//            whose B operands are 8 consecutive values of one w row. A and B use
//            the same permutation of k inside a 16-column step, so the product
//            is the plain contraction;
//   reduce   the four waves' partial tiles go through LDS and are summed in the
//            fixed order w = 0, 1, 2, 3.
// The arithmetic of a row depends only on that row, d and out_dim: calling the
// kernel on any range of rows gives the same bits for those rows.
#include "common.hpp"
#include "kernels.hpp"

namespace dit {

constexpr int FL_BM = 32;    // token rows per workgroup
constexpr int FL_WAVES = 4;  // waves per workgroup; each owns a quarter of d

template <typename T>
__device__ __forceinline__ void load8(const T* p, float v[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(q[j] << 16);
      v[2 * j + 1] = __uint_as_float(q[j] & 0xffff0000u);
    }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
  }
}

__device__ __forceinline__ void load8f(const float* p, float v[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = a[j];
    v[4 + j] = b[j];
  }
}

// T: activation type of x (float or uint16_t = bf16). G: 8-column groups per
// lane in phase 1 (d <= 512 * G). NT: 32-column output tiles.
template <typename T, int G, int NT>
__global__ __launch_bounds__(256) void final_layer_kernel(const T* __restrict__ x, int64_t ldx, int64_t n, int d,
                                                          const float* __restrict__ shift,
                                                          const float* __restrict__ scale,
                                                          const float* __restrict__ w, int out_dim,
                                                          float* __restrict__ out, int64_t ldo, float eps) {
  constexpr int TW = NT * 32;  // padded tile width
  __shared__ float s_mu[FL_BM], s_rs[FL_BM];
  __shared__ float s_part[FL_WAVES][FL_BM][TW];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * FL_BM;

  // Phase 1: row statistics, 8 rows per wave.
  {
    const int ngroups = d >> 3;
    const float inv_d = 1.0f / (float)d;
    for (int rr = 0; rr < FL_BM / FL_WAVES; ++rr) {
      const int r = wave * (FL_BM / FL_WAVES) + rr;
      const int64_t row = m0 + r;
      if (row >= n) break;  // uniform across the wave
      const T* xr = x + row * ldx;
      float v[G][8];
      float s = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int idx = g * 64 + lane;
        if (idx < ngroups) {
          load8(xr + idx * 8, v[g]);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[g][j] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) s += v[g][j];
      }
      const float mu = wave_sum(s) * inv_d;
      float s2 = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (g * 64 + lane < ngroups) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float t = v[g][j] - mu;
            s2 += t * t;
          }
        }
      }
      const float var = wave_sum(s2) * inv_d;
      if (lane == 0) {
        s_mu[r] = mu;
        s_rs[r] = 1.0f / sqrtf(var + eps);
      }
    }
  }
  __syncthreads();

  // Phase 2: this wave's quarter of the contraction.
  const int lr = lane & 31, half = lane >> 5;
  const int64_t row = m0 + lr < n ? m0 + lr : n - 1;  // clamped rows are computed and discarded
  const float mu = m0 + lr < n ? s_mu[lr] : 0.f;
  const float rs = m0 + lr < n ? s_rs[lr] : 0.f;
  const T* xr = x + row * ldx;
  const float* wr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int j = t * 32 + lr;
    wr[t] = w + (int64_t)(j < out_dim ? j : out_dim - 1) * d;  // padded columns are discarded
  }
  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};

  const int kq = d / FL_WAVES;
  const int kbeg = wave * kq, kend = kbeg + kq;
  float xa[8], xb[8], wa[NT][8], wb[NT][8];
  auto fetch = [&](int k0, float xv[8], float wv[NT][8]) {
    const int kk = k0 + 8 * half;
    load8(xr + kk, xv);
#pragma unroll
    for (int t = 0; t < NT; ++t) load8f(wr[t] + kk, wv[t]);
  };
  auto compute = [&](int k0, const float xv[8], const float wv[NT][8]) {
    const int kk = k0 + 8 * half;
    float sc[8], sh[8];
    load8f(scale + kk, sc);
    load8f(shift + kk, sh);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a = (xv[i] - mu) * rs * (1.0f + sc[i]) + sh[i];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = mfma32_f32(a, wv[t][i], acc[t]);
    }
  };
  // kq is a multiple of 16; steps alternate between two register sets so the
  // next step's loads are in flight during this step's MFMAs.
  int k0 = kbeg;
  fetch(k0, xa, wa);
  for (; k0 + 32 <= kend; k0 += 32) {
    fetch(k0 + 16, xb, wb);
    compute(k0, xa, wa);
    if (k0 + 32 < kend) fetch(k0 + 32, xa, wa);
    compute(k0 + 16, xb, wb);
  }
  if (k0 < kend) compute(k0, xa, wa);

  // Cross-wave reduction in a fixed order.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s_part[wave][8 * (r / 4) + 4 * half + (r % 4)][t * 32 + lr] = acc[t][r];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < FL_BM * TW; e += 256) {
    const int r = e / TW, c = e % TW;
    if (m0 + r < n && c < out_dim) {
      const float v = ((s_part[0][r][c] + s_part[1][r][c]) + s_part[2][r][c]) + s_part[3][r][c];
      out[(m0 + r) * ldo + c] = v;
    }
  }
}

template <typename T, int NT>
static hipError_t launch_fl_nt(const void* x, int64_t ldx, int64_t n, int d, const float* shift, const float* scale,
                               const float* w, int out_dim, float* out, int64_t ldo, float eps, hipStream_t st) {
  const int g = (int)ceil_div(d / 8, 64);
  const dim3 grid((unsigned)ceil_div(n, FL_BM)), block(256);
  const T* xx = static_cast<const T*>(x);
#define DIT_FL_CASE(G)                                                                                     \
  case G:                                                                                                  \
    hipLaunchKernelGGL((final_layer_kernel<T, G, NT>), grid, block, 0, st, xx, ldx, n, d, shift, scale, w, \
                       out_dim, out, ldo, eps);                                                            \
    break;
  switch (g) {
    DIT_FL_CASE(1)
    DIT_FL_CASE(2)
    DIT_FL_CASE(3)
    DIT_FL_CASE(4)
    DIT_FL_CASE(5)
    DIT_FL_CASE(6)
    DIT_FL_CASE(7)
    DIT_FL_CASE(8)
    DIT_FL_CASE(9)
    DIT_FL_CASE(10)
    DIT_FL_CASE(11)
    DIT_FL_CASE(12)
    DIT_FL_CASE(13)
    DIT_FL_CASE(14)
    DIT_FL_CASE(15)
    DIT_FL_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef DIT_FL_CASE
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_fl_t(const void* x, int64_t ldx, int64_t n, int d, const float* shift, const float* scale,
                              const float* w, int out_dim, float* out, int64_t ldo, float eps, hipStream_t st) {
  switch ((out_dim + 31) / 32) {
    case 1: return launch_fl_nt<T, 1>(x, ldx, n, d, shift, scale, w, out_dim, out, ldo, eps, st);
    case 2: return launch_fl_nt<T, 2>(x, ldx, n, d, shift, scale, w, out_dim, out, ldo, eps, st);
    case 3: return launch_fl_nt<T, 3>(x, ldx, n, d, shift, scale, w, out_dim, out, ldo, eps, st);
    case 4: return launch_fl_nt<T, 4>(x, ldx, n, d, shift, scale, w, out_dim, out, ldo, eps, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_final_layer(int x_f32, const void* x, int64_t ldx, int64_t n, int d, const float* shift,
                              const float* scale, const float* w, int out_dim, float* out, int64_t ldo, float eps,
                              hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (d < 64 || d % 64 || d > 8192 || out_dim < 1 || out_dim > 128) return hipErrorInvalidValue;
  return x_f32 ? launch_fl_t<float>(x, ldx, n, d, shift, scale, w, out_dim, out, ldo, eps, st)
               : launch_fl_t<uint16_t>(x, ldx, n, d, shift, scale, w, out_dim, out, ldo, eps, st);
}

}  // namespace dit
