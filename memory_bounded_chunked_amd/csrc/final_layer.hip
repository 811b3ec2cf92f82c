// Output head after the last block: adaLN-modulated LayerNorm of each token
// row followed by an fp32 projection to the output width, fused into one
// kernel so that the normalised rows never reach HBM ("LayerStream: H3
// Chunking", "How the slicing works": the fp32 output head; streaming
// proposal, section "Summary": the final projection/modulation is bounded like
// the block).
//
//   out[t][j] = sum_c (LN(x[t])[c] * (1 + scale[c]) + shift[c]) * w[j][c]
//
// A workgroup owns 64 token rows (two 32x32 MFMA row tiles, which share every
// weight fragment) and every output column (out_dim <= 128, i.e. up to 4
// column tiles of 32).
//   phase 1  each wave computes mean and 1/sqrt(var + eps) of 16 rows, two-pass
//            over rows held in registers as stored (fp32 statistics), into LDS;
//   phase 2  wave w contracts columns [w*d/4, (w+1)*d/4) of d: each lane loads
//            8 consecutive x values of its row and normalises/modulates them in
//            registers; those are the A operands of eight 32x32x2 fp32 MFMAs,
//            whose B operands are 8 consecutive values of one w row. A and B use
//            the same permutation of k inside a 16-column step, so the product
//            is the plain contraction;
//   reduce   the four waves' partial tiles are summed through LDS in the fixed
//            order (w0 + w1) + (w2 + w3).
// A 64-row tile (640 KB at d = 5120) does not stay on chip between the
// statistics pass and the contraction, so x is fetched twice.
// The arithmetic of a row depends only on that row, d and out_dim: calling the
// kernel on any range of rows gives the same bits for those rows.
#include "common.hpp"
#include "kernels.hpp"

namespace dit {

constexpr int FL_BM = 64;    // token rows per workgroup: two 32-row MFMA tiles
constexpr int FL_WAVES = 4;  // waves per workgroup; each owns a quarter of d

// Eight consecutive values of a row, as stored: bf16 packed in pairs (one
// u32x4) or fp32 (two u32x4).
template <typename T>
struct Raw8 {
  u32x4 v[sizeof(T) / 2];
};

template <typename T>
__device__ __forceinline__ Raw8<T> load_raw8(const T* p) {
  Raw8<T> r;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i) r.v[i] = reinterpret_cast<const u32x4*>(p)[i];
  return r;
}

template <typename T>
__device__ __forceinline__ float raw_at(const Raw8<T>& r, int j) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w = r.v[0][j >> 1];
    return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
  } else {
    return __uint_as_float(r.v[j >> 2][j & 3]);
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

// Mean and 1/sqrt(var + eps) of R rows (two-pass over registers); lane 0
// writes them to mu_out[q], rs_out[q].
template <typename T, int G, int R>
__device__ __forceinline__ void row_stats(const T* __restrict__ x, int64_t ldx, const int64_t (&rows)[R],
                                          int ngroups, float inv_d, float eps, int lane, float* mu_out,
                                          float* rs_out) {
  Raw8<T> v[R][G];
#pragma unroll
  for (int q = 0; q < R; ++q) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int idx = g * 64 + lane;
      if (idx < ngroups) v[q][g] = load_raw8(x + rows[q] * ldx + idx * 8);
    }
  }
#pragma unroll
  for (int q = 0; q < R; ++q) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (g * 64 + lane < ngroups) {
#pragma unroll
        for (int j = 0; j < 8; ++j) s += raw_at(v[q][g], j);
      }
    const float mu = wave_sum(s) * inv_d;
    float s2 = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (g * 64 + lane < ngroups) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float t = raw_at(v[q][g], j) - mu;
          s2 += t * t;
        }
      }
    const float var = wave_sum(s2) * inv_d;
    if (lane == 0) {
      mu_out[q] = mu;
      rs_out[q] = 1.0f / sqrtf(var + eps);
    }
  }
}

template <typename T, int NT>
struct FlStep {
  Raw8<T> xv[FL_BM / 32];
  float wv[NT][8];
  float sc[8], sh[8];
};

// T: activation type of x (float or uint16_t = bf16). G: 8-column groups per
// lane in phase 1 (d <= 512 * G). NT: 32-column output tiles.
template <typename T, int G, int NT>
__global__ __launch_bounds__(256) void final_layer_kernel(const T* __restrict__ x, int64_t ldx, int64_t n, int d,
                                                          const float* __restrict__ shift,
                                                          const float* __restrict__ scale,
                                                          const float* __restrict__ w, int out_dim,
                                                          float* __restrict__ out, int64_t ldo, float eps) {
  constexpr int TW = NT * 32;  // padded tile width
  constexpr int MT = FL_BM / 32;
  __shared__ float s_mu[FL_BM], s_rs[FL_BM];
  __shared__ float s_red[2][FL_BM][TW];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * FL_BM;

  // Phase 1: row statistics, FL_BM / 4 rows per wave, R rows in flight.
  {
    constexpr int R = (sizeof(T) == 2 && G <= 12) ? 2 : 1;
    constexpr int PER_WAVE = FL_BM / FL_WAVES;
    const int ngroups = d >> 3;
    const float inv_d = 1.0f / (float)d;
    for (int rr = 0; rr < PER_WAVE; rr += R) {
      const int r = wave * PER_WAVE + rr;
      int64_t rows[R];
#pragma unroll
      for (int q = 0; q < R; ++q) rows[q] = m0 + r + q < n ? m0 + r + q : n - 1;  // clamped rows unused
      row_stats<T, G, R>(x, ldx, rows, ngroups, inv_d, eps, lane, s_mu + r, s_rs + r);
    }
  }
  __syncthreads();

  // Phase 2: this wave's quarter of the contraction for all MT row tiles.
  const int lr = lane & 31, half = lane >> 5;
  const T* xr[MT];
  float mu[MT], rs[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int r = m * 32 + lr;
    const int64_t row = m0 + r < n ? m0 + r : n - 1;  // clamped rows are computed and discarded
    xr[m] = x + row * ldx;
    mu[m] = s_mu[r];
    rs[m] = s_rs[r];
  }
  const float* wr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int j = t * 32 + lr;
    wr[t] = w + (int64_t)(j < out_dim ? j : out_dim - 1) * d;  // padded columns are discarded
  }
  f32x16 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][t] = f32x16{};

  auto fetch = [&](int k0, FlStep<T, NT>& s) {
    const int kk = k0 + 8 * half;
#pragma unroll
    for (int m = 0; m < MT; ++m) s.xv[m] = load_raw8(xr[m] + kk);
#pragma unroll
    for (int t = 0; t < NT; ++t) load8f(wr[t] + kk, s.wv[t]);
    load8f(scale + kk, s.sc);
    load8f(shift + kk, s.sh);
  };
  auto compute = [&](const FlStep<T, NT>& s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float g = 1.0f + s.sc[i];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float a = (raw_at(s.xv[m], i) - mu[m]) * rs[m] * g + s.sh[i];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[m][t] = mfma32_f32(a, s.wv[t][i], acc[m][t]);
      }
    }
  };
  // The quarter is a multiple of 16 columns; steps alternate between two
  // register sets so the next step's loads are in flight during this step's MFMAs.
  const int kq = d / FL_WAVES;
  const int kbeg = wave * kq, kend = kbeg + kq;
  FlStep<T, NT> sa, sb;
  int k0 = kbeg;
  fetch(k0, sa);
  for (; k0 + 32 <= kend; k0 += 32) {
    fetch(k0 + 16, sb);
    compute(sa);
    if (k0 + 32 < kend) fetch(k0 + 32, sa);
    compute(sb);
  }
  if (k0 < kend) compute(sa);

  // Cross-wave reduction in the fixed order (w0 + w1) + (w2 + w3).
  auto put = [&](int buf, bool add) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float& dst = s_red[buf][m * 32 + 8 * (r / 4) + 4 * half + (r % 4)][t * 32 + lr];
          dst = add ? dst + acc[m][t][r] : acc[m][t][r];
        }
  };
  if ((wave & 1) == 0) put(wave >> 1, false);
  __syncthreads();
  if (wave & 1) put(wave >> 1, true);
  __syncthreads();
  for (int e = threadIdx.x; e < FL_BM * TW; e += 256) {
    const int r = e / TW, c = e % TW;
    if (m0 + r < n && c < out_dim) out[(m0 + r) * ldo + c] = s_red[0][r][c] + s_red[1][r][c];
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
