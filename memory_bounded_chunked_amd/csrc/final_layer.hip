// Output head after the last block: adaLN-modulated LayerNorm of each token
// row followed by an fp32 projection to the output width, fused into one
// kernel so that the normalised rows never reach HBM ("LayerStream: H3
// Chunking", "How the slicing works": the fp32 output head; streaming
// proposal, section "Summary": the final projection/modulation is bounded like
// the block).
//
//   out[t][j] = sum_c (LN(x[t])[c] * (1 + scale[c]) + shift[c]) * w[j][c]
//
// One pass over x. LayerNorm is linear in the row once its statistics are
// known, so with a per-row shift p (the mean of the row's first 8 values),
// u = x - p, g = 1 + scale:
//
//   out[t][j] = r * (S[j] - (mu - p) * C[j]) + B[j],
//   S[j] = sum_c u[c] g[c] w[j][c],  C[j] = sum_c g[c] w[j][c],  B[j] = sum_c shift[c] w[j][c],
//   mu - p = sum_c u[c] / d,  var = sum_c u[c]^2 / d - (mu - p)^2,  r = 1/sqrt(var + eps).
//
// The shift keeps the moments and S - (mu - p) C free of cancellation (p is
// within a few standard deviations of the mean), and x is read from HBM once
// instead of once for the statistics and again for the contraction.
//
// A workgroup owns 64 token rows (two 32x32 MFMA row tiles, which share every
// weight fragment) and every output column (out_dim <= 128, i.e. up to 4
// column tiles of 32). Wave w contracts columns [w*d/4, (w+1)*d/4) of d: each
// lane loads 8 consecutive x values of its row, forms u g in registers (the A
// operands of eight 32x32x2 fp32 MFMAs, whose B operands are 8 consecutive
// values of one w row; A and B use the same permutation of k inside a
// 16-column step, so the product is the plain contraction) and accumulates the
// row's moments of u; the lanes that hold a w row accumulate C and B for it.
// The four waves' partial tiles, moments and C/B are summed through LDS in the
// fixed order (w0 + w1) + (w2 + w3), and the epilogue applies the formula.
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

template <typename T, int NT>
struct FlStep {
  Raw8<T> xv[FL_BM / 32];
  float wv[NT][8];
  float sc[8], sh[8];
};

// T: activation type of x (float or uint16_t = bf16). NT: 32-column output tiles.
template <typename T, int NT>
__global__ __launch_bounds__(256) void final_layer_kernel(const T* __restrict__ x, int64_t ldx, int64_t n, int d,
                                                          const float* __restrict__ shift,
                                                          const float* __restrict__ scale,
                                                          const float* __restrict__ w, int out_dim,
                                                          float* __restrict__ out, int64_t ldo, float eps) {
  constexpr int TW = NT * 32;  // padded tile width
  constexpr int MT = FL_BM / 32;
  __shared__ float s_red[2][FL_BM][TW];
  __shared__ float s_mom[FL_WAVES][FL_BM][2];  // per-wave sums of u and u^2 per row
  __shared__ float s_cb[FL_WAVES][TW][2];      // per-wave partial C and B per column
  __shared__ float s_dl[FL_BM], s_rs[FL_BM];   // mu - p and 1/sqrt(var + eps) per row
  __shared__ float s_c[TW], s_b[TW];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, half = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * FL_BM;

  const T* xr[MT];
  float p[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t row = m0 + m * 32 + lr < n ? m0 + m * 32 + lr : n - 1;  // clamped rows are computed and discarded
    xr[m] = x + row * ldx;
    const Raw8<T> head = load_raw8(xr[m]);
    float s8 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s8 += raw_at(head, i);
    p[m] = s8 * 0.125f;
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
  float s1[MT], s2[MT], cs[NT], bs[NT];
#pragma unroll
  for (int m = 0; m < MT; ++m) s1[m] = s2[m] = 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t) cs[t] = bs[t] = 0.f;

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
      for (int t = 0; t < NT; ++t) {
        cs[t] = fmaf(g, s.wv[t][i], cs[t]);
        bs[t] = fmaf(s.sh[i], s.wv[t][i], bs[t]);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float u = raw_at(s.xv[m], i) - p[m];
        s1[m] += u;
        s2[m] = fmaf(u, u, s2[m]);
        const float a = u * g;
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

  // Lanes l and l^32 hold the two halves of each 16-column step: combine them.
  auto pair_sum = [](float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const float a1 = pair_sum(s1[m]), a2 = pair_sum(s2[m]);
    if (half == 0) {
      s_mom[wave][m * 32 + lr][0] = a1;
      s_mom[wave][m * 32 + lr][1] = a2;
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float c = pair_sum(cs[t]), b = pair_sum(bs[t]);
    if (half == 0) {
      s_cb[wave][t * 32 + lr][0] = c;
      s_cb[wave][t * 32 + lr][1] = b;
    }
  }

  // Cross-wave sums in the fixed order (w0 + w1) + (w2 + w3).
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
  if (wave & 1) {
    put(wave >> 1, true);
  } else if (wave == 0) {  // row statistics, one row per lane
    const float inv_d = 1.0f / (float)d;
    const float u1 = (s_mom[0][lane][0] + s_mom[1][lane][0]) + (s_mom[2][lane][0] + s_mom[3][lane][0]);
    const float u2 = (s_mom[0][lane][1] + s_mom[1][lane][1]) + (s_mom[2][lane][1] + s_mom[3][lane][1]);
    const float dl = u1 * inv_d;
    const float var = fmaxf(u2 * inv_d - dl * dl, 0.0f);
    s_dl[lane] = dl;
    s_rs[lane] = 1.0f / sqrtf(var + eps);
  } else {  // wave 2: C and B per column
    for (int c = lane; c < TW; c += 64) {
      s_c[c] = (s_cb[0][c][0] + s_cb[1][c][0]) + (s_cb[2][c][0] + s_cb[3][c][0]);
      s_b[c] = (s_cb[0][c][1] + s_cb[1][c][1]) + (s_cb[2][c][1] + s_cb[3][c][1]);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < FL_BM * TW; e += 256) {
    const int r = e / TW, c = e % TW;
    if (m0 + r < n && c < out_dim)
      out[(m0 + r) * ldo + c] = s_rs[r] * ((s_red[0][r][c] + s_red[1][r][c]) - s_dl[r] * s_c[c]) + s_b[c];
  }
}

template <typename T, int NT>
static hipError_t launch_fl_nt(const void* x, int64_t ldx, int64_t n, int d, const float* shift, const float* scale,
                               const float* w, int out_dim, float* out, int64_t ldo, float eps, hipStream_t st) {
  const dim3 grid((unsigned)ceil_div(n, FL_BM)), block(256);
  hipLaunchKernelGGL((final_layer_kernel<T, NT>), grid, block, 0, st, static_cast<const T*>(x), ldx, n, d, shift,
                     scale, w, out_dim, out, ldo, eps);
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
