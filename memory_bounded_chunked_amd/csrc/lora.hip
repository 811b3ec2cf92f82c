// Adapter inputs of activation-space LoRA: t = alpha * (A a) for a slab of
// token rows ("ComfyUI-StaticPipeline", "Activation-space LoRA (bypass
// mode)": the low-rank product runs on the activations, in token chunks).
//
// t is [rows][rank] with rank <= 256 while the contracted length is d or the
// FFN width, so a plain output-tiled GEMM has only rows/256 workgroups. Here a
// workgroup owns 32 token rows and all rank columns, and its NW wavefronts
// split the contraction into NW contiguous parts (the boundaries depend on the
// length and the rank alone; NW waves with PF k-steps of loads in flight each
// keep enough bytes moving to stream the activation rows). Each wave
// multiplies its part with 32x32x16 bf16 MFMAs, operands loaded straight from
// global memory (both are read once per workgroup: the activation rows are
// the workgroup's own, the adapter rows are shared by every workgroup and stay
// in L2). The parts are added in a fixed order through LDS, so a row's t
// depends only on that row: the same bits whatever the slab size or offset.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace dit {

template <int NT>
struct LoraT {
  static constexpr int NW = NT <= 4 ? 8 : 4;                  // wavefronts (parts of k)
  static constexpr int PF = NT <= 2 ? 8 : (NT <= 4 ? 4 : 2);  // k-steps in flight per wave
};

// NT = 32-column tiles of the rank.
template <int NT>
__global__ __launch_bounds__(LoraT<NT>::NW * 64) void lora_t_kernel(const uint16_t* __restrict__ a, int64_t lda,
                                                     const uint16_t* __restrict__ w, int64_t ldw, int64_t m,
                                                     int64_t k, int64_t rank, float alpha, int accumulate,
                                                     float* __restrict__ t, int64_t ldt) {
  constexpr int NW = LoraT<NT>::NW, PF = LoraT<NT>::PF;
  __shared__ f32x16 part[NW - 1][NT][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * 32;
  const int64_t row = m0 + l32;
  const bool a_ok = row < m;
  const int64_t steps = k / 16;
  const int64_t s_begin = steps * wave / NW, s_end = steps * (wave + 1) / NW;

  // lane operands: A[row][16s + 8*half ..] and W[n][16s + 8*half ..]
  const uint16_t* ap = a + (a_ok ? row : 0) * lda + 8 * half;
  const uint16_t* wp[NT];
  bool w_ok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t n = nt * 32 + l32;
    w_ok[nt] = n < rank;
    wp[nt] = w + (w_ok[nt] ? n : 0) * ldw + 8 * half;
  }

  f32x16 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x16{};
  u32x4 af[PF], bf[PF][NT];
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
  auto load = [&](int64_t s, int slot) {
    af[slot] = a_ok ? *reinterpret_cast<const u32x4*>(ap + s * 16) : zero;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bf[slot][nt] = w_ok[nt] ? *reinterpret_cast<const u32x4*>(wp[nt] + s * 16) : zero;
  };
#pragma unroll
  for (int i = 0; i < PF; ++i)
    if (s_begin + i < s_end) load(s_begin + i, i);
  for (int64_t s = s_begin; s < s_end; s += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (s + i < s_end) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt] = mfma32_bf16(__builtin_bit_cast(bf16x8, af[i]), __builtin_bit_cast(bf16x8, bf[i][nt]), acc[nt]);
        if (s + i + PF < s_end) load(s + i + PF, i);
      }
    }
  }

  // parts 1..NW-1 through LDS; wave 0 adds them in order and writes t
  if (wave > 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) part[wave - 1][nt][lane] = acc[nt];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    f32x16 sum = acc[nt];
#pragma unroll
    for (int q = 0; q < NW - 1; ++q) {
      const f32x16 p = part[q][nt][lane];
#pragma unroll
      for (int r = 0; r < 16; ++r) sum[r] += p[r];
    }
    const int64_t n = nt * 32 + l32;
    if (n >= rank) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t mr = m0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (mr >= m) continue;
      float* o = t + mr * ldt + n;
      *o = (accumulate ? *o : 0.f) + alpha * sum[r];
    }
  }
}

hipError_t launch_lora_t(const void* a, int64_t lda, const void* w, int64_t ldw, int64_t m, int64_t k, int64_t rank,
                         float alpha, int accumulate, float* t, int64_t ldt, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  if (k < 16 || k % 16 || rank < 1 || rank > 256 || lda % 8 || ldw % 8 || lda < k || ldw < k || ldt < rank)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)ceil_div(m, 32));
  const auto* ab = static_cast<const uint16_t*>(a);
  const auto* wb = static_cast<const uint16_t*>(w);
  const int nt = (int)ceil_div(rank, 32);
  auto go = [&](auto nt_c) {
    constexpr int NT = decltype(nt_c)::value;
    hipLaunchKernelGGL((lora_t_kernel<NT>), grid, dim3(LoraT<NT>::NW * 64), 0, st, ab, lda, wb, ldw, m, k, rank,
                       alpha, accumulate, t, ldt);
  };
  if (nt <= 1) go(std::integral_constant<int, 1>{});
  else if (nt <= 2) go(std::integral_constant<int, 2>{});
  else if (nt <= 4) go(std::integral_constant<int, 4>{});
  else go(std::integral_constant<int, 8>{});
  return hipGetLastError();
}

}  // namespace dit
