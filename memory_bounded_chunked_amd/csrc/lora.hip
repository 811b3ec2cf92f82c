// Adapter inputs of activation-space LoRA: t = alpha * (A a) for a slab of
// token rows ("ComfyUI-StaticPipeline", "Activation-space LoRA (bypass
// mode)": the low-rank product runs on the activations, in token chunks).
//
// t is [rows][rank] with rank <= 256 while the contracted length is d or the
// FFN width, so a plain output-tiled GEMM has only rows/256 workgroups. Here a
// workgroup owns 32 token rows and every rank column. The contraction runs
// in chunks of CK = 16*NW: the workgroup stages a chunk of its activation rows
// and of the adapter rows through LDS (double buffered; every load instruction
// covers whole 128-byte lines), and wavefront w multiplies k-step w of each
// chunk (32x32x16 bf16 MFMAs). The NW per-wave sums are added in a fixed order
// through LDS. Which k a wave sums depends only on the length and the rank, so
// a row's t depends only on that row: the same bits whatever the slab size or
// offset.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace dit {

template <int NT>  // NT = 32-column tiles of the rank
struct LoraT {
  static constexpr int NW = NT <= 4 ? 8 : 4;   // wavefronts = k-steps per chunk
  static constexpr int NTHR = NW * 64;
  static constexpr int CK = 16 * NW;           // k per chunk
  static constexpr int ROW = CK * 2 + 16;      // LDS row stride (bytes): 16-B reads of 32 rows are conflict-free
  static constexpr int A_BYTES = 32 * ROW, W_BYTES = 32 * NT * ROW;
  static constexpr int STAGE = A_BYTES + W_BYTES;
  static constexpr int PART = (NW - 1) * NT * 64 * 64;  // per-wave sums, f32x16 per lane
  static constexpr int LDS = 2 * STAGE > PART ? 2 * STAGE : PART;
  static_assert(32 * CK / 8 == NTHR, "one 16-byte activation chunk per thread");
};

template <int NT>
__global__ __launch_bounds__(LoraT<NT>::NTHR) void lora_t_kernel(const uint16_t* __restrict__ a, int64_t lda,
                                                                const uint16_t* __restrict__ w, int64_t ldw,
                                                                int64_t m, int64_t k, int64_t rank, float alpha,
                                                                int accumulate, float* __restrict__ t, int64_t ldt) {
  using L = LoraT<NT>;
  constexpr int NW = L::NW, NTHR = L::NTHR, CK = L::CK, ROW = L::ROW, STAGE = L::STAGE;
  constexpr int CPR = CK / 8;  // 16-byte chunks per staged row
  __shared__ __attribute__((aligned(16))) char smem[L::LDS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * 32;
  const int64_t n_chunks = ceil_div(k, (int64_t)CK);

  // global side: thread tid moves chunk (tid % CPR) of activation row tid / CPR
  // and of adapter rows tid / CPR + i * (NTHR / CPR)
  const int crow = tid / CPR, cch = tid % CPR;
  const bool a_ok = m0 + crow < m;
  const uint16_t* a_src = a + (a_ok ? m0 + crow : 0) * lda + cch * 8;
  const uint16_t* w_src[NT];
  bool w_ok[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int64_t n = crow + i * (NTHR / CPR);
    w_ok[i] = n < rank;
    w_src[i] = w + (w_ok[i] ? n : 0) * ldw + cch * 8;
  }
  u32x4 ra, rw[NT];
  const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
  auto load = [&](int64_t c) {
    const int64_t k0 = c * CK;
    const bool k_ok = k0 + cch * 8 < k;
    ra = (a_ok && k_ok) ? *reinterpret_cast<const u32x4*>(a_src + k0) : zero;
#pragma unroll
    for (int i = 0; i < NT; ++i) rw[i] = (w_ok[i] && k_ok) ? *reinterpret_cast<const u32x4*>(w_src[i] + k0) : zero;
  };
  auto store = [&](int buf) {
    char* st = smem + buf * STAGE;
    *reinterpret_cast<u32x4*>(st + crow * ROW + cch * 16) = ra;
#pragma unroll
    for (int i = 0; i < NT; ++i)
      *reinterpret_cast<u32x4*>(st + L::A_BYTES + (crow + i * (NTHR / CPR)) * ROW + cch * 16) = rw[i];
  };

  f32x16 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x16{};
  // wave w: k-step w of each chunk; lane operands A[l32][16w + 8*half ..], W[n][same k]
  const int frag = l32 * ROW + (16 * wave + 8 * half) * 2;
  auto compute = [&](int64_t c, int buf) {
    if (c * CK + 16 * wave >= k) return;  // uniform per wave: past the end of a short last chunk
    const char* st = smem + buf * STAGE;
    const u32x4 af = *reinterpret_cast<const u32x4*>(st + frag);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const u32x4 bf = *reinterpret_cast<const u32x4*>(st + L::A_BYTES + nt * 32 * ROW + frag);
      acc[nt] = mfma32_bf16(__builtin_bit_cast(bf16x8, af), __builtin_bit_cast(bf16x8, bf), acc[nt]);
    }
  };

  // chunk c is multiplied from LDS buffer c % 2 while chunk c+1 goes from the
  // staging registers into the other buffer and chunk c+2 is loaded
  load(0);
  store(0);
  if (n_chunks > 1) load(1);
  __syncthreads();
  for (int64_t c = 0; c < n_chunks; ++c) {
    compute(c, (int)(c & 1));
    if (c + 1 < n_chunks) {
      store((int)((c + 1) & 1));
      if (c + 2 < n_chunks) load(c + 2);
    }
    __syncthreads();
  }

  // per-wave sums 1..NW-1 through LDS (the staging area is free after the
  // last barrier); wave 0 adds them in order and writes t
  f32x16* part = reinterpret_cast<f32x16*>(smem);
  if (wave > 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) part[((wave - 1) * NT + nt) * 64 + lane] = acc[nt];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    f32x16 sum = acc[nt];
#pragma unroll
    for (int q = 0; q < NW - 1; ++q) {
      const f32x16 p = part[(q * NT + nt) * 64 + lane];
#pragma unroll
      for (int r = 0; r < 16; ++r) sum[r] += p[r];
    }
    const int64_t n = nt * 32 + l32;
    if (n >= rank) continue;
    // the 16 previous values are read together, before any store, from
    // clamped rows (no load under a branch), and used only when accumulating
    float prev[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t mr = m0 + 8 * (r >> 2) + 4 * half + (r & 3);
      prev[r] = t[(mr < m ? mr : m - 1) * ldt + n];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t mr = m0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (mr >= m) continue;
      t[mr * ldt + n] = (accumulate ? prev[r] : 0.f) + alpha * sum[r];
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
    hipLaunchKernelGGL((lora_t_kernel<NT>), grid, dim3(LoraT<NT>::NTHR), 0, st, ab, lda, wb, ldw, m, k, rank,
                       alpha, accumulate, t, ldt);
  };
  if (nt <= 1) go(std::integral_constant<int, 1>{});
  else if (nt <= 2) go(std::integral_constant<int, 2>{});
  else if (nt <= 4) go(std::integral_constant<int, 4>{});
  else go(std::integral_constant<int, 8>{});
  return hipGetLastError();
}

}  // namespace dit
