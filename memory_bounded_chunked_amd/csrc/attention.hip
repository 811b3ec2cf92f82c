// K3: softmax attention of a bounded query slice against the global K/V.
//
// Pass 2 of the two-pass scheme ("LayerStream: H3 Chunking", section "How
// the slicing works": attend the slice against the full K/V; the streaming
// proposal's "Attention requires a stronger contract": retain global K/V,
// consume bounded Q, produce output in Q-sized slabs). The kernel never holds
// anything that grows with the key count: K/V tiles stream through LDS and
// the softmax is taken online in fp32.
//
// Work split: one workgroup = 4 wavefronts = 128 query rows of one head; each
// wave owns 32 queries. Per 64-key tile a wave computes S^T = K Q^T (keys
// along the MFMA M dimension, queries along N), so each lane owns one query
// column and a query's row max / row sum need one cross-lane exchange with
// lane^32. P^T is then already laid out as the B operand of O^T += V^T P^T.
// V is stored transposed in HBM ([d][keys]), so both MFMA operands are
// read from LDS as 16-byte, key-contiguous fragments.
//
// Per query the sequence of operations (KV tile size, tile order, MFMA shape)
// is fixed and does not depend on which slice the query belongs to, so O is
// bit-identical for every choice of query slicing.
#include "common.hpp"
#include "kernels.hpp"

namespace dit {

constexpr int ATT_BM = 128;  // queries per workgroup
constexpr int ATT_BN = 64;   // keys per tile

__device__ __forceinline__ int swz(int row, int chunk, int row_bytes) {
  return row * row_bytes + ((chunk ^ (row & 7)) << 4);
}

template <typename T, int DH>
__global__ __launch_bounds__(256, 2) void attention_kernel(const T* __restrict__ q, int64_t ldq,
                                                           const T* __restrict__ k, int64_t ldk,
                                                           const T* __restrict__ vt, int64_t ldvt,
                                                           T* __restrict__ o, int64_t ldo,
                                                           int64_t n_q, int64_t n_kv, float qk_scale_log2) {
  constexpr bool F32 = sizeof(T) == 4;
  constexpr int EPC = 16 / sizeof(T);          // elements per 16-B chunk
  constexpr int KRB = DH * sizeof(T);          // K tile row bytes
  constexpr int VRB = ATT_BN * sizeof(T);      // V^T tile row bytes
  constexpr int KCH = KRB / 16, VCH = VRB / 16;
  constexpr int K_TILE = ATT_BN * KRB, V_TILE = DH * VRB;
  constexpr int STAGE = K_TILE + V_TILE;
  constexpr int K_LD = ATT_BN * KCH / 256, V_LD = DH * VCH / 256;
  constexpr int QS = DH / (2 * EPC);           // k-steps over dh (2 lane halves x one chunk)
  constexpr int OT = DH / 32;                  // O^T tiles along dh
  static_assert(K_LD >= 1 && V_LD >= 1, "tile");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.y;
  const int64_t q0 = (int64_t)blockIdx.x * ATT_BM + wave * 32;
  const int64_t col0 = (int64_t)head * DH;

  // Q^T fragments (B operand): lane holds query q0+l32, dh chunk 2s+half.
  u32x4 qf[QS];
  {
    const int64_t qr = q0 + l32;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      if (qr < n_q)
        qf[s] = *reinterpret_cast<const u32x4*>(q + qr * ldq + col0 + (2 * s + half) * EPC);
      else
        qf[s] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  u32x4 rk[K_LD], rv[V_LD];
  auto load_kv = [&](int64_t kv0) {
#pragma unroll
    for (int i = 0; i < K_LD; ++i) {
      const int c = tid + i * 256;
      const int r = c / KCH, ch = c % KCH;
      const int64_t key = kv0 + r;
      rk[i] = (key < n_kv) ? *reinterpret_cast<const u32x4*>(k + key * ldk + col0 + ch * EPC)
                           : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      const int c = tid + i * 256;
      const int r = c / VCH, ch = c % VCH;
      const int64_t key = kv0 + ch * EPC;
      const T* src = vt + (col0 + r) * ldvt + key;
      if (key + EPC <= n_kv) {
        rv[i] = *reinterpret_cast<const u32x4*>(src);
      } else {
        T tmp[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) tmp[e] = (key + e < n_kv) ? src[e] : T(0);
        rv[i] = __builtin_bit_cast(u32x4, tmp);
      }
    }
  };
  auto store_kv = [&](int buf) {
    char* Ks = smem + buf * STAGE;
    char* Vs = Ks + K_TILE;
#pragma unroll
    for (int i = 0; i < K_LD; ++i) {
      const int c = tid + i * 256;
      *reinterpret_cast<u32x4*>(Ks + swz(c / KCH, c % KCH, KRB)) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      const int c = tid + i * 256;
      const int r = c / VCH, ch = c % VCH;
      if constexpr (F32) {
        *reinterpret_cast<u32x4*>(Vs + swz(r, ch, VRB)) = rv[i];
      } else {
        // keys 16j..16j+15 of a row: slot 2j holds keys {0-3, 8-11}, slot 2j+1
        // holds {4-7, 12-15}, the order in which P^T sits in the S^T registers.
        const int j = ch >> 1, hi = ch & 1;
        *reinterpret_cast<u32x2*>(Vs + swz(r, 2 * j, VRB) + 8 * hi) = u32x2{rv[i][0], rv[i][1]};
        *reinterpret_cast<u32x2*>(Vs + swz(r, 2 * j + 1, VRB) + 8 * hi) = u32x2{rv[i][2], rv[i][3]};
      }
    }
  };

  f32x16 acc_o[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t) acc_o[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  auto compute = [&](int buf, int64_t kv0) {
    const char* Ks = smem + buf * STAGE;
    const char* Vs = Ks + K_TILE;
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int st = 0; st < QS; ++st) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(Ks + swz(mt * 32 + l32, 2 * st + half, KRB));
        if constexpr (F32) {
#pragma unroll
          for (int t = 0; t < 4; ++t) s[mt] = mfma32_f32(__uint_as_float(a[t]), __uint_as_float(qf[st][t]), s[mt]);
        } else {
          s[mt] = mfma32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[st]), s[mt]);
        }
      }
    }
    if (kv0 + ATT_BN > n_kv) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kv0 + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= n_kv) s[mt][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * qk_scale_log2);
    m_run = m_new;
    const float mc = m_new * qk_scale_log2;
    float lsum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[mt][r] * qk_scale_log2 - mc);
        s[mt][r] = p;
        lsum += p;
      }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int t = 0; t < OT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[t][r] *= alpha;

    if constexpr (F32) {
      // B operand of each 32x32x2 MFMA: this lane's own score register r
      // (key 8*(r/4) + 4*half + r%4 of the 32-key tile).
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
#pragma unroll
          for (int t = 0; t < OT; ++t) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(Vs + swz(t * 32 + l32, 8 * mt + 2 * qd + half, VRB));
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc_o[t] = mfma32_f32(__uint_as_float(a[e]), s[mt][4 * qd + e], acc_o[t]);
          }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& sv = s[j >> 1];
        const int r0 = 8 * (j & 1);
        const u32x4 pb = u32x4{pack_bf16x2(sv[r0 + 0], sv[r0 + 1]), pack_bf16x2(sv[r0 + 2], sv[r0 + 3]),
                               pack_bf16x2(sv[r0 + 4], sv[r0 + 5]), pack_bf16x2(sv[r0 + 6], sv[r0 + 7])};
#pragma unroll
        for (int t = 0; t < OT; ++t) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(Vs + swz(t * 32 + l32, 2 * j + half, VRB));
          acc_o[t] = mfma32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pb), acc_o[t]);
        }
      }
    }
  };

  const int64_t n_tiles = ceil_div(n_kv, ATT_BN);
  load_kv(0);
  store_kv(0);
  __syncthreads();
  for (int64_t t = 0; t < n_tiles; ++t) {
    const int cur = (int)(t & 1);
    if (t + 1 < n_tiles) load_kv((t + 1) * ATT_BN);
    compute(cur, t * ATT_BN);
    if (t + 1 < n_tiles) store_kv(cur ^ 1);
    __syncthreads();
  }

  const float l_all = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_all;
  const int64_t qr = q0 + l32;
  if (qr < n_q) {
    T* orow = o + qr * ldo + col0;
#pragma unroll
    for (int t = 0; t < OT; ++t)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int c = t * 32 + 8 * qd + 4 * half;
        const float v0 = acc_o[t][4 * qd] * inv, v1 = acc_o[t][4 * qd + 1] * inv;
        const float v2 = acc_o[t][4 * qd + 2] * inv, v3 = acc_o[t][4 * qd + 3] * inv;
        if constexpr (F32) {
          *reinterpret_cast<f32x4*>(orow + c) = f32x4{v0, v1, v2, v3};
        } else {
          *reinterpret_cast<u32x2*>(orow + c) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        }
      }
  }
}

template <typename T, int DH>
static hipError_t launch_att_t(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* vt,
                               int64_t ldvt, void* o, int64_t ldo, int64_t n_q, int64_t n_kv, int n_heads,
                               hipStream_t st) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)DH);
  dim3 grid((unsigned)ceil_div(n_q, ATT_BM), (unsigned)n_heads), block(256);
  hipLaunchKernelGGL((attention_kernel<T, DH>), grid, block, 0, st, static_cast<const T*>(q), ldq,
                     static_cast<const T*>(k), ldk, static_cast<const T*>(vt), ldvt, static_cast<T*>(o), ldo,
                     n_q, n_kv, scale_log2);
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const void* q, int64_t ldq, const void* k, int64_t ldk,
                            const void* vt, int64_t ldvt, void* o, int64_t ldo, int64_t n_q,
                            int64_t n_kv, int n_heads, int head_dim, hipStream_t st) {
  if (n_q <= 0) return hipSuccess;
  if (n_kv <= 0) return hipErrorInvalidValue;
  if (dtype == F32) {
    if (head_dim == 64) return launch_att_t<float, 64>(q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, n_heads, st);
    if (head_dim == 128) return launch_att_t<float, 128>(q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, n_heads, st);
  } else {
    if (head_dim == 64) return launch_att_t<uint16_t, 64>(q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, n_heads, st);
    if (head_dim == 128) return launch_att_t<uint16_t, 128>(q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, n_heads, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dit
