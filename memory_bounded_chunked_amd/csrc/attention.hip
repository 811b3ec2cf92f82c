// K3: softmax attention of a bounded query slice against the global K/V.
//
// Pass 2 of the two-pass scheme ("LayerStream: H3 Chunking", section "How
// the slicing works": attend the slice against the full K/V; the streaming
// proposal's "Attention requires a stronger contract": retain global K/V,
// consume bounded Q, produce output in Q-sized slabs). The kernel never holds
// anything that grows with the key count: K/V tiles stream through LDS and
// the softmax is taken online in fp32.
//
// Work split: one workgroup = NW wavefronts, each owning 32 query rows of one
// head (8 waves = 256 queries: two waves per SIMD, so one wave's softmax runs
// while the other's matrix products occupy the MFMA unit). Per 64-key tile a
// wave computes S^T = K Q^T (keys along the MFMA M dimension, queries along
// N), so each lane owns one query column and a query's row max and row sum
// need one exchange with lane^32. P^T is then already laid out as the B
// operand of O^T += V^T P^T. V is stored transposed in HBM ([d][keys]), so
// both MFMA operands come from LDS as 16-byte, key-contiguous fragments.
// LDS rows are padded by 16 bytes: consecutive rows start 4 banks apart, so
// 16-byte fragment reads are conflict-free and every read address is a
// per-thread base plus a compile-time offset.
//
// Per query the sequence of operations (KV tile size, tile order, MFMA shape)
// is fixed and does not depend on which slice the query belongs to, so O is
// bit-identical for every choice of query slicing. Skipping the rescale of O
// when no running max moved is exact (the factor would be 1).
#include "common.hpp"
#include "kernels.hpp"

namespace dit {

constexpr int ATT_BN = 64;  // keys per tile
#ifndef DIT_ATT_NW
#define DIT_ATT_NW 8  // wavefronts per workgroup of the bf16 kernel
#endif

template <typename T, int DH, int NW>
struct AttLayout {
  static constexpr bool F32 = sizeof(T) == 4;
  static constexpr int NTHR = NW * 64;
  static constexpr int BM = NW * 32;                 // queries per workgroup
  static constexpr int EPC = 16 / sizeof(T);         // elements per 16-B chunk
  static constexpr int KRB = DH * sizeof(T);         // K tile row bytes (one key)
  static constexpr int VRB = ATT_BN * sizeof(T);     // V^T tile row bytes (one dh)
  static constexpr int KRP = KRB + 16, VRP = VRB + 16;  // padded strides
  static constexpr int KCH = KRB / 16, VCH = VRB / 16;
  static constexpr int K_TILE = ATT_BN * KRP, V_TILE = DH * VRP;
  static constexpr int STAGE = K_TILE + V_TILE;
  static constexpr int K_LD = ATT_BN * KCH / NTHR, V_LD = DH * VCH / NTHR;
  static constexpr int QS = DH / (2 * EPC);          // k-steps over dh
  static constexpr int OT = DH / 32;                 // O^T tiles along dh
  static_assert(ATT_BN * KCH % NTHR == 0 && DH * VCH % NTHR == 0, "tile loads");
};

template <typename T, int DH, int NW>
__global__ __launch_bounds__(NW * 64) void attention_kernel(const T* __restrict__ q, int64_t ldq,
                                                            const T* __restrict__ k, int64_t ldk,
                                                            const T* __restrict__ vt, int64_t ldvt,
                                                            T* __restrict__ o, int64_t ldo, int64_t n_q,
                                                            int64_t n_kv, float qk_scale_log2) {
  using L = AttLayout<T, DH, NW>;
  constexpr bool F32 = L::F32;
  constexpr int EPC = L::EPC, KCH = L::KCH, VCH = L::VCH, KRP = L::KRP, VRP = L::VRP;
  constexpr int STAGE = L::STAGE, K_TILE = L::K_TILE, K_LD = L::K_LD, V_LD = L::V_LD;
  constexpr int QS = L::QS, OT = L::OT, NTHR = L::NTHR;

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.y;
  const int64_t q0 = (int64_t)blockIdx.x * L::BM + wave * 32;
  const int64_t col0 = (int64_t)head * DH;

  // Q^T fragments (B operand): lane holds query q0+l32, dh chunk 2s+half.
  u32x4 qf[QS];
  {
    const int64_t qr = q0 + l32;
#pragma unroll
    for (int s = 0; s < QS; ++s)
      qf[s] = qr < n_q ? *reinterpret_cast<const u32x4*>(q + qr * ldq + col0 + (2 * s + half) * EPC)
                       : u32x4{0u, 0u, 0u, 0u};
  }

  // Cooperative K / V^T tile loads: a uniform per-tile base plus a 32-bit
  // per-thread byte offset, and the LDS destination of each 16-byte chunk.
  const char* kbase = reinterpret_cast<const char*>(k + col0);
  const char* vbase = reinterpret_cast<const char*>(vt + col0 * ldvt);
  const int64_t k_tile_bytes = (int64_t)ATT_BN * ldk * (int64_t)sizeof(T);
  constexpr int64_t v_tile_bytes = (int64_t)ATT_BN * sizeof(T);
  uint32_t koff[K_LD], voff[V_LD];
  int kdst[K_LD], vdst[V_LD], krow[K_LD], vkey[V_LD];
#pragma unroll
  for (int i = 0; i < K_LD; ++i) {
    const int c = tid + i * NTHR;
    krow[i] = c / KCH;
    koff[i] = (uint32_t)(((int64_t)krow[i] * ldk + (c % KCH) * EPC) * (int64_t)sizeof(T));
    kdst[i] = krow[i] * KRP + (c % KCH) * 16;
  }
#pragma unroll
  for (int i = 0; i < V_LD; ++i) {
    const int c = tid + i * NTHR;
    const int r = c / VCH, ch = c % VCH;
    vkey[i] = ch * EPC;
    voff[i] = (uint32_t)(((int64_t)r * ldvt + ch * EPC) * (int64_t)sizeof(T));
    if constexpr (F32) {
      vdst[i] = r * VRP + ch * 16;
    } else {
      // keys 16j..16j+15 of a row: slot 2j holds keys {0-3, 8-11}, slot 2j+1
      // holds {4-7, 12-15}, the order in which P^T sits in the S^T registers
      vdst[i] = r * VRP + (ch >> 1) * 32 + 8 * (ch & 1);
    }
  }

  u32x4 rk[K_LD], rv[V_LD];
  auto load_full = [&](int64_t t) {
    const char* kt = kbase + t * k_tile_bytes;
    const char* vtile = vbase + t * v_tile_bytes;
#pragma unroll
    for (int i = 0; i < K_LD; ++i) rk[i] = *reinterpret_cast<const u32x4*>(kt + koff[i]);
#pragma unroll
    for (int i = 0; i < V_LD; ++i) rv[i] = *reinterpret_cast<const u32x4*>(vtile + voff[i]);
  };
  auto load_tail = [&](int64_t t) {
    const int64_t kv0 = t * ATT_BN;
    const char* kt = kbase + t * k_tile_bytes;
    const char* vtile = vbase + t * v_tile_bytes;
#pragma unroll
    for (int i = 0; i < K_LD; ++i)
      rk[i] = (kv0 + krow[i] < n_kv) ? *reinterpret_cast<const u32x4*>(kt + koff[i]) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      const int64_t key = kv0 + vkey[i];
      const T* src = reinterpret_cast<const T*>(vtile + voff[i]);
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
    for (int i = 0; i < K_LD; ++i) *reinterpret_cast<u32x4*>(Ks + kdst[i]) = rk[i];
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      if constexpr (F32) {
        *reinterpret_cast<u32x4*>(Vs + vdst[i]) = rv[i];
      } else {
        *reinterpret_cast<u32x2*>(Vs + vdst[i]) = u32x2{rv[i][0], rv[i][1]};
        *reinterpret_cast<u32x2*>(Vs + vdst[i] + 16) = u32x2{rv[i][2], rv[i][3]};
      }
    }
  };

  f32x16 acc_o[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t) acc_o[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int k_rd = l32 * KRP + half * 16;  // this lane's K fragment base within a tile
  const int v_rd = l32 * VRP + half * 16;  // this lane's V^T fragment base within a tile

  auto compute = [&](int buf, int64_t kv0, bool tail) {
    const char* Ks = smem + buf * STAGE + k_rd;
    const char* Vs = smem + buf * STAGE + K_TILE + v_rd;
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int st = 0; st < QS; ++st) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(Ks + mt * 32 * KRP + st * 32);
        if constexpr (F32) {
#pragma unroll
          for (int e = 0; e < 4; ++e) s[mt] = mfma32_f32(__uint_as_float(a[e]), __uint_as_float(qf[st][e]), s[mt]);
        } else {
          s[mt] = mfma32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[st]), s[mt]);
        }
      }
    }
    if (tail) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kv0 + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= n_kv) s[mt][r] = -INFINITY;
    }
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
#ifdef DIT_ATT_RESCALE_ALWAYS
    if (true) {
#else
    if (__any(mx > m_run)) {  // wave-uniform: rescale only when some running max moved
#endif
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * qk_scale_log2);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < OT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[t][r] *= alpha;
    }
    const float mc = m_run * qk_scale_log2;
    float lsum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[mt][r] * qk_scale_log2 - mc);
        s[mt][r] = p;
        lsum += p;
      }
    l_run += lsum;

    if constexpr (F32) {
      // B operand of each 32x32x2 MFMA: this lane's own score register r
      // (key 8*(r/4) + 4*half + r%4 of the 32-key tile).
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
#pragma unroll
          for (int t = 0; t < OT; ++t) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(Vs + t * 32 * VRP + (8 * mt + 2 * qd) * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc_o[t] = mfma32_f32(__uint_as_float(a[e]), s[mt][4 * qd + e], acc_o[t]);
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
          const u32x4 a = *reinterpret_cast<const u32x4*>(Vs + t * 32 * VRP + j * 32);
          acc_o[t] = mfma32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pb), acc_o[t]);
        }
      }
    }
  };

  // Full tiles in the loop (no masking anywhere in it); a ragged last tile,
  // if any, after it. Tile t sits in LDS buffer t & 1; tile t+1 is fetched
  // from HBM into registers while tile t is multiplied.
  const int64_t n_full = n_kv / ATT_BN;
  const bool ragged = (n_kv % ATT_BN) != 0;
  if (n_full > 0)
    load_full(0);
  else
    load_tail(0);
  store_kv(0);
  __syncthreads();
  for (int64_t t = 0; t < n_full; ++t) {
    const int cur = (int)(t & 1);
    const bool fetch = t + 1 < n_full || ragged;
    if (t + 1 < n_full)
      load_full(t + 1);
    else if (ragged)
      load_tail(t + 1);
    compute(cur, t * ATT_BN, false);
    if (fetch) store_kv(cur ^ 1);
    __syncthreads();
  }
  if (ragged) compute((int)(n_full & 1), n_full * ATT_BN, true);

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

// bf16 variant with a one-tile software pipeline: the score MFMAs of tile
// t+1 are issued interleaved with the softmax of tile t (VALU and the
// transcendental unit), so the matrix cores stay busy while exponentials are
// taken. K runs one tile ahead of V in the LDS rings: iteration t reads K
// tile t+1 and V tile t, and refills the K slot of tile t (consumed one
// iteration earlier) with tile t+2 and the V slot of tile t-1 with tile t+1.
// The row sum is accumulated from the bf16-rounded P that enters the PV
// product (v_dot2_f32_bf16 against 1.0), two elements per instruction, and O
// is rescaled only when a running max grows by more than 2^8.
template <int DH, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attention_bf16_kernel(const uint16_t* __restrict__ q, int64_t ldq,
                                                                 const uint16_t* __restrict__ k, int64_t ldk,
                                                                 const uint16_t* __restrict__ vt, int64_t ldvt,
                                                                 uint16_t* __restrict__ o, int64_t ldo,
                                                                 int64_t n_q, int64_t n_kv, float qk_scale_log2) {
  using L = AttLayout<uint16_t, DH, NW>;
  constexpr int EPC = L::EPC, KCH = L::KCH, VCH = L::VCH, KRP = L::KRP, VRP = L::VRP;
  constexpr int K_TILE = L::K_TILE, V_TILE = L::V_TILE, K_LD = L::K_LD, V_LD = L::V_LD;
  constexpr int QS = L::QS, OT = L::OT, NTHR = L::NTHR;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf2;
  // Head-major order, contiguous per XCD: the query tiles of one head run on
  // one XCD at the same time and share that head's K/V tiles through its L2,
  // so each head's K/V crosses from HBM about once per launch.
  const int64_t q_tiles = ceil_div(n_q, L::BM);
  const int64_t logical = xcd_contiguous(blockIdx.x, gridDim.x);  // gridDim.x = q_tiles * heads
  const int64_t head_idx = logical / q_tiles, q_tile = logical % q_tiles;

  __shared__ __attribute__((aligned(16))) char smem[2 * K_TILE + 2 * V_TILE];
  char* const kring = smem;
  char* const vring = smem + 2 * K_TILE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t q0 = q_tile * L::BM + wave * 32;
  const int64_t col0 = head_idx * DH;

  u32x4 qf[QS];
  {
    const int64_t qr = q0 + l32;
#pragma unroll
    for (int st = 0; st < QS; ++st)
      qf[st] = qr < n_q ? *reinterpret_cast<const u32x4*>(q + qr * ldq + col0 + (2 * st + half) * EPC)
                        : u32x4{0u, 0u, 0u, 0u};
  }

  const char* kbase = reinterpret_cast<const char*>(k + col0);
  const char* vbase = reinterpret_cast<const char*>(vt + col0 * ldvt);
  const int64_t k_tile_bytes = (int64_t)ATT_BN * ldk * 2;
  uint32_t koff[K_LD], voff[V_LD];
  int kdst[K_LD], vdst[V_LD], krow[K_LD], vkey[V_LD];
#pragma unroll
  for (int i = 0; i < K_LD; ++i) {
    const int c = tid + i * NTHR;
    krow[i] = c / KCH;
    koff[i] = (uint32_t)(((int64_t)krow[i] * ldk + (c % KCH) * EPC) * 2);
    kdst[i] = krow[i] * KRP + (c % KCH) * 16;
  }
#pragma unroll
  for (int i = 0; i < V_LD; ++i) {
    const int c = tid + i * NTHR;
    const int r = c / VCH, ch = c % VCH;
    vkey[i] = ch * EPC;
    voff[i] = (uint32_t)(((int64_t)r * ldvt + ch * EPC) * 2);
    // keys 16j..16j+15 of a row: slot 2j holds keys {0-3, 8-11}, slot 2j+1
    // holds {4-7, 12-15}, the order in which P^T sits in the S^T registers
    vdst[i] = r * VRP + (ch >> 1) * 32 + 8 * (ch & 1);
  }

  u32x4 rk[K_LD], rv[V_LD];
  auto load_k = [&](int64_t t) {
    const char* src = kbase + t * k_tile_bytes;
    const int64_t kv0 = t * ATT_BN;
    if (kv0 + ATT_BN <= n_kv) {
#pragma unroll
      for (int i = 0; i < K_LD; ++i) rk[i] = *reinterpret_cast<const u32x4*>(src + koff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < K_LD; ++i)
        rk[i] = (kv0 + krow[i] < n_kv) ? *reinterpret_cast<const u32x4*>(src + koff[i]) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto load_v = [&](int64_t t) {
    const char* src = vbase + t * (int64_t)ATT_BN * 2;
    const int64_t kv0 = t * ATT_BN;
    if (kv0 + ATT_BN <= n_kv) {
#pragma unroll
      for (int i = 0; i < V_LD; ++i) rv[i] = *reinterpret_cast<const u32x4*>(src + voff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < V_LD; ++i) {
        const int64_t key = kv0 + vkey[i];
        const uint16_t* e = reinterpret_cast<const uint16_t*>(src + voff[i]);
        uint16_t tmp[EPC];
#pragma unroll
        for (int j = 0; j < EPC; ++j) tmp[j] = (key + j < n_kv) ? e[j] : (uint16_t)0;
        rv[i] = __builtin_bit_cast(u32x4, tmp);
      }
    }
  };
  auto store_k = [&](int slot) {
#pragma unroll
    for (int i = 0; i < K_LD; ++i) *reinterpret_cast<u32x4*>(kring + slot * K_TILE + kdst[i]) = rk[i];
  };
  auto store_v = [&](int slot) {
    char* vs = vring + slot * V_TILE;
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      *reinterpret_cast<u32x2*>(vs + vdst[i]) = u32x2{rv[i][0], rv[i][1]};
      *reinterpret_cast<u32x2*>(vs + vdst[i] + 16) = u32x2{rv[i][2], rv[i][3]};
    }
  };

  const int k_rd = l32 * KRP + half * 16;
  const int v_rd = l32 * VRP + half * 16;

  // S^T of one key tile: 2 x (32 keys x 32 queries), 2*QS MFMAs; the K
  // fragments of k-step st+1 are read from LDS while those of st are used.
  auto scores = [&](int slot, f32x16 (&s)[2]) {
    const char* ks = kring + slot * K_TILE + k_rd;
    s[0] = f32x16{};
    s[1] = f32x16{};
    u32x4 a[2][2];
    a[0][0] = *reinterpret_cast<const u32x4*>(ks);
    a[0][1] = *reinterpret_cast<const u32x4*>(ks + 32 * KRP);
#pragma unroll
    for (int st = 0; st < QS; ++st) {
      if (st + 1 < QS) {
        a[(st + 1) & 1][0] = *reinterpret_cast<const u32x4*>(ks + (st + 1) * 32);
        a[(st + 1) & 1][1] = *reinterpret_cast<const u32x4*>(ks + 32 * KRP + (st + 1) * 32);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        s[mt] = mfma32_bf16(__builtin_bit_cast(bf16x8, a[st & 1][mt]), __builtin_bit_cast(bf16x8, qf[st]), s[mt]);
    }
  };

  f32x16 acc_o[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t) acc_o[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const bf2 ones = __builtin_bit_cast(bf2, 0x3f803f80u);

  // Softmax of one tile, in two parts. rescale(): the tile's row max; a
  // query whose max grew by more than 8 (log2 units) past the max in use
  // moves to its new max and rescales its O and row sum. Otherwise the stale
  // max stays in use and P may reach 2^8, which fp32 and bf16 hold without
  // loss of relative precision. The decision is taken per query, from that
  // query's own scores only (other lanes of the wave merely share the branch,
  // with a factor of exactly 1), so O does not depend on which queries share
  // a wavefront, i.e. on how the queries were sliced. exp_tile(): P = exp2 of
  // the scaled scores minus the max in use, packed to bf16, and the row sum
  // accumulated from the packed values.
  //
  // The two lanes of a query (l and l^32) each hold half of its keys; one
  // v_permlane32_swap gives both of them the combined value, in the same
  // operand order.
  auto pair_max = [](float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };
  auto exp_tile = [&](f32x16 (&s)[2], u32x4 (&pb)[4]) {
    const float mc = m_run * qk_scale_log2;
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x16& sv = s[j >> 1];
      const int r0 = 8 * (j & 1);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(sv[r0 + 2 * e] * qk_scale_log2 - mc);
        const float p1 = __builtin_amdgcn_exp2f(sv[r0 + 2 * e + 1] * qk_scale_log2 - mc);
        w[e] = pack_bf16x2(p0, p1);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w[e]), ones, lsum, false);
      }
      pb[j] = u32x4{w[0], w[1], w[2], w[3]};
    }
    return lsum;
  };
  // After a tile's P is formed against the max in use: a query whose tile
  // sum left [0, 2^16] (or is not finite) moves to its new max, rescales its
  // O and row sum, and forms P again; every other query keeps its max and
  // its P (factor exactly 1).
  auto settle = [&](f32x16 (&s)[2], u32x4 (&pb)[4], float ls) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ls), __float_as_uint(ls), false, false);
    const bool move = !(__uint_as_float(r[0]) + __uint_as_float(r[1]) <= 65536.0f);
    if (__any(move)) {
      float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
      for (int q = 2; q < 16; ++q) mx = fmaxf(mx, s[0][q]);
#pragma unroll
      for (int q = 0; q < 16; ++q) mx = fmaxf(mx, s[1][q]);
      mx = pair_max(mx);
      const float m_new = move ? fmaxf(m_run, mx) : m_run;
      const float alpha = move ? __builtin_amdgcn_exp2f((m_run - m_new) * qk_scale_log2) : 1.0f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < OT; ++t)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc_o[t][q] *= alpha;
      ls = exp_tile(s, pb);
    }
    l_run += ls;
  };

  auto pv = [&](int slot, const u32x4 (&pb)[4]) {
    const char* vs = vring + slot * V_TILE + v_rd;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < OT; ++t) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(vs + t * 32 * VRP + j * 32);
        acc_o[t] = mfma32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pb[j]), acc_o[t]);
      }
  };

  const int64_t n_tiles = ceil_div(n_kv, ATT_BN);
  // prologue: K tiles 0 and 1, V tile 0; scores of tile 0
  load_k(0);
  store_k(0);
  if (n_tiles > 1) {
    load_k(1);
    store_k(1);
  }
  load_v(0);
  store_v(0);
  __syncthreads();
  // One pipeline step: scores of tile t+1 into s_nxt, interleaved with the
  // softmax of tile t (in s_cur), then PV of tile t, then the LDS refills.
  auto step = [&](int64_t t, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2]) {
    const bool more_k = t + 2 < n_tiles;
    if (more_k) load_k(t + 2);
    load_v(t + 1);
    u32x4 pb[4];
    scores((int)((t + 1) & 1), s_nxt);
    const float ls = exp_tile(s_cur, pb);
#pragma unroll
    for (int i = 0; i < QS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS fragment reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // 6 VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // 6 VALU
    }
    settle(s_cur, pb, ls);
    pv((int)(t & 1), pb);
    if (more_k) store_k((int)(t & 1));
    store_v((int)((t + 1) & 1));
    __syncthreads();
  };
  // Keys past n_kv in the last tile get -inf. Register r of block mt holds
  // key mt*32 + 8*(r/4) + 4*half + r%4; the lane part is folded into the
  // threshold so that the per-register part stays a literal.
  auto mask_last = [&](f32x16 (&s)[2]) {
    const int thr = (int)(n_kv - (n_tiles - 1) * ATT_BN) - 4 * half;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (mt * 32 + 8 * (r >> 2) + (r & 3) >= thr) s[mt][r] = -INFINITY;
  };
  auto last = [&](f32x16 (&s_cur)[2]) {
    if (n_kv % ATT_BN != 0 && n_tiles > 1) mask_last(s_cur);
    u32x4 pb[4];
    settle(s_cur, pb, exp_tile(s_cur, pb));
    pv((int)((n_tiles - 1) & 1), pb);
  };

  f32x16 sa[2], sb[2];
  scores(0, sa);
  // tile 0 sets each query's running max exactly
  if (n_tiles == 1 && n_kv % ATT_BN != 0) mask_last(sa);
  {
    float mx = fmaxf(sa[0][0], sa[0][1]);
#pragma unroll
    for (int q = 2; q < 16; ++q) mx = fmaxf(mx, sa[0][q]);
#pragma unroll
    for (int q = 0; q < 16; ++q) mx = fmaxf(mx, sa[1][q]);
    m_run = pair_max(mx);
  }
  int64_t t = 0;
  for (; t + 2 < n_tiles; t += 2) {  // only the last tile can be ragged
    step(t, sa, sb);
    step(t + 1, sb, sa);
  }
  if (t + 1 < n_tiles) {
    step(t, sa, sb);
    last(sb);
  } else {
    last(sa);
  }

  const auto lr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float inv = 1.0f / (__uint_as_float(lr[0]) + __uint_as_float(lr[1]));
  const int64_t qr = q0 + l32;
  if (qr < n_q) {
    uint16_t* orow = o + qr * ldo + col0;
#pragma unroll
    for (int t = 0; t < OT; ++t)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int c = t * 32 + 8 * qd + 4 * half;
        *reinterpret_cast<u32x2*>(orow + c) =
            u32x2{pack_bf16x2(acc_o[t][4 * qd] * inv, acc_o[t][4 * qd + 1] * inv),
                  pack_bf16x2(acc_o[t][4 * qd + 2] * inv, acc_o[t][4 * qd + 3] * inv)};
      }
  }
}

template <int DH, int NW>
static hipError_t launch_att_bf16(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* vt,
                                  int64_t ldvt, void* o, int64_t ldo, int64_t n_q, int64_t n_kv, int n_heads,
                                  hipStream_t st) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)DH);
  // one-dimensional grid: the kernel derives (head, query tile) from blockIdx.x
  dim3 grid((unsigned)(ceil_div(n_q, AttLayout<uint16_t, DH, NW>::BM) * n_heads)), block(NW * 64);
  hipLaunchKernelGGL((attention_bf16_kernel<DH, NW>), grid, block, 0, st, static_cast<const uint16_t*>(q), ldq,
                     static_cast<const uint16_t*>(k), ldk, static_cast<const uint16_t*>(vt), ldvt,
                     static_cast<uint16_t*>(o), ldo, n_q, n_kv, scale_log2);
  return hipGetLastError();
}

template <typename T, int DH, int NW>
static hipError_t launch_att_t(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* vt,
                               int64_t ldvt, void* o, int64_t ldo, int64_t n_q, int64_t n_kv, int n_heads,
                               hipStream_t st) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)DH);
  dim3 grid((unsigned)ceil_div(n_q, AttLayout<T, DH, NW>::BM), (unsigned)n_heads), block(NW * 64);
  hipLaunchKernelGGL((attention_kernel<T, DH, NW>), grid, block, 0, st, static_cast<const T*>(q), ldq,
                     static_cast<const T*>(k), ldk, static_cast<const T*>(vt), ldvt, static_cast<T*>(o), ldo,
                     n_q, n_kv, scale_log2);
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const void* q, int64_t ldq, const void* k, int64_t ldk,
                            const void* vt, int64_t ldvt, void* o, int64_t ldo, int64_t n_q,
                            int64_t n_kv, int n_heads, int head_dim, hipStream_t st) {
  if (n_q <= 0) return hipSuccess;
  if (n_kv <= 0) return hipErrorInvalidValue;
  // per-thread offsets into a V^T tile are 32-bit: head_dim rows of ldvt elements
  if ((int64_t)head_dim * ldvt * (dtype == F32 ? 4 : 2) >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
  if (dtype == F32) {
    if (head_dim == 64) return launch_att_t<float, 64, 4>(q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, n_heads, st);
    if (head_dim == 128) return launch_att_t<float, 128, 4>(q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, n_heads, st);
  } else {
    if (head_dim == 64) return launch_att_bf16<64, DIT_ATT_NW>(q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, n_heads, st);
    if (head_dim == 128) return launch_att_bf16<128, DIT_ATT_NW>(q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, n_heads, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dit
