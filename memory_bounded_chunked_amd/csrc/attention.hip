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

// 16 bytes per lane from a raw buffer straight into LDS (buffer_load_dwordx4
// ... lds): lane l writes lds + 16*l.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, char* lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 0);
}
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

// bf16 variant, software-pipelined over three key tiles. Step t of a wave
// issues, interleaved, three independent streams:
//   - the score MFMAs of tile t+1 (S^T = K Q^T from the K ring),
//   - the softmax of tile t (VALU and the transcendental unit),
//   - the PV MFMAs of tile t-1 (O^T += V^T P^T from the V ring),
// so the exponentials of one tile run beside the matrix products of two
// others. The K ring runs two tiles ahead of the V ring: step t writes tile
// t+2 into the K slot of tile t-1 and tile t into the V slot of tile t-2, and
// one barrier per step separates the refills from the reads.
//
// Running max, decided per query ("lazy" rescaling): tile 0 sets each
// query's max exactly. Later tiles are exponentiated against the max in use;
// P may then exceed 1, which is harmless in floating point as long as it
// stays far from overflow. Only when a query's tile sum exceeds 2^16 (or is
// not finite) does that query move to its new max: O and the row sum are
// rescaled after the PV of the previous tile has landed, and the tile's P is
// recomputed. The decision uses nothing but the query's own scores, so the
// result does not depend on which queries share a wavefront, i.e. on how the
// queries were sliced. The row sum is accumulated from the bf16-rounded P
// that enters the PV product (v_dot2_f32_bf16 against 1.0).
template <int DH, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void attention_bf16_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const uint16_t* __restrict__ k, int64_t ldk,
    const uint16_t* __restrict__ vt, int64_t ldvt, uint16_t* __restrict__ o, int64_t ldo, int64_t n_q, int64_t n_kv,
    float qk_scale_log2) {
  using L = AttLayout<uint16_t, DH, NW>;
  constexpr int EPC = L::EPC, KRP = L::KRP;
  constexpr int QS = L::QS, OT = L::OT;
  constexpr int NPV = 4 * OT;  // PV MFMAs per tile (4 key groups of 16 x OT dh tiles)
  static_assert(NPV == 2 * QS, "the interleave pairs one score MFMA with one PV MFMA");
  constexpr int EXP_PER_I = 16 / (2 * QS);  // packed words of P per interleave slot (1 at dh 128, 2 at 64)
  constexpr int VALU_PER_MFMA = 3 * EXP_PER_I;
  constexpr float LAZY_LIMIT = 65536.0f;  // 2^16
  typedef __attribute__((ext_vector_type(2))) __bf16 bf2;

  // LDS tiles are filled by buffer loads that write LDS directly: 16 bytes
  // per lane, so one instruction fills 1 KiB (4 K rows of 256 bytes at dh
  // 128; 8 rows of 128 bytes otherwise), and each 1 KiB group is followed by
  // 16 bytes of padding (1040-byte stride). Rows are placed so that the 16
  // rows whose fragments 16 lanes read together sit in 16 distinct groups
  // (or two rows of one 256-byte bank window apart), which makes the 16-byte
  // fragment reads conflict-free with per-lane base + compile-time offsets.
  // (A 16-byte read is served half a wave at a time: the 32 lanes must hit
  // 32 distinct 16-byte slots modulo 512 bytes.)
  //
  // Keys are permuted within each 16-key group: MFMA row 16a+8c+4h+b of a
  // 32-key block holds key 16a+8h+4c+b (bits 2 and 3 swapped). Then the 8
  // P^T registers a lane feeds to one PV MFMA are 8 consecutive keys, and
  // V^T can stay in natural key order in LDS.
  constexpr int GRP = 1040;
  constexpr int KRB = DH * 2, K_RPG = 1024 / KRB;  // K row bytes, K rows per group
  constexpr int K_NG = ATT_BN / K_RPG, V_NG = DH / 8;  // groups per tile (V^T rows are 128 bytes)
  constexpr int K_TILE = K_NG * GRP, V_TILE = V_NG * GRP;
  constexpr int K_DMA = K_NG / NW, V_DMA = V_NG / NW;  // instructions per wave per tile
  static_assert(K_DMA * NW == K_NG && V_DMA * NW == V_NG, "tile loads");

  // Head-major order, contiguous per XCD: the query tiles of one head run on
  // one XCD at the same time and share that head's K/V tiles through its L2,
  // so each head's K/V crosses from HBM about once per launch.
  const int64_t q_tiles = ceil_div(n_q, L::BM);
  const int64_t logical = xcd_contiguous(blockIdx.x, gridDim.x);  // gridDim.x = q_tiles * heads
  const int64_t head_idx = logical / q_tiles, q_tile = logical % q_tiles;

  // LDS: K ring (3 tiles), V^T ring (2 tiles), and each wave's 32 query rows
  // (the B operand of the score MFMAs, read back by the lane that wrote it).
  // The K ring has a third slot because a wave that moves its running max in
  // step t re-reads tile t's K while faster waves already refill a slot: tile
  // t+2 goes to slot (t+2)%3, whose tile t-1 was last read before the
  // previous barrier.
  __shared__ __attribute__((aligned(16))) char smem[3 * K_TILE + 2 * V_TILE + NW * 32 * KRP];
  char* const kring = smem;
  char* const vring = smem + 3 * K_TILE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t q0 = q_tile * L::BM + wave * 32;
  const int64_t col0 = head_idx * DH;

  // Where row m (0..31) of key block mt, and V^T row dh, live in a tile.
  auto k_place = [](int mt, int m) {  // byte offset of the row start
    if constexpr (K_RPG == 4) return (m & 15) * GRP + (2 * mt + (m >> 4)) * KRB;
    else return (m & 7) * GRP + (4 * mt + 2 * (m >> 4) + ((m >> 3) & 1)) * KRB;
  };
  auto v_place = [](int dh) {
    const int ot = dh >> 5, l = dh & 31;
    if constexpr (V_NG == 16) return (l & 15) * GRP + (2 * (l >> 4) + (ot & 1) + 4 * (ot >> 1)) * 128;
    else return (l & 7) * GRP + ((l >> 3) + 4 * ot) * 128;
  };
  // fragment bases (chunk `half`); block mt / tile ot add compile-time offsets
  const int k_rd = k_place(0, l32) + half * 16;
  const int v_rd = v_place(l32) + half * 16;
  constexpr int K_MT = K_RPG == 4 ? 2 * KRB : 4 * KRB;  // k_place(1, m) - k_place(0, m)
  // v_place(ot*32 + l) - v_place(l)
  auto v_ot = [](int ot) { return V_NG == 16 ? ((ot & 1) + 4 * (ot >> 1)) * 128 : ot * 512; };

  // Q fragment st of this lane: query q0+l32, dh chunk 2st+half.
  const char* const qlds = smem + 3 * K_TILE + 2 * V_TILE + wave * 32 * KRP + l32 * KRP + half * 16;
  {
    const int64_t qr = q0 + l32;
#pragma unroll
    for (int st = 0; st < QS; ++st)
      *reinterpret_cast<u32x4*>(const_cast<char*>(qlds) + st * 32) =
          qr < n_q ? *reinterpret_cast<const u32x4*>(q + qr * ldq + col0 + (2 * st + half) * EPC)
                   : u32x4{0u, 0u, 0u, 0u};
  }
  auto qfrag = [&](int st) { return *reinterpret_cast<const u32x4*>(qlds + st * 32); };

  // Global side of the tile loads: instruction i of this wave fills group
  // g = wave*K_DMA + i; lane l of it moves 16 bytes of one row. k_key / v_dh
  // name that row, k_off / v_off are its byte offsets from the tile start.
  const char* kbase = reinterpret_cast<const char*>(k + col0);
  const char* vbase = reinterpret_cast<const char*>(vt + col0 * ldvt);
  const int64_t k_tile_bytes = (int64_t)ATT_BN * ldk * 2;
  int k_key[K_DMA], k_off[K_DMA], v_off[V_DMA];
#pragma unroll
  for (int i = 0; i < K_DMA; ++i) {
    const int g = wave * K_DMA + i, rig = lane / (KRB / 16), ch = lane % (KRB / 16);
    int mt, m;
    if constexpr (K_RPG == 4) {
      mt = rig >> 1;
      m = g + 16 * (rig & 1);
    } else {
      mt = rig >> 2;
      m = g + 8 * (rig & 1) + 16 * ((rig >> 1) & 1);
    }
    const int row = 32 * mt + m;                                      // MFMA row of the tile
    k_key[i] = (row & ~12) | ((row & 4) << 1) | ((row & 8) >> 1);     // bits 2 and 3 swapped
    k_off[i] = (int)(k_key[i] * ldk * 2 + ch * 16);
  }
#pragma unroll
  for (int i = 0; i < V_DMA; ++i) {
    const int g = wave * V_DMA + i, rig = lane >> 3, ch = lane & 7;
    // the row that v_place puts at row rig of group g
    int dh;
    if constexpr (V_NG == 16) {
      const int ot = (rig & 1) + 2 * (rig >> 2), hi = (rig >> 1) & 1;
      dh = ot * 32 + 16 * hi + g;
    } else {
      dh = (rig >> 2) * 32 + 8 * (rig & 3) + g;
    }
    v_off[i] = (int)(dh * ldvt * 2 + ch * 16);
  }
  constexpr int RSRC_FLAGS = 0x00020000;  // raw buffer, 32-bit data

  // K tile tt into ring slot `slot`. In a ragged last tile, rows past n_kv
  // re-read the last key row: finite values whose scores are masked to -inf.
  auto dma_k = [&](int64_t tt, int slot) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(kbase + tt * k_tile_bytes), (short)0, -1, RSRC_FLAGS);
    const int64_t nk = n_kv - tt * ATT_BN;
#pragma unroll
    for (int i = 0; i < K_DMA; ++i) {
      char* dst = kring + slot * K_TILE + (wave * K_DMA + i) * GRP;
      int off = k_off[i];
      if (nk < ATT_BN && k_key[i] >= nk) off = (int)((nk - 1) * ldk * 2 + (lane % (KRB / 16)) * 16);
      buffer_load_lds16(r, dst, off);
    }
  };
  // Full V^T tile tt into ring slot `slot`.
  auto dma_v = [&](int64_t tt, int slot) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(vbase + tt * ATT_BN * 2), (short)0, -1, RSRC_FLAGS);
#pragma unroll
    for (int i = 0; i < V_DMA; ++i)
      buffer_load_lds16(r, vring + slot * V_TILE + (wave * V_DMA + i) * GRP, v_off[i]);
  };
  // Ragged last V^T tile through registers: keys past n_kv become zero (the
  // columns past n_kv may hold anything, and 0 * NaN would not vanish).
  u32x4 vtail[V_DMA];
  auto load_v_tail = [&](int64_t tt) {
    const int nk = (int)(n_kv - tt * ATT_BN);
    const int key0 = (lane & 7) * 8;
#pragma unroll
    for (int i = 0; i < V_DMA; ++i) {
      const uint16_t* e = reinterpret_cast<const uint16_t*>(vbase + tt * ATT_BN * 2 + v_off[i]);
      uint16_t tmp[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) tmp[j] = key0 + j < nk ? e[j] : (uint16_t)0;
      vtail[i] = __builtin_bit_cast(u32x4, tmp);
    }
  };
  auto store_v_tail = [&](int slot) {
#pragma unroll
    for (int i = 0; i < V_DMA; ++i)
      *reinterpret_cast<u32x4*>(vring + slot * V_TILE + (wave * V_DMA + i) * GRP + lane * 16) = vtail[i];
  };

  // The two lanes of a query (l and l^32) each hold half of its keys. These
  // give both lanes the same combined value, computed in the same order.
  auto pair_max = [](float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };
  auto pair_sum = [](float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };
  auto tile_max = [&](const f32x16 (&s)[2]) {
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    return pair_max(mx);
  };
  auto mask_tail = [&](f32x16 (&s)[2], int64_t t) {  // keys past n_kv in tile t get -inf
    // register r of block mt is MFMA row 8*(r/4) + 4*half + r%4, which holds
    // key mt*32 + 16*(r/8) + 8*half + 4*((r/4)%2) + r%4 (bits 2 and 3 of the
    // row swapped); the lane part (8*half) is folded into the threshold so
    // that the per-register part stays a literal
    const int thr = (int)(n_kv - t * ATT_BN) - 8 * half;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (mt * 32 + 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3) >= thr) s[mt][r] = -INFINITY;
  };

  f32x16 acc_o[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t) acc_o[t] = f32x16{};
  float m_run, l_run = 0.f;
  const bf2 ones = __builtin_bit_cast(bf2, 0x3f803f80u);

  // One packed word of P: scores r, r+1 of the tile; p = 2^(s*scale - mc).
  auto exp_pair = [&](const f32x16 (&s)[2], int i, float mc, u32x4 (&pb)[4], float& lsum) {
    const f32x16& sv = s[i >> 3];
    const int r = 2 * (i & 7);
    const float p0 = __builtin_amdgcn_exp2f(sv[r] * qk_scale_log2 - mc);
    const float p1 = __builtin_amdgcn_exp2f(sv[r + 1] * qk_scale_log2 - mc);
    const uint32_t w = pack_bf16x2(p0, p1);
    pb[i >> 2][i & 3] = w;
    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w), ones, lsum, false);
  };
  auto exp_tile = [&](const f32x16 (&s)[2], u32x4 (&pb)[4]) {
    const float mc = m_run * qk_scale_log2;
    float la = 0.f, lb = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      exp_pair(s, i, mc, pb, la);
      exp_pair(s, i + 1, mc, pb, lb);
    }
    return la + lb;
  };

  auto scores = [&](int slot, f32x16 (&s)[2]) {
    const char* ks = kring + slot * K_TILE + k_rd;
    s[0] = f32x16{};
    s[1] = f32x16{};
    u32x4 b;
#pragma unroll
    for (int i = 0; i < 2 * QS; ++i) {
      const int st = i >> 1, mt = i & 1;
      if (mt == 0) b = qfrag(st);
      const u32x4 a = *reinterpret_cast<const u32x4*>(ks + mt * K_MT + st * 32);
      s[mt] = mfma32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), s[mt]);
    }
  };

  const int64_t n_tiles = ceil_div(n_kv, ATT_BN);
  const bool ragged = (n_kv % ATT_BN) != 0;

  // Step t (see above). s_cur holds the scores of tile t, p_prev the P of
  // tile t-1; s_nxt receives the scores of tile t+1 and p_cur the P of tile t.
  // nxt: tile t+1 exists; prv: t > 0; more_k: tile t+2 exists; mask_nxt:
  // tile t+1 is the ragged last tile; last: t is the last tile. Every call
  // site passes constants (mask_nxt aside, which is `ragged` or false), so no
  // step carries logic for the cases it cannot meet.
  auto step = [&](int64_t t, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2], const u32x4 (&p_prev)[4],
                  u32x4 (&p_cur)[4], const bool nxt, const bool prv, const bool more_k, const bool mask_nxt,
                  const bool last) {
    const int k_slot = (int)t % 3;  // K ring slot of tile t; t+1 and t+2 follow cyclically
    const int k_next = k_slot == 2 ? 0 : k_slot + 1, k_free = k_next == 2 ? 0 : k_next + 1;
    // refills: both target slots were last read before the previous barrier
    if (more_k) dma_k(t + 2, k_free);
    const bool v_ragged = last && ragged;
    if (v_ragged)
      load_v_tail(t);
    else
      dma_v(t, (int)(t & 1));
    const char* ks = kring + k_next * K_TILE + k_rd;
    const char* vs = vring + (int)((t - 1) & 1) * V_TILE + v_rd;
    const float mc = m_run * qk_scale_log2;
    float la = 0.f, lb = 0.f;
    if (nxt) {
      s_nxt[0] = f32x16{};
      s_nxt[1] = f32x16{};
    }
    // 2*QS score MFMAs, NPV PV MFMAs and 16 packed words of P, interleaved.
    // The LDS fragments of slot i+1 are read while slot i's MFMAs run.
    u32x4 fk[2], fv[2], fq[2];
    auto fetch = [&](int i) {
      const int st = i >> 1, mt = i & 1;
      if (nxt) {
        if (mt == 0) fq[st & 1] = qfrag(st);
        fk[i & 1] = *reinterpret_cast<const u32x4*>(ks + mt * K_MT + st * 32);
      }
      if (prv) fv[i & 1] = *reinterpret_cast<const u32x4*>(vs + v_ot(i % OT) + (i / OT) * 32);
    };
    fetch(0);
#pragma unroll
    for (int i = 0; i < 2 * QS; ++i) {
      const int st = i >> 1, mt = i & 1;
      if (i + 1 < 2 * QS) fetch(i + 1);
      if (nxt)
        s_nxt[mt] = mfma32_bf16(__builtin_bit_cast(bf16x8, fk[i & 1]), __builtin_bit_cast(bf16x8, fq[st & 1]),
                                s_nxt[mt]);
#pragma unroll
      for (int e = 0; e < EXP_PER_I; ++e) {
        const int w = i * EXP_PER_I + e;
        if (EXP_PER_I > 1 && e == EXP_PER_I / 2 && prv) {
          const int j = i / OT, ot = i % OT;
          acc_o[ot] = mfma32_bf16(__builtin_bit_cast(bf16x8, fv[i & 1]), __builtin_bit_cast(bf16x8, p_prev[j]),
                                  acc_o[ot]);
        }
        exp_pair(s_cur, w, mc, p_cur, (w & 1) ? lb : la);
      }
      if (EXP_PER_I == 1 && prv) {
        const int j = i / OT, ot = i % OT;
        acc_o[ot] = mfma32_bf16(__builtin_bit_cast(bf16x8, fv[i & 1]), __builtin_bit_cast(bf16x8, p_prev[j]),
                                acc_o[ot]);
      }
    }
    // Issue order per slot: the next slot's LDS fragment reads, then each
    // MFMA followed by its share of the VALU work of P (per packed word: 2
    // FMA, 2 exp, 1 convert, 1 dot).
#pragma unroll
    for (int i = 0; i < QS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // K and V fragment reads (slot 2i+1)
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER_MFMA, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER_MFMA, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // Q, K and V fragment reads (slot 2i+2)
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER_MFMA, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER_MFMA, 0);
    }
    float ls = la + lb;
    // A query whose tile sum left the safe range moves to its new max.
    const float lq = pair_sum(ls);
    const bool move = !(lq <= LAZY_LIMIT);
    if (__any(move)) {
      // s_cur died while P was formed; tile t's K is still in its LDS slot
      // (refilled only below), so recompute the same scores, bit for bit.
      scores(k_slot, s_cur);
      if (ragged && t + 1 == n_tiles) mask_tail(s_cur, t);
      const float mx = tile_max(s_cur);
      const float m_new = move ? fmaxf(m_run, mx) : m_run;
      const float alpha = move ? __builtin_amdgcn_exp2f((m_run - m_new) * qk_scale_log2) : 1.0f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int ot = 0; ot < OT; ++ot)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[ot][r] *= alpha;
      ls = exp_tile(s_cur, p_cur);
    }
    l_run += ls;
    if (mask_nxt) mask_tail(s_nxt, t + 1);
    if (v_ragged) store_v_tail((int)(t & 1));
    __syncthreads();  // also waits for this step's LDS-direct loads
  };

  // prologue: K tiles 0 and 1; scores of tile 0 and its exact max
  dma_k(0, 0);
  if (n_tiles > 1) dma_k(1, 1);
  __syncthreads();
  f32x16 sa[2], sb[2];
  u32x4 pa[4], pb[4];
  scores(0, sa);
  if (n_tiles == 1 && ragged) mask_tail(sa, 0);
  m_run = tile_max(sa);

  // PV of the last tile (after its step's barrier).
  auto final_pv = [&](const u32x4 (&pl)[4]) {
    const char* vs = vring + (int)((n_tiles - 1) & 1) * V_TILE + v_rd;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int ot = 0; ot < OT; ++ot) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(vs + v_ot(ot) + j * 32);
        acc_o[ot] = mfma32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, pl[j]), acc_o[ot]);
      }
  };

  // Step 0, then pairs of inner steps, then the last one to three steps.
  // Scores and P alternate between (sa, pa) and (sb, pb).
  if (n_tiles == 1) {
    step(0, sa, sb, pb, pa, false, false, false, false, true);
    final_pv(pa);
  } else if (n_tiles == 2) {
    step(0, sa, sb, pb, pa, true, false, false, ragged, false);
    step(1, sb, sa, pa, pb, false, true, false, false, true);
    final_pv(pb);
  } else {
    step(0, sa, sb, pb, pa, true, false, true, ragged && n_tiles == 2, false);
    int64_t t = 1;
    for (; t + 1 <= n_tiles - 3; t += 2) {
      step(t, sb, sa, pa, pb, true, true, true, false, false);
      step(t + 1, sa, sb, pb, pa, true, true, true, false, false);
    }
    // steps t .. n_tiles-1 remain, t odd
    const int64_t rem = n_tiles - t;
    if (rem == 1) {
      step(t, sb, sa, pa, pb, false, true, false, false, true);
      final_pv(pb);
    } else if (rem == 2) {
      step(t, sb, sa, pa, pb, true, true, false, ragged, false);
      step(t + 1, sa, sb, pb, pa, false, true, false, false, true);
      final_pv(pa);
    } else {
      step(t, sb, sa, pa, pb, true, true, true, false, false);
      step(t + 1, sa, sb, pb, pa, true, true, false, ragged, false);
      step(t + 2, sb, sa, pa, pb, false, true, false, false, true);
      final_pv(pb);
    }
  }

  const float inv = 1.0f / pair_sum(l_run);
  const int64_t qr = q0 + l32;
  if (qr < n_q) {
    uint16_t* orow = o + qr * ldo + col0;
#pragma unroll
    for (int ot = 0; ot < OT; ++ot)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int c = ot * 32 + 8 * qd + 4 * half;
        *reinterpret_cast<u32x2*>(orow + c) =
            u32x2{pack_bf16x2(acc_o[ot][4 * qd] * inv, acc_o[ot][4 * qd + 1] * inv),
                  pack_bf16x2(acc_o[ot][4 * qd + 2] * inv, acc_o[ot][4 * qd + 3] * inv)};
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
