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

// Key split: the keys of every query are cut into `splits` contiguous ranges
// of whole 64-key tiles, range p = tiles [p*T/splits, (p+1)*T/splits) of the
// T = ceil(n_kv/64) tiles. The cut depends only on n_kv and splits. With
// splits > 1 each workgroup attends one range and writes, per query and head,
// its unnormalised fp32 O and its (running max m, row sum l); the combine
// kernel merges the ranges in order p = 0, 1, ...
struct AttSplit {
  int splits;        // 1: no split (O written normalised, in the output type)
  float* o_part;     // [splits][n_q][d] unnormalised O of each range (splits > 1)
  float* ml_part;    // [splits][n_q][n_heads][2]: m (in score units) and l of each range
};

__device__ __forceinline__ void key_range(int64_t n_tiles, int splits, int p, int64_t& kt0, int64_t& kt1) {
  kt0 = (int64_t)p * n_tiles / splits;
  kt1 = (int64_t)(p + 1) * n_tiles / splits;
}

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

template <typename T, int DH, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void attention_kernel(const T* __restrict__ q, int64_t ldq,
                                                            const T* __restrict__ k, int64_t ldk,
                                                            const T* __restrict__ vt, int64_t ldvt,
                                                            T* __restrict__ o, int64_t ldo, int64_t n_q,
                                                            int64_t n_kv, float qk_scale_log2, AttSplit sp) {
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
    if (__any(mx > m_run)) {  // wave-uniform: rescale only when some running max moved
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

  // Full tiles of the key range in the loop (no masking anywhere in it); the
  // ragged last tile of the sequence, if it is in the range, after it. Tile t
  // sits in LDS buffer (t - kt0) & 1; tile t+1 is fetched from HBM into
  // registers while tile t is multiplied.
  const int64_t n_tiles = ceil_div(n_kv, ATT_BN);
  int64_t kt0 = 0, kt1 = n_tiles;
  if constexpr (SPLIT) key_range(n_tiles, sp.splits, (int)blockIdx.z, kt0, kt1);
  const int64_t n_full = n_kv / ATT_BN;
  const int64_t fe = kt1 < n_full ? kt1 : n_full;  // end of the range's full tiles
  const bool tail = (n_kv % ATT_BN) != 0 && kt1 == n_tiles;
  if (kt0 < fe)
    load_full(kt0);
  else
    load_tail(kt0);
  store_kv(0);
  __syncthreads();
  for (int64_t t = kt0; t < fe; ++t) {
    const int cur = (int)((t - kt0) & 1);
    const bool fetch = t + 1 < fe || tail;
    if (t + 1 < fe)
      load_full(t + 1);
    else if (tail)
      load_tail(t + 1);
    compute(cur, t * ATT_BN, false);
    if (fetch) store_kv(cur ^ 1);
    __syncthreads();
  }
  if (tail) compute((int)((fe - kt0) & 1), n_full * ATT_BN, true);

  const float l_all = l_run + __shfl_xor(l_run, 32, 64);
  const int64_t qr = q0 + l32;
  if constexpr (SPLIT) {  // this range's unnormalised O, its m and l
    if (qr < n_q) {
      const int64_t d = (int64_t)gridDim.y * DH;
      const int64_t prow = (int64_t)blockIdx.z * n_q + qr;
      float* orow = sp.o_part + prow * d + col0;
#pragma unroll
      for (int t = 0; t < OT; ++t)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *reinterpret_cast<f32x4*>(orow + t * 32 + 8 * qd + 4 * half) =
              f32x4{acc_o[t][4 * qd], acc_o[t][4 * qd + 1], acc_o[t][4 * qd + 2], acc_o[t][4 * qd + 3]};
      if (half == 0) {
        float* ml = sp.ml_part + (prow * gridDim.y + head) * 2;
        ml[0] = m_run;
        ml[1] = l_all;
      }
    }
    return;
  }
  const float inv = 1.0f / l_all;
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

// Largest tile sum of P before a query's running max moves (2^64). Every P
// element then stays below 2^64, the row sum below 2^64 per 64-key tile
// (2^80 at 2^16 tiles, four million keys) and |O| below that times max|V|, so
// fp32 (to 2^128) and bf16 P (same exponent range) hold them with room for
// |V| up to 2^40. A high bar keeps moves rare when logits are large (weights
// of the int8 block give logits of tens to hundreds), where every move costs
// a rescale of O and a second exponentiation of the tile.
constexpr float ATT_MOVE_SUM = 18446744073709551616.0f;

// bf16 variant (8 waves) with a two-group schedule. Waves w and w+4 share a
// SIMD, so waves 0-3 and 4-7 form two groups with one wave per SIMD each;
// group 1 runs one phase behind group 0. A key tile is four phases, each
// closed by a workgroup barrier:
//   M1: read the K fragments of tile t from LDS; store K tile t+1 into the
//       other K slot; load K tile t+2 into the staging registers
//   C1: S^T = K Q^T (2 x QS MFMAs)
//   M2: read the V^T fragments of tile t; the softmax of tile t; store V^T
//       tile t+1; load V^T tile t+2
//   C2: O^T += V^T P^T (4 x OT MFMAs)
// so on every SIMD one wave issues MFMAs while the other reads LDS and runs
// the softmax. Tile t+1 is complete in LDS (both groups' stores) a barrier
// before either group reads it, and a slot is overwritten only after both
// groups finished reading the tile it held; both groups pass the same
// number of barriers.
//
// Softmax: fp32, exp2 with log2(e)/sqrt(dh) folded into one multiply-add.
// Tile 0 sets each query's running max exactly. Later tiles are
// exponentiated against the max in use, and only a query whose tile sum
// leaves [0, ATT_MOVE_SUM] moves to its new max (its O and row sum
// rescaled, the tile's P formed again); otherwise P may reach ATT_MOVE_SUM
// per element, which fp32 and bf16 hold without loss of relative precision
// (see ATT_MOVE_SUM for the range). The decision uses only the query's own
// scores, so O does not depend on which queries share a wavefront. P is
// rounded to bf16 and the row sum is accumulated from the rounded values
// (v_dot2_f32_bf16 against 1.0), the ones that enter the PV product; O is
// divided by the row sum at the end.
//
// Loads carry no branch: key rows past n_kv re-read the last key row (their
// scores are masked to -inf), V^T chunks past n_kv re-read the last valid
// chunk (still inside the row: ldvt is a multiple of 8 and at least n_kv)
// and are zeroed when stored, and the tiles after the last reload the last
// tile into a slot no later phase reads. The compiler then waits for each
// staged tile by exact count instead of for every outstanding load.
template <int DH, bool SPLIT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void attention_bf16_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const uint16_t* __restrict__ k, int64_t ldk,
    const uint16_t* __restrict__ vt, int64_t ldvt, uint16_t* __restrict__ o, int64_t ldo, int64_t n_q,
    int64_t n_kv, float qk_scale_log2, AttSplit sp) {
  using L = AttLayout<uint16_t, DH, 8>;
  constexpr int EPC = L::EPC, KCH = L::KCH, VCH = L::VCH, KRP = L::KRP, VRP = L::VRP;
  constexpr int K_TILE = L::K_TILE, V_TILE = L::V_TILE, K_LD = L::K_LD, V_LD = L::V_LD;
  constexpr int QS = L::QS, OT = L::OT, NTHR = L::NTHR;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf2;
  const int64_t q_tiles = ceil_div(n_q, L::BM);
  // gridDim.x = heads * splits * q_tiles; each XCD gets a contiguous range of
  // logical ids, ordered head, key range, query tile, so the workgroups that
  // stream one head's key range run on one XCD and share its L2
  const int64_t logical = xcd_contiguous(blockIdx.x, gridDim.x);
  const int splits = SPLIT ? sp.splits : 1;
  const int64_t head_idx = logical / (splits * q_tiles);
  const int64_t rem = logical % (splits * q_tiles);
  const int part = (int)(rem / q_tiles);
  const int64_t q_tile = rem % q_tiles;

  __shared__ __attribute__((aligned(16))) char smem[2 * K_TILE + 2 * V_TILE];
  char* const kring = smem;
  char* const vring = smem + 2 * K_TILE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int grp = wave >> 2;
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

  const int64_t n_tiles = ceil_div(n_kv, ATT_BN);
  const int64_t last_kv0 = (n_tiles - 1) * ATT_BN;
  const bool ragged = (n_kv % ATT_BN) != 0;
  // this workgroup's key tiles [kt0, kt1); te is the last of them
  int64_t kt0 = 0, kt1 = n_tiles;
  if constexpr (SPLIT) key_range(n_tiles, splits, part, kt0, kt1);
  const int64_t te = kt1 - 1;
  const char* kbase = reinterpret_cast<const char*>(k + col0);
  const char* vbase = reinterpret_cast<const char*>(vt + col0 * ldvt);
  const int64_t k_tile_bytes = (int64_t)ATT_BN * ldk * 2;
  // Per-thread chunks: thread tid moves chunk tid % KCH of K rows tid / KCH +
  // i * (NTHR / KCH), and chunk tid % VCH of V^T rows tid / VCH + i * (NTHR /
  // VCH), so every offset is one per-thread value plus a uniform step in i.
  // In the last tile, K rows past n_kv are read from the last valid row and
  // V^T chunks that start past n_kv from the last valid chunk.
  constexpr int KRS = NTHR / KCH, VRS = NTHR / VCH;  // row steps between a thread's chunks
  static_assert(NTHR % KCH == 0 && NTHR % VCH == 0, "chunk rows");
  const int krow0 = tid / KCH, kch = tid % KCH;
  const int vrow0 = tid / VCH, vch = tid % VCH, vkey = vch * EPC;
  const uint32_t koff0 = (uint32_t)(((int64_t)krow0 * ldk + kch * EPC) * 2);
  const int kv_last = (int)(n_kv - last_kv0);  // valid keys in the last tile, 1..64
  const uint32_t kclamp = (uint32_t)(((int64_t)(kv_last - 1) * ldk + kch * EPC) * 2);
  const uint32_t kstep = (uint32_t)((int64_t)KRS * ldk * 2);
  const int64_t vkl = last_kv0 + vkey < n_kv ? vkey : ((n_kv - 1) & ~(int64_t)(EPC - 1)) - last_kv0;
  const uint32_t voff0 = (uint32_t)(((int64_t)vrow0 * ldvt + vkey) * 2);
  const uint32_t vclamp0 = (uint32_t)(((int64_t)vrow0 * ldvt + vkl) * 2);
  const uint32_t vstep = (uint32_t)((int64_t)VRS * ldvt * 2);
  const int kdst0 = krow0 * KRP + kch * 16;
  // keys 16j..16j+15 of a V^T row: slot 2j holds keys {0-3, 8-11}, slot
  // 2j+1 holds {4-7, 12-15}, the order in which P^T sits in the S^T registers
  const int vdst0 = vrow0 * VRP + (vch >> 1) * 32 + 8 * (vch & 1);

  u32x4 rk[K_LD], rv[V_LD];
  auto load_k = [&](int64_t t) {  // t <= n_tiles - 1
    const char* src = kbase + t * k_tile_bytes;
    const bool lt = t == n_tiles - 1;
#pragma unroll
    for (int i = 0; i < K_LD; ++i) {
      const bool clamp = lt && krow0 + i * KRS >= kv_last;
      rk[i] = *reinterpret_cast<const u32x4*>(src + (clamp ? kclamp : koff0 + i * kstep));
    }
  };
  auto load_v = [&](int64_t t) {
    const char* src = vbase + t * (int64_t)ATT_BN * 2;
    const uint32_t base = t == n_tiles - 1 ? vclamp0 : voff0;
#pragma unroll
    for (int i = 0; i < V_LD; ++i) rv[i] = *reinterpret_cast<const u32x4*>(src + base + i * vstep);
  };
  auto store_k = [&](int slot) {
#pragma unroll
    for (int i = 0; i < K_LD; ++i)
      *reinterpret_cast<u32x4*>(kring + slot * K_TILE + kdst0 + i * KRS * KRP) = rk[i];
  };
  auto store_v = [&](int slot, int64_t t) {  // t: the tile the staging registers hold
    if (ragged && t == n_tiles - 1) {  // keys past n_kv read as zero
      // (the empty asm keeps these compares here rather than hoisted out of
      // the key loop, where their results would hold registers throughout)
      int key = vkey;
      asm volatile("" : "+v"(key));
#pragma unroll
      for (int i = 0; i < V_LD; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo = key + 2 * w < kv_last ? 0x0000ffffu : 0u;
          const uint32_t hi = key + 2 * w + 1 < kv_last ? 0xffff0000u : 0u;
          rv[i][w] &= lo | hi;
        }
    }
    char* vs = vring + slot * V_TILE + vdst0;
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      *reinterpret_cast<u32x2*>(vs + i * VRS * VRP) = u32x2{rv[i][0], rv[i][1]};
      *reinterpret_cast<u32x2*>(vs + i * VRS * VRP + 16) = u32x2{rv[i][2], rv[i][3]};
    }
  };

  const int k_rd = l32 * KRP + half * 16;
  const int v_rd = l32 * VRP + half * 16;

  f32x16 acc_o[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t) acc_o[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const bf2 ones = __builtin_bit_cast(bf2, 0x3f803f80u);

  auto pair_max = [](float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };
  // P = exp2(s * c - m * c): the exponent is one explicit fused multiply-add
  // with m * c rounded first. settle() can run this a second time for a
  // whole wave; spelled out, both runs give a query that did not move the
  // same bits (left to the compiler, the second copy was contracted the
  // other way round, and a query's P then depended on its wave-mates).
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
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r0 + 2 * e], qk_scale_log2, -mc));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r0 + 2 * e + 1], qk_scale_log2, -mc));
        w[e] = pack_bf16x2(p0, p1);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w[e]), ones, lsum, false);
      }
      pb[j] = u32x4{w[0], w[1], w[2], w[3]};
    }
    return lsum;
  };
  auto tile_max = [&](const f32x16 (&s)[2]) {
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int q = 2; q < 16; ++q) mx = fmaxf(mx, s[0][q]);
#pragma unroll
    for (int q = 0; q < 16; ++q) mx = fmaxf(mx, s[1][q]);
    return pair_max(mx);
  };
  auto settle = [&](f32x16 (&s)[2], u32x4 (&pb)[4], float ls) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ls), __float_as_uint(ls), false, false);
    const bool move = !(__uint_as_float(r[0]) + __uint_as_float(r[1]) <= ATT_MOVE_SUM);
    if (__any(move)) {
      const float mx = tile_max(s);
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
  // keys past n_kv in the last tile: -inf (register r of block mt holds key
  // mt*32 + 8*(r/4) + 4*half + r%4)
  auto mask_last = [&](f32x16 (&s)[2]) {
    int thr = kv_last - 4 * half;
    asm volatile("" : "+v"(thr));  // compares stay here, not hoisted out of the key loop
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (mt * 32 + 8 * (r >> 2) + (r & 3) >= thr) s[mt][r] = -INFINITY;
  };
  auto phase_end = []() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: tile kt0 in slot 0, tile kt0+1 (or the range's last tile again)
  // in the staging registers
  load_k(kt0);
  load_v(kt0);
  store_k(0);
  store_v(0, kt0);
  {
    const int64_t t1 = kt0 + 1 < kt1 ? kt0 + 1 : te;
    load_k(t1);
    load_v(t1);
  }
  __syncthreads();
  if (grp == 1) phase_end();
  for (int64_t t = kt0; t < kt1; ++t) {
    const int cur = (int)((t - kt0) & 1);
    const int64_t t2 = t + 2 < kt1 ? t + 2 : te;
    // M1
    u32x4 kf[QS][2];
    {
      const char* ks = kring + cur * K_TILE + k_rd;
#pragma unroll
      for (int st = 0; st < QS; ++st) {
        kf[st][0] = *reinterpret_cast<const u32x4*>(ks + st * 32);
        kf[st][1] = *reinterpret_cast<const u32x4*>(ks + 32 * KRP + st * 32);
      }
    }
    store_k(cur ^ 1);
    load_k(t2);
    phase_end();
    // C1
    f32x16 s[2];
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int st = 0; st < QS; ++st)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        s[mt] = mfma32_bf16(__builtin_bit_cast(bf16x8, kf[st][mt]), __builtin_bit_cast(bf16x8, qf[st]), s[mt]);
    phase_end();
    // M2
    u32x4 vf[4][OT];
    {
      const char* vs = vring + cur * V_TILE + v_rd;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int ot = 0; ot < OT; ++ot) vf[j][ot] = *reinterpret_cast<const u32x4*>(vs + ot * 32 * VRP + j * 32);
    }
    // the LDS traffic of this phase (fragment reads, tile store) is issued
    // first and runs under the softmax
    if (ragged && t == n_tiles - 1) mask_last(s);
    if (t == kt0) m_run = tile_max(s);  // the first tile sets each query's running max exactly
    u32x4 pb[4];
    settle(s, pb, exp_tile(s, pb));
    store_v(cur ^ 1, t + 1 < kt1 ? t + 1 : te);
    load_v(t2);
    phase_end();
    // C2
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int ot = 0; ot < OT; ++ot)
        acc_o[ot] = mfma32_bf16(__builtin_bit_cast(bf16x8, vf[j][ot]), __builtin_bit_cast(bf16x8, pb[j]), acc_o[ot]);
    phase_end();
  }
  if (grp == 0) phase_end();

  const auto lr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float l_all = __uint_as_float(lr[0]) + __uint_as_float(lr[1]);
  // the output address is formed here from the thread id (passed through an
  // empty asm), not kept in registers across the key loop
  int tid_e = tid;
  asm volatile("" : "+v"(tid_e));
  const int64_t qr = q_tile * L::BM + (tid_e >> 6) * 32 + (tid_e & 31);
  if constexpr (SPLIT) {  // this range's unnormalised O, its m and l
    if (qr < n_q) {
      const int64_t n_heads = gridDim.x / ((int64_t)splits * q_tiles);
      const int64_t prow = (int64_t)part * n_q + qr;
      float* orow = sp.o_part + prow * (n_heads * DH) + col0;
#pragma unroll
      for (int t = 0; t < OT; ++t)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *reinterpret_cast<f32x4*>(orow + t * 32 + 8 * qd + 4 * half) =
              f32x4{acc_o[t][4 * qd], acc_o[t][4 * qd + 1], acc_o[t][4 * qd + 2], acc_o[t][4 * qd + 3]};
      if (half == 0) {
        float* ml = sp.ml_part + (prow * n_heads + head_idx) * 2;
        ml[0] = m_run;
        ml[1] = l_all;
      }
    }
    return;
  }
  const float inv = 1.0f / l_all;
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

// Merge of the key ranges, one thread per (query, 4 output columns): m =
// max_p m_p, w_p = exp2((m_p - m) * c), O = (sum_p w_p O_p) / (sum_p w_p l_p),
// the sums taken in order p = 0, 1, ...; every operation is fixed, so a
// query's O depends only on its own partials.
template <typename T>
__global__ __launch_bounds__(256) void attention_combine_kernel(const float* __restrict__ o_part,
                                                                const float* __restrict__ ml_part, T* __restrict__ o,
                                                                int64_t ldo, int64_t n_q, int n_heads, int head_dim,
                                                                int splits, float qk_scale_log2) {
  const int64_t d = (int64_t)n_heads * head_dim;
  const int64_t groups = d / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / groups;
  if (row >= n_q) return;
  const int64_t col = (idx % groups) * 4;
  const int64_t head = col / head_dim;
  float m = -INFINITY;
  for (int p = 0; p < splits; ++p) m = fmaxf(m, ml_part[(((int64_t)p * n_q + row) * n_heads + head) * 2]);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  for (int p = 0; p < splits; ++p) {
    const int64_t prow = (int64_t)p * n_q + row;
    const float* ml = ml_part + (prow * n_heads + head) * 2;
    const float w = __builtin_amdgcn_exp2f((ml[0] - m) * qk_scale_log2);
    l = __builtin_fmaf(w, ml[1], l);
    const f32x4 op = *reinterpret_cast<const f32x4*>(o_part + prow * d + col);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, op[e], acc[e]);
  }
  const float inv = 1.0f / l;
  T* orow = o + row * ldo + col;
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(orow) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  } else {
    *reinterpret_cast<u32x2*>(orow) =
        u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  }
}

template <int DH>
static hipError_t launch_att_bf16(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* vt,
                                  int64_t ldvt, void* o, int64_t ldo, int64_t n_q, int64_t n_kv, int n_heads,
                                  const AttSplit& sp, hipStream_t st) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)DH);
  // one-dimensional grid: the kernel derives (head, key range, query tile) from blockIdx.x
  dim3 grid((unsigned)(ceil_div(n_q, AttLayout<uint16_t, DH, 8>::BM) * n_heads * sp.splits)), block(512);
  if (sp.splits == 1) {
    hipLaunchKernelGGL((attention_bf16_kernel<DH, false>), grid, block, 0, st, static_cast<const uint16_t*>(q), ldq,
                       static_cast<const uint16_t*>(k), ldk, static_cast<const uint16_t*>(vt), ldvt,
                       static_cast<uint16_t*>(o), ldo, n_q, n_kv, scale_log2, sp);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((attention_bf16_kernel<DH, true>), grid, block, 0, st, static_cast<const uint16_t*>(q), ldq,
                     static_cast<const uint16_t*>(k), ldk, static_cast<const uint16_t*>(vt), ldvt,
                     static_cast<uint16_t*>(o), ldo, n_q, n_kv, scale_log2, sp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = n_q * (n_heads * DH / 4);
  hipLaunchKernelGGL((attention_combine_kernel<uint16_t>), dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, st,
                     sp.o_part, sp.ml_part, static_cast<uint16_t*>(o), ldo, n_q, n_heads, DH, sp.splits, scale_log2);
  return hipGetLastError();
}

template <typename T, int DH, int NW>
static hipError_t launch_att_t(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* vt,
                               int64_t ldvt, void* o, int64_t ldo, int64_t n_q, int64_t n_kv, int n_heads,
                               const AttSplit& sp, hipStream_t st) {
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)DH);
  dim3 grid((unsigned)ceil_div(n_q, AttLayout<T, DH, NW>::BM), (unsigned)n_heads, (unsigned)sp.splits),
      block(NW * 64);
  if (sp.splits == 1) {
    hipLaunchKernelGGL((attention_kernel<T, DH, NW, false>), grid, block, 0, st, static_cast<const T*>(q), ldq,
                       static_cast<const T*>(k), ldk, static_cast<const T*>(vt), ldvt, static_cast<T*>(o), ldo,
                       n_q, n_kv, scale_log2, sp);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((attention_kernel<T, DH, NW, true>), grid, block, 0, st, static_cast<const T*>(q), ldq,
                     static_cast<const T*>(k), ldk, static_cast<const T*>(vt), ldvt, static_cast<T*>(o), ldo,
                     n_q, n_kv, scale_log2, sp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = n_q * (n_heads * DH / 4);
  hipLaunchKernelGGL((attention_combine_kernel<T>), dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, st,
                     sp.o_part, sp.ml_part, static_cast<T*>(o), ldo, n_q, n_heads, DH, sp.splits, scale_log2);
  return hipGetLastError();
}

int64_t attention_splits_effective(int64_t splits, int64_t n_kv) {
  const int64_t tiles = ceil_div(n_kv, (int64_t)ATT_BN);
  return splits < tiles ? splits : tiles;
}

hipError_t launch_attention(int dtype, const void* q, int64_t ldq, const void* k, int64_t ldk,
                            const void* vt, int64_t ldvt, void* o, int64_t ldo, int64_t n_q,
                            int64_t n_kv, int n_heads, int head_dim, int64_t splits, float* o_part, float* ml_part,
                            hipStream_t st) {
  if (n_q <= 0) return hipSuccess;
  if (n_kv <= 0 || splits < 1) return hipErrorInvalidValue;
  // per-thread offsets into a V^T tile are 32-bit: head_dim rows of ldvt elements
  if ((int64_t)head_dim * ldvt * (dtype == F32 ? 4 : 2) >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
  AttSplit sp{(int)attention_splits_effective(splits, n_kv), o_part, ml_part};
  if (sp.splits > 1 && (!o_part || !ml_part)) return hipErrorInvalidValue;
  if (dtype == F32) {
    if (head_dim == 64) return launch_att_t<float, 64, 4>(q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, n_heads, sp, st);
    if (head_dim == 128) return launch_att_t<float, 128, 4>(q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, n_heads, sp, st);
  } else {
    if (head_dim == 64) return launch_att_bf16<64>(q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, n_heads, sp, st);
    if (head_dim == 128) return launch_att_bf16<128>(q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, n_heads, sp, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dit
