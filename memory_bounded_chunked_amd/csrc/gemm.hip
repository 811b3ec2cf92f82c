// K2: C[M][N] = A[M][K] * B[N][K]^T on MFMA, with fused epilogues.
//
// A holds token rows (activations), B holds weight rows [out][in]; both are
// K-contiguous, which is the operand layout MFMA consumes directly. A
// 256-row tile of A and a BN-row tile of B are staged through LDS (double
// buffered: the next k-tile's global loads are in flight while the current
// one is multiplied); WM x WN wavefronts (8 for BN = 256 or 128: two per
// SIMD) each compute a (256/WM) x (BN/WN) block with accumulators in VGPRs.
// With 8 waves and bf16 weights the two waves of each SIMD run one phase
// apart (the two-group schedule at the main loop), so one multiplies while
// the other reads LDS.
// LDS rows hold 128 B of k and are padded to 144 B:
// consecutive rows start 4 banks apart, so fragment reads are conflict-free
// and their addresses are a per-lane base plus compile-time offsets.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs, each with its
// own L2. The hardware workgroup id is remapped so that each XCD owns a
// contiguous range of tiles, walked in groups of 4 tile rows; the 32
// workgroups an XCD runs at once then cover a 4 x 8 block of tiles and share
// their A and B k-slices through that XCD's L2.
//
// Each output element is the same fixed sequence: 32x32x16 bf16 MFMA (or
// 32x32x2 fp32 MFMA for the F32 block) accumulations over k in increasing
// k-tile order, followed by the epilogue. That sequence does not depend on
// M, on the tile's position or on which token slab is being projected, so a
// row's result is bit-identical however the tokens are sliced ("How the
// slicing works": the projections and the MLP are token-wise).
//
// Weight-only int8 (W8_BF16): B is int8 in HBM and is widened exactly to bf16
// on its way into LDS (|q| <= 127 needs 7 significant bits); the per-row scale
// multiplies the fp32 accumulator in the epilogue.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace dit {

constexpr int LDS_ROW = 144;  // 128 B of k per row + 16 B pad

__device__ __forceinline__ int lds_slot(int row, int chunk) { return row * LDS_ROW + chunk * 16; }

// Logical tile of hardware workgroup `bid` (see the tile-order note above).
__device__ __forceinline__ void tile_of(int64_t bid, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                        int64_t& tn) {
  constexpr int64_t GM = 4;
  const int64_t l = xcd_contiguous(bid, tiles_m * tiles_n);
  const int64_t grp = l / (GM * tiles_n);
  const int64_t rows = (tiles_m - grp * GM) < GM ? (tiles_m - grp * GM) : GM;
  const int64_t within = l - grp * GM * tiles_n;
  tm = grp * GM + within % rows;
  tn = within / rows;
}

// 16 int8 -> 16 bf16 (exact): each byte converts to fp32 exactly and every
// |q| <= 127 is a bf16 value, so the rounding conversion of each pair
// (v_cvt_pk_bf16_f32) is exact too.
__device__ __forceinline__ void i8x16_to_bf16(const u32x4& q, u32x4& lo, u32x4& hi) {
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t v = q[j];
    const float f0 = (float)(int8_t)(v & 0xff);
    const float f1 = (float)(int8_t)((v >> 8) & 0xff);
    const float f2 = (float)(int8_t)((v >> 16) & 0xff);
    const float f3 = (float)(int8_t)(v >> 24);
    w[2 * j] = pack_bf16x2(f0, f1);
    w[2 * j + 1] = pack_bf16x2(f2, f3);
  }
  lo = u32x4{w[0], w[1], w[2], w[3]};
  hi = u32x4{w[4], w[5], w[6], w[7]};
}

template <typename T>
__device__ __forceinline__ float load_act(const T* p) {
  if constexpr (sizeof(T) == 2)
    return bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
  else
    return *p;
}
template <typename T>
__device__ __forceinline__ void store_act(T* p, float v) {
  if constexpr (sizeof(T) == 2)
    *reinterpret_cast<uint16_t*>(p) = f32_to_bf16(v);
  else
    *p = v;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// Lane data movement inside a row of 16 lanes (DPP), without the LDS crossbar.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_XOR1 = 0xb1;         // quad_perm [1, 0, 3, 2]
constexpr int DPP_XOR2 = 0x4e;         // quad_perm [2, 3, 0, 1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i of 8 <-> 7 - i
constexpr int DPP_MIRROR = 0x140;       // lane i of 16 <-> 15 - i

// Sum over the 32 lanes of each half-wave. Every step adds two values that
// every lane of the pair holds identically (a + b and b + a are the same
// float), so all 32 lanes end with the same bits, and the order of the sum
// is fixed by the lane positions alone.
__device__ __forceinline__ float half_wave_sum(float t) {
  t += dpp_f32<DPP_XOR1>(t);
  t += dpp_f32<DPP_XOR2>(t);
  t += dpp_f32<DPP_HALF_MIRROR>(t);
  t += dpp_f32<DPP_MIRROR>(t);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LO: whether the kernel carries the adapter phase. int8-weight kernels come
// in both forms, because that phase follows their main loop and its
// registers would otherwise cost every int8 launch (spills after the loop);
// the others always carry it (it runs before the loop, or in fp32).
// QKD: head size of the QK RMSNorm / RoPE epilogue (EPI_STORE and EPI_KV
// only; 64 or 128), or 0 for the form without it, which launches without
// those transforms run.
template <typename TA, typename TB, int EPI, int BM, int BN, int WM, int WN, bool LO, int QKD>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(const GemmArgs g) {
  constexpr int NTHR = WM * WN * 64;
  constexpr bool A_F32 = sizeof(TA) == 4;
  constexpr bool B_I8 = sizeof(TB) == 1;
  constexpr int BK = A_F32 ? 32 : 64;  // k elements per tile: 128 B of an A row
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MT = WTM / 32, NTL = WTN / 32;
  constexpr int A_LD = BM * 8 / NTHR;
  constexpr int B_GROW = B_I8 ? 4 : 8;  // 16-B global chunks per B tile row
  constexpr int B_LD = BN * B_GROW / NTHR;
  constexpr int STAGE = (BM + BN) * LDS_ROW;
  static_assert(BM * 8 % NTHR == 0 && BN * B_GROW % NTHR == 0, "tile/threads");
  static_assert(EPI != EPI_GATEUP || NTL % 2 == 0, "gate/up tiles come in pairs");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  constexpr int OUT_BN = (EPI == EPI_GATEUP) ? BN / 2 : BN;
  const int64_t tiles_n = (g.N - g.col0) / OUT_BN;
  int64_t tm, tn;
  tile_of(blockIdx.x, ceil_div(g.M, BM), tiles_n, tm, tn);
  tn += g.col0 / OUT_BN;  // this launch covers output columns [col0, N)
  const int64_t m0 = tm * BM;

  const char* A = static_cast<const char*>(g.a);
  const char* B = static_cast<const char*>(g.b);

  // Global source of B tile row r.
  auto b_row = [&](int r) -> int64_t {
    if constexpr (EPI == EPI_GATEUP) {
      const int grp = r >> 5;
      const int64_t feat = tn * (BN / 2) + (grp >> 1) * 32 + (r & 31);
      return feat + ((grp & 1) ? g.up_offset : 0);
    } else {
      return tn * BN + r;
    }
  };

  // Global loads: a uniform base advanced per k-tile plus a 32-bit byte
  // offset per thread and chunk (row * ld + chunk), fixed for the whole loop.
  // Tile rows past the last token row load that last row again: an output
  // row depends only on its own A row, and rows past M are never stored, so
  // the loads need no branch (which also lets the compiler count them exactly
  // when it waits for them).
  uint32_t aoff[A_LD], boff[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int c = tid + i * NTHR;
    const int64_t gr = m0 + (c >> 3) < g.M ? m0 + (c >> 3) : g.M - 1;
    aoff[i] = (uint32_t)((gr - m0) * g.lda * (int64_t)sizeof(TA) + (c & 7) * 16);
  }
  const int64_t b_first = b_row(0);
  bool bval[B_LD];  // EPI_LORA_T: B rows past n_valid read as zero
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int c = tid + i * NTHR;
    bval[i] = EPI != EPI_LORA_T || b_row(c / B_GROW) < g.n_valid;
    boff[i] = bval[i] ? (uint32_t)((b_row(c / B_GROW) - b_first) * g.ldb * (int64_t)sizeof(TB) + (c % B_GROW) * 16)
                      : 0u;
  }
  const char* a_base = A + m0 * g.lda * (int64_t)sizeof(TA);
  const char* b_base = B + b_first * g.ldb * (int64_t)sizeof(TB);

  // One register staging set: tile kt+1 is written from it to LDS while
  // tile kt is multiplied, then it is refilled with tile kt+2 (see below).
  u32x4 ra[A_LD], rb[B_LD];
  auto load_a = [&](int64_t k0) {
    const char* at = a_base + k0 * (int64_t)sizeof(TA);
#pragma unroll
    for (int i = 0; i < A_LD; ++i)
      ra[i] = *reinterpret_cast<const u32x4*>(at + aoff[i]);
  };
  auto load_b = [&](int64_t k0) {
    const char* bt = b_base + k0 * (int64_t)sizeof(TB);
#pragma unroll
    for (int i = 0; i < B_LD; ++i)
      rb[i] = bval[i] ? *reinterpret_cast<const u32x4*>(bt + boff[i]) : u32x4{0u, 0u, 0u, 0u};
  };
  auto load_tiles = [&](int64_t k0) {
    load_a(k0);
    load_b(k0);
  };
  auto store_a = [&](int buf) {
    char* As = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int c = tid + i * NTHR;
      *reinterpret_cast<u32x4*>(As + lds_slot(c >> 3, c & 7)) = ra[i];
    }
  };
  auto store_b = [&](int buf) {
    char* Bs = smem + buf * STAGE + BM * LDS_ROW;
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int c = tid + i * NTHR;
      const int r = c / B_GROW, ch = c % B_GROW;
      if constexpr (B_I8) {
        u32x4 lo, hi;
        i8x16_to_bf16(rb[i], lo, hi);
        *reinterpret_cast<u32x4*>(Bs + lds_slot(r, 2 * ch)) = lo;
        *reinterpret_cast<u32x4*>(Bs + lds_slot(r, 2 * ch + 1)) = hi;
      } else {
        *reinterpret_cast<u32x4*>(Bs + lds_slot(r, ch)) = rb[i];
      }
    }
  };
  auto store_tiles = [&](int buf) {
    store_a(buf);
    store_b(buf);
  };

  f32x16 acc[MT][NTL];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTL; ++j) acc[i][j] = f32x16{};

  const int arow = wm * WTM + (lane & 31);
  const int brow = wn * WTN + (lane & 31);
  const int half = lane >> 5;

  // ---- activation-space adapter phase (see GemmArgs): the adapter term joins
  // the same fp32 accumulator as the main contraction, so the output is
  // rounded once. Except for int8 weights it runs first, into the zeroed
  // accumulator, while no main-loop state is live. A-operand fragments come from t (fp32; for bf16 as a
  // rounded value plus its residual), B-operand fragments from the adapter's
  // B rows, both straight from global memory (both are small and stay in L2).
  auto lora_phase = [&]() {
    if constexpr (EPI != EPI_LORA_T) {
      // The lane id passes through an empty asm here, so nothing derived from
      // it is computed before the main loop and held in registers across it.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int l32 = ln & 31, hf = ln >> 5;
      int64_t brow[NTL], sidx[NTL];
#pragma unroll
      for (int j = 0; j < NTL; ++j) {
        if constexpr (EPI == EPI_GATEUP) {
          const int64_t f = tn * (BN / 2) + ((wn * NTL + j) >> 1) * 32 + l32;
          brow[j] = f;
          sidx[j] = f + ((j & 1) ? g.up_offset : 0);
        } else {
          const int64_t col = tn * BN + wn * WTN + j * 32 + l32;
          brow[j] = (EPI == EPI_KV && col >= g.split) ? col - g.split : col;
          sidx[j] = col;
        }
      }
      if constexpr (B_I8) {  // the weight's per-row scale belongs to W a only
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
          const float sc = g.bscale[sidx[j]];
#pragma unroll
          for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] *= sc;
        }
      }
      // One k loop per segment; a tile's columns belong to segment `SG` when
      // seg[j] == SG (GATEUP: j parity; KV: the whole tile; else segment 0).
      auto lora_seg = [&](auto sg_c) {
        constexpr int SG = decltype(sg_c)::value;
        constexpr int KS = A_F32 ? 2 : 16;  // k per MFMA
        const int64_t r = g.lora_r[SG];
        const TA* bbase = static_cast<const TA*>(g.lora_b[SG]);
        // bf16: t enters as two bf16 terms, its rounded value (first sweep)
        // and the rounding residual (second sweep), so the adapter adds no
        // rounding point of its own (t is carried to about 2^-17 relative).
        // One term per sweep keeps few registers live.
        auto sweep = [&](auto part_c) {
          constexpr int PART = decltype(part_c)::value;
          for (int64_t k0 = 0; k0 < r; k0 += KS) {
            const int64_t kk = g.lora_toff[SG] + k0 + (A_F32 ? hf : 8 * hf);
            u32x4 bfr[NTL];
            float bf32[NTL];
#pragma unroll
            for (int j = 0; j < NTL; ++j) {
              if (EPI == EPI_GATEUP && (j & 1) != SG) continue;
              const TA* bp = bbase + brow[j] * r + k0;
              if constexpr (A_F32)
                bf32[j] = load_act(bp + hf);
              else
                bfr[j] = *reinterpret_cast<const u32x4*>(bp + 8 * hf);
            }
#pragma unroll
            for (int i = 0; i < MT; ++i) {
              const int64_t row = m0 + wm * WTM + i * 32 + l32;
              const float* tp = g.lora_t + (row < g.M ? row : 0) * g.lora_ldt + kk;
              if constexpr (A_F32) {
                const float av = row < g.M ? *tp : 0.f;
#pragma unroll
                for (int j = 0; j < NTL; ++j)
                  if (EPI != EPI_GATEUP || (j & 1) == SG) acc[i][j] = mfma32_f32(av, bf32[j], acc[i][j]);
              } else {
                f32x4 t0 = f32x4{0.f, 0.f, 0.f, 0.f}, t1 = t0;
                if (row < g.M) {
                  t0 = *reinterpret_cast<const f32x4*>(tp);
                  t1 = *reinterpret_cast<const f32x4*>(tp + 4);
                }
                const float tv[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
                uint32_t wv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  wv[q] = pack_bf16x2(tv[2 * q], tv[2 * q + 1]);
                  if constexpr (PART == 1)
                    wv[q] = pack_bf16x2(tv[2 * q] - __uint_as_float(wv[q] << 16),
                                        tv[2 * q + 1] - __uint_as_float(wv[q] & 0xffff0000u));
                }
                const u32x4 af = u32x4{wv[0], wv[1], wv[2], wv[3]};
#pragma unroll
                for (int j = 0; j < NTL; ++j)
                  if (EPI != EPI_GATEUP || (j & 1) == SG)
                    acc[i][j] = mfma32_bf16(__builtin_bit_cast(bf16x8, af), __builtin_bit_cast(bf16x8, bfr[j]),
                                            acc[i][j]);
              }
            }
          }
        };
        if constexpr (A_F32) {
          sweep(std::integral_constant<int, 0>{});
        } else {
          // bf16: t and the adapter's B rows for this tile are staged through
          // LDS in rank chunks of 64 (all global loads of a chunk in flight
          // at once), then the two sweeps read their fragments from LDS. The
          // accumulation order is that of the two sweeps above.
          constexpr int RC = 64;                      // rank chunk
          constexpr int TROW = RC * 4 + 16;           // LDS row of t (fp32), padded
          constexpr int BROW = RC * 2 + 16;           // LDS row of B (bf16), padded
          constexpr int T_CH = BM * (RC / 4), B_CH = BN * (RC / 8);  // 16-B chunks
          static_assert(BM * TROW + BN * BROW <= 2 * STAGE, "adapter staging fits the tile buffers");
          static_assert(T_CH % NTHR == 0 && B_CH % NTHR == 0, "adapter staging chunks");
          char* const ts = smem;
          char* const bs = smem + BM * TROW;
          // Chunk job j < NTJ moves a 16-B piece of t, job NTJ + q a 16-B piece
          // of B. With int8 weights (this phase then follows the main loop,
          // every accumulator live) the jobs run in batches of 4 to keep the
          // staging registers few; otherwise all loads are in flight at once.
          constexpr int NTJ = T_CH / NTHR, NBJ = B_CH / NTHR, NJ = NTJ + NBJ;
          constexpr int BATCH = B_I8 ? 4 : NJ;
          auto stage = [&](int64_t c0) {
            const int64_t kc = r - c0 < RC ? r - c0 : RC;
            auto load_job = [&](int j) -> u32x4 {
              if (j < NTJ) {
                const int c = tid + j * NTHR, row = c / (RC / 4), ch = c % (RC / 4);
                const int64_t gr = m0 + row < g.M ? m0 + row : g.M - 1;
                const int64_t col = ch * 4 < kc ? g.lora_toff[SG] + c0 + ch * 4 : g.lora_toff[SG] + c0;
                return *reinterpret_cast<const u32x4*>(g.lora_t + gr * g.lora_ldt + col);
              }
              const int c = tid + (j - NTJ) * NTHR, cb = c / (RC / 8), ch = c % (RC / 8);
              int64_t brw;  // adapter row of tile column cb (any valid row for other segments)
              if constexpr (EPI == EPI_GATEUP) {
                brw = tn * (BN / 2) + ((cb >> 5) >> 1) * 32 + (cb & 31);
              } else {
                const int64_t colg = tn * BN + cb;
                brw = (EPI == EPI_KV && colg >= g.split) ? colg - g.split : colg;
              }
              const int64_t kk = ch * 8 < kc ? c0 + ch * 8 : c0;
              return *reinterpret_cast<const u32x4*>(bbase + brw * r + kk);
            };
            auto store_job = [&](int j, const u32x4& v) {
              if (j < NTJ) {
                const int c = tid + j * NTHR;
                *reinterpret_cast<u32x4*>(ts + (c / (RC / 4)) * TROW + (c % (RC / 4)) * 16) = v;
              } else {
                const int c = tid + (j - NTJ) * NTHR;
                *reinterpret_cast<u32x4*>(bs + (c / (RC / 8)) * BROW + (c % (RC / 8)) * 16) = v;
              }
            };
#pragma unroll
            for (int j0 = 0; j0 < NJ; j0 += BATCH) {
              u32x4 rr[BATCH];
#pragma unroll
              for (int q = 0; q < BATCH; ++q)
                if (j0 + q < NJ) rr[q] = load_job(j0 + q);
              if (j0 == 0) __syncthreads();  // every wave is done with the previous contents
#pragma unroll
              for (int q = 0; q < BATCH; ++q)
                if (j0 + q < NJ) store_job(j0 + q, rr[q]);
            }
            __syncthreads();
          };
          auto sweep_lds = [&](auto part_c, int64_t c0) {
            constexpr int PART = decltype(part_c)::value;
            const int64_t kc = r - c0 < RC ? r - c0 : RC;
            for (int64_t k0 = 0; k0 < kc; k0 += 16) {
              u32x4 bfr[NTL];
#pragma unroll
              for (int j = 0; j < NTL; ++j) {
                if (EPI == EPI_GATEUP && (j & 1) != SG) continue;
                bfr[j] = *reinterpret_cast<const u32x4*>(bs + (wn * WTN + j * 32 + l32) * BROW + (k0 + 8 * hf) * 2);
              }
#pragma unroll
              for (int i = 0; i < MT; ++i) {
                const char* tp = ts + (wm * WTM + i * 32 + l32) * TROW + (k0 + 8 * hf) * 4;
                const f32x4 t0 = *reinterpret_cast<const f32x4*>(tp);
                const f32x4 t1 = *reinterpret_cast<const f32x4*>(tp + 16);
                const float tv[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
                uint32_t wv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  wv[q] = pack_bf16x2(tv[2 * q], tv[2 * q + 1]);
                  if constexpr (PART == 1)
                    wv[q] = pack_bf16x2(tv[2 * q] - __uint_as_float(wv[q] << 16),
                                        tv[2 * q + 1] - __uint_as_float(wv[q] & 0xffff0000u));
                }
                const u32x4 af = u32x4{wv[0], wv[1], wv[2], wv[3]};
#pragma unroll
                for (int j = 0; j < NTL; ++j)
                  if (EPI != EPI_GATEUP || (j & 1) == SG)
                    acc[i][j] = mfma32_bf16(__builtin_bit_cast(bf16x8, af), __builtin_bit_cast(bf16x8, bfr[j]),
                                            acc[i][j]);
              }
            }
          };
          if (r <= RC) {
            if (r > 0) {
              stage(0);
              sweep_lds(std::integral_constant<int, 0>{}, 0);
              sweep_lds(std::integral_constant<int, 1>{}, 0);
            }
          } else {
            for (int64_t c0 = 0; c0 < r; c0 += RC) {
              stage(c0);
              sweep_lds(std::integral_constant<int, 0>{}, c0);
            }
            for (int64_t c0 = 0; c0 < r; c0 += RC) {
              stage(c0);
              sweep_lds(std::integral_constant<int, 1>{}, c0);
            }
          }
        }
      };
      if constexpr (EPI == EPI_GATEUP) {
        lora_seg(std::integral_constant<int, 0>{});
        lora_seg(std::integral_constant<int, 1>{});
      } else if constexpr (EPI == EPI_KV) {
        if (tn * BN < g.split)  // uniform per workgroup: the split is tile-aligned
          lora_seg(std::integral_constant<int, 0>{});
        else
          lora_seg(std::integral_constant<int, 1>{});
      } else {
        lora_seg(std::integral_constant<int, 0>{});
      }
    }
  };

  const int a_rd = lds_slot(arow, half), b_rd = lds_slot(brow, half);
  // Fragments of k-steps s0 and s0+1 of the tile in LDS buffer buf, and
  // their MFMAs (for each accumulator, k-step s0 before s0+1).
  auto read_frags = [&](int buf, int s0, u32x4 (&af)[2][MT], u32x4 (&bfr)[2][NTL]) {
    const char* As = smem + buf * STAGE + a_rd;
    const char* Bs = smem + buf * STAGE + BM * LDS_ROW + b_rd;
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
        af[ss][i] = *reinterpret_cast<const u32x4*>(As + i * 32 * LDS_ROW + (s0 + ss) * 32);
#pragma unroll
      for (int j = 0; j < NTL; ++j)
        bfr[ss][j] = *reinterpret_cast<const u32x4*>(Bs + j * 32 * LDS_ROW + (s0 + ss) * 32);
    }
  };
  auto mfma_frags = [&](const u32x4 (&af)[2][MT], const u32x4 (&bfr)[2][NTL]) {
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTL; ++j)
          acc[i][j] = mfma32_bf16(__builtin_bit_cast(bf16x8, af[ss][i]), __builtin_bit_cast(bf16x8, bfr[ss][j]),
                                  acc[i][j]);
  };
  auto compute = [&](int buf) {
    const char* As = smem + buf * STAGE + a_rd;
    const char* Bs = smem + buf * STAGE + BM * LDS_ROW + b_rd;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 af[MT], bfr[NTL];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(As + i * 32 * LDS_ROW + s * 32);
#pragma unroll
      for (int j = 0; j < NTL; ++j)
        bfr[j] = *reinterpret_cast<const u32x4*>(Bs + j * 32 * LDS_ROW + s * 32);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
          if constexpr (A_F32) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
              acc[i][j] = mfma32_f32(__uint_as_float(af[i][t]), __uint_as_float(bfr[j][t]), acc[i][j]);
          } else {
            acc[i][j] = mfma32_bf16(__builtin_bit_cast(bf16x8, af[i]), __builtin_bit_cast(bf16x8, bfr[j]),
                                    acc[i][j]);
          }
        }
    }
  };

  // k-tile kt is multiplied from LDS buffer kt & 1. While it is, tile kt+1
  // (loaded from HBM during the previous iteration) goes from the staging
  // registers into the other buffer, whose previous tile every wave finished
  // before the last barrier, and the staging registers are refilled with
  // tile kt+2. One barrier per k-tile.
  const int KT = (int)(g.K / BK);
  if constexpr (!B_I8) {
    if (g.lora_t != nullptr) {
      lora_phase();
      __syncthreads();  // the adapter staging area is the tile buffers
    }
  }
  load_tiles(0);
  store_tiles(0);
  if (KT > 1) load_tiles(BK);
  __syncthreads();
  // Two-group schedule for 8 waves (bf16 weights). Waves 0-3 and 4-7 each
  // hold one wave per SIMD, and group 1 runs one phase behind group 0, so on
  // every SIMD one wave issues MFMAs while the other reads its next
  // fragments from LDS and moves the next tile in. A k-tile is four phases,
  // each closed by a workgroup barrier:
  //   M1: read fragments of k-steps 0-1; store A of tile kt+1 into the other
  //       buffer, then load A of tile kt+2 into the staging registers
  //   C1: MFMAs of k-steps 0-1
  //   M2: read fragments of k-steps 2-3; store B of tile kt+1, load B of kt+2
  //   C2: MFMAs of k-steps 2-3
  // Tile kt+1 is complete in LDS (both groups' stores) before either group
  // reads it, and the buffer it overwrites was last read (tile kt-1) before
  // the barrier that opens the first store; the barriers count the same for
  // both groups (group 1 takes one more before the loop, group 0 one more
  // after it). Each accumulator still takes k-steps 0, 1, 2, 3 of each tile in
  // order, as in the one-group schedule.
  // With int8 weights the B stores of M2 carry the widening to bf16 (one
  // conversion per weight, one packing conversion per pair).
  constexpr bool PP = !A_F32 && WM * WN == 8;
  int kt = 0;
  if constexpr (PP) {
    const int grp = wave >> 2;
    auto phase_end = []() {
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    if (grp == 1) phase_end();
    u32x4 af[2][MT], bfr[2][NTL];
    // The last two iterations reload the last k-tile and store it into the
    // buffer no later phase reads, so every iteration has the same shape.
    const int64_t k_last = (int64_t)(KT - 1) * BK;
    for (; kt < KT; ++kt) {
      const int cur = kt & 1;
      const int64_t k_next2 = (int64_t)(kt + 2) * BK < k_last ? (int64_t)(kt + 2) * BK : k_last;
      read_frags(cur, 0, af, bfr);
      store_a(cur ^ 1);
      load_a(k_next2);
      phase_end();
      mfma_frags(af, bfr);
      phase_end();
      read_frags(cur, 2, af, bfr);
      store_b(cur ^ 1);
      load_b(k_next2);
      phase_end();
      mfma_frags(af, bfr);
      phase_end();
    }
    if (grp == 0) phase_end();
  } else {
    for (; kt + 2 < KT; ++kt) {
      compute(kt & 1);
      store_tiles((kt + 1) & 1);
      load_tiles((int64_t)(kt + 2) * BK);
      __syncthreads();
    }
    if (kt + 1 < KT) {
      compute(kt & 1);
      store_tiles((kt + 1) & 1);
      __syncthreads();
      ++kt;
    }
    compute(kt & 1);
  }

  // int8 weights: the adapter term joins after the contraction and the
  // per-row scale (which belongs to W a only) is applied before it.
  bool scaled = B_I8;  // the per-row weight scale still has to be applied
  if constexpr (B_I8 && LO) {
    if (g.lora_t != nullptr) {
      lora_phase();
      scaled = false;
    }
  }
  // Weight scale of output column c. The load carries no branch (the scale
  // array is always present with int8 weights): a value loaded under a
  // branch makes the compiler wait for every outstanding memory operation,
  // stores included, wherever the value is used.
  auto col_scale = [&](int64_t c) -> float {
    if constexpr (B_I8) {
      const float v = g.bscale[c];
      return scaled ? v : 1.f;
    } else {
      return 1.f;
    }
  };

  // QK RMSNorm and RoPE of the stored columns (Q, and the K columns of the K|V
  // launch), on the fp32 accumulators before the one rounding to the output
  // type. A wave's columns are 64 wide (WTN = 64 for every tile shape): one
  // head of 64, or half a head of 128 whose other half is in wave wn ^ 1. Per
  // token row and head: t <- t / sqrt(mean(t^2) + eps) * w, then (t[2j],
  // t[2j+1]) <- (a c - b s, a s + b c) with c, s the row's angle j. The sum of
  // squares is reduced over the 32 lanes of a half-wave (half_wave_sum) and,
  // for heads of 128, added to the partner wave's through LDS as (even wave) +
  // (odd wave); every step is fixed, so a row's result depends only on that
  // row, whatever tile computes it.
  auto qk_apply = [&]() {
    static_assert(WTN == 64, "qk epilogue assumes 64-column wave tiles");
    constexpr int HD = QKD > 0 ? QKD : 64, HP = HD / 2;  // head size, angles per row
    const int l32 = lane & 31;
    if constexpr (B_I8) {  // the per-row scale belongs to the projection, before the norm
#pragma unroll
      for (int j = 0; j < NTL; ++j) {
        const float sc = col_scale(tn * BN + wn * WTN + j * 32 + l32);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] *= sc;
      }
      scaled = false;
    }
    // One 32-row block of every wave at a time. The rows' RoPE angles (cos
    // then sin) are staged through LDS with coalesced 16-byte loads: for every
    // block at once when they fit beside the partial sums (256-wide tiles),
    // else block by block. The partial sums of squares go through LDS to the
    // partner wave.
    const bool norm = g.qk_w != nullptr, rope = g.rope_cs != nullptr;
    constexpr int SROWS = WM * 32;               // rows of one block over the workgroup
    constexpr int RED = WN * SROWS * 4;          // bytes of the partial sums
    constexpr int CPR = HP / 4;                  // 16-byte angle chunks per row
    constexpr bool ALL = (int)sizeof(smem) >= MT * SROWS * HP * 8 + RED;  // stage every block at once
    constexpr int NB = ALL ? MT : 1;             // blocks per staging
    float* const ang = reinterpret_cast<float*>(smem);  // [NB][2][SROWS][HP]: cos, then sin
    float* const red = ang + NB * 2 * SROWS * HP;       // [WN][SROWS]
    auto stage = [&](int i0) {  // angles of blocks i0 .. i0 + NB - 1
      constexpr int CHUNKS = NB * SROWS * CPR;   // per table
      for (int c = tid; c < 2 * CHUNKS; c += NTHR) {
        const int tab = c >= CHUNKS, cc = c - tab * CHUNKS;
        const int bi = cc / (SROWS * CPR), sr = (cc / CPR) % SROWS, ch = cc % CPR;
        int64_t row = m0 + (sr >> 5) * WTM + (i0 + bi) * 32 + (sr & 31);
        row = row < g.M ? row : g.M - 1;
        const float* src = (tab ? g.rope_sn : g.rope_cs) + row * g.ld_rope + ch * 4;
        *reinterpret_cast<f32x4*>(ang + ((bi * 2 + tab) * SROWS + sr) * HP + ch * 4) =
            *reinterpret_cast<const f32x4*>(src);
      }
    };
    float wv[NTL];
#pragma unroll
    for (int j = 0; j < NTL; ++j) wv[j] = norm ? g.qk_w[(wn * WTN + j * 32 + l32) % HD] : 1.f;
    const int jp0 = ((wn * WTN + l32) % HD) >> 1;  // angle index of this lane's pair in column block 0
    // rotation of a pair (a, b) = (t[2j], t[2j+1]): the even lane forms
    // a c - b s, the odd lane b c + a s, i.e. self * c + other * (+-s)
    const float sgn = (l32 & 1) ? 1.f : -1.f;
    if (ALL) {
      __syncthreads();  // the tile buffers are no longer read
      if (rope) stage(0);
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      float ss[16];
      if (norm) {
        // the 16 rows' sums side by side, step by step (independent chains)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float t = 0.f;
#pragma unroll
          for (int j = 0; j < NTL; ++j) t = __builtin_fmaf(acc[i][j][r], acc[i][j][r], t);
          ss[r] = t;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) ss[r] += dpp_f32<DPP_XOR1>(ss[r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) ss[r] += dpp_f32<DPP_XOR2>(ss[r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) ss[r] += dpp_f32<DPP_HALF_MIRROR>(ss[r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) ss[r] += dpp_f32<DPP_MIRROR>(ss[r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(ss[r]), __float_as_uint(ss[r]), false, false);
          ss[r] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        }
      }
      const int bi = ALL ? i : 0;  // the block's place in the staged angles
      if (!ALL || (norm && HD == 128)) {
        __syncthreads();  // the previous block's angles and sums (or the tile buffers) are no longer read
        if (!ALL && rope) stage(i);
        if (norm && HD == 128 && l32 == 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) red[wn * SROWS + wm * 32 + 8 * (r >> 2) + 4 * half + (r & 3)] = ss[r];
        }
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int br = wm * 32 + 8 * (r >> 2) + 4 * half + (r & 3);  // the row's place in the staged block
        if (norm) {
          const float tot = HD == 128 ? red[(wn & ~1) * SROWS + br] + red[(wn | 1) * SROWS + br] : ss[r];
          const float rr = 1.0f / sqrtf(tot * (1.0f / HD) + g.qk_eps);
#pragma unroll
          for (int j = 0; j < NTL; ++j) acc[i][j][r] = acc[i][j][r] * rr * wv[j];
        }
      }
      if (rope) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int br = wm * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const float* ac = ang + (bi * 2) * SROWS * HP + br * HP;
          const float* as = ac + SROWS * HP;
#pragma unroll
          for (int j = 0; j < NTL; ++j) {
            const int jp = (jp0 + j * 16) % HP;  // column block j is 32 columns, 16 pairs, further on
            const float self = acc[i][j][r];
            const float other = dpp_f32<DPP_XOR1>(self);
            acc[i][j][r] = __builtin_fmaf(other, as[jp] * sgn, self * ac[jp]);
          }
        }
      }
    }
  };

  // ---- epilogue: lane holds C[8*(r/4) + 4*half + r%4][lane%32] of each 32x32 tile
  if constexpr (EPI == EPI_GATEUP) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int p = 0; p < NTL / 2; ++p) {
        const int64_t f = tn * (BN / 2) + ((wn * NTL + 2 * p) >> 1) * 32 + (lane & 31);
        const float sg = col_scale(f), su = col_scale(f + g.up_offset);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (row < g.M) {
            const float gv = acc[i][2 * p][r] * sg;
            const float uv = acc[i][2 * p + 1][r] * su;
            store_act(static_cast<TA*>(g.out) + row * g.ldo + f, silu_f32(gv) * uv);
          }
        }
      }
  } else if constexpr (EPI == EPI_STORE_T || EPI == EPI_KV) {
    // transposed store: four consecutive rows of one column per 8-byte write
    auto store_t = [&](TA* out, int64_t ldo, int64_t col_base) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
          const int64_t col = tn * BN + wn * WTN + j * 32 + (lane & 31);
          const float sc = col_scale(col);
          TA* orow = out + (col - col_base) * ldo;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t row0 = m0 + wm * WTM + i * 32 + 8 * q + 4 * half;
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = acc[i][j][4 * q + t] * sc;
            if (row0 + 3 < g.M) {
              if constexpr (sizeof(TA) == 2) {
                *reinterpret_cast<u32x2*>(orow + row0) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
              } else {
                *reinterpret_cast<f32x4*>(orow + row0) = f32x4{v[0], v[1], v[2], v[3]};
              }
            } else {
#pragma unroll
              for (int t = 0; t < 4; ++t)
                if (row0 + t < g.M) store_act(orow + row0 + t, v[t]);
            }
          }
        }
    };
    if constexpr (EPI == EPI_KV) {
      if (tn * BN < g.split) {  // uniform per workgroup: the split is tile-aligned
        if constexpr (QKD != 0) qk_apply();
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int j = 0; j < NTL; ++j) {
            const int64_t col = tn * BN + wn * WTN + j * 32 + (lane & 31);
            const float sc = col_scale(col);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int64_t row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
              if (row < g.M) store_act(static_cast<TA*>(g.out) + row * g.ldo + col, acc[i][j][r] * sc);
            }
          }
      } else {
        store_t(static_cast<TA*>(g.out2), g.ldo2, g.split);
      }
    } else {
      store_t(static_cast<TA*>(g.out), g.ldo, 0);
    }
  } else if constexpr (EPI == EPI_LORA_T) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NTL; ++j) {
        const int64_t col = tn * BN + wn * WTN + j * 32 + (lane & 31);
        if (col >= g.n_valid) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (row >= g.M) continue;
          float* o = static_cast<float*>(g.out) + row * g.ldo + col;
          *o = (g.accumulate ? *o : 0.f) + g.alpha * acc[i][j][r];
        }
      }
  } else {
    if constexpr (EPI == EPI_STORE && QKD != 0) qk_apply();
    // Per 32x32 block: the 16 operand values this lane needs (x for RESID,
    // the fp32 stage for ACCUM and FINAL) are loaded together before any
    // result is stored, so the block waits for memory once rather than once
    // per element (the compiler may not move a load above a store that
    // could alias it).
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NTL; ++j) {
        const int64_t col = tn * BN + wn * WTN + j * 32 + (lane & 31);
        const float sc = col_scale(col);
        const float gt = (EPI == EPI_STORE) ? 1.f : g.gate[col];
        const int64_t row0 = m0 + wm * WTM + i * 32 + 4 * half;  // + 8 * (r / 4) + r % 4
        float av[16];
        if constexpr (EPI != EPI_STORE) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            // rows past M read row M-1 (no branch around the load); their
            // results are not stored
            int64_t row = row0 + 8 * (r >> 2) + (r & 3);
            row = row < g.M ? row : g.M - 1;
            if constexpr (EPI == EPI_RESID)
              av[r] = load_act(static_cast<const TA*>(g.aux) + row * g.ldaux + col);
            else if constexpr (EPI == EPI_ACCUM)
              av[r] = static_cast<const float*>(g.out)[row * g.ldo + col];
            else  // EPI_FINAL
              av[r] = static_cast<const float*>(g.aux)[row * g.ldaux + col];
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = row0 + 8 * (r >> 2) + (r & 3);
          if (row >= g.M) continue;
          const float v = acc[i][j][r] * sc;
          if constexpr (EPI == EPI_STORE)
            store_act(static_cast<TA*>(g.out) + row * g.ldo + col, v);
          else if constexpr (EPI == EPI_RESID || EPI == EPI_ACCUM)
            static_cast<float*>(g.out)[row * g.ldo + col] = av[r] + gt * v;
          else  // EPI_FINAL
            store_act(static_cast<TA*>(g.out) + row * g.ldo + col, av[r] + gt * v);
        }
      }
  }
}

template <typename TA, typename TB, int EPI, int BN, int WM, int WN, int QKD>
static hipError_t launch_tile_qk(const GemmArgs& g, hipStream_t st) {
  constexpr int BM = 256;
  constexpr int OUT_BN = (EPI == EPI_GATEUP) ? BN / 2 : BN;
  const int64_t tiles = ceil_div(g.M, BM) * ((g.N - g.col0) / OUT_BN);
  if constexpr (sizeof(TB) == 1) {
    if (g.lora_t == nullptr) {
      hipLaunchKernelGGL((gemm_kernel<TA, TB, EPI, BM, BN, WM, WN, false, QKD>), dim3((unsigned)tiles),
                         dim3(WM * WN * 64), 0, st, g);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_kernel<TA, TB, EPI, BM, BN, WM, WN, true, QKD>), dim3((unsigned)tiles),
                     dim3(WM * WN * 64), 0, st, g);
  return hipGetLastError();
}

template <typename TA, typename TB, int EPI, int BN, int WM, int WN>
static hipError_t launch_tile(const GemmArgs& g, hipStream_t st) {
  if constexpr (EPI == EPI_STORE || EPI == EPI_KV) {
    if (g.qk_w || g.rope_cs) {
      if (g.qk_head_dim == 64) return launch_tile_qk<TA, TB, EPI, BN, WM, WN, 64>(g, st);
      if (g.qk_head_dim == 128) return launch_tile_qk<TA, TB, EPI, BN, WM, WN, 128>(g, st);
      return hipErrorInvalidValue;
    }
  }
  return launch_tile_qk<TA, TB, EPI, BN, WM, WN, 0>(g, st);
}

// Compute units of the current device (cached per device; concurrent callers
// may both query, and store the same value).
static int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Column split between 256-wide B tiles (wb output columns each: 256, or 128
// features for GATEUP) and 128-wide B tiles (wb/2 columns): columns [0, na)
// in the first kind, [na, N) in the second, with na chosen so that the two
// launches fill whole rounds of the compute units. Cost model: one round of
// 256-wide tiles = 1, one round of 128-wide tiles = 0.6 (measured: 0.58 on
// the down projection). At 8192 rows on 256 CUs: N = 5120 gives na = 4096,
// i.e. 512 + 256 tiles = 2 + 1 rounds (2.6) against 5 rounds of 128-wide
// tiles (3.0); gate/up with F = 13824 gives 13 + 1 rounds (13.6) against
// 13.5 rounded up to 14.
static int64_t wide_split(int64_t m, int64_t n, int cus, int64_t wb) {
  const int64_t mt = ceil_div(m, (int64_t)256);
  double best = 1e300;
  int64_t na_best = 0;
  for (int64_t na = 0; na <= n; na += wb) {
    const double c = (double)ceil_div(mt * (na / wb), (int64_t)cus) +
                     0.6 * (double)ceil_div(mt * ((n - na) / (wb / 2)), (int64_t)cus);
    if (c <= best) {  // ties: more 256-wide tiles
      best = c;
      na_best = na;
    }
  }
  return na_best;
}

template <typename TA, typename TB, int EPI>
static hipError_t launch_epi(const GemmArgs& g, hipStream_t st) {
  // The tile shapes depend on M, N, the epilogue and the compute-unit count,
  // but which tile computes an element does not change its value (every tile
  // shape runs the same MFMA over the same k sequence), so every token row
  // gets the same bits whatever the slab size. 8 wavefronts (2 per SIMD) per 256-row tile: while one wave waits on
  // LDS or a barrier, the other keeps the matrix core busy.
  if constexpr (EPI == EPI_KV || EPI == EPI_LORA_T) {
    if (g.N % 256 == 0 && g.N >= 8192) return launch_tile<TA, TB, EPI, 256, 2, 4>(g, st);
    if (g.N % 128 == 0) return launch_tile<TA, TB, EPI, 128, 4, 2>(g, st);
    if (g.N % 64 == 0) return launch_tile<TA, TB, EPI, 64, 4, 1>(g, st);
  } else {
    constexpr int64_t WB = (EPI == EPI_GATEUP) ? 128 : 256;  // output columns of a 256-wide B tile
    if (g.N % WB == 0) {
      const int64_t na = wide_split(g.M, g.N, cu_count(), WB);
      if (na > 0) {
        GemmArgs ga = g;
        ga.N = na;
        const hipError_t e = launch_tile<TA, TB, EPI, 256, 2, 4>(ga, st);
        if (e != hipSuccess || na == g.N) return e;
      }
      GemmArgs gb = g;
      gb.col0 = na;
      return launch_tile<TA, TB, EPI, 128, 4, 2>(gb, st);
    }
    if (g.N % (WB / 2) == 0) return launch_tile<TA, TB, EPI, 128, 4, 2>(g, st);
    if constexpr (EPI != EPI_GATEUP)
      if (g.N % 64 == 0) return launch_tile<TA, TB, EPI, 64, 4, 1>(g, st);
  }
  return hipErrorInvalidValue;
}

template <typename TA, typename TB>
static hipError_t launch_types(Epilogue epi, const GemmArgs& g, hipStream_t st) {
  switch (epi) {
    case EPI_STORE: return launch_epi<TA, TB, EPI_STORE>(g, st);
    case EPI_STORE_T: return launch_epi<TA, TB, EPI_STORE_T>(g, st);
    case EPI_RESID: return launch_epi<TA, TB, EPI_RESID>(g, st);
    case EPI_GATEUP: return launch_epi<TA, TB, EPI_GATEUP>(g, st);
    case EPI_ACCUM: return launch_epi<TA, TB, EPI_ACCUM>(g, st);
    case EPI_FINAL: return launch_epi<TA, TB, EPI_FINAL>(g, st);
    case EPI_KV: return launch_epi<TA, TB, EPI_KV>(g, st);
    case EPI_LORA_T:
      if constexpr (sizeof(TB) == 1) return hipErrorInvalidValue;  // adapters are never int8
      else return launch_epi<TA, TB, EPI_LORA_T>(g, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(int dtype, Epilogue epi, const GemmArgs& g_in, hipStream_t st) {
  GemmArgs g = g_in;
  g.col0 = 0;
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (!gemm_offsets_fit(dtype, g.lda, g.ldb, epi == EPI_GATEUP ? g.up_offset + 256 : 256))
    return hipErrorInvalidValue;
  const int bk = dtype == F32 ? 32 : 64;
  if (g.K <= 0 || g.K % bk) return hipErrorInvalidValue;
  switch (dtype) {
    case F32: return launch_types<float, float>(epi, g, st);
    case BF16: return launch_types<uint16_t, uint16_t>(epi, g, st);
    case W8_BF16: return launch_types<uint16_t, int8_t>(epi, g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dit
