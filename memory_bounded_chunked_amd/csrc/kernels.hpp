// Host-side launchers of the gfx950 kernels (internal interface of the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

// K1: modulated LayerNorm of `rows` rows of length d (d % 8 == 0, d <= 8192).
hipError_t launch_modnorm(int in_f32, int out_f32, const void* x, int64_t ldx, const float* shift,
                          const float* scale, void* out, int64_t ldo, int64_t rows, int d,
                          float eps, hipStream_t st);

// K2 epilogues.
enum Epilogue : int {
  EPI_STORE = 0,    // out[m][n] = acc                        (activation type)
  EPI_STORE_T = 1,  // out[n][m] = acc                        (transposed store)
  EPI_RESID = 2,    // out[m][n] (fp32) = aux[m][n] + gate[n] * acc     aux: activation type
  EPI_GATEUP = 3,   // out[m][f] = silu(acc_gate) * acc_up    (B rows paired gate/up)
  EPI_ACCUM = 4,    // out[m][n] (fp32) += gate[n] * acc
  EPI_FINAL = 5,    // out[m][n] = aux[m][n] (fp32) + gate[n] * acc     out: activation type
  EPI_KV = 6,       // columns [0, split): out[m][n] = acc; columns [split, N):
                    // out2[n - split][m] = acc (K row-major and V transposed, one launch)
  EPI_LORA_T = 7,   // adapter input product: out (fp32) [m][n] = (accumulate ? out[m][n] : 0)
                    // + alpha * acc for n < n_valid; B rows >= n_valid read as zero
};

struct GemmArgs {
  const void* a;        // [M][K] activations (bf16, or fp32 for the F32 block)
  int64_t lda;
  const void* b;        // [N][K] weight rows (bf16, fp32 or int8); GATEUP: first gate row
  int64_t ldb;
  const float* bscale;  // int8 weights: fp32 scale per B row (same offset as b), else null
  int64_t up_offset;    // GATEUP: rows from a gate row to its up row (F)
  int64_t M, N, K;      // N = output columns (GATEUP: features)
  void* out;
  int64_t ldo;
  const void* aux;      // RESID: x rows; FINAL: fp32 stage rows
  int64_t ldaux;
  const float* gate;    // RESID/ACCUM/FINAL: gate vector indexed by output column
  void* out2;           // KV: transposed destination of the columns from `split` on
  int64_t ldo2;
  int64_t split;        // KV: first column stored transposed (a multiple of the tile width)
  // EPI_LORA_T
  float alpha;
  int accumulate;
  int64_t n_valid;
  // Activation-space adapter phase of the main epilogues (lora_t == null: none).
  // After the contraction, output column n of segment s gains
  //   sum_j t[m][lora_toff[s] + j] * lora_b[s][row_s(n)][j],  j < lora_r[s],
  // with t fp32 [M][lora_ldt] (rounded to the activation type on use) and
  // lora_b[s] [rows][lora_r[s]] in the activation type. Segments: KV: 0 = K
  // columns, 1 = V columns; GATEUP: 0 = gate, 1 = up (row = feature); else 0.
  // For int8 weights the per-row scale is applied before this phase.
  const float* lora_t;
  int64_t lora_ldt;
  const void* lora_b[2];
  int64_t lora_r[2];
  int64_t lora_toff[2];
  // QK RMSNorm (qk_w: fp32 [qk_head_dim], or null) and RoPE (rope_cs /
  // rope_sn: fp32 [M][ld_rope] angles of this launch's rows, or null) of the
  // stored columns, per head of qk_head_dim (64 or 128) columns, before the
  // output is rounded: EPI_STORE, and the first `split` columns of EPI_KV.
  const float* qk_w;
  const float* rope_cs;
  const float* rope_sn;
  int64_t ld_rope;
  int qk_head_dim;
  float qk_eps;
  // Set by launch_gemm only: a launch covers output columns [col0, N).
  int64_t col0;
};

// dtype: 0 = F32, 1 = BF16, 2 = W8_BF16 (activations bf16, weights int8).
hipError_t launch_gemm(int dtype, Epilogue epi, const GemmArgs& g, hipStream_t st);

// The GEMM kernel reaches the rows of one tile through 32-bit byte offsets
// from the tile's first row: 256 rows of A (leading dimension lda) and
// b_rows_span rows of B (256, or up_offset + 256 for gate/up pairs). True when
// both stay below 2^32 bytes.
inline bool gemm_offsets_fit(int dtype, int64_t lda, int64_t ldb, int64_t b_rows_span) {
  const int64_t ea = dtype == 0 ? 4 : 2, eb = dtype == 0 ? 4 : (dtype == 1 ? 2 : 1);
  const int64_t lim = (int64_t)1 << 32;
  return 256 * lda * ea < lim && b_rows_span * ldb * eb < lim;
}

// Adapter input of activation-space LoRA, bf16 operands: t[r][n] =
// (accumulate ? t[r][n] : 0) + alpha * sum_k a[r][k] * w[n][k] for r < m,
// n < rank (<= 256); k % 16 == 0, lda and ldw multiples of 8, 16-B aligned.
hipError_t launch_lora_t(const void* a, int64_t lda, const void* w, int64_t ldw, int64_t m, int64_t k, int64_t rank,
                         float alpha, int accumulate, float* t, int64_t ldt, hipStream_t st);

// Optional QK RMSNorm (w: [head_dim] or null) and RoPE (cs/sn: [rows][ld_rope]
// or null), in place on `rows` token rows of width d.
hipError_t launch_qk_transform(int f32, void* x, int64_t ldx, int64_t rows, int d, int head_dim, const float* w,
                               const float* cs, const float* sn, int64_t ld_rope, float eps, hipStream_t st);

// Output head: out[t][j] = sum_c (LN(x[t])[c] * (1 + scale[c]) + shift[c]) * w[j][c],
// fp32 arithmetic; x [n][ldx] (fp32 or bf16), w [out_dim][d] fp32, out [n][ldo] fp32.
// d % 64 == 0, 64 <= d <= 8192, 1 <= out_dim <= 128.
hipError_t launch_final_layer(int x_f32, const void* x, int64_t ldx, int64_t n, int d, const float* shift,
                              const float* scale, const float* w, int out_dim, float* out, int64_t ldo, float eps,
                              hipStream_t st);

// K3: softmax attention of n_q query rows against n_kv keys for all heads.
// q [n_q][ldq], k [n_kv][ldk], vt [n_heads*head_dim][ldvt] (V transposed),
// o [n_q][ldo]; head h owns columns h*head_dim.. of q, k, o and rows of vt.
// splits > 1: each query's keys in attention_splits_effective(splits, n_kv)
// contiguous ranges of 64-key tiles, merged by a second kernel; o_part
// [S][n_q][n_heads*head_dim] and ml_part [S][n_q][n_heads][2] fp32 hold the
// ranges' partial results (S = the effective split count).
hipError_t launch_attention(int dtype, const void* q, int64_t ldq, const void* k, int64_t ldk,
                            const void* vt, int64_t ldvt, void* o, int64_t ldo, int64_t n_q,
                            int64_t n_kv, int n_heads, int head_dim, int64_t splits, float* o_part, float* ml_part,
                            hipStream_t st);
// Key ranges actually used for `splits` requested: at most one per 64-key tile.
int64_t attention_splits_effective(int64_t splits, int64_t n_kv);

}  // namespace dit
