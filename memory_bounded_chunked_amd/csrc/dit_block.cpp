// C ABI of the block: argument validation, the closed-form workspace, the
// workspace carve and the two-pass, token-chunked schedule.
//
// Schedule ("LayerStream: H3 Chunking", sections "How the slicing works" and
// "The two numbers you set"; streaming proposal, "Attention requires a
// stronger contract" and "MLP planning"):
//   pass 1   for each slab of Ca tokens: norm1 -> K rows and V^T columns of the
//            global K/V (only the K and V weight rows are multiplied);
//   pass 2   for each super-slice of S = max(Ca, Cm) tokens:
//              for each Ca-slab: norm1 -> Q -> attention vs global K/V -> O
//                                -> stage = x + gate1 * (O Wo^T)        (fp32)
//              for each Cm-slab: norm2(stage) -> SwiGLU (per FFN feature slice)
//                                -> x = stage + gate2 * (h Wd^T)        (in place)
// Pass 1 ends before anything writes x; afterwards each super-slice reads and
// writes only its own rows of x. The residual after attention stays in fp32
// in `stage` and the block output is rounded once, when it is written to x.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/dit_block.h"
#include "../../include/dit_block_profile.h"
#include "../../include/dit_block_steps.h"
#include "../../include/dit_final_layer.h"
#include "kernels.hpp"

struct dit_block {
  dit_block_desc desc;
  dit_block_weights w;
  dit_block_lora lora;  // rank 0 = no adapter
  int64_t att_splits;   // key ranges per query in attention (1 = none)
};

// Workspace of dit_block_forward_noalloc: one copy per GPU, loaded with the
// library's code object and held until the process ends. In host code this
// name is only a handle for the runtime; the device address of each GPU's
// copy comes from hipGetSymbolAddress and is the only form host code passes on.
static __device__ __align__(256) unsigned char scratch[DIT_STATIC_WORKSPACE_BYTES];

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int64_t act_bytes(int dtype) { return dtype == DIT_F32 ? 4 : 2; }

struct Plan {
  int64_t n, ca, cm, fc, s, np, splits;
  size_t off_k, off_vt, off_stage, off_slab, slab_b, off_opart, off_ml, off_lora, total;
};

// Bytes of the partial results of `splits` (effective) key ranges for n_q queries.
size_t split_part_bytes(int64_t splits, int64_t n_q, int64_t d, int64_t heads, size_t* ml_off) {
  if (splits <= 1) {
    *ml_off = 0;
    return 0;
  }
  const size_t o_bytes = round_up((size_t)splits * n_q * d * 4, kAlign);
  *ml_off = o_bytes;
  return o_bytes + round_up((size_t)splits * n_q * heads * 2 * 4, kAlign);
}

// Adapter ranks of one handle (0 = none).
struct Ranks {
  int64_t q, k, v, o, gate, up, down;
  int64_t attn() const { return std::max({k + v, q, o}); }  // widest t of one attention launch group
  int64_t mlp() const { return gate + up + down; }          // t of gate/up and down, live together
  bool any() const { return q || k || v || o || gate || up || down; }
};
Ranks ranks_of(const dit_block* h) {
  const dit_block_lora& l = h->lora;
  return {l.q.rank, l.k.rank, l.v.rank, l.o.rank, l.gate.rank, l.up.rank, l.down.rank};
}

int make_plan(const dit_block* h, int64_t n, int64_t attn_chunk, int64_t mlp_chunk, int64_t ffn_chunk,
              Plan* p) {
  if (!h || !p) return DIT_EINVAL;
  if (n < 1 || attn_chunk < 0 || mlp_chunk < 1 || ffn_chunk < 0 || ffn_chunk % 64) return DIT_EINVAL;
  const int64_t d = h->desc.d, f = h->desc.ffn, e = act_bytes(h->desc.dtype);
  p->n = n;
  p->ca = attn_chunk == 0 ? n : std::min(attn_chunk, n);
  p->cm = std::min(mlp_chunk, n);
  p->fc = ffn_chunk == 0 ? f : std::min(ffn_chunk, f);
  p->s = std::max(p->ca, p->cm);
  p->np = (n + 63) / 64 * 64;
  // the attention kernel addresses a head's V^T rows with 32-bit offsets
  if (h->desc.head_dim * p->np * e >= ((int64_t)1 << 32)) return DIT_EINVAL;
  const size_t k_bytes = round_up((size_t)n * d * e, kAlign);
  const size_t vt_bytes = round_up((size_t)d * p->np * e, kAlign);
  const size_t stage_bytes = round_up((size_t)p->s * d * 4, kAlign);
  const size_t attn_a = round_up((size_t)p->ca * d * e, kAlign);
  const size_t mlp_a = round_up((size_t)p->cm * d * e, kAlign);
  const size_t mlp_h = round_up((size_t)p->cm * p->fc * e, kAlign);
  const Ranks r = ranks_of(h);
  const size_t lora_bytes =
      r.any() ? round_up((size_t)4 * std::max(p->ca * r.attn(), p->cm * r.mlp()), kAlign) : 0;
  p->splits = dit::attention_splits_effective(h->att_splits, n);
  size_t ml_off = 0;
  const size_t part_bytes = split_part_bytes(p->splits, p->ca, d, h->desc.n_heads, &ml_off);
  p->off_k = 0;
  p->off_vt = k_bytes;
  p->off_stage = p->off_vt + vt_bytes;
  p->off_slab = p->off_stage + stage_bytes;
  p->slab_b = attn_a;  // offset of the Q slab within the slab region
  p->off_opart = p->off_slab + std::max(2 * attn_a, mlp_a + mlp_h);
  p->off_ml = p->off_opart + ml_off;
  p->off_lora = p->off_opart + part_bytes;
  p->total = p->off_lora + lora_bytes;
  return DIT_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DIT_OK : DIT_EHIP; }

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DIT_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return DIT_EINVAL;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DIT_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DIT_OK;
}

// Optional per-kernel event timing (dit_block_profile.h).
struct Profiler {
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<Rec> recs;

  hipEvent_t take() {
    if (used == pool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
};
Profiler g_prof;

// Runs one launch, bracketed by events when profiling is on.
template <typename F>
hipError_t run_step(int kind, hipStream_t st, F&& launch) {
  if (!g_prof.on) return launch();
  std::lock_guard<std::mutex> lock(g_prof.mu);
  hipEvent_t a = g_prof.take(), b = g_prof.take();
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, st);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, st);
  if (e == hipSuccess) g_prof.recs.push_back({kind, a, b});
  return e;
}

}  // namespace

extern "C" {

const char* dit_block_strerror(int code) {
  switch (code) {
    case DIT_OK: return "ok";
    case DIT_EINVAL: return "invalid argument";
    case DIT_ENOSPC: return "workspace too small";
    case DIT_EHIP: return "HIP launch error";
    case DIT_ETOOBIG: return "sizes need more than the library's static workspace";
    default: return "unknown error";
  }
}

int dit_block_create(const dit_block_desc* desc, const dit_block_weights* w, dit_block** out) {
  if (!desc || !w || !out) return DIT_EINVAL;
  const dit_block_desc& d = *desc;
  if (d.dtype != DIT_F32 && d.dtype != DIT_BF16 && d.dtype != DIT_W8_BF16) return DIT_EINVAL;
  if (d.head_dim != 64 && d.head_dim != 128) return DIT_EINVAL;
  if (d.n_heads < 1 || d.d != d.n_heads * d.head_dim || d.d > 8192) return DIT_EINVAL;
  if (d.ffn < 64 || d.ffn % 64) return DIT_EINVAL;
  if (!(d.eps > 0.f)) return DIT_EINVAL;
  // the projection kernels address a tile's weight rows with 32-bit offsets
  if (!dit::gemm_offsets_fit(d.dtype, d.d, d.d, d.ffn + 256) ||
      !dit::gemm_offsets_fit(d.dtype, d.ffn, d.ffn, 256))
    return DIT_EINVAL;
  const void* ptrs[4] = {w->w_qkv, w->w_o, w->w_gu, w->w_down};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return DIT_EINVAL;
  if (d.dtype == DIT_W8_BF16) {
    if (!w->s_qkv || !w->s_o || !w->s_gu || !w->s_down) return DIT_EINVAL;
  }
  if ((w->q_norm && !aligned16(w->q_norm)) || (w->k_norm && !aligned16(w->k_norm))) return DIT_EINVAL;
  dit_block* h = new (std::nothrow) dit_block;
  if (!h) return DIT_EINVAL;
  h->desc = d;
  h->w = *w;
  std::memset(&h->lora, 0, sizeof(h->lora));
  h->att_splits = 1;
  *out = h;
  return DIT_OK;
}

int dit_block_set_lora(dit_block* h, const dit_block_lora* lora) {
  if (!h) return DIT_EINVAL;
  if (!lora) {
    std::memset(&h->lora, 0, sizeof(h->lora));
    return DIT_OK;
  }
  const dit_lora* all[7] = {&lora->q, &lora->k, &lora->v, &lora->o, &lora->gate, &lora->up, &lora->down};
  for (const dit_lora* l : all) {
    if (l->rank < 0 || l->rank % 16 || l->rank > 256) return DIT_EINVAL;
    if (l->rank == 0) continue;
    if (!l->a || !l->b || !aligned16(l->a) || !aligned16(l->b)) return DIT_EINVAL;
    if (!std::isfinite(l->alpha)) return DIT_EINVAL;
  }
  h->lora = *lora;
  dit_lora* mine[7] = {&h->lora.q, &h->lora.k, &h->lora.v, &h->lora.o, &h->lora.gate, &h->lora.up, &h->lora.down};
  for (dit_lora* l : mine)
    if (l->rank == 0) *l = dit_lora{nullptr, nullptr, 0, 0.f};
  return DIT_OK;
}

int dit_block_set_attention_splits(dit_block* h, int64_t splits) {
  if (!h || splits < 1 || splits > 64) return DIT_EINVAL;
  h->att_splits = splits;
  return DIT_OK;
}

void dit_block_destroy(dit_block* h) { delete h; }

int dit_block_peak_workspace(const dit_block* h, int64_t n_tokens, int64_t attn_chunk_tokens,
                             int64_t mlp_chunk_tokens, int64_t ffn_chunk_features, size_t* bytes_out) {
  if (!bytes_out) return DIT_EINVAL;
  Plan p;
  const int rc = make_plan(h, n_tokens, attn_chunk_tokens, mlp_chunk_tokens, ffn_chunk_features, &p);
  if (rc != DIT_OK) return rc;
  *bytes_out = p.total;
  return DIT_OK;
}

int dit_block_plan_chunks(const dit_block* h, int64_t n_tokens, size_t budget_bytes, int64_t* attn_chunk_tokens,
                          int64_t* mlp_chunk_tokens, int64_t* ffn_chunk_features) {
  if (!h || !attn_chunk_tokens || !mlp_chunk_tokens || !ffn_chunk_features || n_tokens < 1) return DIT_EINVAL;
  const int64_t f = h->desc.ffn;
  auto fits = [&](int64_t c, int64_t fc) {
    Plan p;
    return make_plan(h, n_tokens, c, c, fc == f ? 0 : fc, &p) == DIT_OK && p.total <= budget_bytes;
  };
  int64_t best_c = 0, best_fc = 0;
  for (int64_t fc = f; fc >= 64 && fc % 64 == 0; fc = (fc % 128 == 0) ? fc / 2 : 0) {
    int64_t c = 0;
    if (fits(n_tokens, fc)) {
      c = n_tokens;
    } else {
      // workspace grows with C, so the largest fitting multiple of 256 is found by bisection
      int64_t lo = 0, hi = (n_tokens - 1) / 256;  // in units of 256 tokens
      while (lo < hi) {
        const int64_t mid = (lo + hi + 1) / 2;
        if (fits(mid * 256, fc))
          lo = mid;
        else
          hi = mid - 1;
      }
      c = lo * 256;
    }
    if (c > best_c) {
      best_c = c;
      best_fc = fc;
    }
    if (best_c == n_tokens) break;
  }
  if (best_c == 0) return DIT_ENOSPC;
  *attn_chunk_tokens = best_c >= n_tokens ? 0 : best_c;
  *mlp_chunk_tokens = best_c;
  *ffn_chunk_features = best_fc == f ? 0 : best_fc;
  return DIT_OK;
}

int dit_block_forward(dit_block* h, void* x, const float* mod, int64_t n_tokens, int64_t attn_chunk_tokens,
                      int64_t mlp_chunk_tokens, int64_t ffn_chunk_features, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return dit_block_forward_rope(h, x, mod, nullptr, nullptr, n_tokens, attn_chunk_tokens, mlp_chunk_tokens,
                                ffn_chunk_features, workspace, workspace_bytes, stream);
}

int dit_block_forward_rope(dit_block* h, void* x, const float* mod, const float* rope_cos, const float* rope_sin,
                           int64_t n_tokens, int64_t attn_chunk_tokens, int64_t mlp_chunk_tokens,
                           int64_t ffn_chunk_features, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  const int rc = make_plan(h, n_tokens, attn_chunk_tokens, mlp_chunk_tokens, ffn_chunk_features, &p);
  if (rc != DIT_OK) return rc;
  if (!x || !mod || !workspace) return DIT_EINVAL;
  if (!aligned16(x) || !aligned16(mod) || !aligned16(workspace)) return DIT_EINVAL;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return DIT_EINVAL;
  if (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))) return DIT_EINVAL;
  if (workspace_bytes < p.total) return DIT_ENOSPC;

  using namespace dit;
  const dit_block_desc& dsc = h->desc;
  const int dt = dsc.dtype;
  const int f32 = dt == DIT_F32;
  const int64_t d = dsc.d, ffn = dsc.ffn, e = act_bytes(dt), n = p.n;
  const bool w8 = dt == DIT_W8_BF16;
  const int64_t wb = w8 ? 1 : e;  // bytes per weight element
  hipStream_t st = static_cast<hipStream_t>(stream);

  char* ws = static_cast<char*>(workspace);
  char* kbuf = ws + p.off_k;
  char* vtbuf = ws + p.off_vt;
  float* stage = reinterpret_cast<float*>(ws + p.off_stage);
  char* slab_a = ws + p.off_slab;
  char* slab_b = ws + p.off_slab + p.slab_b;
  char* xb = static_cast<char*>(x);

  const float *sh1 = mod, *sc1 = mod + d, *g1 = mod + 2 * d;
  const float *sh2 = mod + 3 * d, *sc2 = mod + 4 * d, *g2 = mod + 5 * d;
  const char* wqkv = static_cast<const char*>(h->w.w_qkv);
  const float* s_qkv = w8 ? h->w.s_qkv : nullptr;
  const int64_t dh = dsc.head_dim, ld_rope = dh / 2;
  auto rope_rows = [&](const float* t, int64_t r0) { return t ? t + r0 * ld_rope : nullptr; };

  hipError_t err = hipSuccess;
#define DIT_TRY(kind, call)                                  \
  do {                                                       \
    err = run_step((kind), st, [&]() { return (call); });    \
    if (err != hipSuccess) return DIT_EHIP;                  \
  } while (0)

  // Activation-space adapters: t = alpha * (A a) of one launch group, fp32
  // [rows][ldt] at column offset toff of the adapter region; `accumulate`
  // adds into t (the down adapter over FFN feature slices). A rank-0 adapter
  // launches nothing.
  const dit_block_lora& lo = h->lora;
  const Ranks rk = ranks_of(h);
  float* tbuf = reinterpret_cast<float*>(ws + p.off_lora);
  const int lora_dt = f32 ? DIT_F32 : DIT_BF16;  // adapters are never int8
  auto lora_in = [&](const dit_lora& ad, const void* a, int64_t lda, int64_t rows, int64_t in, int64_t col0,
                     int64_t ld_in, int64_t ldt, int64_t toff, int accumulate) -> hipError_t {
    if (ad.rank == 0) return hipSuccess;
    if (!f32)
      return launch_lora_t(a, lda, static_cast<const char*>(ad.a) + col0 * e, ld_in, rows, in, ad.rank, ad.alpha,
                           accumulate, tbuf + toff, ldt, st);
    GemmArgs g{};
    g.a = a;
    g.lda = lda;
    g.M = rows;
    g.K = in;
    g.b = static_cast<const char*>(ad.a) + col0 * e;
    g.ldb = ld_in;
    g.N = (ad.rank + 63) / 64 * 64;
    g.n_valid = ad.rank;
    g.out = tbuf + toff;
    g.ldo = ldt;
    g.alpha = ad.alpha;
    g.accumulate = accumulate;
    return launch_gemm(lora_dt, EPI_LORA_T, g, st);
  };
  auto with_lora = [&](GemmArgs& g, const dit_lora& a0, int64_t b0_row, const dit_lora* a1, int64_t b1_row,
                       int64_t ldt, int64_t toff1) {
    if (a0.rank == 0 && (!a1 || a1->rank == 0)) return;
    g.lora_t = tbuf;
    g.lora_ldt = ldt;
    g.lora_b[0] = a0.rank ? static_cast<const char*>(a0.b) + b0_row * a0.rank * e : nullptr;
    g.lora_r[0] = a0.rank;
    g.lora_toff[0] = 0;
    if (a1) {
      g.lora_b[1] = a1->rank ? static_cast<const char*>(a1->b) + b1_row * a1->rank * e : nullptr;
      g.lora_r[1] = a1->rank;
      g.lora_toff[1] = toff1;
    }
  };

  // ---- pass 1: K and V for all tokens, in slabs of Ca tokens
  for (int64_t s0 = 0; s0 < n; s0 += p.ca) {
    const int64_t c = std::min(p.ca, n - s0);
    DIT_TRY(DIT_K_MODNORM, launch_modnorm(f32, f32, xb + s0 * d * e, d, sh1, sc1, slab_a, d, c, (int)d, dsc.eps, st));
    GemmArgs g{};
    g.a = slab_a;
    g.lda = d;
    g.M = c;
    g.K = d;
    g.ldb = d;
    g.b = wqkv + d * d * wb;  // K rows then V rows of w_qkv
    g.bscale = s_qkv ? s_qkv + d : nullptr;
    g.out = kbuf + s0 * d * e;
    g.ldo = d;
    // K's RMSNorm and RoPE in the projection's epilogue
    g.qk_w = h->w.k_norm;
    g.rope_cs = rope_rows(rope_cos, s0);
    g.rope_sn = rope_rows(rope_sin, s0);
    g.ld_rope = ld_rope;
    g.qk_head_dim = (int)dh;
    g.qk_eps = dsc.eps;
    const int64_t ldt_kv = rk.k + rk.v;
    if (lo.k.rank || lo.v.rank) {
      if (lo.k.rank) DIT_TRY(DIT_K_LORA, lora_in(lo.k, slab_a, d, c, d, 0, d, ldt_kv, 0, 0));
      if (lo.v.rank) DIT_TRY(DIT_K_LORA, lora_in(lo.v, slab_a, d, c, d, 0, d, ldt_kv, rk.k, 0));
    }
    if (d % 256 == 0) {  // one launch: K row-major, V transposed
      g.N = 2 * d;
      g.out2 = vtbuf + s0 * e;
      g.ldo2 = p.np;
      g.split = d;
      with_lora(g, lo.k, 0, &lo.v, 0, ldt_kv, rk.k);
      DIT_TRY(DIT_K_KV_PROJ, launch_gemm(dt, EPI_KV, g, st));
    } else {
      g.N = d;
      GemmArgs gk = g;
      with_lora(gk, lo.k, 0, nullptr, 0, ldt_kv, 0);
      DIT_TRY(DIT_K_KV_PROJ, launch_gemm(dt, EPI_STORE, gk, st));
      g.b = wqkv + 2 * d * d * wb;
      g.bscale = s_qkv ? s_qkv + 2 * d : nullptr;
      g.out = vtbuf + s0 * e;
      g.ldo = p.np;
      g.qk_w = nullptr;  // V is not transformed
      g.rope_cs = g.rope_sn = nullptr;
      with_lora(g, lo.v, 0, nullptr, 0, ldt_kv, 0);
      if (g.lora_t) g.lora_t = tbuf + rk.k;  // V's t columns follow K's
      DIT_TRY(DIT_K_KV_PROJ, launch_gemm(dt, EPI_STORE_T, g, st));
    }
  }

  // ---- pass 2: super-slices of S tokens
  for (int64_t t0 = 0; t0 < n; t0 += p.s) {
    const int64_t tn = std::min(p.s, n - t0);
    for (int64_t s0 = t0; s0 < t0 + tn; s0 += p.ca) {
      const int64_t c = std::min(p.ca, t0 + tn - s0);
      DIT_TRY(DIT_K_MODNORM, launch_modnorm(f32, f32, xb + s0 * d * e, d, sh1, sc1, slab_a, d, c, (int)d, dsc.eps, st));
      GemmArgs g{};
      g.a = slab_a;
      g.lda = d;
      g.M = c;
      g.N = d;
      g.K = d;
      g.b = wqkv;
      g.ldb = d;
      g.bscale = s_qkv;
      g.out = slab_b;
      g.ldo = d;
      // Q's RMSNorm and RoPE in the projection's epilogue
      g.qk_w = h->w.q_norm;
      g.rope_cs = rope_rows(rope_cos, s0);
      g.rope_sn = rope_rows(rope_sin, s0);
      g.ld_rope = ld_rope;
      g.qk_head_dim = (int)dh;
      g.qk_eps = dsc.eps;
      if (lo.q.rank) DIT_TRY(DIT_K_LORA, lora_in(lo.q, slab_a, d, c, d, 0, d, rk.q, 0, 0));
      with_lora(g, lo.q, 0, nullptr, 0, rk.q, 0);
      DIT_TRY(DIT_K_Q_PROJ, launch_gemm(dt, EPI_STORE, g, st));
      DIT_TRY(DIT_K_ATTENTION, launch_attention(dt, slab_b, d, kbuf, d, vtbuf, p.np, slab_a, d, c, n, (int)dsc.n_heads,
                                                (int)dsc.head_dim, p.splits, reinterpret_cast<float*>(ws + p.off_opart),
                                                reinterpret_cast<float*>(ws + p.off_ml), st));
      GemmArgs o{};
      o.a = slab_a;
      o.lda = d;
      o.M = c;
      o.N = d;
      o.K = d;
      o.b = h->w.w_o;
      o.ldb = d;
      o.bscale = w8 ? h->w.s_o : nullptr;
      o.out = stage + (s0 - t0) * d;
      o.ldo = d;
      o.aux = xb + s0 * d * e;
      o.ldaux = d;
      o.gate = g1;
      if (lo.o.rank) DIT_TRY(DIT_K_LORA, lora_in(lo.o, slab_a, d, c, d, 0, d, rk.o, 0, 0));
      with_lora(o, lo.o, 0, nullptr, 0, rk.o, 0);
      DIT_TRY(DIT_K_OUT_PROJ, launch_gemm(dt, EPI_RESID, o, st));
    }
    for (int64_t m0 = t0; m0 < t0 + tn; m0 += p.cm) {
      const int64_t c = std::min(p.cm, t0 + tn - m0);
      float* srows = stage + (m0 - t0) * d;
      char* n2 = slab_a;
      char* hbuf = slab_a + round_up((size_t)p.cm * d * e, kAlign);
      DIT_TRY(DIT_K_NORM2, launch_modnorm(1, f32, srows, d, sh2, sc2, n2, d, c, (int)d, dsc.eps, st));
      // adapter inputs of this slab: [gate | up | down] columns of one t
      const int64_t ldt_m = rk.mlp();
      if (lo.gate.rank) DIT_TRY(DIT_K_LORA, lora_in(lo.gate, n2, d, c, d, 0, d, ldt_m, 0, 0));
      if (lo.up.rank) DIT_TRY(DIT_K_LORA, lora_in(lo.up, n2, d, c, d, 0, d, ldt_m, rk.gate, 0));
      for (int64_t f0 = 0; f0 < ffn; f0 += p.fc) {
        const int64_t fl = std::min(p.fc, ffn - f0);
        GemmArgs gu{};
        gu.a = n2;
        gu.lda = d;
        gu.M = c;
        gu.N = fl;
        gu.K = d;
        gu.b = static_cast<const char*>(h->w.w_gu) + f0 * d * wb;
        gu.ldb = d;
        gu.up_offset = ffn;
        gu.bscale = w8 ? h->w.s_gu + f0 : nullptr;
        gu.out = hbuf;
        gu.ldo = p.fc;
        with_lora(gu, lo.gate, f0, &lo.up, f0, ldt_m, rk.gate);
        DIT_TRY(DIT_K_GATE_UP, launch_gemm(dt, EPI_GATEUP, gu, st));
        const bool last = f0 + fl >= ffn;
        // the down adapter's A h, accumulated over the feature slices
        if (lo.down.rank) DIT_TRY(DIT_K_LORA, lora_in(lo.down, hbuf, p.fc, c, fl, f0, ffn, ldt_m, rk.gate + rk.up, f0 > 0));
        GemmArgs dn{};
        dn.a = hbuf;
        dn.lda = p.fc;
        dn.M = c;
        dn.N = d;
        dn.K = fl;
        dn.b = static_cast<const char*>(h->w.w_down) + f0 * wb;
        dn.ldb = ffn;
        dn.bscale = w8 ? h->w.s_down : nullptr;
        dn.gate = g2;
        if (last) {
          dn.out = xb + m0 * d * e;
          dn.ldo = d;
          dn.aux = srows;
          dn.ldaux = d;
          with_lora(dn, lo.down, 0, nullptr, 0, ldt_m, 0);
          if (dn.lora_t) dn.lora_t = tbuf + rk.gate + rk.up;
          DIT_TRY(DIT_K_DOWN, launch_gemm(dt, EPI_FINAL, dn, st));
        } else {
          dn.out = srows;
          dn.ldo = d;
          DIT_TRY(DIT_K_DOWN, launch_gemm(dt, EPI_ACCUM, dn, st));
        }
      }
    }
  }
#undef DIT_TRY
  (void)err;
  return DIT_OK;
}

int dit_block_forward_noalloc(dit_block* h, void* x, const float* mod, const float* rope_cos,
                              const float* rope_sin, int64_t n_tokens, int64_t attn_chunk_tokens,
                              int64_t mlp_chunk_tokens, int64_t ffn_chunk_features, void* stream) {
  Plan p;
  const int rc = make_plan(h, n_tokens, attn_chunk_tokens, mlp_chunk_tokens, ffn_chunk_features, &p);
  if (rc != DIT_OK) return rc;
  if (p.total > DIT_STATIC_WORKSPACE_BYTES) return DIT_ETOOBIG;
  void* ws = nullptr;
  const int sc = scratch_of_current_device(&ws);
  if (sc != DIT_OK) return sc;
  return dit_block_forward_rope(h, x, mod, rope_cos, rope_sin, n_tokens, attn_chunk_tokens, mlp_chunk_tokens,
                                ffn_chunk_features, ws, DIT_STATIC_WORKSPACE_BYTES, stream);
}

// ---------------------------------------------------------------- profiling

int dit_profile_enable(int on) {
  std::lock_guard<std::mutex> lock(g_prof.mu);
  if (on) {
    g_prof.recs.clear();
    g_prof.used = 0;
  }
  g_prof.on = on != 0;
  return DIT_OK;
}

int dit_profile_read(int kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= DIT_K_COUNT || !total_ms || !launches) return DIT_EINVAL;
  std::lock_guard<std::mutex> lock(g_prof.mu);
  double t = 0.0;
  int64_t n = 0;
  for (const auto& r : g_prof.recs) {
    if (r.kind != kind) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return DIT_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return DIT_EHIP;
    t += ms;
    ++n;
  }
  *total_ms = t;
  *launches = n;
  return DIT_OK;
}

// ---------------------------------------------------------------- step-level entry points

int dit_modnorm(int32_t in_dtype, int32_t out_dtype, const void* x, int64_t ldx, const float* shift,
                const float* scale, void* out, int64_t ldo, int64_t rows, int64_t d, float eps, void* stream) {
  if ((in_dtype != DIT_F32 && in_dtype != DIT_BF16) || (out_dtype != DIT_F32 && out_dtype != DIT_BF16))
    return DIT_EINVAL;
  if (!x || !shift || !scale || !out || rows < 0 || d < 8 || d > 8192 || d % 8) return DIT_EINVAL;
  if (ldx < d || ldo < d || ldx % 8 || ldo % 8 || !(eps > 0.f)) return DIT_EINVAL;
  if (!aligned16(x) || !aligned16(out) || !aligned16(shift) || !aligned16(scale)) return DIT_EINVAL;
  if (rows == 0) return DIT_OK;
  return hip_status(dit::launch_modnorm(in_dtype == DIT_F32, out_dtype == DIT_F32, x, ldx, shift, scale, out,
                                        ldo, rows, (int)d, eps, static_cast<hipStream_t>(stream)));
}

int dit_qk_transform(int32_t dtype, void* x, int64_t ldx, int64_t rows, int64_t n_heads, int64_t head_dim,
                     const float* norm_w, const float* rope_cos, const float* rope_sin, int64_t ld_rope, float eps,
                     void* stream) {
  if (dtype != DIT_F32 && dtype != DIT_BF16) return DIT_EINVAL;
  if (!x || rows < 0 || n_heads < 1 || (head_dim != 64 && head_dim != 128)) return DIT_EINVAL;
  const int64_t d = n_heads * head_dim;
  if (d > 8192 || ldx < d || ldx % 8 || !(eps > 0.f) || !aligned16(x)) return DIT_EINVAL;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return DIT_EINVAL;
  if (rope_cos && (ld_rope < head_dim / 2 || ld_rope % 4 || !aligned16(rope_cos) || !aligned16(rope_sin)))
    return DIT_EINVAL;
  if (norm_w && !aligned16(norm_w)) return DIT_EINVAL;
  if (rows == 0) return DIT_OK;
  return hip_status(dit::launch_qk_transform(dtype == DIT_F32, x, ldx, rows, (int)d, (int)head_dim, norm_w,
                                             rope_cos, rope_sin, ld_rope, eps, static_cast<hipStream_t>(stream)));
}

int dit_attention(int32_t dtype, const void* q, int64_t ldq, const void* k, int64_t ldk, const void* vt,
                  int64_t ldvt, void* o, int64_t ldo, int64_t n_q, int64_t n_kv, int64_t n_heads,
                  int64_t head_dim, void* stream) {
  if (dtype != DIT_F32 && dtype != DIT_BF16) return DIT_EINVAL;
  if (!q || !k || !vt || !o || n_q < 0 || n_kv < 1 || n_heads < 1) return DIT_EINVAL;
  if (head_dim != 64 && head_dim != 128) return DIT_EINVAL;
  const int64_t d = n_heads * head_dim;
  if (ldq < d || ldk < d || ldo < d || ldvt < n_kv) return DIT_EINVAL;
  if (ldq % 8 || ldk % 8 || ldo % 8 || ldvt % 8) return DIT_EINVAL;
  if (head_dim * ldvt * (dtype == DIT_F32 ? 4 : 2) >= ((int64_t)1 << 32)) return DIT_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o)) return DIT_EINVAL;
  if (n_q == 0) return DIT_OK;
  return hip_status(dit::launch_attention(dtype, q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, (int)n_heads,
                                          (int)head_dim, 1, nullptr, nullptr, static_cast<hipStream_t>(stream)));
}

int dit_attention_split_workspace(int64_t n_q, int64_t n_kv, int64_t n_heads, int64_t head_dim, int64_t splits,
                                  size_t* bytes_out) {
  if (!bytes_out || n_q < 0 || n_kv < 1 || n_heads < 1 || head_dim < 1 || splits < 1 || splits > 64)
    return DIT_EINVAL;
  size_t ml_off = 0;
  *bytes_out = split_part_bytes(dit::attention_splits_effective(splits, n_kv), n_q, n_heads * head_dim, n_heads,
                                &ml_off);
  return DIT_OK;
}

int dit_attention_split(int32_t dtype, const void* q, int64_t ldq, const void* k, int64_t ldk, const void* vt,
                        int64_t ldvt, void* o, int64_t ldo, int64_t n_q, int64_t n_kv, int64_t n_heads,
                        int64_t head_dim, int64_t splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (splits < 1 || splits > 64) return DIT_EINVAL;
  size_t need = 0;
  if (n_q >= 0 && n_kv >= 1 && n_heads >= 1 &&
      dit_attention_split_workspace(n_q, n_kv, n_heads, head_dim, splits, &need) != DIT_OK)
    return DIT_EINVAL;
  const int64_t s_eff = n_kv >= 1 ? dit::attention_splits_effective(splits, n_kv) : 1;
  if (s_eff == 1) return dit_attention(dtype, q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, n_heads, head_dim, stream);
  if (dtype != DIT_F32 && dtype != DIT_BF16) return DIT_EINVAL;
  if (!q || !k || !vt || !o || n_q < 0 || n_heads < 1) return DIT_EINVAL;
  if (head_dim != 64 && head_dim != 128) return DIT_EINVAL;
  const int64_t d = n_heads * head_dim;
  if (ldq < d || ldk < d || ldo < d || ldvt < n_kv) return DIT_EINVAL;
  if (ldq % 8 || ldk % 8 || ldo % 8 || ldvt % 8) return DIT_EINVAL;
  if (head_dim * ldvt * (dtype == DIT_F32 ? 4 : 2) >= ((int64_t)1 << 32)) return DIT_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o)) return DIT_EINVAL;
  if (!workspace || !aligned16(workspace)) return DIT_EINVAL;
  if (workspace_bytes < need) return DIT_ENOSPC;
  if (n_q == 0) return DIT_OK;
  size_t ml_off = 0;
  split_part_bytes(s_eff, n_q, d, n_heads, &ml_off);
  char* ws = static_cast<char*>(workspace);
  return hip_status(dit::launch_attention(dtype, q, ldq, k, ldk, vt, ldvt, o, ldo, n_q, n_kv, (int)n_heads,
                                          (int)head_dim, splits, reinterpret_cast<float*>(ws),
                                          reinterpret_cast<float*>(ws + ml_off), static_cast<hipStream_t>(stream)));
}

int dit_linear(int32_t dtype, int32_t epilogue, const void* a, int64_t lda, const void* w, int64_t ldw,
               const float* w_scale, int64_t up_offset, int64_t m, int64_t n, int64_t k, void* out,
               int64_t ldo, const void* aux, int64_t ldaux, const float* gate, void* stream) {
  if (dtype != DIT_F32 && dtype != DIT_BF16 && dtype != DIT_W8_BF16) return DIT_EINVAL;
  if (epilogue < DIT_EPI_STORE || epilogue > DIT_EPI_FINAL) return DIT_EINVAL;
  if (!a || !w || !out || m < 0 || n < 64 || n % 64 || k < 1) return DIT_EINVAL;
  if (k % (dtype == DIT_F32 ? 32 : 64)) return DIT_EINVAL;
  if (lda < k || ldw < k || lda % 8 || ldo % 8 || ldw % (dtype == DIT_W8_BF16 ? 16 : 8)) return DIT_EINVAL;
  if ((dtype == DIT_W8_BF16) != (w_scale != nullptr)) return DIT_EINVAL;
  const bool needs_aux = epilogue == DIT_EPI_RESID || epilogue == DIT_EPI_FINAL;
  const bool needs_gate = needs_aux || epilogue == DIT_EPI_ACCUM;
  if (needs_aux && (!aux || ldaux < n || ldaux % 8)) return DIT_EINVAL;
  if (needs_gate && !gate) return DIT_EINVAL;
  if (epilogue == DIT_EPI_GATEUP && up_offset < n) return DIT_EINVAL;
  if (epilogue == DIT_EPI_STORE_T ? ldo < m : ldo < n) return DIT_EINVAL;
  if (!aligned16(a) || !aligned16(w) || !aligned16(out) || (aux && !aligned16(aux))) return DIT_EINVAL;
  if (!dit::gemm_offsets_fit(dtype, lda, ldw, epilogue == DIT_EPI_GATEUP ? up_offset + 256 : 256))
    return DIT_EINVAL;
  if (m == 0) return DIT_OK;
  dit::GemmArgs g{};
  g.a = a;
  g.lda = lda;
  g.b = w;
  g.ldb = ldw;
  g.bscale = w_scale;
  g.up_offset = up_offset;
  g.M = m;
  g.N = n;
  g.K = k;
  g.out = out;
  g.ldo = ldo;
  g.aux = aux;
  g.ldaux = ldaux;
  g.gate = gate;
  return hip_status(dit::launch_gemm(dtype, static_cast<dit::Epilogue>(epilogue), g,
                                     static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- output head

int dit_final_layer(int32_t x_dtype, const void* x, int64_t ldx, int64_t n_tokens, int64_t d, const float* shift,
                    const float* scale, const float* w_out, int64_t out_dim, float* out, int64_t ldo, float eps,
                    void* stream) {
  if (x_dtype != DIT_F32 && x_dtype != DIT_BF16) return DIT_EINVAL;
  if (!shift || !scale || !w_out || n_tokens < 0) return DIT_EINVAL;
  if (n_tokens > 0 && (!x || !out)) return DIT_EINVAL;  // an empty row range may pass NULL rows
  if (d < 64 || d > 8192 || d % 64 || out_dim < 1 || out_dim > 128) return DIT_EINVAL;
  if (ldx < d || ldx % 8 || ldo < out_dim || !(eps > 0.f)) return DIT_EINVAL;
  if (!aligned16(x) || !aligned16(shift) || !aligned16(scale) || !aligned16(w_out)) return DIT_EINVAL;
  if (reinterpret_cast<uintptr_t>(out) & 3u) return DIT_EINVAL;
  if (n_tokens == 0) return DIT_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(run_step(DIT_K_FINAL, st, [&] {
    return dit::launch_final_layer(x_dtype == DIT_F32, x, ldx, n_tokens, (int)d, shift, scale, w_out, (int)out_dim,
                                   out, ldo, eps, st);
  }));
}

}  // extern "C"
