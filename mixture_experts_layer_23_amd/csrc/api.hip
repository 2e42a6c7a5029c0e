// api.hip -- the C ABI: argument validation, workspace layout, launch order,
// error reporting and optional per-kernel timing.  Host code only.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace moe {

static thread_local char g_err[512] = "";

void set_error(const char* where, hipError_t e) {
  snprintf(g_err, sizeof g_err, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

// --- timing ----------------------------------------------------------------
// Events come from a pool that grows on demand and is reused after each
// report, so that timing a run creates no events inside it after the first.
struct TimedLaunch {
  std::string name;
  hipEvent_t a, b;
};
static bool g_timing = false;
static std::string g_only;               // time only launches of this name ("" = all)
static std::vector<TimedLaunch> g_records;
static std::vector<hipEvent_t> g_pool;
static size_t g_pool_next = 0;
static bool g_last_timed = false;

bool timing_on() { return g_timing; }

static bool pool_event(hipEvent_t* e) {
  if (g_pool_next == g_pool.size()) {
    hipEvent_t n;
    if (hipEventCreate(&n) != hipSuccess) return false;
    g_pool.push_back(n);
  }
  *e = g_pool[g_pool_next++];
  return true;
}

void timing_before(const char* name, hipStream_t s) {
  g_last_timed = false;
  if (!g_only.empty() && g_only != name) return;
  TimedLaunch r;
  r.name = name;
  if (!pool_event(&r.a) || !pool_event(&r.b)) return;
  (void)hipEventRecord(r.a, s);
  g_records.push_back(r);
  g_last_timed = true;
}

void timing_after(hipStream_t s) {
  if (g_last_timed && !g_records.empty()) (void)hipEventRecord(g_records.back().b, s);
  g_last_timed = false;
}

// --- configuration ----------------------------------------------------------
static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static int check_cfg(const moe_config* c) {
  if (!c) return MOE_EINVAL;
  if (c->T < 0 || c->D <= 0 || c->F <= 0 || c->E < 1 || c->E > 1024) return MOE_EINVAL;
  if (c->D % 64 || c->F % 64) return MOE_EINVAL;
  // the grouped GEMMs address one tile's rows of D or 2F elements with 32-bit
  // byte offsets inside a descriptor based at the tile: D and F up to 2^20
  // keep 256 rows of 2F bf16 under 2^31 bytes
  if (c->D > kMaxDim || c->F > kMaxDim) return MOE_EINVAL;
  if (c->routing != MOE_TOKEN_CHOICE && c->routing != MOE_EXPERT_CHOICE) return MOE_EINVAL;
  if (c->K < 1 || c->K > c->E) return MOE_EINVAL;
  if (c->routing == MOE_TOKEN_CHOICE && c->K > 64) return MOE_EINVAL;
  if (c->expert_lo < 0 || c->expert_lo > c->expert_hi || c->expert_hi > c->E) return MOE_EINVAL;
  if (c->n_shared < 0 || c->n_shared > 1) return MOE_EINVAL;
  if (c->score_fn != MOE_SCORE_SOFTMAX && c->score_fn != MOE_SCORE_SIGMOID) return MOE_EINVAL;
  if (c->gating != MOE_GATE_TRUNCATED && c->gating != MOE_GATE_RENORM) return MOE_EINVAL;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_EDTYPE;
  if (!std::isfinite(c->capacity_factor)) return MOE_EINVAL;
  // expert choice weighs a pair by its softmax probability (gating A)
  if (c->routing == MOE_EXPERT_CHOICE &&
      (c->score_fn != MOE_SCORE_SOFTMAX || c->gating != MOE_GATE_TRUNCATED))
    return MOE_EINVAL;
  // row indices, slot indices and element offsets of row buffers fit the
  // kernels' int32 / int64 arithmetic
  const int64_t rows = routed_rows_max(*c) + (int64_t)c->n_shared * c->T;
  if (rows > INT32_MAX / 2) return MOE_EINVAL;
  if ((int64_t)c->T * slot_width(*c) > INT32_MAX / 2) return MOE_EINVAL;
  return MOE_OK;
}

static int capacity_of(const moe_config& c) {
  if (c.routing == MOE_EXPERT_CHOICE) return (int)ec_capacity(c);
  if (!(c.capacity_factor > 0.0)) return -1;
  const double v = std::ceil((c.capacity_factor * (double)c.T * (double)c.K) / (double)c.E);
  return v > (double)INT32_MAX ? INT32_MAX : (int)v;
}

static size_t al(size_t b) { return (b + 255) & ~(size_t)255; }

static int groups(const moe_config& c) { return (c.expert_hi - c.expert_lo) + c.n_shared; }

Workspace workspace_layout(const moe_config& c) {
  Workspace L = {};
  const bool ec = c.routing == MOE_EXPERT_CHOICE;
  const int64_t TK = (int64_t)c.T * c.K;
  const int64_t TW = (int64_t)c.T * slot_width(c);
  const int64_t rows = routed_rows_max(c) + (int64_t)c.n_shared * c.T;
  const size_t esz = c.dtype == MOE_BF16 ? 2 : 4;
  L.ntiles = ec ? 1 : (int)std::max<int64_t>(1, cdiv(TK, kSlotTile));
  L.aux_blocks = (int)std::max<int64_t>(1, cdiv(c.T, aux_tokens_per_block(c.E)));
  if (c.E <= 16) {
    // token chunks of the few-expert router weight gradient: about 320
    // workgroups, and for long batches chunks of at most 64 tokens (up to
    // 2048 chunks) so that the per-wave token loops stay short; chunks of at
    // least 16 tokens
    const int64_t dblk = cdiv(c.D, 64 * router_wgrad_width(c));
    int64_t nchunk = std::max<int64_t>(1, cdiv(320, dblk));
    nchunk = std::max<int64_t>(nchunk, std::min<int64_t>(cdiv(c.T, 64), 2048));
    nchunk = std::min<int64_t>(nchunk, std::max<int64_t>(1, cdiv(c.T, 16)));
    // every chunk must be non-empty: re-derive the count from the chunk length
    const int64_t len = cdiv(std::max<int64_t>(c.T, 1), nchunk);
    L.dwr_splits = (int)std::max<int64_t>(1, cdiv(std::max<int64_t>(c.T, 1), len));
  } else {
    // token splits of the many-expert router weight gradient: about 1024
    // workgroups of 128 x 128 (matrix-core path, E a multiple of 4) or
    // 64 x 64 (SIMT path) output tiles, splits of at least 256 tokens
    const int64_t tb = (c.E % 4 == 0) ? 128 : 64;
    const int64_t tiles = cdiv(c.E, tb) * cdiv(c.D, tb);
    int64_t s = cdiv(1024, tiles);
    s = std::min<int64_t>(s, std::max<int64_t>(1, c.T / 256));
    L.dwr_splits = (int)std::max<int64_t>(1, s);
  }
  size_t o = 0;
  L.tile_counts = o; o += al((size_t)L.ntiles * c.E * 4);
  L.tile_base = o;   o += al((size_t)L.ntiles * c.E * 4);
  L.aux_part = o;    o += al((size_t)L.aux_blocks * (c.E + 1) * 4);
  L.d_o = o;         o += al((size_t)rows * c.D * esz);
  L.dact = o;        o += al((size_t)rows * 2 * c.F * esz);
  L.dx_perm = o;     o += al((size_t)rows * c.D * esz);
  L.dg = o;          o += al((size_t)TW * 4);
  L.ds = o;          o += al((size_t)c.T * c.E * 4);
  L.dxr = o;         o += (c.E > 16) ? al((size_t)c.T * c.D * 4) : 0;
  L.dwr_part = o;    o += al((size_t)L.dwr_splits * (((size_t)c.E * c.D + c.E + 3) & ~(size_t)3) * 4);
  // router-bias partials (large E): chunks of at least 128 tokens, at most 64
  {
    const int64_t T1 = std::max<int64_t>(c.T, 1);
    const int64_t len = std::max<int64_t>(128, cdiv(T1, 64));
    L.rb_splits = (int)cdiv(T1, len);
  }
  L.rb_part = o;     o += al((size_t)L.rb_splits * (((size_t)c.E + 3) & ~(size_t)3) * 4);
  L.seq_part = o;    o += al((size_t)std::max(c.T, 1) * 4);
  L.seq_blk_n = o;   o += al((size_t)std::max(c.T, 1) * c.E * 4);
  L.seq_blk_p = o;   o += al((size_t)std::max(c.T, 1) * c.E * 4);
  L.ec_keys = o;     o += ec ? al((size_t)(c.expert_hi - c.expert_lo) * std::max(c.T, 1) * 4) : 0;
  {
    const bool fold = !ec && c.E <= 16;
    L.fold_counts = o; o += fold ? al((size_t)cdiv(std::max(c.T, 1), 16) * c.E * 4) : 0;
    L.fold_rank = o;   o += fold ? al((size_t)std::max<int64_t>(TK, 1) * 4) : 0;
  }
  L.total = o;
  return L;
}

// --- allocation-free permute ----------------------------------------------
// The tiled permute's per-tile expert histograms and bases (2 * ntiles * E
// int32, ntiles = ceil(T*K / 256)) live in this static device array for
// moe_permute_noalloc.  Every GPU the library runs on holds its own copy for
// the life of the process; each call on a GPU reuses it (nothing in it must
// start at zero: the histogram kernel writes every entry it later reads).
constexpr size_t kScratchBytes = 8u << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

// Host code may not pass `scratch` itself to a kernel (on the host that name
// is a stand-in, not the device address): the address is looked up once per
// device, with that device current, and kept.
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static int scratch_on_current_device(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error("hipGetDevice", e);
    return MOE_ELAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return MOE_EINVAL;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error("hipGetSymbolAddress(scratch)", e);
      return MOE_ELAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return MOE_OK;
}

// scratch bytes the permute needs: the tile histograms and, after them, the
// tile bases (the first two regions of the workspace layout)
static size_t permute_scratch_bytes(const moe_config& c, const Workspace& L) {
  return L.tile_base + al((size_t)L.ntiles * c.E * 4);
}

}  // namespace moe

using namespace moe;

#define REQ(p) \
  do { if (!(p)) return MOE_EINVAL; if (!aligned16(p)) return MOE_EALIGN; } while (0)
#define OPT(p) \
  do { if ((p) && !aligned16(p)) return MOE_EALIGN; } while (0)

extern "C" {

int moe_capacity(const moe_config* cfg, int32_t* capacity) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!capacity) return MOE_EINVAL;
  *capacity = capacity_of(*cfg);
  return MOE_OK;
}

int moe_rows_max(const moe_config* cfg, int64_t* rows) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!rows) return MOE_EINVAL;
  *rows = routed_rows_max(*cfg) + (int64_t)cfg->n_shared * cfg->T;
  return MOE_OK;
}

int moe_workspace_size(const moe_config* cfg, size_t* bytes) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!bytes) return MOE_EINVAL;
  *bytes = workspace_layout(*cfg).total;
  return MOE_OK;
}

int moe_route_ex(const moe_config* cfg, const void* x, const float* w_r, const float* r_bias,
                 const float* sel_bias, const float* jitter, const float* w_noise,
                 const float* noise_eps, float* noise_logits, float* logits, int32_t* topk_idx,
                 float* topk_w, float* lse, int32_t flags, moe_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (cfg->routing != MOE_TOKEN_CHOICE) return MOE_EINVAL;
  if (flags & ~MOE_ROUTE_LOGITS_GIVEN) return MOE_EINVAL;
  const bool given = (flags & MOE_ROUTE_LOGITS_GIVEN) != 0;
  if (!given) { REQ(x); REQ(w_r); OPT(r_bias); }
  OPT(sel_bias); OPT(jitter);
  if (w_noise) {
    // noisy top-K is defined on softmax scores; it needs x, eps and the
    // noise-logit output
    if (cfg->score_fn != MOE_SCORE_SOFTMAX) return MOE_EINVAL;
    REQ(x); REQ(w_noise); REQ(noise_eps); REQ(noise_logits);
  }
  REQ(logits); REQ(topk_idx); REQ(topk_w); OPT(lse);
  if (cfg->T == 0) return MOE_OK;
  return launch_route(*cfg, x, w_r, r_bias, sel_bias, jitter, w_noise, noise_eps, noise_logits,
                      logits, topk_idx, topk_w, lse, given, (hipStream_t)stream);
}

int moe_route(const moe_config* cfg, const void* x, const float* w_r, const float* r_bias,
              const float* sel_bias, float* logits, int32_t* topk_idx, float* topk_w, float* lse,
              int32_t flags, moe_stream_t stream) {
  return moe_route_ex(cfg, x, w_r, r_bias, sel_bias, nullptr, nullptr, nullptr, nullptr, logits,
                      topk_idx, topk_w, lse, flags, stream);
}

int moe_route_permute(const moe_config* cfg, const void* x, const float* w_r,
                      const float* r_bias, const float* sel_bias, float* logits,
                      int32_t* topk_idx, float* topk_w, float* lse, int32_t* counts_all,
                      int32_t* offsets, int32_t* slot_row, int32_t* row_token, int32_t* row_slot,
                      int32_t* n_dropped, void* x_perm, void* ws, size_t ws_bytes,
                      moe_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (cfg->routing != MOE_TOKEN_CHOICE) return MOE_EINVAL;
  REQ(x); REQ(w_r); OPT(r_bias); OPT(sel_bias);
  REQ(logits); REQ(topk_idx); REQ(topk_w); OPT(lse);
  REQ(counts_all); REQ(offsets); REQ(slot_row); REQ(row_token); REQ(row_slot); REQ(n_dropped);
  REQ(x_perm); REQ(ws);
  const Workspace L = workspace_layout(*cfg);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  return launch_route_permute(*cfg, x, w_r, r_bias, sel_bias, logits, topk_idx, topk_w, lse,
                              capacity_of(*cfg), counts_all, offsets, slot_row, row_token,
                              row_slot, n_dropped, x_perm, (char*)ws, L, (hipStream_t)stream);
}

int moe_route_expert_choice(const moe_config* cfg, const void* x, const float* w_r,
                            const float* r_bias, float* logits, float* gate_w, float* lse,
                            int32_t* counts_all, int32_t* offsets, int32_t* slot_row,
                            int32_t* row_token, int32_t* row_slot, void* x_perm, int32_t flags,
                            void* ws, size_t ws_bytes, moe_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (cfg->routing != MOE_EXPERT_CHOICE) return MOE_EINVAL;
  if (flags & ~MOE_ROUTE_LOGITS_GIVEN) return MOE_EINVAL;
  const bool given = (flags & MOE_ROUTE_LOGITS_GIVEN) != 0;
  REQ(x);
  if (!given) { REQ(w_r); OPT(r_bias); }
  REQ(logits); REQ(gate_w); OPT(lse); REQ(counts_all); REQ(offsets); REQ(slot_row);
  REQ(row_token); REQ(row_slot); REQ(x_perm); REQ(ws);
  const Workspace L = workspace_layout(*cfg);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  return launch_route_ec(*cfg, x, w_r, r_bias, logits, gate_w, lse, counts_all, offsets, slot_row,
                         row_token, row_slot, x_perm, given, (char*)ws, L, (hipStream_t)stream);
}

int moe_permute(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                int32_t* counts_all, int32_t* offsets, int32_t* slot_row, int32_t* row_token,
                int32_t* row_slot, int32_t* n_dropped, void* x_perm, void* ws, size_t ws_bytes,
                moe_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (cfg->routing != MOE_TOKEN_CHOICE) return MOE_EINVAL;
  REQ(topk_idx); REQ(x); REQ(counts_all); REQ(offsets); REQ(slot_row); REQ(row_token);
  REQ(row_slot); REQ(n_dropped); REQ(x_perm); REQ(ws);
  const Workspace L = workspace_layout(*cfg);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  return launch_permute(*cfg, capacity_of(*cfg), topk_idx, x, counts_all, offsets, slot_row,
                        row_token, row_slot, n_dropped, x_perm, (char*)ws, L, (hipStream_t)stream);
}

int moe_permute_noalloc(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                        int32_t* counts_all, int32_t* offsets, int32_t* slot_row,
                        int32_t* row_token, int32_t* row_slot, int32_t* n_dropped, void* x_perm,
                        moe_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (cfg->routing != MOE_TOKEN_CHOICE) return MOE_EINVAL;
  REQ(topk_idx); REQ(x); REQ(counts_all); REQ(offsets); REQ(slot_row); REQ(row_token);
  REQ(row_slot); REQ(n_dropped); REQ(x_perm);
  const Workspace L = workspace_layout(*cfg);
  if (permute_scratch_bytes(*cfg, L) > kScratchBytes) return MOE_EWORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  char* ws = nullptr;
  if ((rc = scratch_on_current_device(&ws))) return rc;
  return launch_permute(*cfg, capacity_of(*cfg), topk_idx, x, counts_all, offsets, slot_row,
                        row_token, row_slot, n_dropped, x_perm, ws, L, (hipStream_t)stream);
}

int moe_expert_ffn(const moe_config* cfg, const void* x, const void* x_perm, const int32_t* offsets,
                   const void* w_gate, const void* w_up, const void* w_down, void* act, void* h,
                   void* o_perm, moe_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  REQ(x); REQ(x_perm); REQ(offsets); REQ(act); REQ(h); REQ(o_perm);
  if (groups(*cfg) > 0) { REQ(w_gate); REQ(w_up); REQ(w_down); }
  if (cfg->T == 0 || groups(*cfg) == 0) return MOE_OK;
  hipStream_t st = (hipStream_t)stream;
  if ((rc = gemm_swiglu_fwd(*cfg, x, x_perm, offsets, w_gate, w_up, act, h, st))) return rc;
  return gemm_down_fwd(*cfg, offsets, h, w_down, o_perm, st);
}

int moe_combine(const moe_config* cfg, const void* o_perm, const int32_t* offsets,
                const int32_t* slot_row, const float* topk_w, void* y, moe_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  REQ(o_perm); REQ(offsets); REQ(slot_row); REQ(topk_w); REQ(y);
  if (cfg->T == 0) return MOE_OK;
  return launch_combine(*cfg, o_perm, offsets, slot_row, topk_w, y, (hipStream_t)stream);
}

int aux_balance_loss(const moe_config* cfg, const float* logits, const int32_t* counts_all,
                     float alpha, float z_lambda, float* losses, float* d_logits, void* ws,
                     size_t ws_bytes, moe_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (cfg->score_fn != MOE_SCORE_SOFTMAX) return MOE_EINVAL;
  if (!std::isfinite(alpha) || !std::isfinite(z_lambda)) return MOE_EINVAL;
  REQ(logits); REQ(counts_all); REQ(losses); OPT(d_logits); REQ(ws);
  const Workspace L = workspace_layout(*cfg);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  return launch_aux(*cfg, logits, counts_all, alpha, z_lambda, losses, d_logits, (char*)ws, L,
                    (hipStream_t)stream);
}

int moe_bias_update(const moe_config* cfg, const int32_t* counts_all, float gamma,
                    float* sel_bias, moe_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (cfg->routing != MOE_TOKEN_CHOICE) return MOE_EINVAL;
  if (!std::isfinite(gamma)) return MOE_EINVAL;
  REQ(counts_all); REQ(sel_bias);
  return launch_bias_update(*cfg, counts_all, gamma, sel_bias, (hipStream_t)stream);
}

int aux_seq_loss(const moe_config* cfg, const float* logits, const int32_t* topk_idx,
                 int32_t seq_len, float alpha, float* loss, float* d_logits, int32_t accumulate,
                 void* ws, size_t ws_bytes, moe_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (cfg->routing != MOE_TOKEN_CHOICE) return MOE_EINVAL;
  if (!std::isfinite(alpha) || seq_len <= 0) return MOE_EINVAL;
  if (cfg->T % seq_len) return MOE_EINVAL;
  REQ(logits); REQ(topk_idx); REQ(loss); OPT(d_logits); REQ(ws);
  const Workspace L = workspace_layout(*cfg);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  return launch_seq_aux(*cfg, logits, topk_idx, seq_len, alpha, loss, d_logits, accumulate != 0,
                        (char*)ws, L, (hipStream_t)stream);
}

int moe_backward_ex(const moe_config* cfg, const void* x, const float* w_r, const float* logits,
                    const int32_t* topk_idx, const float* topk_w, const int32_t* offsets,
                    const int32_t* slot_row, const void* x_perm, const void* act, const void* h,
                    const void* o_perm, const void* w_gate, const void* w_up, const void* w_down,
                    const void* dy, const float* d_logits_extra, const float* jitter, void* dx,
                    float* dw_r, float* d_rbias, void* dw_gate, void* dw_up, void* dw_down,
                    float* d_logits_out, void* ws, size_t ws_bytes, moe_stream_t stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  REQ(x); REQ(w_r); REQ(logits); REQ(topk_w); REQ(offsets); REQ(slot_row);
  REQ(x_perm); REQ(act); REQ(h); REQ(o_perm); REQ(dy);
  // expert choice indexes its [T][E] tables by expert: no top-K list
  if (cfg->routing == MOE_EXPERT_CHOICE) topk_idx = nullptr;
  else REQ(topk_idx);
  OPT(d_logits_extra); OPT(jitter); REQ(dx); REQ(dw_r); OPT(d_rbias); OPT(d_logits_out); REQ(ws);
  if (groups(*cfg) > 0) {
    REQ(w_gate); REQ(w_up); REQ(w_down); REQ(dw_gate); REQ(dw_up); REQ(dw_down);
  }
  const Workspace L = workspace_layout(*cfg);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  if (cfg->T == 0) return MOE_OK;
  return launch_backward(*cfg, x, w_r, logits, topk_idx, topk_w, offsets, slot_row, x_perm, act,
                         h, o_perm, w_gate, w_up, w_down, dy, d_logits_extra, jitter, dx, dw_r,
                         d_rbias, dw_gate, dw_up, dw_down, d_logits_out, (char*)ws, L,
                         (hipStream_t)stream);
}

int moe_backward(const moe_config* cfg, const void* x, const float* w_r, const float* logits,
                 const int32_t* topk_idx, const float* topk_w, const int32_t* offsets,
                 const int32_t* slot_row, const void* x_perm, const void* act, const void* h,
                 const void* o_perm, const void* w_gate, const void* w_up, const void* w_down,
                 const void* dy, const float* d_logits_extra, void* dx, float* dw_r,
                 float* d_rbias, void* dw_gate, void* dw_up, void* dw_down, float* d_logits_out,
                 void* ws, size_t ws_bytes, moe_stream_t stream) {
  return moe_backward_ex(cfg, x, w_r, logits, topk_idx, topk_w, offsets, slot_row, x_perm, act, h,
                         o_perm, w_gate, w_up, w_down, dy, d_logits_extra, nullptr, dx, dw_r,
                         d_rbias, dw_gate, dw_up, dw_down, d_logits_out, ws, ws_bytes, stream);
}

const char* moe_error_string(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (size, range, enum or NULL pointer)";
    case MOE_EALIGN: return "pointer not 16-byte aligned";
    case MOE_EDTYPE: return "unsupported dtype";
    case MOE_ELAUNCH: return g_err[0] ? g_err : "HIP launch failed";
    case MOE_EWORKSPACE: return "workspace smaller than moe_workspace_size()";
    default: return "unknown error code";
  }
}

int moe_timing_enable(int32_t on) {
  g_timing = on != 0;
  return MOE_OK;
}

int moe_timing_select(const char* kernel_name) {
  g_only = kernel_name ? kernel_name : "";
  return MOE_OK;
}

int moe_timing_report(char* buf, size_t len) {
  if (!buf || len == 0) return MOE_EINVAL;
  std::map<std::string, std::pair<int, double>> agg;
  std::vector<std::string> order;
  for (auto& r : g_records) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      if (!agg.count(r.name)) order.push_back(r.name);
      agg[r.name].first += 1;
      agg[r.name].second += ms;
    }
  }
  g_records.clear();
  g_pool_next = 0;
  std::string out;
  for (auto& n : order) {
    char line[256];
    snprintf(line, sizeof line, "%s\t%d\t%.6f\n", n.c_str(), agg[n].first, agg[n].second);
    out += line;
  }
  strncpy(buf, out.c_str(), len - 1);
  buf[len - 1] = 0;
  return MOE_OK;
}

}  // extern "C"
