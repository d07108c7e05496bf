// Host side of the C ABI declared in include/moe.h: validation, workspace
// layout and the order of kernel launches for each entry point. No entry
// point allocates, frees, synchronises or prints.
#include "moe.h"

#include <climits>
#include <cmath>

#include "moe_internal.h"

namespace moe {
thread_local StageEvents t_stage_events;
}

namespace {

using namespace moe;

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t ntiles_of(int64_t T) { return (T + kTileTokens - 1) / kTileTokens; }

// tokens per top-k block: quarter tiles when whole tiles would leave most of
// the chip idle (bf16 layers; their logits kernel clears the histograms the
// quarter-tile blocks add into)
int topk_block_tokens(const moe_config& c) {
  return (c.dtype == MOE_BF16 && ntiles_of(c.T) < 256) ? 16 : 64;
}

int64_t max_rows_of(const moe_config& c) {
  const int64_t a = c.T * c.k;
  const int64_t b = static_cast<int64_t>(c.E) * c.capacity;
  return a < b ? a : b;
}

int elem_size(const moe_config& c) { return c.dtype == MOE_BF16 ? 2 : 4; }

// candidates per token the route keeps: the top-k, plus the next candidates
// re-routing may need (each round uses at most k more per token)
int n_cand_of(const moe_config& c) {
  if (c.reroute <= 0) return c.k;
  const int64_t n = static_cast<int64_t>(c.k) * (1 + static_cast<int64_t>(c.reroute));
  return static_cast<int>(n < c.E ? n : c.E);
}

// priority order or re-routing: the general dispatch path
bool general_rule(const moe_config& c) { return c.priority != MOE_PRIORITY_TOKEN || c.reroute > 0; }

// The layer's first expert GEMM reads token rows straight from x through
// row_token (32-bit byte offsets into x); only a larger x needs the permuted
// copy materialised in the workspace.
bool layer_gathers(const moe_config& c) {
  return c.T * static_cast<int64_t>(c.d) * elem_size(c) < (static_cast<int64_t>(1) << 32);
}

int32_t check_cfg(const moe_config* c) {
  if (c == nullptr) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->E < 1 || c->E > MOE_MAX_EXPERTS || c->k < 1 || c->k > c->E ||
      c->k > MOE_MAX_TOPK || c->d < 1 || c->d_ff < 1 || c->capacity < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->T > 0 && c->capacity < 1) return MOE_ERR_INVALID_ARG;
  if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->act != MOE_ACT_RELU && c->act != MOE_ACT_GELU_TANH) return MOE_ERR_INVALID_ARG;
  if (c->priority != MOE_PRIORITY_TOKEN && c->priority != MOE_PRIORITY_RANK) return MOE_ERR_INVALID_ARG;
  if (c->reroute < 0 || c->reroute > MOE_MAX_TOPK) return MOE_ERR_INVALID_ARG;
  if (n_cand_of(*c) > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  // rows, slots and per-token indices are int32; tiles index a 32-bit grid
  if (c->T > (static_cast<int64_t>(INT32_MAX) / c->k)) return MOE_ERR_UNSUPPORTED;
  if (c->dtype == MOE_BF16 && (c->d % 64 != 0 || c->d_ff % 64 != 0)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

struct Layout {
  size_t logits, prob_part, hist, base, ids, gates, counts, offsets, prob_sum, slot, row_of,
      row_token, x_perm, h, y_perm, y_perm2, nsplit, rr_col, rr_served, rr_next, rr_fill, rr_fill0, rr_hist,
      rr_base, served_ids, cgates, total;
};

Layout layout_of(const moe_config& c) {
  Layout L{};
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    const size_t o = off;
    off += round_up(static_cast<size_t>(bytes > 0 ? bytes : 0));
    return o;
  };
  const int64_t T = c.T, E = c.E, k = c.k, R = max_rows_of(c), nt = ntiles_of(c.T);
  const int es = elem_size(c);
  L.logits = take(T * E * 4);
  L.prob_part = take((T + 15) / 16 * E * 4);  // per route block (16, 32 or 64 tokens)
  L.hist = take((T + 15) / 16 * E * 4);       // per-expert counts in rows of 16, 32 or 64 tokens
  L.base = take(nt * E * 4);
  L.ids = take(T * n_cand_of(c) * 4);
  L.gates = take(T * n_cand_of(c) * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.prob_sum = take(E * 4);
  L.slot = take(T * k * 4);
  L.row_of = take(T * k * 4);
  L.row_token = take(R * 4);
  L.x_perm = take(layer_gathers(c) ? 0 : R * c.d * es);
  L.h = take(R * c.d_ff * es);
  // y_perm in the layer's dtype (it holds the part-0 partial sums of the
  // rows the second GEMM splits in K, in place)
  L.y_perm = take(R * c.d * es);
  // the other K parts' partial sums of those rows (bf16 layers; bf16 rows)
  L.y_perm2 = take(c.dtype == MOE_BF16 ? R * c.d * 2 : 0);
  L.nsplit = take(3 * 4);  // parts, first split row, split rows (second GEMM)
  // state of the general dispatch (priority order, re-routing rounds); small
  // next to h, so every layout has it and moe_dispatch_reroute works for any
  // config
  const int64_t ntv = reroute_tiles(T, c.k);
  L.rr_col = take(T * k * 4);
  L.rr_served = take(T * k * 4);
  L.rr_next = take(T * 4);
  L.rr_fill = take(E * 4);
  L.rr_fill0 = take(E * 4);
  L.rr_hist = take(ntv * E * 4);
  L.rr_base = take(ntv * E * 4);
  L.served_ids = take(T * k * 4);
  L.cgates = take(T * k * 4);
  L.total = off;
  return L;
}

// workspace of moe_layer_backward
struct BwdLayout {
  size_t logits, W1t, W2t, x_perm, dy_perm, u, Z, h, du, dY, dxp, row_expert, row_gate, dg_row, ds,
      dsT, range_T, range_E, part, poff, At, Bt, colsum, total;
  int router_splits, router_dsplits;
  int64_t ldp;     // columns of the transposed weight-gradient operands (0: not used)
};

// bf16 weight gradients run on the MFMA grouped GEMM with transposed operands
// whose expert row ranges are padded to multiples of 64: at most R + 63 E
// columns. Its DMA offsets are 32-bit (256 rows of ldp bf16 values).
int64_t wgrad_ld_of(const moe_config& c) {
  if (c.dtype != MOE_BF16) return 0;
  const int64_t ldp = ((max_rows_of(c) + 64LL * c.E) + 63) / 64 * 64;
  if (256 * ldp * 2 >= (static_cast<int64_t>(1) << 32)) return 0;
  return ldp;
}

// row slices of dW_r = ds^T x (one group, K = T rows): enough blocks to fill
// the chip, slices of at least 256 rows
// token slices of the direct router weight gradient (few experts): 64 tokens
// or more per slice, about 1024 blocks of 256 columns at most
int router_direct_splits_of(const moe_config& c) {
  const int64_t col_blocks = (c.d + 255) / 256;
  int64_t sp = c.T / 64;
  const int64_t cap = 1024 / col_blocks;
  if (sp > cap) sp = cap;
  return sp < 1 ? 1 : static_cast<int>(sp);
}

int router_splits_of(const moe_config& c) {
  const int64_t tiles = ((c.E + 63) / 64) * ((c.d + 1 + 63) / 64);
  int64_t sp = (1024 + tiles - 1) / tiles;
  const int64_t by_rows = c.T / 256;
  if (sp > by_rows) sp = by_rows;
  if (sp > 256) sp = 256;
  return sp < 1 ? 1 : static_cast<int>(sp);
}

BwdLayout bwd_layout_of(const moe_config& c) {
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    const size_t o = off;
    off += round_up(static_cast<size_t>(bytes > 0 ? bytes : 0));
    return o;
  };
  const int64_t T = c.T, E = c.E, R = max_rows_of(c), d = c.d, f = c.d_ff;
  const int es = elem_size(c);
  const bool gather = layer_gathers(c);
  L.logits = take(T * E * 4);
  // transposed expert weights (fp32 layers only: the bf16 GEMM reads W1
  // and W2 as stored for the dgrad products)
  L.W1t = take(c.dtype == MOE_BF16 ? 0 : E * d * f * es);
  L.W2t = take(c.dtype == MOE_BF16 ? 0 : E * d * f * es);
  L.x_perm = take(gather ? 0 : R * d * es);
  L.dy_perm = take(gather ? 0 : R * d * es);
  L.u = take(R * f * 4);
  L.Z = take(R * f * 4);
  L.h = take(R * f * es);
  L.du = take(R * f * es);
  L.dY = take(R * d * es);
  L.dxp = take(R * d * 4);
  L.row_expert = take(R * 4);
  L.row_gate = take(R * 4);
  L.dg_row = take(R * 4);
  L.ds = take(T * E * 4);
  L.dsT = take(T * E * 4);
  L.range_T = take(8);
  L.range_E = take(8);
  L.router_splits = router_splits_of(c);
  L.router_dsplits = router_direct_splits_of(c);
  {
    const int64_t sp = E <= kRouterDirectMaxE ? L.router_dsplits : L.router_splits;
    L.part = take(sp > 1 ? sp * E * (d + 1) * 4 : 0);
  }
  L.ldp = wgrad_ld_of(c);
  const int64_t wide = d > f ? d : f;
  L.poff = take((E + 1) * 4);
  L.At = take(L.ldp * wide * es);
  L.Bt = take(L.ldp * wide * es);
  // per 64-row tile column sums of the transposed du and dY (bias gradients)
  L.colsum = take(L.ldp / 64 * wide * 4);
  L.total = off;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int32_t check_ws(const moe_config& c, void* ws, size_t ws_bytes) {
  if (ws == nullptr || !aligned(ws, kAlign) || ws_bytes < layout_of(c).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

#define MOE_HIP(call)                               \
  do {                                              \
    if ((call) != hipSuccess) return MOE_ERR_HIP;   \
  } while (0)

// ---- stages (arguments already validated)

// logits_out (nullable): the caller's logits output; logits_ws: workspace
// for them otherwise. hist (nullable): per-expert counts of the first k
// choices in rows of *hist_tokens tokens (16 or 32 from the fused route, 64
// otherwise), as the dispatch takes them.
// defer_rows (nullable): the caller's dispatch can sum the probability
// partials (a plain-rule dispatch whose scan runs in one launch); when the
// route leaves them to it, *defer_rows is the number of partial rows, else 0.
int32_t route_stage(const moe_config& c, const void* x, const void* Wr, const float* br,
                    int32_t* ids, float* gates, float* prob_sum, float* logits_out, float* logits_ws,
                    float* prob_part, int32_t* hist, int* hist_tokens, int* defer_rows, hipStream_t s) {
  *hist_tokens = kTileTokens;
  if (defer_rows != nullptr) *defer_rows = 0;
  const int fused = c.dtype == MOE_BF16 ? route_fused_tokens(c.T, c.E) : 0;
  if (fused > 0 && logits_out == nullptr &&
      (hist == nullptr || fused_scan_fits((c.T + fused - 1) / fused, c.E))) {
    // logits, softmax, top-k, gates and counts in one launch
    MOE_HIP(launch_route_fused_bf16(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(Wr), br, c.T,
                                    c.d, c.E, c.k, n_cand_of(c), c.renormalize, ids, gates,
                                    prob_sum != nullptr ? prob_part : nullptr, hist, s));
    const int prows = static_cast<int>((c.T + fused - 1) / fused);
    *hist_tokens = fused;
    if (prob_sum != nullptr) {
      if (defer_rows != nullptr && hist != nullptr) *defer_rows = prows;
      else MOE_HIP(launch_prob_reduce(prob_part, prows, c.E, prob_sum, s));
    }
    return MOE_OK;
  }
  float* logits = logits_out != nullptr ? logits_out : logits_ws;
  const int tb = topk_block_tokens(c);
  int32_t* zero = (hist != nullptr && tb < kTileTokens) ? hist : nullptr;  // cleared for the quarter-tile sums
  if (c.dtype == MOE_BF16)
    MOE_HIP(launch_logits_bf16(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(Wr), br,
                               logits, c.T, c.d, c.E, zero, zero != nullptr ? ntiles_of(c.T) * c.E : 0,
                               s));
  else
    MOE_HIP(launch_logits_f32(static_cast<const float*>(x), static_cast<const float*>(Wr), br, logits,
                              c.T, c.d, c.E, s));
  MOE_HIP(launch_topk(logits, c.T, c.E, c.k, n_cand_of(c), c.renormalize, ids, gates,
                      prob_sum != nullptr ? prob_part : nullptr, hist, tb, s));
  if (prob_sum != nullptr) {
    const int prows = static_cast<int>((c.T + tb - 1) / tb);
    if (defer_rows != nullptr && hist != nullptr && fused_scan_fits(ntiles_of(c.T), c.E))
      *defer_rows = prows;
    else
      MOE_HIP(launch_prob_reduce(prob_part, prows, c.E, prob_sum, s));
  }
  return MOE_OK;
}

// x_perm may be null: the row copy is then skipped (the layer gathers rows in
// its first GEMM instead). hist_ready: hist holds the route's counts in rows
// of hist_tokens tokens; else they are counted here (64-token rows).
// prob_rows > 0: also sum the route's probability partials (prob_part
// [prob_rows, E]) into prob_sum; only with the one-launch scan, which the
// route checked before leaving them here.
int32_t dispatch_stage(const moe_config& c, const void* x, const int32_t* ids, bool hist_ready,
                       int32_t* hist, int hist_tokens, int32_t* base, int32_t* counts,
                       int32_t* offsets, int32_t* slot, int32_t* row_of, int32_t* row_token,
                       void* x_perm, const float* prob_part, int prob_rows, float* prob_sum,
                       hipStream_t s) {
  if (!hist_ready) {
    MOE_HIP(launch_hist(ids, c.T, c.k, c.E, hist, s));
    hist_tokens = kTileTokens;
  }
  const int nt = static_cast<int>(ntiles_of(c.T));
  if (fused_scan_fits((c.T + hist_tokens - 1) / hist_tokens, c.E)) {
    MOE_HIP(launch_permute_scan(x, ids, hist, hist_tokens, c.T, c.k, c.E, c.capacity, c.d * elem_size(c),
                                counts, offsets, slot, row_of, row_token, x_perm, prob_part, prob_rows,
                                prob_rows > 0 ? prob_sum : nullptr, s));
    return MOE_OK;
  }
  // the separate scan takes 64-token rows (the fused route is used only when
  // its rows fit the one-launch path)
  MOE_HIP(launch_scan(hist, nt, c.E, c.capacity, base, counts, offsets, s));
  MOE_HIP(launch_permute(x, ids, base, offsets, c.T, c.k, c.E, c.capacity, c.d * elem_size(c), slot,
                         row_of, row_token, x_perm, s));
  return MOE_OK;
}

// the general capacity rule (priority order, re-routing rounds); cand has
// n_cand_of(c) columns; cand_gates, served_ids, cgates and x_perm may be null
int32_t dispatch_general_stage(const moe_config& c, void* ws, const void* x, const int32_t* cand,
                               const float* cand_gates, int32_t* counts, int32_t* offsets,
                               int32_t* slot, int32_t* row_of, int32_t* row_token,
                               int32_t* served_ids, float* cgates, void* x_perm, hipStream_t s) {
  const Layout L = layout_of(c);
  const ReroutePlan plan{at<int32_t>(ws, L.rr_col),  at<int32_t>(ws, L.rr_served),
                         at<int32_t>(ws, L.rr_next), at<int32_t>(ws, L.rr_fill),
                         at<int32_t>(ws, L.rr_fill0), at<int32_t>(ws, L.rr_hist),
                         at<int32_t>(ws, L.rr_base)};
  MOE_HIP(launch_dispatch_reroute(x, cand, cand_gates, c.T, c.k, n_cand_of(c), c.E, c.capacity,
                                  c.priority == MOE_PRIORITY_RANK, c.reroute,
                                  c.d * elem_size(c), plan, counts, offsets, slot, row_of,
                                  row_token, served_ids, cgates, x_perm, s));
  return MOE_OK;
}

// A is x_perm (row_idx null) or x with row r of the problem at row_idx[r].
int32_t gemm1_stage(const moe_config& c, const void* A, const int32_t* row_idx,
                    const int32_t* offsets, const void* W1, const float* b1, void* h,
                    hipStream_t s) {
  const int64_t R = max_rows_of(c);
  const int per_expert = static_cast<int>(c.T < c.capacity ? c.T : c.capacity);
  if (c.dtype == MOE_BF16)
    MOE_HIP(launch_gemm_bf16(static_cast<const uint16_t*>(A), row_idx, static_cast<const uint16_t*>(W1), b1,
                             h, nullptr, nullptr, kGemmOutBf16, c.act, offsets, c.E, c.d_ff, c.d, R,
                             per_expert, s));
  else
    MOE_HIP(launch_gemm_f32(static_cast<const float*>(A), row_idx, static_cast<const float*>(W1), b1,
                            static_cast<float*>(h), c.act, offsets, c.E, c.d_ff, c.d, per_expert, s));
  return MOE_OK;
}

// y_perm in the layer's dtype. y_perm2/nsplit (nullable, bf16 only): let the
// GEMM run some tiles as K parts; their rows in y_perm and y_perm2 then hold
// bf16 partial sums, and nsplit says which (see launch_gemm_bf16).
int32_t gemm2_stage(const moe_config& c, const void* h, const int32_t* offsets, const void* W2,
                    const float* b2, void* y_perm, void* y_perm2, int32_t* nsplit, hipStream_t s) {
  const int64_t R = max_rows_of(c);
  const int per_expert = static_cast<int>(c.T < c.capacity ? c.T : c.capacity);
  if (c.dtype == MOE_BF16)
    MOE_HIP(launch_gemm_bf16(static_cast<const uint16_t*>(h), nullptr, static_cast<const uint16_t*>(W2), b2,
                             y_perm, y_perm2, nsplit, kGemmOutYperm, kActNone, offsets, c.E, c.d, c.d_ff, R,
                             per_expert, s));
  else
    MOE_HIP(launch_gemm_f32(static_cast<const float*>(h), nullptr, static_cast<const float*>(W2), b2,
                            static_cast<float*>(y_perm), kActNone, offsets, c.E, c.d, c.d_ff, per_expert, s));
  return MOE_OK;
}

// y_perm2/nsplit: as gemm2_stage wrote them (null for fp32 layers and for
// a caller's y_perm)
int32_t combine_stage(const moe_config& c, const void* y_perm, const void* y_perm2,
                      const int32_t* nsplit, const int32_t* row_of, const float* gates, void* y,
                      hipStream_t s) {
  const bool bf = c.dtype == MOE_BF16;
  MOE_HIP(launch_combine(y_perm, bf, bf ? y_perm2 : nullptr, bf ? nsplit : nullptr, row_of, gates, c.T,
                         c.k, c.d, bf, y, s));
  return MOE_OK;
}

// Clears the stage kernel events of this thread when a layer call returns
// (also on an early error return).
struct StageEventsGuard {
  ~StageEventsGuard() { t_stage_events = StageEvents{}; }
};

#define MOE_TRY(expr)              \
  do {                             \
    const int32_t st_ = (expr);    \
    if (st_ != MOE_OK) return st_; \
  } while (0)

}  // namespace

extern "C" {

int32_t moe_capacity(int64_t T, int32_t k, int32_t E, double c, int32_t* C_out) {
  if (C_out == nullptr || T < 0 || k < 1 || E < 1 || !std::isfinite(c) || !(c > 0.0))
    return MOE_ERR_INVALID_ARG;
  if (T == 0) {
    *C_out = 0;
    return MOE_OK;
  }
  // c = m * 2^-s exactly, m a 53-bit integer; C = ceil(m*T*k / (E * 2^s)).
  int ex = 0;
  const double f = std::frexp(c, &ex);  // c = f * 2^ex, f in [0.5, 1)
  if (ex < -39 || ex > 41) return MOE_ERR_INVALID_ARG;  // c outside [2^-40, 2^40]
  const int64_t m = static_cast<int64_t>(std::ldexp(f, 53));
  const int s = 53 - ex;  // in [12, 92]
  if (T > (static_cast<int64_t>(1) << 62) / k) return MOE_ERR_INVALID_ARG;
  const __int128 num = static_cast<__int128>(m) * T * k;
  const __int128 den = static_cast<__int128>(E) << s;
  const __int128 q = (num + den - 1) / den;
  if (q > INT32_MAX) return MOE_ERR_INVALID_ARG;
  *C_out = static_cast<int32_t>(q);
  return MOE_OK;
}

int32_t moe_candidates(const moe_config* cfg, int32_t* n_cand) {
  MOE_TRY(check_cfg(cfg));
  if (n_cand == nullptr) return MOE_ERR_INVALID_ARG;
  *n_cand = n_cand_of(*cfg);
  return MOE_OK;
}

int32_t moe_max_rows(const moe_config* cfg, int64_t* rows) {
  MOE_TRY(check_cfg(cfg));
  if (rows == nullptr) return MOE_ERR_INVALID_ARG;
  *rows = max_rows_of(*cfg);
  return MOE_OK;
}

int32_t moe_workspace_size(const moe_config* cfg, size_t* bytes) {
  MOE_TRY(check_cfg(cfg));
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  *bytes = layout_of(*cfg).total;
  return MOE_OK;
}

int32_t moe_set_gemm_max_blocks(int32_t blocks) {
  if (blocks < 0) return MOE_ERR_INVALID_ARG;
  set_gemm_max_blocks(blocks);
  return MOE_OK;
}

int32_t moe_route(const moe_config* cfg, const void* x, const void* W_r, const float* b_r,
                  int32_t* topk_ids, float* topk_gates, float* prob_sum, float* logits, void* ws,
                  size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (x == nullptr || W_r == nullptr || topk_ids == nullptr || topk_gates == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(W_r, 16) || !aligned(b_r, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_gates, 4) || !aligned(prob_sum, 4) || !aligned(logits, 4))
    return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(c, ws, ws_bytes));
  const Layout L = layout_of(c);
  int hist_tokens = 0;
  return route_stage(c, x, W_r, b_r, topk_ids, topk_gates, prob_sum, logits, at<float>(ws, L.logits),
                     at<float>(ws, L.prob_part), nullptr, &hist_tokens, nullptr, stream);
}

int32_t moe_dispatch(const moe_config* cfg, const void* x, const int32_t* topk_ids,
                     int32_t* expert_counts, int32_t* expert_offsets, int32_t* slot,
                     int32_t* row_of, int32_t* row_token, void* x_perm, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (x == nullptr || topk_ids == nullptr || expert_counts == nullptr ||
      expert_offsets == nullptr || slot == nullptr || row_of == nullptr || row_token == nullptr ||
      x_perm == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(x_perm, 16) || !aligned(topk_ids, 4) ||
      !aligned(expert_counts, 4) || !aligned(expert_offsets, 4) || !aligned(slot, 4) ||
      !aligned(row_of, 4) || !aligned(row_token, 4))
    return MOE_ERR_INVALID_ARG;
  if (c.reroute != 0) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(c, ws, ws_bytes));
  const Layout L = layout_of(c);
  if (general_rule(c))
    return dispatch_general_stage(c, ws, x, topk_ids, nullptr, expert_counts, expert_offsets, slot,
                                  row_of, row_token, nullptr, nullptr, x_perm, stream);
  return dispatch_stage(c, x, topk_ids, false, at<int32_t>(ws, L.hist), kTileTokens, at<int32_t>(ws, L.base),
                        expert_counts, expert_offsets, slot, row_of, row_token, x_perm, nullptr, 0, nullptr,
                        stream);
}

int32_t moe_dispatch_reroute(const moe_config* cfg, const void* x, const int32_t* cand_ids,
                             const float* cand_gates, int32_t* expert_counts,
                             int32_t* expert_offsets, int32_t* slot, int32_t* row_of,
                             int32_t* row_token, int32_t* served_ids, float* combine_gates,
                             void* x_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (cand_ids == nullptr || cand_gates == nullptr || expert_counts == nullptr ||
      expert_offsets == nullptr || slot == nullptr || row_of == nullptr || row_token == nullptr ||
      combine_gates == nullptr || (x_perm != nullptr && x == nullptr))
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(x_perm, 16) || !aligned(cand_ids, 4) || !aligned(cand_gates, 4) ||
      !aligned(expert_counts, 4) || !aligned(expert_offsets, 4) || !aligned(slot, 4) ||
      !aligned(row_of, 4) || !aligned(row_token, 4) || !aligned(served_ids, 4) ||
      !aligned(combine_gates, 4))
    return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(c, ws, ws_bytes));
  return dispatch_general_stage(c, ws, x, cand_ids, cand_gates, expert_counts, expert_offsets,
                                slot, row_of, row_token, served_ids, combine_gates, x_perm,
                                stream);
}

int32_t moe_expert_ffn(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                       const void* W1, const float* b1, const void* W2, const float* b2, void* h,
                       void* y_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (x_perm == nullptr || expert_offsets == nullptr || W1 == nullptr || W2 == nullptr ||
      h == nullptr || y_perm == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x_perm, 16) || !aligned(W1, 16) || !aligned(W2, 16) || !aligned(b1, 16) ||
      !aligned(b2, 16) || !aligned(h, 16) || !aligned(y_perm, 16) || !aligned(expert_offsets, 4))
    return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(c, ws, ws_bytes));
  MOE_TRY(gemm1_stage(c, x_perm, nullptr, expert_offsets, W1, b1, h, stream));
  return gemm2_stage(c, h, expert_offsets, W2, b2, y_perm, nullptr, nullptr, stream);
}

int32_t moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* row_of,
                    const float* topk_gates, void* y, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (y_perm == nullptr || row_of == nullptr || topk_gates == nullptr || y == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(y_perm, 16) || !aligned(y, 16) || !aligned(row_of, 4) || !aligned(topk_gates, 4))
    return MOE_ERR_INVALID_ARG;
  return combine_stage(c, y_perm, nullptr, nullptr, row_of, topk_gates, y, stream);
}

int32_t moe_layer_forward(const moe_config* cfg, const void* x, const void* W_r,
                          const float* b_r, const void* W1, const float* b1, const void* W2,
                          const float* b2, void* y, const moe_route_info* info, void* ws,
                          size_t ws_bytes, hipEvent_t* stage_events, hipEvent_t* kernel_events,
                          hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (x == nullptr || W_r == nullptr || W1 == nullptr || W2 == nullptr || y == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(W_r, 16) || !aligned(W1, 16) || !aligned(W2, 16) ||
      !aligned(y, 16) || !aligned(b_r, 4) || !aligned(b1, 16) || !aligned(b2, 16))
    return MOE_ERR_INVALID_ARG;
  moe_route_info in{};
  if (info != nullptr) in = *info;
  if (!aligned(in.topk_ids, 4) || !aligned(in.topk_gates, 4) || !aligned(in.prob_sum, 4) ||
      !aligned(in.expert_counts, 4) || !aligned(in.expert_offsets, 4) || !aligned(in.slot, 4) ||
      !aligned(in.row_of, 4) || !aligned(in.row_token, 4) || !aligned(in.served_ids, 4) ||
      !aligned(in.combine_gates, 4) || !aligned(in.h, 16))
    return MOE_ERR_INVALID_ARG;
  if (stage_events != nullptr)
    for (int i = 0; i <= MOE_NUM_STAGES; ++i)
      if (stage_events[i] == nullptr) return MOE_ERR_INVALID_ARG;
  if (kernel_events != nullptr)
    for (int i = 0; i < 2 * MOE_NUM_STAGES; ++i)
      if (kernel_events[i] == nullptr) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(c, ws, ws_bytes));
  // every argument is valid: nothing below returns an error before a HIP call
  // has failed

  const Layout L = layout_of(c);
  int32_t* ids = in.topk_ids != nullptr ? in.topk_ids : at<int32_t>(ws, L.ids);
  float* gates = in.topk_gates != nullptr ? in.topk_gates : at<float>(ws, L.gates);
  int32_t* counts = in.expert_counts != nullptr ? in.expert_counts : at<int32_t>(ws, L.counts);
  int32_t* offsets = in.expert_offsets != nullptr ? in.expert_offsets : at<int32_t>(ws, L.offsets);
  int32_t* slot = in.slot != nullptr ? in.slot : at<int32_t>(ws, L.slot);
  int32_t* row_of = in.row_of != nullptr ? in.row_of : at<int32_t>(ws, L.row_of);
  int32_t* row_token = in.row_token != nullptr ? in.row_token : at<int32_t>(ws, L.row_token);
  const bool gather = layer_gathers(c);
  void* x_perm = gather ? nullptr : at<char>(ws, L.x_perm);
  void* h = in.h != nullptr ? in.h : at<char>(ws, L.h);
  void* y_perm = at<char>(ws, L.y_perm);
  const bool bf = c.dtype == MOE_BF16;
  void* y_perm2 = bf ? at<char>(ws, L.y_perm2) : nullptr;
  int32_t* nsplit = bf ? at<int32_t>(ws, L.nsplit) : nullptr;
  int32_t* hist = at<int32_t>(ws, L.hist);
  const bool gen = general_rule(c);
  float* cgates = gates;  // combine weights
  if (gen) cgates = in.combine_gates != nullptr ? in.combine_gates : at<float>(ws, L.cgates);

  StageEventsGuard guard;
  // stage st begins: its boundary event, and its kernels' start/end events
  auto begin = [&](int st) -> int32_t {
    if (stage_events != nullptr && hipEventRecord(stage_events[st], stream) != hipSuccess)
      return MOE_ERR_HIP;
    if (kernel_events != nullptr) t_stage_events = StageEvents{kernel_events[2 * st], kernel_events[2 * st + 1]};
    return MOE_OK;
  };
  // a stage that launched no kernel (no rows) marks its place on the stream
  auto end = [&](int st) -> int32_t {
    if (kernel_events != nullptr) {
      const bool none = t_stage_events.start != nullptr;
      t_stage_events = StageEvents{};
      if (none && (hipEventRecord(kernel_events[2 * st], stream) != hipSuccess ||
                   hipEventRecord(kernel_events[2 * st + 1], stream) != hipSuccess))
        return MOE_ERR_HIP;
    }
    return MOE_OK;
  };
  MOE_TRY(begin(MOE_STAGE_ROUTE));
  int hist_tokens = kTileTokens;
  int prob_rows = 0;  // > 0: the dispatch sums the route's probability partials
  MOE_TRY(route_stage(c, x, W_r, b_r, ids, gates, in.prob_sum, nullptr, at<float>(ws, L.logits),
                      at<float>(ws, L.prob_part), gen ? nullptr : hist, &hist_tokens, &prob_rows, stream));
  MOE_TRY(end(MOE_STAGE_ROUTE));
  MOE_TRY(begin(MOE_STAGE_DISPATCH));
  if (gen)
    MOE_TRY(dispatch_general_stage(c, ws, x, ids, gates, counts, offsets, slot, row_of, row_token,
                                   in.served_ids, cgates, x_perm, stream));
  else
    MOE_TRY(dispatch_stage(c, x, ids, true, hist, hist_tokens, at<int32_t>(ws, L.base), counts, offsets,
                           slot, row_of, row_token, x_perm, at<float>(ws, L.prob_part), prob_rows,
                           in.prob_sum, stream));
  MOE_TRY(end(MOE_STAGE_DISPATCH));
  MOE_TRY(begin(MOE_STAGE_GEMM1));
  MOE_TRY(gemm1_stage(c, gather ? x : x_perm, gather ? row_token : nullptr, offsets, W1, b1, h, stream));
  MOE_TRY(end(MOE_STAGE_GEMM1));
  MOE_TRY(begin(MOE_STAGE_GEMM2));
  MOE_TRY(gemm2_stage(c, h, offsets, W2, b2, y_perm, y_perm2, nsplit, stream));
  MOE_TRY(end(MOE_STAGE_GEMM2));
  MOE_TRY(begin(MOE_STAGE_COMBINE));
  MOE_TRY(combine_stage(c, y_perm, y_perm2, nsplit, row_of, cgates, y, stream));
  MOE_TRY(end(MOE_STAGE_COMBINE));
  if (stage_events != nullptr && hipEventRecord(stage_events[MOE_NUM_STAGES], stream) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int32_t moe_load_stats(const moe_config* cfg, const int32_t* expert_counts,
                       const int32_t* expert_offsets, const float* prob_sum, double aux_alpha,
                       int32_t* kept, int32_t* dropped, double* stats, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.T == 0) return MOE_OK;
  if (expert_counts == nullptr || expert_offsets == nullptr || stats == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(aux_alpha) || !aligned(expert_counts, 4) || !aligned(expert_offsets, 4) ||
      !aligned(prob_sum, 4) || !aligned(kept, 4) || !aligned(dropped, 4) || !aligned(stats, 8))
    return MOE_ERR_INVALID_ARG;
  MOE_HIP(launch_load_stats(expert_counts, expert_offsets, prob_sum, c.E, c.capacity, c.T, c.k, aux_alpha, kept,
                            dropped, stats, stream));
  return MOE_OK;
}

int32_t moe_backward_workspace_size(const moe_config* cfg, size_t* bytes) {
  MOE_TRY(check_cfg(cfg));
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  *bytes = bwd_layout_of(*cfg).total;
  return MOE_OK;
}

int32_t moe_layer_backward(const moe_config* cfg, const void* x, const void* W_r, const float* b_r,
                           const void* W1, const float* b1, const void* W2, const float* b2,
                           const moe_route_info* fwd, const void* dy, float aux_alpha, float* dx,
                           float* dW_r, float* db_r, float* dW1, float* db1, float* dW2, float* db2,
                           void* ws, size_t ws_bytes, hipEvent_t* stage_events, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_config& c = *cfg;
  if (c.reroute != 0) return MOE_ERR_UNSUPPORTED;
  if (c.T == 0) return MOE_OK;
  if (x == nullptr || W_r == nullptr || W1 == nullptr || W2 == nullptr || fwd == nullptr ||
      dy == nullptr || dx == nullptr || dW_r == nullptr || dW1 == nullptr || dW2 == nullptr)
    return MOE_ERR_INVALID_ARG;
  const moe_route_info& f = *fwd;
  if (f.topk_ids == nullptr || f.topk_gates == nullptr || f.expert_counts == nullptr ||
      f.expert_offsets == nullptr || f.row_of == nullptr || f.row_token == nullptr)
    return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(aux_alpha)) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(W_r, 16) || !aligned(W1, 16) || !aligned(W2, 16) ||
      !aligned(dy, 16) || !aligned(b_r, 4) || !aligned(b1, 16) || !aligned(b2, 16) ||
      !aligned(dx, 4) || !aligned(dW_r, 4) || !aligned(db_r, 4) || !aligned(dW1, 4) ||
      !aligned(db1, 4) || !aligned(dW2, 4) || !aligned(db2, 4) || !aligned(f.topk_ids, 4) ||
      !aligned(f.topk_gates, 4) || !aligned(f.expert_counts, 4) || !aligned(f.expert_offsets, 4) ||
      !aligned(f.row_of, 4) || !aligned(f.row_token, 4))
    return MOE_ERR_INVALID_ARG;
  if (stage_events != nullptr)
    for (int i = 0; i <= MOE_BWD_NUM_STAGES; ++i)
      if (stage_events[i] == nullptr) return MOE_ERR_INVALID_ARG;
  const BwdLayout L = bwd_layout_of(c);
  if (ws == nullptr || !aligned(ws, kAlign) || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  auto mark = [&](int i) -> int32_t {
    if (stage_events != nullptr && hipEventRecord(stage_events[i], stream) != hipSuccess)
      return MOE_ERR_HIP;
    return MOE_OK;
  };

  hipStream_t s = stream;
  const bool bf = c.dtype == MOE_BF16;
  const int es = elem_size(c);
  const int64_t R = max_rows_of(c);
  const int per_expert = static_cast<int>(c.T < c.capacity ? c.T : c.capacity);
  const int32_t* offsets = f.expert_offsets;
  const int32_t* row_token = f.row_token;
  float* logits = at<float>(ws, L.logits);
  void* W1t = at<char>(ws, L.W1t);
  void* W2t = at<char>(ws, L.W2t);
  float* u = at<float>(ws, L.u);
  float* Z = at<float>(ws, L.Z);
  void* h = at<char>(ws, L.h);
  void* du = at<char>(ws, L.du);
  void* dY = at<char>(ws, L.dY);
  float* dxp = at<float>(ws, L.dxp);
  int32_t* row_expert = at<int32_t>(ws, L.row_expert);
  float* row_gate = at<float>(ws, L.row_gate);
  float* dg_row = at<float>(ws, L.dg_row);
  float* ds = at<float>(ws, L.ds);
  float* dsT = at<float>(ws, L.dsT);
  int32_t* range_T = at<int32_t>(ws, L.range_T);
  int32_t* range_E = at<int32_t>(ws, L.range_E);

  MOE_TRY(mark(MOE_BWD_STAGE_RECOMPUTE));
  // router logits again (the probabilities of every expert are needed)
  if (bf)
    MOE_HIP(launch_logits_bf16(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W_r), b_r,
                               logits, c.T, c.d, c.E, nullptr, 0, s));
  else
    MOE_HIP(launch_logits_f32(static_cast<const float*>(x), static_cast<const float*>(W_r), b_r,
                              logits, c.T, c.d, c.E, s));
  // fp32 layers: transposed expert weights for the dgrad GEMMs,
  // W1t[e] [d, d_ff], W2t[e] [d_ff, d] (the bf16 GEMM reads W1 and W2 as
  // stored, K-major)
  if (!bf) {
    MOE_HIP(launch_transpose(W1, W1t, c.E, c.d_ff, c.d, false, s));
    MOE_HIP(launch_transpose(W2, W2t, c.E, c.d, c.d_ff, false, s));
  }
  // token rows of x and dy for the kept rows (read through row_token, or copied)
  const bool gather = layer_gathers(c);
  const void* xa = x;
  const void* dya = dy;
  const int32_t* ridx = row_token;
  if (!gather) {
    MOE_HIP(launch_gather_rows(x, row_token, offsets, c.E, R, c.d * es, at<char>(ws, L.x_perm), s));
    MOE_HIP(launch_gather_rows(dy, row_token, offsets, c.E, R, c.d * es, at<char>(ws, L.dy_perm), s));
    xa = at<char>(ws, L.x_perm);
    dya = at<char>(ws, L.dy_perm);
    ridx = nullptr;
  }
  // u = x W1_e^T + b1_e (pre-activation, fp32); Z = dy W2_e (fp32)
  if (bf) {
    MOE_HIP(launch_gemm_bf16(static_cast<const uint16_t*>(xa), ridx, static_cast<const uint16_t*>(W1), b1,
                             u, nullptr, nullptr, kGemmOutF32, kActNone, offsets, c.E, c.d_ff, c.d, R,
                             per_expert, s));
    MOE_HIP(launch_gemm_bf16_wt(static_cast<const uint16_t*>(dya), ridx, static_cast<const uint16_t*>(W2),
                                nullptr, Z, offsets, c.E, c.d_ff, c.d, R, per_expert, s));
  } else {
    MOE_HIP(launch_gemm_f32(static_cast<const float*>(xa), ridx, static_cast<const float*>(W1), b1, u,
                            kActNone, offsets, c.E, c.d_ff, c.d, per_expert, s));
    MOE_HIP(launch_gemm_f32(static_cast<const float*>(dya), ridx, static_cast<const float*>(W2t), nullptr,
                            Z, kActNone, offsets, c.E, c.d_ff, c.d, per_expert, s));
  }
  // per row: h, du, dY and the combine-weight gradient
  MOE_TRY(mark(MOE_BWD_STAGE_ROWS));
  MOE_HIP(launch_row_info(f.topk_ids, f.topk_gates, f.row_of, c.T, c.k, row_expert, row_gate, s));
  MOE_HIP(launch_bwd_rows(u, Z, row_token, row_gate, row_expert, offsets, c.E, dy, b2, c.d, c.d_ff, R,
                          bf, c.act, h, du, dY, dg_row, s));
  // dx_perm = du W1_e
  MOE_TRY(mark(MOE_BWD_STAGE_DGRAD));
  if (bf)
    MOE_HIP(launch_gemm_bf16_wt(static_cast<const uint16_t*>(du), nullptr, static_cast<const uint16_t*>(W1),
                                nullptr, dxp, offsets, c.E, c.d, c.d_ff, R, per_expert, s));
  else
    MOE_HIP(launch_gemm_f32(static_cast<const float*>(du), nullptr, static_cast<const float*>(W1t), nullptr,
                            dxp, kActNone, offsets, c.E, c.d, c.d_ff, per_expert, s));
  // expert weight and bias gradients
  MOE_TRY(mark(MOE_BWD_STAGE_WGRAD));
  if (L.ldp > 0) {
    // MFMA path: K-contiguous operands (expert rows as padded columns)
    int32_t* poff = at<int32_t>(ws, L.poff);
    auto* At = at<uint16_t>(ws, L.At);
    auto* Bt = at<uint16_t>(ws, L.Bt);
    const int ld = static_cast<int>(L.ldp);
    MOE_HIP(launch_pad_offsets(offsets, c.E, poff, s));
    float* colsum = at<float>(ws, L.colsum);
    MOE_HIP(launch_padded_transpose(du, nullptr, offsets, poff, c.E, c.d_ff, L.ldp, ld, true, At,
                                    db1 != nullptr ? colsum : nullptr, s));
    if (db1 != nullptr) MOE_HIP(launch_seg_colsum(colsum, poff, c.E, c.d_ff, db1, s));
    MOE_HIP(launch_padded_transpose(x, row_token, offsets, poff, c.E, c.d, L.ldp, ld, true, Bt, nullptr,
                                    s));
    MOE_HIP(launch_wgrad_bf16(At, Bt, poff, c.E, c.d_ff, c.d, ld, dW1, s));
    MOE_HIP(launch_padded_transpose(dY, nullptr, offsets, poff, c.E, c.d, L.ldp, ld, true, At,
                                    db2 != nullptr ? colsum : nullptr, s));
    if (db2 != nullptr) MOE_HIP(launch_seg_colsum(colsum, poff, c.E, c.d, db2, s));
    MOE_HIP(launch_padded_transpose(h, nullptr, offsets, poff, c.E, c.d_ff, L.ldp, ld, true, Bt, nullptr,
                                    s));
    MOE_HIP(launch_wgrad_bf16(At, Bt, poff, c.E, c.d, c.d_ff, ld, dW2, s));
    MOE_HIP(launch_zero_empty(offsets, c.E, static_cast<int64_t>(c.d) * c.d_ff, dW1, s));
    MOE_HIP(launch_zero_empty(offsets, c.E, static_cast<int64_t>(c.d) * c.d_ff, dW2, s));
  } else {
    MOE_HIP(launch_wgrad(du, bf, x, bf, row_token, offsets, c.E, c.d_ff, c.d, dW1, db1, false, 1,
                         nullptr, s));
    MOE_HIP(launch_wgrad(dY, bf, h, bf, nullptr, offsets, c.E, c.d, c.d_ff, dW2, db2, false, 1,
                         nullptr, s));
  }
  // router: ds, then dW_r = ds^T x, db_r, and dx = gathered dx_perm + ds W_r
  MOE_TRY(mark(MOE_BWD_STAGE_ROUTER));
  const double aux = static_cast<double>(aux_alpha) * c.E / (static_cast<double>(c.T) * c.T);
  MOE_HIP(launch_router_bwd(logits, f.topk_ids, f.row_of, dg_row, f.expert_counts, c.T, c.E, c.k,
                            c.renormalize, static_cast<float>(aux), ds, dsT, s));
  if (c.E <= kRouterDirectMaxE) {
    // few experts: one pass over x for all E sums per column, and the router
    // term of dx (E products per element) inside the dx gather
    MOE_HIP(launch_router_wgrad(ds, x, bf, c.T, c.E, c.d, L.router_dsplits, at<float>(ws, L.part), dW_r,
                                db_r, s));
    MOE_HIP(launch_router_dx(dxp, f.row_of, ds, W_r, bf, c.T, c.k, c.E, c.d, dx, s));
  } else {
    MOE_HIP(launch_range(range_T, static_cast<int32_t>(c.T), s));
    MOE_HIP(launch_range(range_E, c.E, s));
    MOE_HIP(launch_wgrad(ds, false, x, bf, nullptr, range_T, 1, c.E, c.d, dW_r, db_r, false,
                         L.router_splits, at<float>(ws, L.part), s));
    MOE_HIP(launch_router_dx(dxp, f.row_of, nullptr, nullptr, bf, c.T, c.k, c.E, c.d, dx, s));
    MOE_HIP(launch_wgrad(dsT, false, W_r, bf, nullptr, range_E, 1, static_cast<int>(c.T), c.d, dx,
                         nullptr, true, 1, nullptr, s));
  }
  return mark(MOE_BWD_NUM_STAGES);
}

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "HIP launch or event error";
    default: return "unknown status";
  }
}

}  // extern "C"
