// Recompute policy: the activation-memory ledger of a transformer layer and
// the choice, layer by layer, of what to store and what to recompute.
//
// Ledger ("Recomputing Activations" plate, "What you will learn", the
// per-token byte formula): per layer, sbh(34 + 5as/h) bytes when nothing is
// recomputed, 34sbh once the attention-score activations are dropped and
// rebuilt (selective), and 2sbh when a layer keeps nothing but its input
// (full).  Under
// tensor parallelism of size t the layer norms and the dropouts after
// attention and the MLP (10sbh) stay whole on every rank and the rest divides
// by t; sequence parallelism divides the 10sbh as well (LIT-736 record, Key
// takeaways bullets 1-2).
//
// Compute: a fully recomputed layer runs its forward pass a second time, one
// extra forward on top of forward plus backward, so about a third more
// training FLOPs (the plate's second paragraph); a selectively recomputed one
// re-does only the attention-score FLOPs.
//
// Every quantity is kept as an exact integer: bytes scaled by t, FLOPs per
// token scaled by L, so the planner's comparisons have no rounding.
#include <cmath>
#include <cstdint>
#include <string>

#include "../../include/srat.h"

namespace srat {

typedef __int128 i128;

namespace {

struct Ledger {
  i128 mem_t[3];     // bytes of one layer on this device, times t (none, selective, full)
  i128 cost_l[3];    // extra FLOPs per token of one layer under each policy, times L
  i128 base_l;       // training FLOPs per token of all layers, times L
  int64_t t, layers;
};

bool check(const srat_layer_desc* d, std::string* err) {
  if (!d) { *err = "layer desc is NULL"; return false; }
  if (d->s <= 0 || d->b <= 0 || d->h <= 0 || d->a <= 0 || d->layers <= 0) {
    *err = "s, b, h, a and layers must be > 0";
    return false;
  }
  if (d->t < 1) { *err = "t must be >= 1"; return false; }
  if (d->n_params < 0) { *err = "n_params must be >= 0"; return false; }
  if ((d->sequence_parallel != 0 && d->sequence_parallel != 1) || (d->causal != 0 && d->causal != 1)) {
    *err = "sequence_parallel and causal must be 0 or 1";
    return false;
  }
  // bounds under which no product below overflows 128 bits: with
  // s, b, h, a < 2^31, layers, t < 2^20, N < 2^50, sbh < 2^60 and as^2b < 2^70,
  // a layer's bytes times t stay below 2^85 and times the layer count below
  // 2^105; A = 4sh < 2^64, so the extra FLOPs (times L) stay below 2^105 and
  // the base L (6N + 3LA) below 2^127
  const int64_t lim = (int64_t)1 << 31;
  if (d->s >= lim || d->b >= lim || d->h >= lim || d->a >= lim || d->layers >= ((int64_t)1 << 20) ||
      d->t >= ((int64_t)1 << 20) || d->n_params >= ((int64_t)1 << 50) ||
      (i128)d->s * d->b * d->h >= ((i128)1 << 60) || (i128)d->s * d->s * d->a * d->b >= ((i128)1 << 70)) {
    *err = "sizes out of range";
    return false;
  }
  return true;
}

Ledger ledger(const srat_layer_desc* d) {
  Ledger g;
  const i128 sbh = (i128)d->s * d->b * d->h;
  const i128 as2b = (i128)d->a * d->s * d->s * d->b;
  const i128 t = d->t;
  // replicated part (10sbh) whole on each rank unless sequence parallel
  const i128 repl_t = d->sequence_parallel ? 10 * sbh : 10 * sbh * t;
  g.mem_t[SRAT_RECOMPUTE_NONE] = repl_t + 24 * sbh + 5 * as2b;
  g.mem_t[SRAT_RECOMPUTE_SELECTIVE] = repl_t + 24 * sbh;
  g.mem_t[SRAT_RECOMPUTE_FULL] = d->sequence_parallel ? 2 * sbh : 2 * sbh * t;
  const i128 L = d->layers;
  const i128 A = (i128)(d->causal ? 2 : 4) * d->s * d->h;   // score FLOPs per token, one layer
  g.cost_l[SRAT_RECOMPUTE_NONE] = 0;
  g.cost_l[SRAT_RECOMPUTE_SELECTIVE] = A * L;
  g.cost_l[SRAT_RECOMPUTE_FULL] = 2 * (i128)d->n_params + A * L;
  g.base_l = L * (6 * (i128)d->n_params + 3 * L * A);
  g.t = d->t;
  g.layers = d->layers;
  return g;
}

}  // namespace

int activation_bytes(const srat_layer_desc* d, int policy, double* bytes, double* extra, std::string* err) {
  if (!check(d, err)) return SRAT_ERR_INVALID;
  if (policy < SRAT_RECOMPUTE_NONE || policy > SRAT_RECOMPUTE_FULL) {
    *err = "unknown recompute policy";
    return SRAT_ERR_INVALID;
  }
  const Ledger g = ledger(d);
  if (bytes) *bytes = (double)g.mem_t[policy] / (double)g.t;
  if (extra) *extra = (double)(g.cost_l[policy] * g.layers) / (double)g.base_l;
  return SRAT_OK;
}

int plan_recompute(const srat_layer_desc* d, double budget, srat_recompute_plan* plan, std::string* err) {
  if (!plan) { *err = "plan is NULL"; return SRAT_ERR_INVALID; }
  *plan = srat_recompute_plan{0, 0, 0, 0.0, 0.0};
  if (!check(d, err)) return SRAT_ERR_INVALID;
  if (std::isnan(budget) || budget < 0) { *err = "budget must be a number >= 0"; return SRAT_ERR_INVALID; }
  const Ledger g = ledger(d);
  const i128 L = g.layers;
  const i128 mn = g.mem_t[SRAT_RECOMPUTE_NONE], ms = g.mem_t[SRAT_RECOMPUTE_SELECTIVE],
             mf = g.mem_t[SRAT_RECOMPUTE_FULL];
  // stored bytes * t must not exceed budget * t; every need is below 2^105,
  // so larger budgets are "everything fits"
  const long double bt = std::floor((long double)budget * (long double)g.t);
  const i128 cap = bt >= 1e36L ? ((i128)1 << 120) : (i128)bt;

  // For a fixed number nf of fully recomputed layers, the cheapest fit
  // recomputes the fewest layers selectively: every layer not fully
  // recomputed stores mn, and each selective one saves mn - ms.
  bool found = false;
  i128 best_cost = 0, best_mem = 0;
  int64_t best_nf = 0, best_ns = 0;
  for (int64_t nf = 0; nf <= g.layers; ++nf) {
    const i128 rest = L - nf;
    const i128 need = rest * mn + (i128)nf * mf;     // with no selective layer
    i128 ns = 0;
    if (need > cap) ns = (need - cap + (mn - ms) - 1) / (mn - ms);
    if (ns > rest) continue;
    const i128 cost = ns * g.cost_l[SRAT_RECOMPUTE_SELECTIVE] + (i128)nf * g.cost_l[SRAT_RECOMPUTE_FULL];
    const i128 mem = need - ns * (mn - ms);
    if (!found || cost < best_cost || (cost == best_cost && mem < best_mem)) {
      found = true;
      best_cost = cost;
      best_mem = mem;
      best_nf = nf;
      best_ns = (int64_t)ns;
    }
  }
  if (!found) {
    *err = "budget below the bytes of full recomputation of every layer";
    return SRAT_ERR_UNSUPPORTED;
  }
  plan->layers_full = best_nf;
  plan->layers_selective = best_ns;
  plan->layers_none = g.layers - best_nf - best_ns;
  plan->activation_bytes = (double)best_mem / (double)g.t;
  plan->extra_compute = (double)best_cost / (double)g.base_l;
  return SRAT_OK;
}

}  // namespace srat
