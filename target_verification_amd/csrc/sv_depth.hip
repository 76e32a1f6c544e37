// Adaptive draft depth: a host-side policy that picks the next round's draft
// depth d (nt = d + 1) from the acceptance the rounds observed and the round
// times measured for each nt (the minfer plan's status notes, doc 95:
// per-depth acceptance with Beta smoothing, the minimum of the last four
// costs per depth, a 10% switch hysteresis, optimism for depths not yet
// seen, and a depth cap).
//
// Model.  c_j is the probability that draft j is accepted given drafts
// 1..j-1 were; with Beta(a0, b0) smoothing, c_j = (a0 + s_j) / (a0 + b0 +
// s_j + f_j), s_j and f_j counting acceptances and first rejections at depth
// j.  A depth never observed is taken to be at least as good as the one
// before it (optimism).  The expected committed tokens of a round at depth d
// are E(d) = 1 + sum_{k=1..d} prod_{j=1..k} c_j (for a constant c this is the
// DFlash/DSpark page's A = (1 - c^(d+1)) / (1 - c), "Is it worth it?").
// A round at depth d costs T(d + 1) + d * t_draft, T(nt) the minimum of the
// last four measured round times at that nt; an nt never measured is priced
// by the cost line through the measured ones (the weights-once model: a
// fixed weight stream plus a per-row term), optimistically when only one nt
// has been measured.  The policy moves to the depth that maximises
// E(d) / cost(d) only when that beats the current depth's rate by the
// hysteresis factor.
#include <algorithm>
#include <cmath>
#include <new>
#include <vector>

#include "sv_internal.h"

struct sv_depth {
  int dmax = 0;
  double a0 = 1, b0 = 1, hyst = 0.1, draft_ms = 0;
  std::vector<double> succ, fail;        // [1..dmax]
  std::vector<std::vector<double>> win;  // [1..dmax+1] last four costs per nt
  std::vector<int> wpos;
  int cur = 1;
};

namespace {

constexpr int kWindow = 4;

double accept_mean(const sv_depth *p, int j, double prev) {
  const double n = p->succ[j] + p->fail[j];
  const double mean = (p->a0 + p->succ[j]) / (p->a0 + p->b0 + n);
  if (n > 0) return mean;
  const double prior = p->a0 / (p->a0 + p->b0);
  return std::max(prior, prev);            // unseen: optimistic
}

double expected_tokens(const sv_depth *p, int d) {
  double e = 1.0, run = 1.0, prev = 0.0;
  for (int j = 1; j <= d; ++j) {
    const double c = accept_mean(p, j, prev);
    run *= c;
    e += run;
    prev = c;
  }
  return e;
}

bool measured(const sv_depth *p, int nt) { return !p->win[nt].empty(); }

double wmin(const sv_depth *p, int nt) {
  return *std::min_element(p->win[nt].begin(), p->win[nt].end());
}

// Round time at nt: the window minimum where measured; elsewhere the least-
// squares line T = w + nt * t_row through the measured minima (two or more
// measured nt), or, from a single measured nt_m, T_m for deeper rounds and
// T_m * nt / nt_m for shallower ones (optimistic both ways, so that an
// unmeasured depth gets tried).
double cost_nt(const sv_depth *p, int nt) {
  if (measured(p, nt)) return wmin(p, nt);
  double n = 0, sx = 0, sy = 0, sxx = 0, sxy = 0;
  int only = 0;
  for (int k = 1; k <= p->dmax + 1; ++k) {
    if (!measured(p, k)) continue;
    const double y = wmin(p, k);
    n += 1;
    sx += k;
    sy += y;
    sxx += (double)k * k;
    sxy += k * y;
    only = k;
  }
  if (n == 0) return 1.0;   // nothing measured yet: every depth costs the same
  if (n == 1) return nt > only ? wmin(p, only) : wmin(p, only) * nt / only;
  const double slope = (n * sxy - sx * sy) / (n * sxx - sx * sx);
  const double icpt = (sy - slope * sx) / n;
  const double lo = 1e-3 * (sy / n);
  return std::max(icpt + slope * nt, lo);
}

double rate(const sv_depth *p, int d) {
  return expected_tokens(p, d) / (cost_nt(p, d + 1) + d * p->draft_ms);
}

}  // namespace

extern "C" {

int sv_depth_create(int32_t d_max, int32_t d_start, float prior_a, float prior_b,
                    float hysteresis, float draft_ms, sv_depth **out) {
  if (!out) return SV_E_INVALID;
  *out = nullptr;
  if (d_max < 1 || d_max > SV_MAX_NT - 1 || d_start < 0 || d_start > d_max) return SV_E_INVALID;
  if (!(prior_a > 0.f) || !(prior_b > 0.f) || !(hysteresis >= 0.f) || !(draft_ms >= 0.f))
    return SV_E_INVALID;
  sv_depth *p = new (std::nothrow) sv_depth();
  if (!p) return SV_E_NOMEM;
  p->dmax = d_max;
  p->a0 = prior_a;
  p->b0 = prior_b;
  p->hyst = hysteresis;
  p->draft_ms = draft_ms;
  p->succ.assign(d_max + 1, 0.0);
  p->fail.assign(d_max + 1, 0.0);
  p->win.assign(d_max + 2, {});
  p->wpos.assign(d_max + 2, 0);
  p->cur = d_start;
  *out = p;
  return SV_OK;
}

void sv_depth_destroy(sv_depth *p) { delete p; }

int sv_depth_observe(sv_depth *p, int32_t d, int32_t n_seq, const int32_t *accepted_len,
                     double round_ms) {
  if (!p || d < 0 || d > p->dmax || n_seq < 0 || (n_seq > 0 && !accepted_len))
    return SV_E_INVALID;
  for (int s = 0; s < n_seq; ++s) {
    const int a = accepted_len[s];
    if (a < 0) continue;                   // a sequence that failed this round
    if (a > d) return SV_E_INVALID;
    for (int j = 1; j <= a; ++j) p->succ[j] += 1.0;
    if (a < d) p->fail[a + 1] += 1.0;
  }
  if (round_ms > 0.0) {
    auto &w = p->win[d + 1];
    if ((int)w.size() < kWindow) {
      w.push_back(round_ms);
    } else {
      w[p->wpos[d + 1]] = round_ms;
    }
    p->wpos[d + 1] = (p->wpos[d + 1] + 1) % kWindow;
  }
  return SV_OK;
}

int32_t sv_depth_next(sv_depth *p) {
  if (!p) return SV_E_INVALID;
  int best = p->cur;
  double best_rate = rate(p, best);
  for (int d = 0; d <= p->dmax; ++d) {
    const double r = rate(p, d);
    if (r > best_rate) {
      best = d;
      best_rate = r;
    }
  }
  if (best != p->cur && best_rate > (1.0 + p->hyst) * rate(p, p->cur)) p->cur = best;
  return p->cur;
}

int sv_depth_estimates(const sv_depth *p, double *accept, double *cost_ms, double *tok_per_ms) {
  if (!p) return SV_E_INVALID;
  double prev = 0.0;
  for (int j = 1; j <= p->dmax; ++j) {
    const double c = accept_mean(p, j, prev);
    if (accept) accept[j - 1] = c;
    prev = c;
  }
  for (int d = 0; d <= p->dmax; ++d) {
    if (cost_ms) cost_ms[d] = cost_nt(p, d + 1) + d * p->draft_ms;
    if (tok_per_ms) tok_per_ms[d] = rate(p, d);
  }
  return SV_OK;
}

}  // extern "C"
