// alloc.cpp — lifetime-aware bit allocation over the units of a model (host code).
//
// STEPQuant talk preview (qingkeai.online), "STEPQuant 核心设计…": the time
// axis gives each unit (a GDN head, a KDA key row) a width from its error at
// each width and how long it lives, under a fixed memory budget; e-cogni
// STEPQuant analysis, "O que os autores propõem": the allocation minimises a
// lifetime-weighted distortion under a fixed bit budget and keeps the
// riskiest units in binary16 as sparse pivots; "Como funciona": the lifetime
// weight decays about exponentially; gpt-diffusion analysis, "Qué dice
// realmente el «6-bit»": pivots are counted apart from the nominal budget.
//
// Problem (every open point is fixed in the contract header):
//   w_u = sum_{t>=0} 2^(-t/h_u) = 1 / (1 - 2^(-1/h_u))      (lifetime weight)
//   pivots: the n_piv units of largest w_u err_u(8), ties to the lower index
//   minimise sum_{u not pivot} w_u err_u(b_u), b_u in {4, 6, 8},
//   subject to sum_u (b_u - 4) / 2 <= K = floor((budget - 4) m / 2).
// Exact by dynamic programming over (unit, width steps spent) while the table
// has at most 2^26 cells; beyond that, greedy upgrades along each unit's
// lower convex hull (optimal for the linear relaxation up to the last unit
// that does not fit).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <queue>
#include <vector>

#include "stq.h"

namespace {

double lifetime_weight(double h) { return -1.0 / std::expm1(-M_LN2 / h); }

// exact: dp over the steps spent so far (at most k), one unit at a time
void solve_dp(int m, int64_t K, const std::vector<double>& c, std::vector<int>& steps) {
  std::vector<double> dp(K + 1, 0.0), nx(K + 1);
  std::vector<uint8_t> ch((size_t)m * (K + 1));
  for (int i = 0; i < m; i++) {
    for (int64_t k = 0; k <= K; k++) {
      double best = dp[k] + c[3 * i];
      uint8_t arg = 0;
      for (int o = 1; o <= 2 && o <= k; o++) {
        const double v = dp[k - o] + c[3 * i + o];
        if (v < best) { best = v; arg = (uint8_t)o; }
      }
      nx[k] = best;
      ch[(size_t)i * (K + 1) + k] = arg;
    }
    dp.swap(nx);
  }
  int64_t k = K;
  for (int i = m - 1; i >= 0; i--) {
    const int o = ch[(size_t)i * (K + 1) + k];
    steps[i] = o;
    k -= o;
  }
}

// greedy along each unit's lower convex hull of (steps, weighted error)
void solve_greedy(int m, int64_t K, const std::vector<double>& c, std::vector<int>& steps) {
  struct Up { double gain; int unit, from, to; };
  auto worse = [](const Up& a, const Up& b) {        // priority: gain per step, then the lower unit
    return a.gain < b.gain || (a.gain == b.gain && a.unit > b.unit);
  };
  std::priority_queue<Up, std::vector<Up>, decltype(worse)> q(worse);
  for (int i = 0; i < m; i++) {
    // the middle width is on the lower hull only when its gain per step is at least the next one's
    const double e0 = c[3 * i], e1 = c[3 * i + 1], e2 = c[3 * i + 2];
    const double g1 = e0 - e1, g2 = e1 - e2;
    if (g1 >= g2) {                                  // convex: one step at a time
      if (g1 > 0) q.push({g1, i, 0, 1});
      else if (e0 - e2 > 0) q.push({(e0 - e2) / 2, i, 0, 2});
    } else if (e0 - e2 > 0) {
      q.push({(e0 - e2) / 2, i, 0, 2});              // off the hull: straight to 8 bits
    }
  }
  int64_t left = K;
  while (!q.empty() && left > 0) {
    const Up u = q.top();
    q.pop();
    const int cost = u.to - u.from;
    if (cost > left) continue;                       // the next best that still fits
    steps[u.unit] = u.to;
    left -= cost;
    if (u.to == 1) {
      const double g = c[3 * u.unit + 1] - c[3 * u.unit + 2];
      if (g > 0) q.push({g, u.unit, 1, 2});
    }
  }
}

}  // namespace

extern "C" stq_status stq_allocate_bits(int32_t n, const double* err, const double* half_life, int32_t n_pivots,
                                        double budget_bits, int32_t* bits_out, double* objective_out) {
  if (n < 1 || !err || !half_life || !bits_out || n_pivots < 0 || n_pivots > n) return STQ_ERR_ARG;
  if (!(budget_bits >= 4.0) || !(budget_bits <= 1e9)) return STQ_ERR_ARG;
  std::vector<double> w(n);
  for (int u = 0; u < n; u++) {
    const double h = half_life[u];
    if (!(h > 0.0) || !std::isfinite(h)) return STQ_ERR_ARG;
    for (int k = 0; k < 3; k++)
      if (!(err[3 * u + k] >= 0.0) || !std::isfinite(err[3 * u + k])) return STQ_ERR_ARG;
    w[u] = lifetime_weight(h);
  }
  // pivots: largest lifetime-weighted 8-bit error, ties to the lower index
  std::vector<int> order(n);
  for (int u = 0; u < n; u++) order[u] = u;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return w[a] * err[3 * a + 2] > w[b] * err[3 * b + 2]; });
  std::vector<char> piv(n, 0);
  for (int i = 0; i < n_pivots; i++) piv[order[i]] = 1;
  std::vector<int> rest;
  for (int u = 0; u < n; u++)
    if (!piv[u]) rest.push_back(u);
  const int m = (int)rest.size();
  int64_t K = (int64_t)std::floor((budget_bits - 4.0) * m / 2.0);
  K = std::min<int64_t>(K, 2 * (int64_t)m);
  std::vector<double> c(3 * (size_t)m);
  for (int i = 0; i < m; i++)
    for (int k = 0; k < 3; k++) c[3 * i + k] = w[rest[i]] * err[3 * rest[i] + k];
  std::vector<int> steps(m, 0);
  if (m > 0) {
    if ((double)m * (double)(K + 1) <= (double)(1 << 26)) solve_dp(m, K, c, steps);
    else solve_greedy(m, K, c, steps);
  }
  double obj = 0.0;
  for (int u = 0; u < n; u++) bits_out[u] = 16;
  for (int i = 0; i < m; i++) {
    bits_out[rest[i]] = 4 + 2 * steps[i];
    obj += c[3 * i + steps[i]];
  }
  if (objective_out) *objective_out = obj;
  return STQ_OK;
}
