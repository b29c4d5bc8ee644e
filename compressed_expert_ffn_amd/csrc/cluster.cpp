// Host routine of moe_cluster.h: dual-similarity clustering of the experts
// and the shared-base + truncated-SVD compression ("Breaking the MoE LLM
// Trilemma", key designs 1 and 2).  Plain C++ in float64; the readings of
// the page it follows are listed in include/moe_cluster.h.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "moe.h"
#include "moe_cluster.h"
#include "pack.h"

using cefn::report_error;

struct moe_cluster {
  moe_cluster_config cfg{};
  std::vector<double> mu;               // [E][d] activation centroids
  bool have_cache = false;
  std::vector<std::vector<float>> cvec;  // cached vec(W_i)
  std::vector<double> cnorm;             // their norms
  std::vector<int> age;
  std::vector<double> S_param;           // [E][E] cosine of cached vectors
};

namespace {

double dot_f(const float* a, const float* b, int64_t n) {
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += (double)a[i] * (double)b[i];
  return s;
}

double cos_of(double dot, double na, double nb) { return (na > 0.0 && nb > 0.0) ? dot / (na * nb) : 0.0; }

// k-medoids with k-means++ seeding from the uniforms u (moe_cluster.h)
void kmedoids(const std::vector<double>& D, int E, int G, const double* u, std::vector<int>& assign,
              std::vector<int>& med) {
  auto Dx = [&](int i, int j) { return D[(size_t)i * E + j]; };
  med.assign(1, std::min((int)(u[0] * E), E - 1));
  std::vector<double> d2(E);
  for (int j = 1; j < G; ++j) {
    double total = 0.0;
    for (int i = 0; i < E; ++i) {
      double m = Dx(i, med[0]);
      for (size_t q = 1; q < med.size(); ++q) m = std::min(m, Dx(i, med[q]));
      d2[i] = m * m;
      total += d2[i];
    }
    auto chosen = [&](int i) { return std::find(med.begin(), med.end(), i) != med.end(); };
    int pick = -1;
    if (total <= 0.0) {
      for (int i = 0; i < E && pick < 0; ++i)
        if (!chosen(i)) pick = i;
    } else {
      const double target = u[j] * total;
      double acc = 0.0;
      for (int i = 0; i < E; ++i) {
        acc += d2[i];
        if (acc > target && !chosen(i)) {
          pick = i;
          break;
        }
      }
      if (pick < 0)
        for (int i = E - 1; i >= 0 && pick < 0; --i)
          if (!chosen(i)) pick = i;
    }
    med.push_back(pick);
  }
  assign.assign(E, 0);
  for (int it = 0; it < 100; ++it) {
    for (int i = 0; i < E; ++i) {
      int best = 0;
      for (int g = 1; g < G; ++g)
        if (Dx(i, med[g]) < Dx(i, med[best])) best = g;
      assign[i] = best;
    }
    std::vector<int> nm = med;
    for (int g = 0; g < G; ++g) {
      int bi = -1;
      double bc = 0.0;
      for (int a = 0; a < E; ++a) {
        if (assign[a] != g) continue;
        double c = 0.0;
        for (int b = 0; b < E; ++b)
          if (assign[b] == g) c += Dx(a, b);
        if (bi < 0 || c < bc) {
          bi = a;
          bc = c;
        }
      }
      if (bi >= 0) nm[g] = bi;
    }
    if (nm == med) break;
    med = nm;
  }
}

// greedy evening out to exactly K per group (moe_cluster.h)
void even_out(const std::vector<double>& D, int E, int G, int K, const std::vector<int>& med, std::vector<int>& assign) {
  std::vector<int> size(G, 0);
  for (int i = 0; i < E; ++i) ++size[assign[i]];
  for (;;) {
    bool over = false;
    for (int g = 0; g < G; ++g) over |= size[g] > K;
    if (!over) break;
    int bi = -1, bh = -1;
    double bc = 0.0;
    for (int i = 0; i < E; ++i) {
      const int g = assign[i];
      if (size[g] <= K) continue;
      for (int h = 0; h < G; ++h) {
        if (size[h] >= K) continue;
        const double c = D[(size_t)i * E + med[h]] - D[(size_t)i * E + med[g]];
        if (bi < 0 || c < bc) {  // strict: keeps the lower (i, h) on ties
          bi = i;
          bh = h;
          bc = c;
        }
      }
    }
    --size[assign[bi]];
    ++size[bh];
    assign[bi] = bh;
  }
}

// ---- truncated SVD by block subspace iteration (float64) --------------

// counter-based start block: SplitMix64 of (seed, index) mapped to [-1, 1)
double start_value(uint64_t i) {
  uint64_t z = i + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0;
}

// Orthonormalise the b columns of M [m][b] (row-major) by modified
// Gram-Schmidt, twice; a column that vanishes is replaced by zeros.
void orthonormalise(std::vector<double>& M, int m, int b) {
  for (int pass = 0; pass < 2; ++pass)
    for (int j = 0; j < b; ++j) {
      for (int q = 0; q < j; ++q) {
        double d = 0.0;
        for (int i = 0; i < m; ++i) d += M[(size_t)i * b + q] * M[(size_t)i * b + j];
        for (int i = 0; i < m; ++i) M[(size_t)i * b + j] -= d * M[(size_t)i * b + q];
      }
      double n = 0.0;
      for (int i = 0; i < m; ++i) n += M[(size_t)i * b + j] * M[(size_t)i * b + j];
      n = std::sqrt(n);
      const double inv = n > 1e-300 ? 1.0 / n : 0.0;
      for (int i = 0; i < m; ++i) M[(size_t)i * b + j] *= inv;
    }
}

// One-sided Jacobi SVD of M [m][b] (columns rotated in place until
// orthogonal); returns the rotation J [b][b] and the column norms.
void jacobi_columns(std::vector<double>& M, int m, int b, std::vector<double>& J, std::vector<double>& sv) {
  J.assign((size_t)b * b, 0.0);
  for (int i = 0; i < b; ++i) J[(size_t)i * b + i] = 1.0;
  for (int sweep = 0; sweep < 60; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < b - 1; ++p)
      for (int q = p + 1; q < b; ++q) {
        double a = 0.0, bb = 0.0, c = 0.0;
        for (int i = 0; i < m; ++i) {
          const double x = M[(size_t)i * b + p], y = M[(size_t)i * b + q];
          a += x * x;
          bb += y * y;
          c += x * y;
        }
        if (std::fabs(c) <= 1e-15 * std::sqrt(a * bb) || c == 0.0) continue;
        off = std::max(off, std::fabs(c) / std::sqrt(a * bb));
        const double zeta = (bb - a) / (2.0 * c);
        const double t = (zeta >= 0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
        const double cs = 1.0 / std::sqrt(1.0 + t * t), sn = cs * t;
        for (int i = 0; i < m; ++i) {
          const double x = M[(size_t)i * b + p], y = M[(size_t)i * b + q];
          M[(size_t)i * b + p] = cs * x - sn * y;
          M[(size_t)i * b + q] = sn * x + cs * y;
        }
        for (int i = 0; i < b; ++i) {
          const double x = J[(size_t)i * b + p], y = J[(size_t)i * b + q];
          J[(size_t)i * b + p] = cs * x - sn * y;
          J[(size_t)i * b + q] = sn * x + cs * y;
        }
      }
    if (off <= 1e-15) break;
  }
  sv.assign(b, 0.0);
  for (int j = 0; j < b; ++j) {
    double n = 0.0;
    for (int i = 0; i < m; ++i) n += M[(size_t)i * b + j] * M[(size_t)i * b + j];
    sv[j] = std::sqrt(n);
  }
}

// Rank-r truncated SVD of R [m][n] (row-major): A [m][r] = U_r sqrt(s),
// B [n][r] = V_r sqrt(s).
void tsvd(const std::vector<double>& R, int m, int n, int r, std::vector<double>& A, std::vector<double>& B) {
  A.assign((size_t)m * r, 0.0);
  B.assign((size_t)n * r, 0.0);
  if (r == 0) return;
  const int b = std::min(std::min(m, n), r + 8);
  // Q = orth(R Om)
  std::vector<double> Q((size_t)m * b, 0.0), Z((size_t)n * b, 0.0);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < b; ++j) Z[(size_t)i * b + j] = start_value((uint64_t)i * 1315423911ull + j);
  auto mul_R = [&](const std::vector<double>& In, std::vector<double>& Out) {  // Out[m][b] = R In[n][b]
    std::fill(Out.begin(), Out.end(), 0.0);
    for (int i = 0; i < m; ++i)
      for (int k = 0; k < n; ++k) {
        const double v = R[(size_t)i * n + k];
        if (v == 0.0) continue;
        for (int j = 0; j < b; ++j) Out[(size_t)i * b + j] += v * In[(size_t)k * b + j];
      }
  };
  auto mul_Rt = [&](const std::vector<double>& In, std::vector<double>& Out) {  // Out[n][b] = R^T In[m][b]
    std::fill(Out.begin(), Out.end(), 0.0);
    for (int i = 0; i < m; ++i)
      for (int k = 0; k < n; ++k) {
        const double v = R[(size_t)i * n + k];
        if (v == 0.0) continue;
        for (int j = 0; j < b; ++j) Out[(size_t)k * b + j] += v * In[(size_t)i * b + j];
      }
  };
  mul_R(Z, Q);
  orthonormalise(Q, m, b);
  std::vector<double> prev(r, -1.0), J, sv, M((size_t)n * b);
  for (int it = 0; it < 200; ++it) {
    mul_Rt(Q, Z);  // Z = R^T Q
    // singular value estimates of R on span(Q): those of Z
    M = Z;
    jacobi_columns(M, n, b, J, sv);
    std::vector<double> s = sv;
    std::sort(s.begin(), s.end(), std::greater<double>());
    double change = 0.0;
    for (int j = 0; j < r; ++j) change = std::max(change, std::fabs(s[j] - prev[j]) / std::max(s[0], 1e-300));
    prev.assign(s.begin(), s.begin() + r);
    if (it >= 3 && change <= 1e-15) break;
    orthonormalise(Z, n, b);
    mul_R(Z, Q);
    orthonormalise(Q, m, b);
  }
  // R ~ Q Q^T R = Q (R^T Q)^T; with R^T Q = M_rot J^T (columns of M_rot
  // orthogonal, norms sv): R ~ (Q J) diag(sv) (M_rot / sv)^T
  std::vector<int> order(b);
  for (int j = 0; j < b; ++j) order[j] = j;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return sv[x] > sv[y]; });
  for (int c = 0; c < r && c < b; ++c) {
    const int j = order[c];
    const double s = sv[j];
    if (!(s > 0.0)) continue;
    const double root = std::sqrt(s);
    for (int i = 0; i < m; ++i) {
      double u = 0.0;
      for (int q = 0; q < b; ++q) u += Q[(size_t)i * b + q] * J[(size_t)q * b + j];
      A[(size_t)i * r + c] = u * root;
    }
    for (int i = 0; i < n; ++i) B[(size_t)i * r + c] = M[(size_t)i * b + j] / s * root;
  }
}

}  // namespace

extern "C" {

int moe_cluster_create(const moe_cluster_config* cfg, moe_cluster** out) {
  if (!cfg || !out) return report_error(MOE_ERR_INVALID_ARG, "null config or output");
  *out = nullptr;
  const moe_cluster_config& c = *cfg;
  if (c.E <= 0 || c.G <= 0 || c.E % c.G || c.d <= 0 || c.n_param <= 0)
    return report_error(MOE_ERR_INVALID_ARG, "need E, G, d, n_param > 0 and E % G == 0");
  if (!(c.alpha >= 0.0 && c.alpha <= 1.0) || !(c.beta >= 0.0 && c.beta <= 1.0) || !(c.eps >= 0.0) ||
      c.cache_life < 1)
    return report_error(MOE_ERR_INVALID_ARG, "alpha, beta in [0, 1], eps >= 0, cache_life >= 1");
  moe_cluster* s = new moe_cluster();
  s->cfg = c;
  s->mu.assign((size_t)c.E * c.d, 0.0);
  *out = s;
  return MOE_OK;
}

int moe_cluster_destroy(moe_cluster* c) {
  delete c;
  return MOE_OK;
}

int moe_cluster_get_centroids(const moe_cluster* c, double* mu) {
  if (!c || !mu) return report_error(MOE_ERR_INVALID_ARG, "null argument");
  std::memcpy(mu, c->mu.data(), sizeof(double) * c->mu.size());
  return MOE_OK;
}

int moe_cluster_set_centroids(moe_cluster* c, const double* mu) {
  if (!c || !mu) return report_error(MOE_ERR_INVALID_ARG, "null argument");
  std::memcpy(c->mu.data(), mu, sizeof(double) * c->mu.size());
  return MOE_OK;
}

int moe_cluster_observe(moe_cluster* c, const float* X, int32_t T, const int32_t* idx, int32_t k) {
  if (!c) return report_error(MOE_ERR_INVALID_ARG, "null state");
  if (T < 0 || k <= 0 || (T > 0 && (!X || !idx))) return report_error(MOE_ERR_INVALID_ARG, "bad batch");
  const int E = c->cfg.E, d = c->cfg.d;
  for (int64_t i = 0; i < (int64_t)T * k; ++i)
    if (idx[i] < 0 || idx[i] >= E) return report_error(MOE_ERR_INVALID_ARG, "expert id %d out of range", idx[i]);
  std::vector<double> sum((size_t)E * d, 0.0);
  std::vector<int64_t> cnt(E, 0);
  for (int t = 0; t < T; ++t)
    for (int a = 0; a < k; ++a) {
      const int e = idx[(size_t)t * k + a];
      bool seen = false;  // a row counts once per expert
      for (int b = 0; b < a; ++b) seen |= idx[(size_t)t * k + b] == e;
      if (seen) continue;
      ++cnt[e];
      for (int j = 0; j < d; ++j) sum[(size_t)e * d + j] += X[(size_t)t * d + j];
    }
  const double beta = c->cfg.beta;
  for (int e = 0; e < E; ++e) {
    if (!cnt[e]) continue;
    for (int j = 0; j < d; ++j) {
      const double xbar = sum[(size_t)e * d + j] / (double)cnt[e];
      c->mu[(size_t)e * d + j] = (1.0 - beta) * c->mu[(size_t)e * d + j] + beta * xbar;
    }
  }
  return MOE_OK;
}

int moe_cluster_regroup(moe_cluster* c, const float* const* W, const double* u, int32_t* group_of,
                        int32_t* members, double* S_out, int32_t* fresh_out) {
  if (!c || !W || !u || !group_of || !members) return report_error(MOE_ERR_INVALID_ARG, "null argument");
  const moe_cluster_config& cf = c->cfg;
  const int E = cf.E, G = cf.G, K = E / G, d = cf.d;
  const int64_t n = cf.n_param;
  for (int e = 0; e < E; ++e)
    if (!W[e]) return report_error(MOE_ERR_INVALID_ARG, "W[%d] is null", e);
  for (int g = 0; g < G; ++g)
    if (!(u[g] >= 0.0 && u[g] < 1.0)) return report_error(MOE_ERR_INVALID_ARG, "u[%d] outside [0, 1)", g);
  // S_param cache: which rows to recompute
  std::vector<int> fresh(E, 0);
  if (!c->have_cache) {
    c->cvec.assign(E, std::vector<float>());
    c->cnorm.assign(E, 0.0);
    c->age.assign(E, 0);
    c->S_param.assign((size_t)E * E, 0.0);
    std::fill(fresh.begin(), fresh.end(), 1);
  } else {
    for (int e = 0; e < E; ++e) {
      const std::vector<float>& old = c->cvec[e];
      double diff = 0.0;
      for (int64_t i = 0; i < n; ++i) {
        const double t = (double)W[e][i] - (double)old[i];
        diff += t * t;
      }
      const bool moved = std::sqrt(diff) > cf.eps * c->cnorm[e];
      if (c->age[e] + 1 >= cf.cache_life || moved) {
        fresh[e] = 1;
      } else {
        ++c->age[e];
      }
    }
  }
  for (int e = 0; e < E; ++e)
    if (fresh[e]) {
      c->cvec[e].assign(W[e], W[e] + n);
      c->cnorm[e] = std::sqrt(dot_f(W[e], W[e], n));
      c->age[e] = 0;
    }
  {
    // rows and columns of the recomputed experts, one thread per row
    std::vector<int> rows;
    for (int e = 0; e < E; ++e)
      if (fresh[e]) rows.push_back(e);
    cefn::parallel_for((int)rows.size(), [&](int q) {
      const int i = rows[q];
      for (int j = 0; j < E; ++j) {
        if (fresh[j] && j < i) continue;  // the pair is done in row j
        const double s = (i == j) ? 1.0
                                  : cos_of(dot_f(c->cvec[i].data(), c->cvec[j].data(), n), c->cnorm[i], c->cnorm[j]);
        c->S_param[(size_t)i * E + j] = s;
        c->S_param[(size_t)j * E + i] = s;
      }
    });
  }
  c->have_cache = true;
  // S_task from the centroids
  std::vector<double> mn(E);
  for (int e = 0; e < E; ++e) {
    double s = 0.0;
    for (int j = 0; j < d; ++j) s += c->mu[(size_t)e * d + j] * c->mu[(size_t)e * d + j];
    mn[e] = std::sqrt(s);
  }
  std::vector<double> S((size_t)E * E), D((size_t)E * E);
  for (int i = 0; i < E; ++i)
    for (int j = 0; j < E; ++j) {
      double st = 1.0;
      if (i != j) {
        double dt = 0.0;
        for (int q = 0; q < d; ++q) dt += c->mu[(size_t)i * d + q] * c->mu[(size_t)j * d + q];
        st = cos_of(dt, mn[i], mn[j]);
      }
      double s = cf.alpha * c->S_param[(size_t)i * E + j] + (1.0 - cf.alpha) * st;
      if (s < cf.tau) s = 0.0;
      if (i == j) s = 1.0;
      S[(size_t)i * E + j] = s;
      D[(size_t)i * E + j] = 1.0 - s;
    }
  std::vector<int> assign, med;
  kmedoids(D, E, G, u, assign, med);
  even_out(D, E, G, K, med, assign);
  std::vector<int> fill(G, 0);
  for (int e = 0; e < E; ++e) {
    group_of[e] = assign[e];
    members[(size_t)assign[e] * K + fill[assign[e]]++] = e;
  }
  if (S_out) std::memcpy(S_out, S.data(), sizeof(double) * S.size());
  if (fresh_out)
    for (int e = 0; e < E; ++e) fresh_out[e] = fresh[e];
  return MOE_OK;
}

int moe_compress_projection(int32_t E, int32_t G, const int32_t* members, int32_t d_in, int32_t d_out, int32_t r,
                            const float* const* W, float* base, float* A, float* B, double* rel_err,
                            int32_t n_threads) {
  if (E <= 0 || G <= 0 || E % G || d_in <= 0 || d_out <= 0 || r < 0 || r > std::min(d_in, d_out))
    return report_error(MOE_ERR_INVALID_ARG, "bad sizes (E %% G == 0, 0 <= r <= min(d_in, d_out))");
  if (!members || !W || !base || (r > 0 && (!A || !B))) return report_error(MOE_ERR_INVALID_ARG, "null argument");
  const int K = E / G;
  std::vector<int> seen(E, 0);
  for (int i = 0; i < E; ++i) {
    if (members[i] < 0 || members[i] >= E || seen[members[i]]++)
      return report_error(MOE_ERR_INVALID_ARG, "members is not a permutation of the experts");
    if (!W[members[i]]) return report_error(MOE_ERR_INVALID_ARG, "W[%d] is null", members[i]);
  }
  const size_t mn = (size_t)d_in * d_out;
  // group bases: the mean of the members, summed in member order
  for (int g = 0; g < G; ++g) {
    std::vector<double> acc(mn, 0.0);
    for (int j = 0; j < K; ++j) {
      const float* w = W[members[(size_t)g * K + j]];
      for (size_t q = 0; q < mn; ++q) acc[q] += (double)w[q];
    }
    for (size_t q = 0; q < mn; ++q) base[(size_t)g * mn + q] = (float)(acc[q] / K);
  }
  // residual factors, one expert per task
  std::vector<std::thread> pool;
  unsigned nt = n_threads > 0 ? (unsigned)n_threads : std::max(1u, std::thread::hardware_concurrency());
  nt = std::min<unsigned>(nt, (unsigned)E);
  auto work = [&](int slot) {
    const int g = slot / K, e = members[slot];
    const float* w = W[e];
    std::vector<double> Rm(mn);
    std::vector<double> acc(mn, 0.0);
    for (int j = 0; j < K; ++j) {
      const float* wj = W[members[(size_t)g * K + j]];
      for (size_t q = 0; q < mn; ++q) acc[q] += (double)wj[q];
    }
    for (size_t q = 0; q < mn; ++q) Rm[q] = (double)w[q] - acc[q] / K;
    std::vector<double> a, b;
    tsvd(Rm, d_in, d_out, r, a, b);
    for (size_t q = 0; q < (size_t)d_in * r; ++q) A[(size_t)slot * d_in * r + q] = (float)a[q];
    for (size_t q = 0; q < (size_t)d_out * r; ++q) B[(size_t)slot * d_out * r + q] = (float)b[q];
    if (rel_err) {
      const float* bs = base + (size_t)g * mn;
      const float* As = A + (size_t)slot * d_in * r;
      const float* Bs = B + (size_t)slot * d_out * r;
      double num = 0.0, den = 0.0;
      for (int i = 0; i < d_in; ++i)
        for (int j = 0; j < d_out; ++j) {
          double v = bs[(size_t)i * d_out + j];
          for (int q = 0; q < r; ++q) v += (double)As[(size_t)i * r + q] * (double)Bs[(size_t)j * r + q];
          const double x = w[(size_t)i * d_out + j];
          num += (x - v) * (x - v);
          den += x * x;
        }
      rel_err[slot] = den > 0.0 ? std::sqrt(num / den) : 0.0;
    }
  };
  if (r == 0 && !rel_err) return MOE_OK;
  for (unsigned t = 0; t < nt; ++t)
    pool.emplace_back([&, t] {
      for (int s = (int)t; s < E; s += (int)nt) work(s);
    });
  for (auto& th : pool) th.join();
  return MOE_OK;
}

}  // extern "C"
