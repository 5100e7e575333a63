// Reference oracle for the speculative-decoding verify step -- TEST
// INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
// CPU-baseline leg load this library; the product path never does.
//
// A plain, slow, obviously-correct CPU implementation in float64.  It shares
// no code, header, table or constant with the GPU path.  Every logit value
// (fp32 or bf16) widens to double exactly, every temperature is the stored
// float32 widened to double, and every sum over the vocabulary is a
// Neumaier-compensated sum taken in ascending token order.
//
// What is computed, per request b (gamma_b draft positions; target rows
// i = 0..gamma_b, draft rows i = 0..gamma_b-1; packed one request after the
// other):
//
//  * Temperature-scaled log-softmax of a row (the softmax(logits/T) of the
//    "Chain of Draft" page, section 3.2 compute_nkl listing, and of the
//    "投机采样" page's verification loop):
//        l(y) = x_y/T - L,  L = M + log sum_k exp(x_k/T - M),  M = max_k x_k/T.
//  * Stochastic mode -- modified rejection sampling ("投机采样" page, section
//    "核心算法数学原理"): alpha_i = min(1, p_i(x_i)/q_i(x_i)); token i is accepted
//    when u_i <= alpha_i; at the first rejection j the token is redrawn from
//    the normalised residual max(0, p_j - q_j) and drafting stops.  If all
//    gamma tokens are accepted, a bonus token is drawn from target row gamma
//    (the page computes gamma+1 target rows; drawing the extra token is the
//    plain reading).  Draws use one uniform per request and the inverse CDF
//    in ascending token order: y* = min{y : C_y > u*S}.
//  * Greedy mode (Gemma-4 MTP page, section 2.3 "接受/拒绝决策"): accept d_i iff
//    d_i == argmax of target row i (lowest index on ties); at the first
//    mismatch emit the target row's argmax; if all accepted emit argmax of
//    row gamma.
//  * NKL mode ("Chain of Draft" page, section 3.2): nkl_i = KL(q_i || p_i) / ln V
//    at the request's temperature, accepted while nkl_i < delta; at the first
//    failure emit argmax of target row j.  With per-position positions
//    ("Chain of Draft" page, section 4.3, position-adaptive threshold) the
//    threshold of draft token i is
//        delta_i = min(delta_max, delta * (1 + alpha * log2(pos_i + 1))),
//    pos_i >= 0 being the token's 0-based position in the generated sequence
//    (so the first token has delta_i = delta, as in the page's examples).
//  * Row sampling (sv_oracle_sample_rows): the drafter's draw of a token from
//    softmax(x/T) of one row, by the same inverse CDF.
//  * Block-accept mode ("Chain of Draft" page, section 3.3 Block-Accept Mode,
//    and section 2.2 "block mode": accept runs of >= 3 agreeing tokens): with
//    agreement a_i = [d_i == argmax of target row i], i < gamma, take the
//    first (lowest start) longest run of consecutive agreements; if it has at
//    least min_len positions and ends at e, the draft tokens before e are kept
//    (including any before the run, as the page's listing keeps them) and the
//    target row e gives the next token (its argmax); with no such run nothing
//    is kept and slot 0 gets the argmax of target row 0.  The strict
//    token-by-token policy of the same section is greedy mode.
//  * Tree mode ("Parallel Drafting" page, section 2.2 tree draft; Gemma-4 MTP
//    page, section 6.2 "longest accepted path"): node n (parent pi(n)) is
//    accepted iff its parent is accepted and its token equals argmax of the
//    parent's target row; the output is the path to the deepest accepted node
//    (lowest node id on ties) followed by that node's argmax.
//
// Flags (stochastic mode) mark requests whose result is decided within 1e-5
// of a boundary: an acceptance decision with |u_i - alpha_i| < 1e-5, or a draw
// whose uniform lies within 1e-5 of a CDF step.  In NKL mode a decision with
// |nkl_i - delta_i| < 1e-6*delta_i is flagged.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

enum { M_STOCH = 0, M_GREEDY = 1, M_NKL = 2, M_TREE = 3, M_BLOCK = 4 };
enum { FLAG_ACCEPT_BAND = 1, FLAG_DRAW_BAND = 2, FLAG_NKL_BAND = 4, FLAG_EMPTY_RESIDUAL = 8, FLAG_INVALID = 16 };

const double kNaN = std::numeric_limits<double>::quiet_NaN();

// Neumaier (improved Kahan-Babuska) compensated summation.
struct NSum {
  double s = 0.0, c = 0.0;
  void add(double v) {
    double t = s + v;
    if (std::fabs(s) >= std::fabs(v))
      c += (s - t) + v;
    else
      c += (v - t) + s;
    s = t;
  }
  double value() const { return s + c; }
};

double widen(const void* base, int dtype, int64_t row, int64_t V, int64_t y) {
  if (dtype == 0) return (double)((const float*)base)[row * V + y];
  uint16_t h = ((const uint16_t*)base)[row * V + y];
  uint32_t w = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &w, 4);
  return (double)f;
}

void load_row(const void* base, int dtype, int64_t row, int64_t V, std::vector<double>& out) {
  out.resize((size_t)V);
  for (int64_t y = 0; y < V; ++y) out[(size_t)y] = widen(base, dtype, row, V, y);
}

// l(y) = x_y/T - logsumexp(x/T)
void log_softmax(const std::vector<double>& x, double T, std::vector<double>& l) {
  const size_t V = x.size();
  l.resize(V);
  double M = -std::numeric_limits<double>::infinity();
  for (size_t y = 0; y < V; ++y) {
    l[y] = x[y] / T;
    if (l[y] > M) M = l[y];
  }
  NSum s;
  for (size_t y = 0; y < V; ++y) s.add(std::exp(l[y] - M));
  const double L = M + std::log(s.value());
  for (size_t y = 0; y < V; ++y) l[y] -= L;
}

// lowest index attaining the maximum raw logit
int32_t argmax_row(const std::vector<double>& x) {
  int32_t best = 0;
  for (size_t y = 1; y < x.size(); ++y)
    if (x[y] > x[(size_t)best]) best = (int32_t)y;
  return best;
}

// Inverse-CDF draw over non-negative weights r in ascending token order:
// y* = min{y : C_y > u*S}; if rounding leaves no such y, the last y with
// r(y) > 0.  Returns y*, and the distance (in units of S) from u to the
// nearer edge of y*'s CDF step.
int32_t inverse_cdf(const std::vector<double>& r, double S, double u, double* margin) {
  const double target = u * S;
  NSum c;
  double prev = 0.0;
  for (size_t y = 0; y < r.size(); ++y) {
    c.add(r[y]);
    const double C = c.value();
    if (C > target) {
      if (margin) *margin = std::fmin(u - prev / S, C / S - u);
      return (int32_t)y;
    }
    prev = C;
  }
  for (size_t y = r.size(); y-- > 0;)
    if (r[y] > 0.0) {
      if (margin) *margin = 0.0;
      return (int32_t)y;
    }
  if (margin) *margin = 0.0;
  return (int32_t)r.size() - 1;
}

struct Args {
  const void* target;
  const void* draft;
  int dtype;
  int32_t B;
  int32_t V;
  const int32_t* tokens;
  const int32_t* gamma;
  const float* temperature;
  const float* u_accept;
  const float* u_resample;
  int32_t mode;
  float delta;
  const int32_t* nkl_position;  // NULL: the constant threshold delta
  float nkl_alpha, nkl_delta_max;
  const int32_t* parents;
  int32_t block_min_len;  // block-accept mode: shortest run that is kept
  int32_t max_gamma;
  int32_t* out_tokens;
  int32_t* out_num_accepted;
  double* out_nkl;
  double* out_p_x;
  double* out_q_x;
  double* out_alpha;
  double* out_resid_mass;
  int32_t* out_tree_node;
  int32_t* out_flags;
  double* out_accept_margin;
  double* out_draw_margin;
};

void mark_invalid(const Args& a, int32_t b, int64_t t0, int64_t d0, int32_t g) {
  a.out_num_accepted[b] = -1;
  for (int64_t k = 0; k <= g; ++k) a.out_tokens[t0 + k] = -1;
  for (int64_t k = 0; k < g; ++k) {
    if (a.out_nkl) a.out_nkl[d0 + k] = kNaN;
    if (a.out_p_x) a.out_p_x[d0 + k] = kNaN;
    if (a.out_q_x) a.out_q_x[d0 + k] = kNaN;
    if (a.out_alpha) a.out_alpha[d0 + k] = kNaN;
  }
  if (a.out_resid_mass) a.out_resid_mass[b] = kNaN;
  if (a.out_tree_node) a.out_tree_node[b] = -1;
  if (a.out_flags) a.out_flags[b] = FLAG_INVALID;
}

bool u_ok(float u) { return u >= 0.0f && u < 1.0f; }  // NaN fails both

// Position-adaptive NKL threshold ("Chain of Draft" page, section 4.3): the
// base threshold grows with the log of the position in the generated
// sequence, up to a cap.  float64 throughout.
double nkl_threshold(float delta, float alpha, float delta_max, int32_t pos) {
  const double grown = (double)delta * (1.0 + (double)alpha * std::log2((double)pos + 1.0));
  return std::fmin((double)delta_max, grown);
}
bool t_ok(float t) { return std::isfinite(t) && t > 0.0f; }

void verify_request(const Args& a, int32_t b, int64_t t0, int64_t d0) {
  const int32_t g = a.gamma[b];
  const int64_t V = a.V;
  if (g > a.max_gamma) return mark_invalid(a, b, t0, d0, g);
  for (int32_t i = 0; i < g; ++i)
    if (a.tokens[d0 + i] < 0 || a.tokens[d0 + i] >= a.V) return mark_invalid(a, b, t0, d0, g);
  if (a.mode == M_STOCH || a.mode == M_NKL)
    if (!t_ok(a.temperature[b])) return mark_invalid(a, b, t0, d0, g);
  if (a.mode == M_STOCH) {
    for (int32_t i = 0; i < g; ++i)
      if (!u_ok(a.u_accept[d0 + i])) return mark_invalid(a, b, t0, d0, g);
    if (!u_ok(a.u_resample[b])) return mark_invalid(a, b, t0, d0, g);
  }
  if (a.mode == M_NKL && a.nkl_position)
    for (int32_t i = 0; i < g; ++i)
      if (a.nkl_position[d0 + i] < 0) return mark_invalid(a, b, t0, d0, g);
  if (a.mode == M_TREE)
    for (int32_t k = 1; k <= g; ++k) {
      const int32_t p = a.parents[d0 + k - 1];
      if (p < 0 || p >= k) return mark_invalid(a, b, t0, d0, g);
    }

  int32_t flags = 0;
  std::vector<double> xt, xd, lt, ld;
  // temperatures are read in the soft modes only (greedy, tree and block modes may pass none)
  const double T = (a.mode == M_STOCH || a.mode == M_NKL) ? (double)a.temperature[b] : 1.0;
  int32_t j = g;          // first failing position
  int32_t terminal = -1;  // token emitted at slot j

  if (a.mode == M_STOCH) {
    std::vector<double> alpha((size_t)g);
    for (int32_t i = 0; i < g; ++i) {
      load_row(a.target, a.dtype, t0 + i, V, xt);
      load_row(a.draft, a.dtype, d0 + i, V, xd);
      log_softmax(xt, T, lt);
      log_softmax(xd, T, ld);
      const int32_t x = a.tokens[d0 + i];
      const double lp = lt[(size_t)x], lq = ld[(size_t)x];
      alpha[(size_t)i] = std::fmin(1.0, std::exp(lp - lq));
      if (a.out_p_x) a.out_p_x[d0 + i] = std::exp(lp);
      if (a.out_q_x) a.out_q_x[d0 + i] = std::exp(lq);
      if (a.out_alpha) a.out_alpha[d0 + i] = alpha[(size_t)i];
      if (a.out_nkl) {
        NSum kl;
        for (int64_t y = 0; y < V; ++y) kl.add(std::exp(ld[(size_t)y]) * (ld[(size_t)y] - lt[(size_t)y]));
        a.out_nkl[d0 + i] = V > 1 ? kl.value() / std::log((double)V) : 0.0;
      }
    }
    double amargin = std::numeric_limits<double>::infinity();
    for (int32_t i = 0; i < g; ++i) {
      const double u = (double)a.u_accept[d0 + i];
      amargin = std::fmin(amargin, std::fabs(u - alpha[(size_t)i]));
      if (!(u <= alpha[(size_t)i])) {
        j = i;
        break;
      }
    }
    if (amargin < 1e-5) flags |= FLAG_ACCEPT_BAND;
    if (a.out_accept_margin) a.out_accept_margin[b] = amargin;

    // terminal distribution: residual of row j, or target row gamma (bonus)
    std::vector<double> r((size_t)V);
    load_row(a.target, a.dtype, t0 + j, V, xt);
    log_softmax(xt, T, lt);
    if (j < g) {
      load_row(a.draft, a.dtype, d0 + j, V, xd);
      log_softmax(xd, T, ld);
      for (int64_t y = 0; y < V; ++y)
        r[(size_t)y] = std::fmax(0.0, std::exp(lt[(size_t)y]) - std::exp(ld[(size_t)y]));
    } else {
      for (int64_t y = 0; y < V; ++y) r[(size_t)y] = std::exp(lt[(size_t)y]);
    }
    NSum s;
    for (int64_t y = 0; y < V; ++y) s.add(r[(size_t)y]);
    double S = s.value();
    if (j < g && !(S > 0.0)) {  // cannot happen in exact arithmetic after a rejection
      flags |= FLAG_EMPTY_RESIDUAL;
      for (int64_t y = 0; y < V; ++y) r[(size_t)y] = std::exp(lt[(size_t)y]);
      NSum s2;
      for (int64_t y = 0; y < V; ++y) s2.add(r[(size_t)y]);
      S = s2.value();
    }
    if (a.out_resid_mass) a.out_resid_mass[b] = (j < g) ? S : 1.0;
    double dmargin = 0.0;
    terminal = inverse_cdf(r, S, (double)a.u_resample[b], &dmargin);
    if (dmargin < 1e-5) flags |= FLAG_DRAW_BAND;
    if (a.out_draw_margin) a.out_draw_margin[b] = dmargin;
  } else if (a.mode == M_GREEDY) {
    for (int32_t i = 0; i <= g; ++i) {
      load_row(a.target, a.dtype, t0 + i, V, xt);
      const int32_t am = argmax_row(xt);
      if (i == g || a.tokens[d0 + i] != am) {
        j = i;
        terminal = am;
        break;
      }
    }
  } else if (a.mode == M_NKL) {
    const double lnV = std::log((double)V);
    std::vector<double> nkl((size_t)g);
    for (int32_t i = 0; i < g; ++i) {
      load_row(a.target, a.dtype, t0 + i, V, xt);
      load_row(a.draft, a.dtype, d0 + i, V, xd);
      log_softmax(xt, T, lt);
      log_softmax(xd, T, ld);
      NSum kl;
      for (int64_t y = 0; y < V; ++y) kl.add(std::exp(ld[(size_t)y]) * (ld[(size_t)y] - lt[(size_t)y]));
      // A one-token vocabulary makes KL/ln V = 0/0: both distributions are the
      // same point mass, so NKL is taken as 0.
      nkl[(size_t)i] = V > 1 ? kl.value() / lnV : 0.0;
      if (a.out_nkl) a.out_nkl[d0 + i] = nkl[(size_t)i];
      if (a.out_p_x) a.out_p_x[d0 + i] = std::exp(lt[(size_t)a.tokens[d0 + i]]);
      if (a.out_q_x) a.out_q_x[d0 + i] = std::exp(ld[(size_t)a.tokens[d0 + i]]);
    }
    for (int32_t i = 0; i < g; ++i) {
      const double delta = a.nkl_position
                               ? nkl_threshold(a.delta, a.nkl_alpha, a.nkl_delta_max, a.nkl_position[d0 + i])
                               : (double)a.delta;
      if (std::fabs(nkl[(size_t)i] - delta) < 1e-6 * delta) flags |= FLAG_NKL_BAND;
      if (!(nkl[(size_t)i] < delta)) {
        j = i;
        break;
      }
    }
    load_row(a.target, a.dtype, t0 + j, V, xt);
    terminal = argmax_row(xt);
  } else if (a.mode == M_BLOCK) {
    // the argmax of every target row, then the first longest run of
    // positions whose draft token equals it
    std::vector<int32_t> am((size_t)g + 1);
    for (int32_t i = 0; i <= g; ++i) {
      load_row(a.target, a.dtype, t0 + i, V, xt);
      am[(size_t)i] = argmax_row(xt);
    }
    int32_t best_len = 0, best_start = 0;
    for (int32_t start = 0; start < g; ++start) {
      int32_t len = 0;
      while (start + len < g && a.tokens[d0 + start + len] == am[(size_t)(start + len)]) ++len;
      if (len > best_len) {
        best_len = len;
        best_start = start;
      }
    }
    j = best_len >= a.block_min_len ? best_start + best_len : 0;
    terminal = am[(size_t)j];
  } else {  // tree
    const int32_t N = g + 1;
    std::vector<int32_t> am((size_t)N), depth((size_t)N, 0);
    std::vector<char> acc((size_t)N, 0);
    for (int32_t n = 0; n < N; ++n) {
      load_row(a.target, a.dtype, t0 + n, V, xt);
      am[(size_t)n] = argmax_row(xt);
    }
    acc[0] = 1;
    int32_t best = 0;
    for (int32_t n = 1; n < N; ++n) {
      const int32_t p = a.parents[d0 + n - 1];
      depth[(size_t)n] = depth[(size_t)p] + 1;
      acc[(size_t)n] = acc[(size_t)p] && a.tokens[d0 + n - 1] == am[(size_t)p];
      if (acc[(size_t)n] && depth[(size_t)n] > depth[(size_t)best]) best = n;
    }
    j = depth[(size_t)best];
    std::vector<int32_t> path;
    for (int32_t n = best; n != 0; n = a.parents[d0 + n - 1]) path.push_back(a.tokens[d0 + n - 1]);
    for (int32_t k = 0; k < j; ++k) a.out_tokens[t0 + k] = path[(size_t)(j - 1 - k)];
    terminal = am[(size_t)best];
    if (a.out_tree_node) a.out_tree_node[b] = best;
  }

  if (a.mode != M_TREE)
    for (int32_t k = 0; k < j; ++k) a.out_tokens[t0 + k] = a.tokens[d0 + k];
  a.out_tokens[t0 + j] = terminal;
  for (int32_t k = j + 1; k <= g; ++k) a.out_tokens[t0 + k] = -1;
  a.out_num_accepted[b] = j;
  if (a.out_flags) a.out_flags[b] = flags;
}

}  // namespace

extern "C" {

// Returns 0 on success, -1 on an argument error (nothing written).
//   target_logits [sum(gamma+1)][V], draft_logits [sum(gamma)][V] (NULL allowed in
//   greedy/tree mode), dtype 0 = float32, 1 = bf16 (uint16 patterns).
//   All arrays are host memory.  Optional outputs may be NULL.
//   Whole-call layout errors (a negative gamma, or sum(gamma) != total_draft_rows)
//   mark every request invalid (num_accepted = -1, tokens = -1).
//   nkl_position (NKL mode, may be NULL): int32 [sum(gamma)], 0-based position of each
//   draft token in the generated sequence; the threshold of token i is then
//   min(nkl_delta_max, delta * (1 + nkl_alpha * log2(pos_i + 1))), and a negative
//   position makes its request invalid.
//   block_min_len (block-accept mode): the shortest run of agreeing positions that is kept (>= 1).
int sv_oracle_verify(const void* target_logits, const void* draft_logits, int32_t dtype, int32_t batch,
                     int32_t vocab, const int32_t* draft_tokens, const int32_t* gamma_per_req,
                     const float* temperature, const float* u_accept, const float* u_resample, int32_t mode,
                     float delta, const int32_t* nkl_position, float nkl_alpha, float nkl_delta_max,
                     const int32_t* tree_parents, int32_t block_min_len, int32_t max_gamma, int64_t total_draft_rows,
                     int32_t* out_tokens, int32_t* out_num_accepted, double* out_nkl, double* out_p_x,
                     double* out_q_x, double* out_alpha, double* out_resid_mass, int32_t* out_tree_node,
                     int32_t* out_flags, double* out_accept_margin, double* out_draw_margin, int32_t nthreads) {
  if (batch <= 0 || vocab <= 0 || (dtype != 0 && dtype != 1) || mode < 0 || mode > 4) return -1;
  if (mode == M_BLOCK && block_min_len < 1) return -1;
  if (!target_logits || !gamma_per_req || !out_tokens || !out_num_accepted) return -1;
  if ((mode == M_STOCH || mode == M_NKL) && (!draft_logits || !temperature)) return -1;
  if (mode == M_STOCH && (!u_accept || !u_resample)) return -1;
  if (mode == M_TREE && !tree_parents) return -1;
  if (mode == M_NKL && !std::isfinite(delta)) return -1;
  if (mode == M_NKL && nkl_position && !(std::isfinite(nkl_alpha) && std::isfinite(nkl_delta_max))) return -1;
  if (total_draft_rows > 0 && !draft_tokens) return -1;

  Args a{target_logits, draft_logits, dtype, batch, vocab, draft_tokens, gamma_per_req, temperature, u_accept,
         u_resample, mode, delta, mode == M_NKL ? nkl_position : nullptr, nkl_alpha, nkl_delta_max, tree_parents,
         block_min_len, max_gamma, out_tokens, out_num_accepted, out_nkl, out_p_x,
         out_q_x, out_alpha, out_resid_mass, out_tree_node, out_flags, out_accept_margin, out_draw_margin};

  std::vector<int64_t> t_off((size_t)batch + 1, 0), d_off((size_t)batch + 1, 0);
  bool layout_ok = true;
  for (int32_t b = 0; b < batch; ++b) {
    if (gamma_per_req[b] < 0) layout_ok = false;
    const int64_t g = gamma_per_req[b] < 0 ? 0 : gamma_per_req[b];
    t_off[(size_t)b + 1] = t_off[(size_t)b] + g + 1;
    d_off[(size_t)b + 1] = d_off[(size_t)b] + g;
  }
  if (d_off[(size_t)batch] != total_draft_rows) layout_ok = false;
  if (!layout_ok) {
    // The packed layout is undefined: only num_accepted is written.
    for (int32_t b = 0; b < batch; ++b) {
      out_num_accepted[b] = -1;
      if (out_flags) out_flags[b] = FLAG_INVALID;
    }
    return 0;
  }

#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int32_t b = 0; b < batch; ++b) verify_request(a, b, t_off[(size_t)b], d_off[(size_t)b]);
  return 0;
}

// Draft-side sampling, the drafter's step before verification (draft tokens
// "drawn from the draft softmax"; the "投机采样" page's draft loop draws
// x_i ~ q_i): the token of row r is the inverse-CDF draw from
// softmax(x_r / T_r) with the uniform u_r, y* = min{y : C_y > u*S} in ascending
// token order (the rule of the verify step's bonus draw).  A row whose
// temperature is not > 0 and finite, or whose uniform is outside [0, 1), gets
// -1.  out_margin (may be NULL): the distance from u_r to the nearer edge of
// y*'s CDF step (NaN for invalid rows).  Returns -1 on an argument error.
int sv_oracle_sample_rows(const void* logits, int32_t dtype, int64_t rows, int32_t vocab, const float* temperature,
                          const float* u, int32_t* out_tokens, double* out_margin, int32_t nthreads) {
  if (rows < 0 || vocab <= 0 || (dtype != 0 && dtype != 1)) return -1;
  if (rows > 0 && (!logits || !temperature || !u || !out_tokens)) return -1;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t r = 0; r < rows; ++r) {
    if (!t_ok(temperature[r]) || !u_ok(u[r])) {
      out_tokens[r] = -1;
      if (out_margin) out_margin[r] = kNaN;
      continue;
    }
    std::vector<double> x, l, p((size_t)vocab);
    load_row(logits, dtype, r, vocab, x);
    log_softmax(x, (double)temperature[r], l);
    NSum s;
    for (int64_t y = 0; y < vocab; ++y) {
      p[(size_t)y] = std::exp(l[(size_t)y]);
      s.add(p[(size_t)y]);
    }
    double margin = 0.0;
    out_tokens[r] = inverse_cdf(p, s.value(), (double)u[r], &margin);
    if (out_margin) out_margin[r] = margin;
  }
  return 0;
}

// Top-k of each row (the children of a tree draft node are the top-k tokens of
// its draft row: "Parallel Drafting" page, section 2.2 tree draft): the k
// indices with the largest logits, largest first, the lower index first among
// equal logits.  Returns -1 on an argument error (k outside [1, V]).
int sv_oracle_topk_rows(const void* logits, int32_t dtype, int64_t rows, int32_t vocab, int32_t k,
                        int32_t* out_idx, int32_t nthreads) {
  if (rows < 0 || vocab <= 0 || (dtype != 0 && dtype != 1) || k < 1 || k > vocab) return -1;
  if (rows > 0 && (!logits || !out_idx)) return -1;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t r = 0; r < rows; ++r) {
    std::vector<double> x;
    load_row(logits, dtype, r, vocab, x);
    std::vector<int32_t> idx((size_t)vocab);
    for (int32_t y = 0; y < vocab; ++y) idx[(size_t)y] = y;
    std::partial_sort(idx.begin(), idx.begin() + k, idx.end(), [&](int32_t a, int32_t b) {
      return x[(size_t)a] > x[(size_t)b] || (x[(size_t)a] == x[(size_t)b] && a < b);
    });
    for (int32_t i = 0; i < k; ++i) out_idx[r * k + i] = idx[(size_t)i];
  }
  return 0;
}

// Consensus across K drafts ("Chain of Draft" page, section 4.4, Consensus-Aware
// Accept: the pairwise NKL matrix of the drafts; some pair below 0.1 is a
// consensus, every pair above 0.15 a divergence).  Request b has gamma_b
// positions; position i of request b (packed index n = d_off[b] + i) holds K
// draft rows, row n*K + a for draft a, all at the request's temperature.  Per
// position:
//   M[a][b] = KL(q_a || q_b) / ln V  (log space, Neumaier sums; 0 for V == 1),
//   the distance of a pair a < b is the symmetrised s_ab = (M[a][b] + M[b][a]) / 2,
//   pair = the pair with the smallest distance (lowest (a, b) on ties),
//   state = 1 (consensus) if that distance < delta_c, 2 (divergence) if it is
//   > delta_d (so every pair is), else 0.
// Flags: 1 if the smallest distance lies within 1e-6 relative of delta_c, 2
// within 1e-6 of delta_d, 4 if another pair's distance lies within 1e-6
// relative of the smallest (the closest pair is then a near tie).  A request
// with a temperature that is not > 0 and finite gets state -1, pair -1 and NaN
// distances.  out_nkl: [positions][K][K] (diagonal 0).  Returns -1 on an
// argument error.
int sv_oracle_consensus(const void* draft_logits, int32_t dtype, int32_t batch, int32_t num_drafts, int32_t vocab,
                        const int32_t* gamma_per_req, const float* temperature, float delta_c, float delta_d,
                        double* out_nkl, int32_t* out_state, int32_t* out_pair, int32_t* out_flags,
                        int32_t nthreads) {
  const int32_t K = num_drafts;
  if (batch <= 0 || vocab <= 0 || K < 2 || (dtype != 0 && dtype != 1)) return -1;
  if (!draft_logits || !gamma_per_req || !temperature || !out_state || !out_pair) return -1;
  std::vector<int64_t> d_off((size_t)batch + 1, 0);
  for (int32_t b = 0; b < batch; ++b) {
    if (gamma_per_req[b] < 0) return -1;
    d_off[(size_t)b + 1] = d_off[(size_t)b] + gamma_per_req[b];
  }
  const int64_t npos = d_off[(size_t)batch];
  const double lnV = std::log((double)vocab);
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t n = 0; n < npos; ++n) {
    int32_t b = 0;
    while (d_off[(size_t)b + 1] <= n) ++b;
    double* M = out_nkl ? out_nkl + n * K * K : nullptr;
    if (!t_ok(temperature[b])) {
      out_state[n] = -1;
      out_pair[n] = -1;
      if (out_flags) out_flags[n] = FLAG_INVALID;
      if (M)
        for (int32_t k = 0; k < K * K; ++k) M[k] = kNaN;
      continue;
    }
    const double T = (double)temperature[b];
    std::vector<std::vector<double>> l((size_t)K);
    std::vector<double> x;
    for (int32_t a = 0; a < K; ++a) {
      load_row(draft_logits, dtype, n * K + a, vocab, x);
      log_softmax(x, T, l[(size_t)a]);
    }
    std::vector<double> m((size_t)K * K, 0.0);
    for (int32_t a = 0; a < K; ++a)
      for (int32_t c = 0; c < K; ++c) {
        if (a == c) continue;
        NSum kl;
        for (int64_t y = 0; y < vocab; ++y)
          kl.add(std::exp(l[(size_t)a][(size_t)y]) * (l[(size_t)a][(size_t)y] - l[(size_t)c][(size_t)y]));
        m[(size_t)(a * K + c)] = vocab > 1 ? kl.value() / lnV : 0.0;
      }
    if (M)
      for (int32_t k = 0; k < K * K; ++k) M[k] = m[(size_t)k];
    double best = std::numeric_limits<double>::infinity();
    int32_t pair = -1;
    for (int32_t a = 0; a < K; ++a)
      for (int32_t c = a + 1; c < K; ++c) {
        const double sd = 0.5 * (m[(size_t)(a * K + c)] + m[(size_t)(c * K + a)]);
        if (sd < best) {
          best = sd;
          pair = a * K + c;
        }
      }
    int32_t flags = 0;
    for (int32_t a = 0; a < K; ++a)
      for (int32_t c = a + 1; c < K; ++c) {
        const double sd = 0.5 * (m[(size_t)(a * K + c)] + m[(size_t)(c * K + a)]);
        if (a * K + c != pair && std::fabs(sd - best) <= 1e-6 * best) flags |= 4;
      }
    if (std::fabs(best - (double)delta_c) < 1e-6 * (double)delta_c) flags |= 1;
    if (std::fabs(best - (double)delta_d) < 1e-6 * (double)delta_d) flags |= 2;
    out_state[n] = best < (double)delta_c ? 1 : (best > (double)delta_d ? 2 : 0);
    out_pair[n] = pair;
    if (out_flags) out_flags[n] = flags;
  }
  return 0;
}

// The position-adaptive NKL threshold of a draft token at 0-based position pos.
double sv_oracle_nkl_threshold(float delta, float alpha, float delta_max, int32_t pos) {
  return nkl_threshold(delta, alpha, delta_max, pos);
}

int sv_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"
