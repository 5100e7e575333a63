// Internal layout shared by the host entry points (api.cpp) and the gfx950
// kernels (kernels.hip).  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "specverify.h"

namespace sv {

constexpr int kThreads = 256;    // threads per workgroup (4 wave64s)
constexpr int kPrepThreads = 1024;
constexpr int kUA = 2;           // 16-byte vectors per thread per row per chunk, row-statistics pass
constexpr int kUC = 2;           // 16-byte vectors per thread per row, draw pass
constexpr int kLdsBatch = 4096;  // batches up to this size scan their offsets in LDS (no prep kernel)

constexpr int elems_per_vec(int dtype) { return dtype == SV_DTYPE_BF16 ? 8 : 4; }
constexpr int elem_size(int dtype) { return dtype == SV_DTYPE_BF16 ? 2 : 4; }
// vocabulary elements covered by one workgroup of each pass
constexpr int64_t chunk_a(int dtype) { return (int64_t)kThreads * kUA * elems_per_vec(dtype); }
constexpr int64_t chunk_c(int dtype) { return (int64_t)kThreads * kUC * elems_per_vec(dtype); }

enum TermKind : int32_t { kTermNone = 0, kTermResidual = 1, kTermBonus = 2 };

// Partial statistics of one (task, vocabulary chunk).  m_* are raw-logit maxima,
// s_* = sum exp((x - m)/T) over the chunk, w = sum exp((d - m_d)/T) * (d - t),
// idx = lowest index attaining m_t.
struct PartA {
  double s_t, s_d, w;
  float m_t, m_d;
  int32_t idx;
  int32_t pad;
};

// Merged statistics of one task (a whole row, or a target/draft row pair);
// kl = KL(q || p) in nats for pair tasks whose KL is requested.
struct TaskStat {
  double s_t, s_d, w;
  float m_t, m_d, kl;
  int32_t idx;
};

// Terminal record of a request, written by the decision step for the draw pass.
struct Term {
  int32_t kind;  // TermKind
  int32_t j;     // slot of the terminal token (= number of accepted drafts)
  int32_t trow;  // target row of the terminal distribution
  int32_t drow;  // draft row (residual only)
  float m_t;     // exact maximum of the target row (residual only)
  float m_d;     // exact maximum of the draft row (residual only)
  float k0;      // s_t / s_d from the statistics pass (residual only)
  int32_t pad;
};

// Partial sums of the draw pass for one (request, chunk), in float64.
struct PartC {
  double a, b, ap, bp;  // sum a, sum b, and the same over {y : a_y > k0 * b_y}
  float m;              // chunk maximum (bonus draws)
  int32_t pad[3];
};

struct Layout {
  size_t off_hdr, off_toff, off_doff, off_pair2req, off_row2req, off_part_a, off_stat, off_gat, off_cnt_task,
      off_cnt_req, off_term, off_part_c, off_cnt_draw, total;
  int64_t n_task_max;
  int64_t nch_a, nch_c;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline Layout make_layout(int64_t B, int64_t V, int dtype, int64_t R_d) {
  Layout L{};
  L.nch_a = (V + chunk_a(dtype) - 1) / chunk_a(dtype);
  L.nch_c = (V + chunk_c(dtype) - 1) / chunk_c(dtype);
  L.n_task_max = R_d + B;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.off_hdr = take(256);
  L.off_toff = take(sizeof(int32_t) * (B + 1));
  L.off_doff = take(sizeof(int32_t) * (B + 1));
  L.off_pair2req = take(sizeof(int32_t) * (R_d > 0 ? R_d : 1));
  L.off_row2req = take(sizeof(int32_t) * (R_d + B));
  L.off_part_a = take(sizeof(PartA) * L.n_task_max * L.nch_a);
  L.off_stat = take(sizeof(TaskStat) * L.n_task_max);
  L.off_gat = take(sizeof(float) * 2 * (R_d > 0 ? R_d : 1));
  L.off_cnt_task = take(sizeof(uint32_t) * L.n_task_max);
  L.off_cnt_req = take(sizeof(uint32_t) * B);
  L.off_term = take(sizeof(Term) * B);
  L.off_part_c = take(sizeof(PartC) * B * L.nch_c);
  L.off_cnt_draw = take(sizeof(uint32_t) * B);
  L.total = o;
  return L;
}

// Everything a kernel needs, passed by value.
struct Params {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* gamma;
  const float* temp;
  const float* ua;
  const float* ur;
  const int32_t* parents;
  int32_t* out_tokens;
  int32_t* out_num;
  float* out_nkl;
  float* out_p_x;
  float* out_q_x;
  float* out_resid;
  int32_t* out_tree_node;
  int32_t B, V, max_gamma, mode, dtype;
  int32_t R_d;     // total draft rows
  int32_t n_task;  // tasks of the row-statistics pass
  int32_t nch_a, nch_c;
  float delta;
  int32_t want_w;  // compute the KL cross term (NKL mode, or stochastic with out_nkl)
  // workspace
  int32_t* hdr;  // hdr[0]: layout error flag
  int32_t* t_off;
  int32_t* d_off;
  int32_t* pair2req;
  int32_t* row2req;
  PartA* part_a;
  TaskStat* stat;
  float* gat;  // [2 * R_d]: target and draft logit at the drafted token
  uint32_t* cnt_task;
  uint32_t* cnt_req;
  Term* term;
  PartC* part_c;
  uint32_t* cnt_draw;
};

// kernel launchers (kernels.hip); return the hipError_t of the launch as int
int launch_prep(const Params& p, void* stream);
int launch_rowstats(const Params& p, bool vec, void* stream);
int launch_draw(const Params& p, bool vec, void* stream);

}  // namespace sv
