// Internal layout shared by the host entry points (api.cpp) and the gfx950
// kernels (kernels.hip).  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "specverify.h"

namespace sv {

constexpr int kThreads = 256;    // threads per workgroup (4 wave64s)
constexpr int kPrepThreads = 1024;
// 16-byte vectors per thread per row per chunk in the row-statistics pass:
// modes that stream one row per task use larger chunks (same bytes per chunk)
constexpr int stats_vectors_per_thread(int mode) {
  return (mode == SV_MODE_GREEDY || mode == SV_MODE_TREE_GREEDY || mode == SV_MODE_BLOCK) ? 4 : 2;
}
constexpr int kUA = 2;           // smallest of the above: sizes the partial arrays
constexpr int kUT = 4;           // 16-byte vectors per thread per row in one slice of k_decide's second look
constexpr int kSelCache = 256;   // draw records a token selection keeps in LDS
constexpr int kLdsBatch = 1024;  // batches up to this size scan their offsets in LDS (no prep kernel)
constexpr int kFusedItemsPerWg = 64;  // longest statistics pass (items per resident workgroup) run in one dispatch
constexpr int kFusedPerCu = 4;        // resident workgroups per compute unit of the single dispatch
constexpr int kFusedNodes = 257;      // tree / block requests of the single dispatch: at most 256 positions
// per-request arrival counters sit 256 bytes apart: increments of different
// requests' counters would otherwise queue behind each other on one line
constexpr int kCntStride = 64;     // in 32-bit words (KL second-pass counters)
constexpr int kArrStride = 32;     // in 64-bit words (epoch-tagged helper counters)
constexpr int kTopkMax = 16;  // largest k of the per-row top-k
constexpr int kConsMaxDrafts = 4;  // largest number of drafts of the consensus pass
constexpr int kModeConsensus = 16;  // internal mode value of the consensus calls (k_prep builds the position map)
// vocabulary elements of one consensus chunk: kThreads x 4 vectors of each row

constexpr int elems_per_vec(int dtype) { return dtype == SV_DTYPE_BF16 ? 8 : 4; }
// Elements of one consensus chunk (one workgroup, kConsVec vectors per thread and row).
constexpr int kConsVec = 16;
constexpr int64_t chunk_cons(int dtype) { return (int64_t)kThreads * kConsVec * elems_per_vec(dtype); }
constexpr int elem_size(int dtype) { return dtype == SV_DTYPE_BF16 ? 2 : 4; }
// vocabulary elements covered by one chunk of each pass
constexpr int64_t chunk_a(int dtype) { return (int64_t)kThreads * kUA * elems_per_vec(dtype); }
constexpr int64_t chunk_stats(int dtype, int mode) {
  return (int64_t)kThreads * stats_vectors_per_thread(mode) * elems_per_vec(dtype);
}
// vocabulary slice of one k_decide helper
constexpr int64_t chunk_t(int dtype) { return (int64_t)kThreads * kUT * elems_per_vec(dtype); }

enum TermKind : int32_t { kTermNone = 0, kTermResidual = 1, kTermBonus = 2 };

// Partial statistics of one task over the vocabulary chunks one workgroup of
// the statistics pass streamed.  m_* are raw-logit maxima, s_* = sum
// 2^((x - m) L) with L = log2(e)/T, w = sum 2^((d - m_d) L) (d - t) and
// z = sum 2^((d - m_d) L) |d - t| over the draft row, idx = lowest index
// attaining m_t.  The single dispatch (whose helpers read the partials during
// the same dispatch) stores self-tagged 64-bit words, (epoch << 32) | 32-bit
// payload, in the same 48 bytes instead: six for a stochastic pair (m_t, s_t
// low and high half, m_d, s_d low and high half), two for a greedy-family row
// (m_t, idx).
struct PartA {
  double s_t, s_d, w, z;
  float m_t, m_d;
  int32_t idx;
  uint32_t pad;
};

// A position queued for the KL second pass, with the constants of its terms:
// p_y = 2^(t_y L - ct) kt, q_y = 2^(d_y L - cd) kd and
// log(p_y / q_y) = (t_y - d_y) L ln 2 + lw (L = Lhi = log2(e) / T).
struct RefItem {
  int32_t pos;   // packed position = draft row
  int32_t b;     // request
  int32_t trow;  // target row
  float Lhi;
  float ct, cd, kt, kd, lw;
  int32_t pad;
};

// Per request: what the KL second pass needs to complete it.
struct ReqFin {
  int32_t d0, g;
  int32_t jnn;      // NKL: decision taken with every queued position accepted
  int32_t pending;  // positions queued; -1: the request failed its input checks
};

// Record space of the terminal draw for one (request, wave-chunk); a slice of
// kThreads x kUT vectors holds four wave-chunks.  The record (DrawRec in
// kernels.hip) takes its first 24 bytes.
struct PartC {
  uint64_t words[6];
};

struct Layout {
  size_t off_hdr, off_doff, off_pair2req, off_row2req, off_part_a, off_cnt, off_cnt_kl, off_req_fin, off_part_c,
      off_ref_list, off_kl_need, off_tidx, off_kl_part, off_topk, total;
  int64_t n_task_max;
  int64_t nch_a, nch_t;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace of a consensus call (B requests, npos positions, K drafts each).
struct ConsLayout {
  size_t off_hdr, off_doff, off_pos2req, off_cnt, off_stats, off_tz, total;
  int64_t nch;
};
inline ConsLayout make_cons_layout(int64_t B, int64_t V, int dtype, int64_t npos, int64_t K) {
  ConsLayout L{};
  L.nch = (V + chunk_cons(dtype) - 1) / chunk_cons(dtype);
  const int64_t P1 = npos > 0 ? npos : 1;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.off_hdr = take(256);
  L.off_doff = take(sizeof(int32_t) * (B + 1));
  L.off_pos2req = take(sizeof(int32_t) * P1);
  L.off_cnt = take(sizeof(uint64_t) * (size_t)P1 * kArrStride);  // per-position arrival counters
  L.off_stats = take(16 * (size_t)(P1 * K * L.nch));
  L.off_tz = take(2 * sizeof(double) * (size_t)(P1 * L.nch * K * (K - 1)));
  L.total = o;
  return L;
}

inline Layout make_layout(int64_t B, int64_t V, int dtype, int64_t R_d) {
  Layout L{};
  L.nch_a = (V + chunk_a(dtype) - 1) / chunk_a(dtype);
  L.nch_t = (V + chunk_t(dtype) - 1) / chunk_t(dtype);
  L.n_task_max = R_d + B;
  const int64_t R1 = R_d > 0 ? R_d : 1;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.off_hdr = take(256);
  // the helpers' arrival counters sit at an offset that depends on B only
  L.off_cnt = take(sizeof(uint64_t) * B * kArrStride);
  L.off_doff = take(sizeof(int32_t) * (B + 1));
  L.off_pair2req = take(sizeof(int32_t) * R1);
  L.off_row2req = take(sizeof(int32_t) * (R_d + B));
  L.off_part_a = take(sizeof(PartA) * L.n_task_max * L.nch_a);
  L.off_cnt_kl = take(sizeof(uint32_t) * B * kCntStride);
  L.off_req_fin = take(sizeof(ReqFin) * B);
  L.off_part_c = take(sizeof(PartC) * B * L.nch_t * (kThreads / 64));
  L.off_ref_list = take(sizeof(RefItem) * R1);
  L.off_kl_need = take(sizeof(int32_t) * R1);
  L.off_tidx = take(sizeof(int32_t) * (R_d + B));
  L.off_kl_part = take(sizeof(double) * R1 * L.nch_t);
  L.off_topk = take(sizeof(uint64_t) * B * kThreads);  // top-k candidates: kThreads per row
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
  int32_t R_d;         // total draft rows
  int32_t n_task;      // tasks of the row-statistics pass
  int32_t nch;         // vocabulary chunks per task in the row-statistics pass
  int32_t stats_grid;  // workgroups of the row-statistics pass
  int32_t grp_log2;    // log2 of the lanes that merge one task's partials
  int32_t maxseg;      // most statistics partials (segments) of one task
  int32_t helpers;     // k_decide workgroups per request (1 in greedy and tree modes)
  int32_t nslices;     // vocabulary slices per row (chunk_t elements each)
  int32_t slices_per_helper;
  float delta;
  const int32_t* nkl_pos;    // NKL: generation position of every draft row (NULL: constant delta)
  float nkl_alpha, nkl_dmax;  // NKL with positions: growth and cap of the threshold
  int32_t want_kl;  // compute KL(q || p) (NKL mode, or stochastic with out_nkl)
  int32_t block_min_len;  // block-accept mode: shortest kept run (>= 1)
  uint32_t epoch;      // this call's tag: fused statistics partials and arrival counters (never 0 or ~0)
  int32_t wait_polls;  // single dispatch: polls of a partial before a helper computes it itself
  // workspace
  int32_t* hdr;  // hdr[0]: layout error flag, hdr[1]: positions queued for the KL second pass
  int32_t* d_off;
  int32_t* pair2req;
  int32_t* row2req;
  PartA* part_a;
  // Per-request arrival counters of the helpers (terminal draw, row sampling,
  // top-k): (epoch << 32) | arrivals, one every kArrStride words.  A helper
  // claims the word for its call (compare-and-swap of a word with another
  // epoch to (epoch << 32)) before it counts itself, so the counters need no
  // reset and any leftover value in the workspace is harmless.
  uint64_t* cnt;      // [B * kArrStride]
  // KL second-pass items done per request: zeroed by the offsets scan of the
  // same call, wrapped back to zero by the last arrival
  uint32_t* cnt_kl;   // [B * kCntStride]
  ReqFin* req_fin;    // [B] completion record of the KL second pass
  PartC* part_c;      // [B * nslices * 4] draw records per wave-chunk
  RefItem* ref_list;  // [R_d] positions queued for the KL second pass (hdr[1] of them)
  int32_t* kl_need;   // [R_d] 1 where the KL of the position comes from the second pass
  int32_t* tidx;      // [R_d + B] argmax of every target row (NKL)
  double* kl_part;    // [R_d * nslices] second-pass KL sums per slice
  uint64_t* topk_cand;  // [B * kThreads] top-k candidates: helper h of row b at b * kThreads + h * topk
  int32_t topk;         // k of the per-row top-k
  // consensus across drafts: K draft rows per position (row pos * K + a)
  int32_t cons_k;
  float cons_dc, cons_dd;   // consensus / divergence thresholds of the closest pair's distance
  float* cons_nkl;          // [positions][K][K] (NULL: not written)
  int32_t* cons_state;      // [positions]
  int32_t* cons_pair;       // [positions]
  float* cons_stats;        // [positions][K][nch] x {m, pad, S (2 floats as a double)}: row-chunk statistics
  double* cons_tz;          // [positions][nch][K(K-1)] x {t, z}: one-pass cross sums per chunk and ordered pair
  int32_t cons_lds;         // 1: each workgroup finds its position's request by a scan of gamma in LDS
};

// kernel launchers (kernels.hip); return the hipError_t of the launch as int
int launch_prep(const Params& p, void* stream);
// picks the grid of the statistics pass: fills p.stats_grid and p.grp_log2
int plan_stats(Params& p, bool vec);
// picks the k_decide grid: fills p.nslices, p.helpers and p.slices_per_helper
int plan_decide(Params& p, bool vec);
// ev_start / ev_stop: optional hipEvent_t handles that take the dispatch's own
// start and end timestamps (NULL = plain launch)
int launch_stats(const Params& p, bool vec, void* stream, void* ev_start, void* ev_stop);
int launch_decide(const Params& p, bool vec, void* stream);
// KL second pass over the queue k_decide fills (NKL mode, or stochastic with out_nkl)
int launch_refine(const Params& p, bool vec, void* stream);
// One kernel for the whole step (batches up to kLdsBatch, a short statistics
// pass, not NKL mode and no KL output; tree and block requests of at most
// kFusedNodes - 1 positions): plan_fused fills p.stats_grid,
// p.grp_log2, p.nslices, p.helpers and p.slices_per_helper and returns the
// grid, or 0 when the step should take the separate kernels; launch_fused
// enqueues it.
int plan_fused(Params& p, bool vec);
// Draft-side row sampling (rows = p.B): plan_sample fills p.nslices, p.helpers
// and p.slices_per_helper; launch_sample enqueues k_sample.
int plan_sample(Params& p, bool vec);
int launch_sample(const Params& p, bool vec, void* stream, void* ev_start, void* ev_stop);
// Per-row top-k (rows = p.B, k = p.topk): plan_topk fills p.nslices,
// p.helpers and p.slices_per_helper; launch_topk enqueues k_topk.
int plan_topk(Params& p, bool vec);
int launch_topk(const Params& p, bool vec, void* stream, void* ev_start, void* ev_stop);
int launch_fused(const Params& p, bool vec, int grid, void* stream, void* ev_start, void* ev_stop);
// Consensus across drafts: k_prep (position -> request map), then the row
// statistics, the exact KL sums and the final per-position decision.
int launch_consensus(const Params& p, bool vec, void* stream, void* ev_start, void* ev_stop);
// plain-read probe over `bytes` (a multiple of 16 KB is read) with wgs_per_cu workgroups per CU
int launch_read_probe(const void* buf, int64_t bytes, int wgs_per_cu, void* sink, void* stream, void* ev_start,
                      void* ev_stop);

}  // namespace sv
