// gfx950 kernels of the speculative-decoding verify step.
//
// Three launches per call:
//   k_prep      one workgroup: exclusive scans of gamma (packed offsets), the
//               row -> request maps, counter reset, layout validation.
//   k_rowstats  one workgroup per (task, vocabulary chunk).  A task is a
//               (target row, draft row) pair (stochastic / NKL) or a single
//               target row (greedy / tree / NKL bonus row).  Each workgroup
//               streams its chunk with 16-byte loads and reduces it to
//               (max, sum exp, argmax, KL cross term); the last workgroup of a
//               task merges the chunk partials, and the last task of a request
//               runs the per-request decision (first-reject scan, tree
//               resolve) and writes the outputs.
//   k_draw      stochastic mode only: one workgroup per (request, chunk) of
//               the terminal row; float64 chunk sums of the residual
//               max(0, p - q) (or of p for a bonus token); the last workgroup
//               of a request selects the chunk and draws the token by a
//               block-wide prefix sum.
//
// Formulas follow these passages:
//   softmax(logits / T), p(x), q(x)     -- "Chain of Draft" page, section 3.2
//                                          (compute_nkl); "投机采样" page,
//                                          verification loop of the engine.
//   alpha = min(1, p/q), accept u<=alpha,
//   redraw from max(0, p-q)/norm        -- "投机采样" page, section 核心算法数学原理.
//   greedy accept d_i == argmax P_i     -- Gemma-4 MTP page, section 2.3.
//   NKL = KL(q||p) / ln V, accept < delta -- "Chain of Draft" page, section 3.2.
//   tree drafts, longest accepted path   -- "Parallel Drafting" page, section 2.2;
//                                          Gemma-4 MTP page, section 6.2.

#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cstdint>

#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr double kLog2eD = 1.44269504088896340736;
constexpr float kLn2 = 0.693147180559945309417f;

// ----------------------------------------------------------------------------
// element access
// ----------------------------------------------------------------------------

template <int DT>
struct Elem;
template <>
struct Elem<SV_DTYPE_BF16> {
  static constexpr int P = 8;
  static constexpr uint32_t kPadPair = 0xFF7FFF7Fu;  // two bf16 -3.39e38 (pad for positions >= V)
  static constexpr float kPad = -3.38953139e38f;      // the pad's value (bf16 0xFF7F)
};
template <>
struct Elem<SV_DTYPE_F32> {
  static constexpr int P = 4;
  static constexpr uint32_t kPadPair = 0xFF7FFFFFu;  // -FLT_MAX
  static constexpr float kPad = -FLT_MAX;
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Raw 16 bytes holding elements [e0, e0 + P) of `row`; positions >= V hold the
// pad pattern.  VEC: rows are 16-byte aligned, so full vectors use one load.
template <int DT, bool VEC>
__device__ __forceinline__ uint4 fetch(const void* base, int64_t row, int64_t V, int64_t e0) {
  constexpr int P = Elem<DT>::P;
  if (VEC && e0 + P <= V) {
    const char* ptr = static_cast<const char*>(base) + (row * V + e0) * (DT == SV_DTYPE_BF16 ? 2 : 4);
    return *reinterpret_cast<const uint4*>(ptr);
  }
  uint32_t w[4] = {Elem<DT>::kPadPair, Elem<DT>::kPadPair, Elem<DT>::kPadPair, Elem<DT>::kPadPair};
  if (DT == SV_DTYPE_BF16) {
    const uint16_t* r = static_cast<const uint16_t*>(base) + row * V;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e0 + e < V) {
        const uint32_t h = r[e0 + e];
        const int sh = (e & 1) * 16;
        w[e >> 1] = (w[e >> 1] & ~(0xFFFFu << sh)) | (h << sh);
      }
    }
  } else {
    const uint32_t* r = static_cast<const uint32_t*>(base) + row * V;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e0 + e < V) w[e] = r[e0 + e];
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int DT>
__device__ __forceinline__ void unpack(const uint4& q, float* v) {
  if (DT == SV_DTYPE_BF16) {
    v[0] = bf_lo(q.x); v[1] = bf_hi(q.x); v[2] = bf_lo(q.y); v[3] = bf_hi(q.y);
    v[4] = bf_lo(q.z); v[5] = bf_hi(q.z); v[6] = bf_lo(q.w); v[7] = bf_hi(q.w);
  } else {
    v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
    v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
  }
}

template <int DT>
__device__ __forceinline__ float load_scalar(const void* base, int64_t row, int64_t V, int64_t y) {
  if (DT == SV_DTYPE_BF16) return __uint_as_float((uint32_t)(static_cast<const uint16_t*>(base)[row * V + y]) << 16);
  return static_cast<const float*>(base)[row * V + y];
}

// ----------------------------------------------------------------------------
// wave64 reductions (DPP within rows of 16 lanes, then the four row results).
// Every lane of the wave must be active.  Deterministic: the combination
// order is fixed by lane position.
// ----------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v, int old) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float lanef(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v, v));   // quad_perm(1,0,3,2)
  v = fmaxf(v, dpp<0x4E>(v, v));   // quad_perm(2,3,0,1)
  v = fmaxf(v, dpp<0x124>(v, v));  // row_ror:4
  v = fmaxf(v, dpp<0x128>(v, v));  // row_ror:8
  return fmaxf(fmaxf(lanef(v, 0), lanef(v, 16)), fmaxf(lanef(v, 32), lanef(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = v + dpp<0xB1>(v, 0.f);
  v = v + dpp<0x4E>(v, 0.f);
  v = v + dpp<0x124>(v, 0.f);
  v = v + dpp<0x128>(v, 0.f);
  return (lanef(v, 0) + lanef(v, 16)) + (lanef(v, 32) + lanef(v, 48));
}
__device__ __forceinline__ int wave_min_int(int v) {
  v = min(v, dppi<0xB1>(v, v));
  v = min(v, dppi<0x4E>(v, v));
  v = min(v, dppi<0x124>(v, v));
  v = min(v, dppi<0x128>(v, v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_max_int(int v) {
  v = max(v, dppi<0xB1>(v, v));
  v = max(v, dppi<0x4E>(v, v));
  v = max(v, dppi<0x124>(v, v));
  v = max(v, dppi<0x128>(v, v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
// butterfly sum: every lane ends with the same bits (a + b == b + a in IEEE)
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// workgroup-wide reductions through LDS (all threads must call)
__device__ __forceinline__ int block_min_int(int v, int* sh) {
  v = wave_min_int(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  int r = sh[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r = min(r, sh[k]);
  return r;
}
__device__ __forceinline__ int block_max_int(int v, int* sh) {
  v = wave_max_int(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  int r = sh[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r = max(r, sh[k]);
  return r;
}
__device__ __forceinline__ float block_max(float v, float* sh) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r = fmaxf(r, sh[k]);
  return r;
}
__device__ __forceinline__ double block_sum_d(double v, double* sh) {
  v = wave_sum_d(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  double r = sh[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) r += sh[k];
  return r;
}

// exclusive prefix sum over the workgroup's threads in float64; returns the
// exclusive prefix of this thread, `total` receives the sum.
__device__ __forceinline__ double block_exclusive_scan_d(double v, double* sh, double& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  __syncthreads();
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  double before = 0.0;
  for (int k = 0; k < w; ++k) before += sh[k];
  double tot = 0.0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) tot += sh[k];
  total = tot;
  return before + incl - v;
}

__device__ __forceinline__ bool unit_ok(float u) { return u >= 0.0f && u < 1.0f; }
__device__ __forceinline__ bool temp_ok(float t) { return t > 0.0f && t <= FLT_MAX; }

// exp((x - m) / T) = exp2(dx * L), L = log2(e)/T split as Lhi + Llo (float32);
// the rounding error of dx*Lhi is recovered exactly by an fma, so the
// exponent carries no systematic rounding (no effective temperature shift).
__device__ __forceinline__ float exp_hp(float dx, float Lhi, float Llo) {
  const float p1 = dx * Lhi;
  const float err = fmaf(dx, Lhi, -p1);
  const float corr = fmaf(dx, Llo, err);
  const float E = __builtin_amdgcn_exp2f(p1);
  const float e = fmaf(E * kLn2, corr, E);
  return p1 >= -160.0f ? e : 0.0f;
}

// ----------------------------------------------------------------------------
// Cross-workgroup publication.  Records that one workgroup hands to another
// inside a launch are written and read with device-scope (sc1) accesses, which
// go to the device-coherent level instead of an XCD's private L2; the writer
// waits for its stores to complete before it bumps the completion counter, and
// the reader only loads after it has seen the final count.  This gives the
// release/acquire ordering the merge needs without an L2 writeback per
// workgroup (an agent-scope release fence flushes the whole L2 of the XCD).
// ----------------------------------------------------------------------------

template <class T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_dev(T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// all earlier memory operations of this thread have completed
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }
// counter increment after the thread's published stores completed; returns the old count
__device__ __forceinline__ unsigned signal_n(uint32_t* cnt, unsigned n) {
  wait_stores();
  return __hip_atomic_fetch_add(cnt, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned signal(uint32_t* cnt) { return signal_n(cnt, 1u); }

__device__ __forceinline__ void put_part_a(PartA* q, const PartA& v) {
  st_dev(&q->s_t, v.s_t);
  st_dev(&q->s_d, v.s_d);
  st_dev(&q->w, v.w);
  st_dev(&q->m_t, v.m_t);
  st_dev(&q->m_d, v.m_d);
  st_dev(&q->idx, v.idx);
}
__device__ __forceinline__ PartA get_part_a(PartA* q) {
  PartA v;
  v.s_t = ld_dev(&q->s_t);
  v.s_d = ld_dev(&q->s_d);
  v.w = ld_dev(&q->w);
  v.m_t = ld_dev(&q->m_t);
  v.m_d = ld_dev(&q->m_d);
  v.idx = ld_dev(&q->idx);
  v.pad = 0;
  return v;
}
__device__ __forceinline__ void put_stat(TaskStat* q, const TaskStat& v) {
  st_dev(&q->s_t, v.s_t);
  st_dev(&q->s_d, v.s_d);
  st_dev(&q->w, v.w);
  st_dev(&q->m_t, v.m_t);
  st_dev(&q->m_d, v.m_d);
  st_dev(&q->kl, v.kl);
  st_dev(&q->idx, v.idx);
}
__device__ __forceinline__ TaskStat get_stat(TaskStat* q) {
  TaskStat v;
  v.s_t = ld_dev(&q->s_t);
  v.s_d = ld_dev(&q->s_d);
  v.w = ld_dev(&q->w);
  v.m_t = ld_dev(&q->m_t);
  v.m_d = ld_dev(&q->m_d);
  v.kl = ld_dev(&q->kl);
  v.idx = ld_dev(&q->idx);
  return v;
}
__device__ __forceinline__ int get_idx(TaskStat* q) { return ld_dev(&q->idx); }
__device__ __forceinline__ void put_part_c(PartC* q, const PartC& v) {
  st_dev(&q->a, v.a);
  st_dev(&q->b, v.b);
  st_dev(&q->ap, v.ap);
  st_dev(&q->bp, v.bp);
  st_dev(&q->m, v.m);
}
__device__ __forceinline__ PartC get_part_c(PartC* q) {
  PartC v;
  v.a = ld_dev(&q->a);
  v.b = ld_dev(&q->b);
  v.ap = ld_dev(&q->ap);
  v.bp = ld_dev(&q->bp);
  v.m = ld_dev(&q->m);
  v.pad[0] = v.pad[1] = v.pad[2] = 0;
  return v;
}

// ----------------------------------------------------------------------------
// k_prep
// ----------------------------------------------------------------------------

__global__ __launch_bounds__(kPrepThreads) void k_prep(Params p) {
  __shared__ long long sh_w[kPrepThreads / 64];
  __shared__ int sh_bad;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  long long carry = 0;  // 64-bit: a bogus gamma cannot wrap the sum around
  for (int base = 0; base < p.B; base += kPrepThreads) {
    const int b = base + tid;
    long long g = 0;
    if (b < p.B) {
      g = p.gamma[b];
      if (g < 0) {
        sh_bad = 1;  // benign race: every writer stores 1
        g = 0;
      }
    }
    long long incl = g;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) sh_w[w] = incl;
    __syncthreads();
    long long before = 0, tile = 0;
    for (int k = 0; k < kPrepThreads / 64; ++k) {
      if (k < w) before += sh_w[k];
      tile += sh_w[k];
    }
    if (b < p.B) {
      const long long excl = carry + before + incl - g;
      // values are only used when the whole layout checks out (sum == R_d < 2^31)
      p.d_off[b] = (int)excl;
      p.t_off[b] = (int)(excl + b);
    }
    carry += tile;
    __syncthreads();
  }
  if (tid == 0) {
    p.d_off[p.B] = (int)carry;
    p.t_off[p.B] = (int)(carry + p.B);
  }
  const bool bad = sh_bad != 0 || carry != (long long)p.R_d;
  if (tid == 0) p.hdr[0] = bad ? 1 : 0;
  if (bad) {
    for (int b = tid; b < p.B; b += kPrepThreads) p.out_num[b] = -1;
    return;
  }
  for (int i = tid; i < p.n_task; i += kPrepThreads) p.cnt_task[i] = 0u;
  for (int b = tid; b < p.B; b += kPrepThreads) {
    p.cnt_req[b] = 0u;
    p.cnt_draw[b] = 0u;
  }
  __syncthreads();  // offsets written by other threads of this workgroup
  for (int b = tid; b < p.B; b += kPrepThreads) {
    const int g = p.gamma[b], d0 = p.d_off[b], t0 = p.t_off[b];
    for (int k = 0; k < g; ++k) p.pair2req[d0 + k] = b;
    for (int k = 0; k <= g; ++k) p.row2req[t0 + k] = b;
  }
}

// ----------------------------------------------------------------------------
// per-request decisions (run by the workgroup that completes a request's last
// task; every thread of the workgroup calls them)
// ----------------------------------------------------------------------------

struct DecideShared {
  int i[kWaves];
  int bad;
};

__device__ void finish_invalid(const Params& p, int b, int t0, int g) {
  for (int k = threadIdx.x; k <= g; k += kThreads) p.out_tokens[t0 + k] = -1;
  if (threadIdx.x == 0) {
    p.out_num[b] = -1;
    if (p.out_resid) p.out_resid[b] = __builtin_nanf("");
    if (p.out_tree_node) p.out_tree_node[b] = -1;
  }
}

// NKL = KL(q || p) / ln V.  The KL comes from the task's merged statistics:
// KL = (W/s_d - (m_d - m_t)) / T - log(s_d / s_t), W = sum e^{(d-m_d)/T} (d - t),
// or from the second pass when that form loses too much to cancellation.
// With a single token both distributions are the same point mass: NKL = 0.
__device__ __forceinline__ float nkl_of(const TaskStat& s, int V) { return V > 1 ? s.kl / logf((float)V) : 0.0f; }

__device__ void decide_stochastic(const Params& p, int b, int g, int t0, int d0, DecideShared& sh) {
  const float T = p.temp[b];
  bool bad = !(g <= p.max_gamma) || !temp_ok(T) || !unit_ok(p.ur[b]);
  int first = INT_MAX;
  for (int i = threadIdx.x; i < g; i += kThreads) {
    const int x = p.tokens[d0 + i];
    const float u = p.ua[d0 + i];
    if (x < 0 || x >= p.V || !unit_ok(u)) {
      bad = true;
      continue;
    }
    const TaskStat s = get_stat(p.stat + d0 + i);
    const float tx = ld_dev(p.gat + 2 * (d0 + i)), dx = ld_dev(p.gat + 2 * (d0 + i) + 1);
    // log p(x) - log q(x) = ((t_x - m_t) - (d_x - m_d)) / T + log(s_d / s_t)
    const float lr = ((tx - s.m_t) - (dx - s.m_d)) / T + (float)log(s.s_d / s.s_t);
    const float alpha = fminf(1.0f, expf(lr));
    if (!(u <= alpha)) first = min(first, i);
    if (p.out_p_x) p.out_p_x[d0 + i] = (float)((double)expf((tx - s.m_t) / T) / s.s_t);
    if (p.out_q_x) p.out_q_x[d0 + i] = (float)((double)expf((dx - s.m_d) / T) / s.s_d);
    if (p.out_nkl) p.out_nkl[d0 + i] = nkl_of(s, p.V);
  }
  if (threadIdx.x == 0) sh.bad = 0;
  __syncthreads();
  if (bad) sh.bad = 1;
  const int j0 = block_min_int(first, sh.i);  // contains barriers
  const int j = j0 == INT_MAX ? g : j0;
  if (sh.bad) {
    finish_invalid(p, b, t0, g);
    if (threadIdx.x == 0) p.term[b].kind = kTermNone;
    return;
  }
  for (int k = threadIdx.x; k <= g; k += kThreads)
    if (k != j) p.out_tokens[t0 + k] = k < j ? p.tokens[d0 + k] : -1;
  if (threadIdx.x == 0) {
    p.out_num[b] = j;
    Term tm;
    tm.j = j;
    tm.trow = t0 + j;
    tm.pad = 0;
    if (j < g) {
      const TaskStat s = get_stat(p.stat + d0 + j);
      tm.kind = kTermResidual;
      tm.drow = d0 + j;
      tm.m_t = s.m_t;
      tm.m_d = s.m_d;
      tm.k0 = (float)(s.s_t / s.s_d);
    } else {
      tm.kind = kTermBonus;
      tm.drow = -1;
      tm.m_t = tm.m_d = tm.k0 = 0.0f;
    }
    p.term[b] = tm;
  }
}

// greedy (mode 1) and NKL (mode 2)
template <int MODE>
__device__ void decide_argmax_chain(const Params& p, int b, int g, int t0, int d0, DecideShared& sh) {
  bool bad = !(g <= p.max_gamma);
  float T = 1.0f;
  if (MODE == SV_MODE_NKL) {
    T = p.temp[b];
    bad = bad || !temp_ok(T);
  }
  int first = INT_MAX;
  for (int i = threadIdx.x; i < g; i += kThreads) {
    const int x = p.tokens[d0 + i];
    if (x < 0 || x >= p.V) {
      bad = true;
      continue;
    }
    bool acc;
    if (MODE == SV_MODE_GREEDY) {
      acc = (x == get_idx(p.stat + t0 + i));
    } else {
      const TaskStat s = get_stat(p.stat + t0 + i);  // NKL tasks are target rows
      const float nkl = nkl_of(s, p.V);
      p.out_nkl[d0 + i] = nkl;
      if (p.out_p_x || p.out_q_x) {
        const float tx = ld_dev(p.gat + 2 * (d0 + i)), dx = ld_dev(p.gat + 2 * (d0 + i) + 1);
        if (p.out_p_x) p.out_p_x[d0 + i] = (float)((double)expf((tx - s.m_t) / T) / s.s_t);
        if (p.out_q_x) p.out_q_x[d0 + i] = (float)((double)expf((dx - s.m_d) / T) / s.s_d);
      }
      acc = nkl < p.delta;
    }
    if (!acc) first = min(first, i);
  }
  if (threadIdx.x == 0) sh.bad = 0;
  __syncthreads();
  if (bad) sh.bad = 1;
  const int j0 = block_min_int(first, sh.i);
  const int j = j0 == INT_MAX ? g : j0;
  if (sh.bad) {
    finish_invalid(p, b, t0, g);
    return;
  }
  int term_tok;
  if (MODE == SV_MODE_GREEDY)
    term_tok = get_idx(p.stat + t0 + j);
  else
    term_tok = get_idx(p.stat + t0 + j);
  for (int k = threadIdx.x; k <= g; k += kThreads)
    p.out_tokens[t0 + k] = k < j ? p.tokens[d0 + k] : (k == j ? term_tok : -1);
  if (threadIdx.x == 0) p.out_num[b] = j;
}

// Tree resolve.  node_info[n] packs (depth << 1) | accepted; parents precede
// children, so one ordered pass settles every node.
__device__ void decide_tree(const Params& p, int b, int g, int t0, int d0, DecideShared& sh, int16_t* node_info,
                            int16_t* par) {
  const int N = g + 1;
  bool bad = !(g <= p.max_gamma);
  if (threadIdx.x == 0) sh.bad = 0;
  __syncthreads();
  if (!bad) {
    for (int n = 1 + threadIdx.x; n < N; n += kThreads) {
      const int pa = p.parents[d0 + n - 1];
      const int x = p.tokens[d0 + n - 1];
      if (pa < 0 || pa >= n || x < 0 || x >= p.V) {
        bad = true;
        continue;
      }
      par[n] = (int16_t)pa;
      node_info[n] = (int16_t)((x == get_idx(p.stat + t0 + pa)) ? 1 : 0);  // edge match, before ancestry
    }
  }
  if (bad) sh.bad = 1;
  __syncthreads();
  if (sh.bad) {
    finish_invalid(p, b, t0, g);
    return;
  }
  if (threadIdx.x == 0) {
    node_info[0] = 1;  // root: depth 0, accepted
    for (int n = 1; n < N; ++n) {
      const int pi = node_info[par[n]];
      node_info[n] = (int16_t)((((pi >> 1) + 1) << 1) | (pi & node_info[n] & 1));
    }
  }
  __syncthreads();
  // deepest accepted node, lowest id on ties
  int key = -1;
  for (int n = threadIdx.x; n < N; n += kThreads) {
    const int ni = node_info[n];
    if (ni & 1) key = max(key, ((ni >> 1) << 13) | (8191 - n));
  }
  const int best_key = block_max_int(key, sh.i);
  const int best = 8191 - (best_key & 8191);
  const int depth = best_key >> 13;
  for (int k = depth + 1 + threadIdx.x; k <= g; k += kThreads) p.out_tokens[t0 + k] = -1;
  if (threadIdx.x == 0) {
    for (int v = best; v != 0; v = par[v]) p.out_tokens[t0 + (node_info[v] >> 1) - 1] = p.tokens[d0 + v - 1];
    p.out_tokens[t0 + depth] = get_idx(p.stat + t0 + best);
    p.out_num[b] = depth;
    if (p.out_tree_node) p.out_tree_node[b] = best;
  }
}

// ----------------------------------------------------------------------------
// k_rowstats
// ----------------------------------------------------------------------------

struct RowShared {
  float m[2][kWaves];
  float s[2][kWaves];
  float w[kWaves];
  int i[kWaves];
  double d[2 + kWaves];
  int last_chunk;  // this workgroup completed the task
  int last_task;   // ... and the request
  int refine;
  DecideShared dec;
};

// g(w) = e^w - 1 - w >= 0, accurate for small |w| (Taylor series to w^9)
__device__ __forceinline__ float g_small(float w) {
  float t = fmaf(w, 1.0f / 362880.0f, 1.0f / 40320.0f);
  t = fmaf(w, t, 1.0f / 5040.0f);
  t = fmaf(w, t, 1.0f / 720.0f);
  t = fmaf(w, t, 1.0f / 120.0f);
  t = fmaf(w, t, 1.0f / 24.0f);
  t = fmaf(w, t, 1.0f / 6.0f);
  t = fmaf(w, t, 0.5f);
  return w * w * t;
}

// KL(q || p) of one row pair in a second pass, written as the sum of the
// non-negative terms q_y * g(w_y), w_y = log(p_y / q_y).  Because
// sum q e^w = sum p = 1, this equals sum q log(q/p) exactly, has no
// cancellation, and an error eps in the log normaliser ratio only adds
// g(eps) = O(eps^2).  Run by all threads of one workgroup.
template <int DT, bool VEC>
__device__ double kl_second_pass(const Params& p, int trow, int drow, float m_t, float m_d, double s_t, double s_d,
                                 float T, float Lhi, double* shd) {
  constexpr int P = Elem<DT>::P;
  constexpr int U = 4;
  const int64_t V = p.V;
  const float invT = (float)(1.0 / (double)T);
  const float lr = (float)log(s_d / s_t);
  const float inv_sd = (float)(1.0 / s_d), inv_st = (float)(1.0 / s_t);
  double acc = 0.0;
  for (int64_t base = 0; base < V; base += (int64_t)kThreads * P * U) {
    uint4 qt[U], qd[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t e0 = base + ((int64_t)k * kThreads + threadIdx.x) * P;
      qt[k] = fetch<DT, VEC>(p.target, trow, V, e0);
      qd[k] = fetch<DT, VEC>(p.draft, drow, V, e0);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      float vt[P], vd[P];
      unpack<DT>(qt[k], vt);
      unpack<DT>(qd[k], vd);
      float part = 0.f;  // P non-negative terms in float32, then float64
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const float dt = vt[e] - m_t, dd = vd[e] - m_d;
        const float q = __builtin_amdgcn_exp2f(dd * Lhi) * inv_sd;
        const float w = fmaf(dt - dd, invT, lr);
        float term;
        if (fabsf(w) < 0.5f) {
          term = q * g_small(w);
        } else {
          // q g(w) = p - q - q w; also right where q underflows but p does not
          const float pp = __builtin_amdgcn_exp2f(dt * Lhi) * inv_st;
          term = (pp - q) - q * w;
        }
        part += term;  // positions past the end of the row give p = q = 0
      }
      acc += (double)part;
    }
  }
  return block_sum_d(acc, shd);
}

// Lane-level running statistics of one row over the chunks a workgroup streams.
struct LaneRow {
  float m;    // running maximum (raw logits)
  float s;    // sum exp2((x - m) * L) over the lane's elements so far
  int idx;    // lowest index attaining m (argmax rows)
};

// Folds NE new elements v (positions pos0 + e, e in vector order) into r.
template <int NE, int P, bool IDX>
__device__ __forceinline__ void fold_row(LaneRow& r, const float* v, float Lhi, bool soft, int64_t pos_base,
                                         int64_t pos_stride, float pad) {
  float mc = v[0];
#pragma unroll
  for (int e = 1; e < NE; ++e) mc = fmaxf(mc, v[e]);
  if (mc == pad) return;  // every element of this lane lies past the end of the row
  if (IDX && mc > r.m) {
    int ic = INT_MAX;
#pragma unroll
    for (int e = NE - 1; e >= 0; --e)
      if (v[e] == mc) ic = (int)(pos_base + (int64_t)(e / P) * pos_stride + (e % P));
    r.idx = ic;
  }
  const float M = fmaxf(r.m, mc);
  if (soft) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int e = 0; e < NE; e += 4) {
      a0 += __builtin_amdgcn_exp2f((v[e] - M) * Lhi);
      a1 += __builtin_amdgcn_exp2f((v[e + 1] - M) * Lhi);
      a2 += __builtin_amdgcn_exp2f((v[e + 2] - M) * Lhi);
      a3 += __builtin_amdgcn_exp2f((v[e + 3] - M) * Lhi);
    }
    r.s = r.s * __builtin_amdgcn_exp2f((r.m - M) * Lhi) + ((a0 + a1) + (a2 + a3));
  }
  r.m = M;
}

// Draft row of a pair, with the KL cross term W = sum e^{(d - m_d)/T} (d - t);
// the same accumulation pattern as fold_row keeps identical rows bit-identical.
template <int NE>
__device__ __forceinline__ void fold_draft_w(LaneRow& r, float& W, const float* vd, const float* vt, float Lhi,
                                             float pad) {
  float mc = vd[0];
#pragma unroll
  for (int e = 1; e < NE; ++e) mc = fmaxf(mc, vd[e]);
  if (mc == pad) return;
  const float M = fmaxf(r.m, mc);
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f, w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f;
#pragma unroll
  for (int e = 0; e < NE; e += 4) {
    const float e0 = __builtin_amdgcn_exp2f((vd[e] - M) * Lhi);
    const float e1 = __builtin_amdgcn_exp2f((vd[e + 1] - M) * Lhi);
    const float e2 = __builtin_amdgcn_exp2f((vd[e + 2] - M) * Lhi);
    const float e3 = __builtin_amdgcn_exp2f((vd[e + 3] - M) * Lhi);
    a0 += e0;
    a1 += e1;
    a2 += e2;
    a3 += e3;
    w0 = fmaf(e0, vd[e] - vt[e], w0);
    w1 = fmaf(e1, vd[e + 1] - vt[e + 1], w1);
    w2 = fmaf(e2, vd[e + 2] - vt[e + 2], w2);
    w3 = fmaf(e3, vd[e + 3] - vt[e + 3], w3);
  }
  const float f = __builtin_amdgcn_exp2f((r.m - M) * Lhi);
  r.s = r.s * f + ((a0 + a1) + (a2 + a3));
  W = W * f + ((w0 + w1) + (w2 + w3));
  r.m = M;
}

// Request of a task (task index = draft row for stochastic pairs, target row
// otherwise): offsets come from LDS (small batches) or from the prep kernel.
struct ReqInfo {
  int b, g, t0, d0;
};

template <int MODE>
__device__ __forceinline__ ReqInfo locate(const Params& p, const int* s_off, bool lds, int task) {
  ReqInfo r;
  if (lds) {
    // last b with off(b) <= task, off = d_off (pairs) or t_off = d_off + b (rows)
    int lo = 0, hi = p.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      const int off = MODE == SV_MODE_STOCHASTIC ? s_off[mid] : s_off[mid] + mid;
      if (off <= task) lo = mid; else hi = mid - 1;
    }
    r.b = lo;
    r.d0 = s_off[lo];
    r.g = s_off[lo + 1] - s_off[lo];
  } else {
    r.b = MODE == SV_MODE_STOCHASTIC ? p.pair2req[task] : p.row2req[task];
    r.d0 = p.d_off[r.b];
    r.g = p.d_off[r.b + 1] - r.d0;
  }
  r.t0 = r.d0 + r.b;
  return r;
}

struct StatsShared {
  float m[2][kWaves];
  float s[2][kWaves];
  float w[kWaves];
  int i[kWaves];
  double d[2 + kWaves];
  int flag;
  int refine;
  int scan[kThreads / 64];
  DecideShared dec;
};

// Persistent row-statistics kernel.  The (task, chunk) items, task-major, are
// split into one contiguous range per workgroup; a workgroup streams its
// range with the next chunk's loads in flight while it folds the current one,
// and publishes one partial per task segment.  The last segment of a task
// merges the partials (in vocabulary order), and the last task of a request
// runs the decision.
template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void k_stats(Params p) {
  constexpr int P = Elem<DT>::P;
  constexpr int NE = kUA * P;  // elements per thread per row per chunk
  constexpr int64_t CH = (int64_t)kThreads * NE;
  constexpr float kPad = Elem<DT>::kPad;
  constexpr bool IDX = MODE != SV_MODE_STOCHASTIC;
  __shared__ int s_off[kLdsBatch + 1];
  __shared__ StatsShared sh;
  __shared__ int16_t tree_info[MODE == SV_MODE_TREE_GREEDY ? SV_MAX_GAMMA + 1 : 1];
  __shared__ int16_t tree_par[MODE == SV_MODE_TREE_GREEDY ? SV_MAX_GAMMA + 1 : 1];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t V = p.V;
  const bool lds = p.B <= kLdsBatch;

  // ---- packed offsets: exclusive scan of gamma in LDS (every workgroup)
  if (lds) {
    if (tid == 0) sh.flag = 0;
    __syncthreads();
    int carry = 0;
    for (int base = 0; base < p.B; base += kThreads) {
      const int bb = base + tid;
      int g = bb < p.B ? p.gamma[bb] : 0;
      if (g < 0 || g > p.R_d) {
        sh.flag = 1;  // every writer stores 1
        g = 0;
      }
      int incl = g;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      if (lane == 63) sh.scan[wv] = incl;
      __syncthreads();
      int before = 0, tile = 0;
#pragma unroll
      for (int k = 0; k < kWaves; ++k) {
        if (k < wv) before += sh.scan[k];
        tile += sh.scan[k];
      }
      if (bb < p.B) s_off[bb] = carry + before + incl - g;
      carry += tile;  // at most B * R_d: bounded because each g <= R_d
      __syncthreads();
    }
    if (tid == 0) s_off[p.B] = carry;
    __syncthreads();
    const bool bad = sh.flag != 0 || carry != p.R_d;
    if (blockIdx.x == 0) {
      // offsets for the draw kernel; layout flag
      for (int bb = tid; bb <= p.B; bb += kThreads) {
        p.d_off[bb] = s_off[bb];
        p.t_off[bb] = s_off[bb] + bb;
      }
      if (tid == 0) p.hdr[0] = bad ? 1 : 0;
      if (bad)
        for (int bb = tid; bb < p.B; bb += kThreads) p.out_num[bb] = -1;
    }
    if (bad) return;
  } else if (p.hdr[0] != 0) {
    return;  // layout error found by k_prep
  }

  // ---- this workgroup's items
  const int nch = p.nch_a;
  const int64_t N = (int64_t)p.n_task * nch;
  const int64_t G = gridDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * N / G, i1 = ((int64_t)blockIdx.x + 1) * N / G;
  if (i0 >= i1) return;

  // segment state (uniform across the workgroup)
  int task = -1, b = 0, g = 0, t0 = 0, d0 = 0, trow = 0, drow = -1, seg_first = 0, x = -1;
  bool pair = false;
  float T = 1.0f, Lhi = 0.0f, Llo = 0.0f;
  LaneRow rt{kPad, 0.f, INT_MAX}, rd{kPad, 0.f, INT_MAX};
  float W = 0.f;
  float gx_t = 0.f, gx_d = 0.f;
  bool gathered = false;

  auto rows_of = [&](int tk, int& tr, int& dr, bool& pr, ReqInfo& ri) {
    ri = locate<MODE>(p, s_off, lds, tk);
    if (MODE == SV_MODE_STOCHASTIC) {
      tr = tk + ri.b;
      dr = tk;
      pr = true;
    } else {
      tr = tk;
      const int i = tk - ri.t0;
      pr = (MODE == SV_MODE_NKL) && i < ri.g;
      dr = pr ? ri.d0 + i : -1;
    }
  };

  // prefetch the first chunk
  uint4 cur_t[kUA], cur_d[kUA], nxt_t[kUA], nxt_d[kUA];
  int n_trow, n_drow;
  bool n_pair;
  {
    ReqInfo ri;
    rows_of((int)(i0 / nch), n_trow, n_drow, n_pair, ri);
    const int64_t e0 = (i0 % nch) * CH;
#pragma unroll
    for (int k = 0; k < kUA; ++k) {
      nxt_t[k] = fetch<DT, VEC>(p.target, n_trow, V, e0 + ((int64_t)k * kThreads + tid) * P);
      if (n_pair) nxt_d[k] = fetch<DT, VEC>(p.draft, n_drow, V, e0 + ((int64_t)k * kThreads + tid) * P);
    }
  }

  for (int64_t it = i0; it < i1; ++it) {
    const int tk = (int)(it / nch);
    const int chunk = (int)(it - (int64_t)tk * nch);
#pragma unroll
    for (int k = 0; k < kUA; ++k) {
      cur_t[k] = nxt_t[k];
      cur_d[k] = nxt_d[k];
    }
    if (tk != task) {  // a new task segment starts
      ReqInfo ri;
      rows_of(tk, trow, drow, pair, ri);
      task = tk;
      b = ri.b;
      g = ri.g;
      t0 = ri.t0;
      d0 = ri.d0;
      seg_first = chunk;
      rt = LaneRow{kPad, 0.f, INT_MAX};
      rd = LaneRow{kPad, 0.f, INT_MAX};
      W = 0.f;
      gathered = false;
      if (pair) {
        T = p.temp[b];
        const double Ld = kLog2eD / (double)T;
        Lhi = (float)Ld;
        Llo = (float)(Ld - (double)Lhi);
        x = p.tokens[drow];
      }
    }
    // next chunk's loads go out before this one is folded
    if (it + 1 < i1) {
      const int tk2 = (int)((it + 1) / nch);
      if (tk2 != task) {
        ReqInfo ri;
        rows_of(tk2, n_trow, n_drow, n_pair, ri);
      } else {
        n_trow = trow;
        n_drow = drow;
        n_pair = pair;
      }
      const int64_t e1 = ((it + 1) - (int64_t)tk2 * nch) * CH;
#pragma unroll
      for (int k = 0; k < kUA; ++k) {
        nxt_t[k] = fetch<DT, VEC>(p.target, n_trow, V, e1 + ((int64_t)k * kThreads + tid) * P);
        if (n_pair) nxt_d[k] = fetch<DT, VEC>(p.draft, n_drow, V, e1 + ((int64_t)k * kThreads + tid) * P);
      }
    }
    const int64_t e_chunk = (int64_t)chunk * CH;
    // gather of the logits at the drafted token
    if (pair && tid == 0 && x >= e_chunk && x < e_chunk + CH && x < V) {
      gx_t = load_scalar<DT>(p.target, trow, V, x);
      gx_d = load_scalar<DT>(p.draft, drow, V, x);
      gathered = true;
    }
    // fold this chunk
    float vt[NE];
#pragma unroll
    for (int k = 0; k < kUA; ++k) unpack<DT>(cur_t[k], vt + k * P);
    fold_row<NE, P, IDX>(rt, vt, Lhi, pair, e_chunk + (int64_t)tid * P, (int64_t)kThreads * P, kPad);
    if (pair) {
      float vd[NE];
#pragma unroll
      for (int k = 0; k < kUA; ++k) unpack<DT>(cur_d[k], vd + k * P);
      if (p.want_w)
        fold_draft_w<NE>(rd, W, vd, vt, Lhi, kPad);
      else
        fold_row<NE, P, false>(rd, vd, Lhi, true, 0, 0, kPad);
    }

    const bool seg_end = (it + 1 == i1) || (chunk + 1 == nch);
    if (!seg_end) continue;

    // ---- end of a task segment: workgroup reduction and publication
    const float Mt = wave_max(rt.m);
    int It = INT_MAX;
    if (IDX) It = wave_min_int(rt.m == Mt ? rt.idx : INT_MAX);
    float St = 0.f, Md = kPad, Sd = 0.f, Wd = 0.f;
    if (pair) {
      St = wave_sum(rt.s * exp_hp(rt.m - Mt, Lhi, Llo));
      Md = wave_max(rd.m);
      const float f = exp_hp(rd.m - Md, Lhi, Llo);
      Sd = wave_sum(rd.s * f);
      if (p.want_w) Wd = wave_sum(W * f);
    }
    __syncthreads();  // LDS of the previous segment is no longer read
    if (lane == 0) {
      sh.m[0][wv] = Mt;
      sh.s[0][wv] = St;
      sh.m[1][wv] = Md;
      sh.s[1][wv] = Sd;
      sh.w[wv] = Wd;
      sh.i[wv] = It;
    }
    __syncthreads();
    const int64_t w_lo = (((int64_t)task * nch + 1) * G - 1) / N;  // first workgroup of the task
    if (tid == 0) {
      PartA pa;
      float M = sh.m[0][0], M2 = sh.m[1][0];
      for (int k = 1; k < kWaves; ++k) {
        M = fmaxf(M, sh.m[0][k]);
        M2 = fmaxf(M2, sh.m[1][k]);
      }
      int I = INT_MAX;
      double S = 0.0, S2 = 0.0, W2 = 0.0;
      for (int k = 0; k < kWaves; ++k) {
        if (sh.m[0][k] == M) I = min(I, sh.i[k]);
        if (pair) {
          S += (double)sh.s[0][k] * (double)exp_hp(sh.m[0][k] - M, Lhi, Llo);
          const double f = (double)exp_hp(sh.m[1][k] - M2, Lhi, Llo);
          S2 += (double)sh.s[1][k] * f;
          W2 += (double)sh.w[k] * f;
        }
      }
      pa.m_t = M;
      pa.s_t = S;
      pa.m_d = M2;
      pa.s_d = S2;
      pa.w = W2;
      pa.idx = I;
      pa.pad = 0;
      put_part_a(p.part_a + (int64_t)task * nch + ((int64_t)blockIdx.x - w_lo), pa);
      if (gathered) {
        st_dev(p.gat + 2 * drow, gx_t);
        st_dev(p.gat + 2 * drow + 1, gx_d);
      }
      const unsigned mine = (unsigned)(chunk + 1 - seg_first);
      const unsigned old = signal_n(p.cnt_task + task, mine);
      sh.flag = (old + mine == (unsigned)nch);
    }
    __syncthreads();
    if (!sh.flag) continue;

    // ---- this workgroup completed the task: merge the partials in order
    const int64_t w_hi = (((int64_t)task * nch + nch) * G - 1) / N;
    const int nseg = (int)(w_hi - w_lo + 1);
    if (wv == 0) {
      float m1 = -FLT_MAX, m2 = -FLT_MAX;
      double s1 = 0.0, s2 = 0.0, w2 = 0.0;
      int i1x = INT_MAX;
      for (int sg = lane; sg < nseg; sg += 64) {
        const PartA q = get_part_a(p.part_a + (int64_t)task * nch + sg);
        if (q.m_t > m1) {
          if (pair) s1 = s1 * (double)exp_hp(m1 - q.m_t, Lhi, Llo) + q.s_t;
          m1 = q.m_t;
          i1x = q.idx;
        } else {
          if (pair) s1 += q.s_t * (double)exp_hp(q.m_t - m1, Lhi, Llo);
          if (q.m_t == m1) i1x = min(i1x, q.idx);
        }
        if (pair) {
          if (q.m_d > m2) {
            const double f = (double)exp_hp(m2 - q.m_d, Lhi, Llo);
            s2 = s2 * f + q.s_d;
            w2 = w2 * f + q.w;
            m2 = q.m_d;
          } else {
            const double f = (double)exp_hp(q.m_d - m2, Lhi, Llo);
            s2 += q.s_d * f;
            w2 += q.w * f;
          }
        }
      }
      const float M1 = wave_max(m1);
      const int I1 = wave_min_int(m1 == M1 ? i1x : INT_MAX);
      double S1 = 0.0, S2 = 0.0, W2 = 0.0;
      float M2 = 0.f;
      if (pair) {
        S1 = wave_sum_d(s1 * (double)exp_hp(m1 - M1, Lhi, Llo));
        M2 = wave_max(m2);
        const double f = (double)exp_hp(m2 - M2, Lhi, Llo);
        S2 = wave_sum_d(s2 * f);
        W2 = wave_sum_d(w2 * f);
      }
      if (lane == 0) {
        TaskStat ts;
        ts.m_t = M1;
        ts.s_t = S1;
        ts.m_d = M2;
        ts.s_d = S2;
        ts.w = W2;
        ts.idx = I1;
        ts.kl = 0.0f;
        int refine = 0;
        if (pair && p.want_w) {
          // one-pass KL and a bound on its rounding error (a few 1e-7 of the
          // magnitude of the terms that cancel)
          const double a = W2 / S2 / (double)T, bm = ((double)M2 - (double)M1) / (double)T, lg = log(S2 / S1);
          const double kl = a - bm - lg;
          const double err = 4e-7 * (fabs(a) + fabs(bm) + fabs(lg) + 1.0);
          refine = err > 1e-5 * kl;
          if (MODE == SV_MODE_NKL && p.V > 1) {
            const double lnV = log((double)p.V);
            refine |= fabs(kl / lnV - (double)p.delta) < 2.0 * err / lnV;
          }
          ts.kl = (float)kl;
        }
        put_stat(p.stat + task, ts);
        sh.refine = refine;
        sh.d[0] = S1;
        sh.d[1] = S2;
        sh.m[0][0] = M1;
        sh.m[1][0] = M2;
      }
    }
    __syncthreads();
    if (sh.refine) {
      const double kl =
          kl_second_pass<DT, VEC>(p, trow, drow, sh.m[0][0], sh.m[1][0], sh.d[0], sh.d[1], T, Lhi, sh.d + 2);
      if (tid == 0) st_dev(&p.stat[task].kl, (float)kl);
    }
    if (tid == 0) {
      st_dev(p.cnt_task + task, 0u);
      const unsigned need = (unsigned)(MODE == SV_MODE_STOCHASTIC ? g : g + 1);
      const unsigned old = signal_n(p.cnt_req + b, 1u);
      sh.flag = (old + 1 == need);
    }
    __syncthreads();
    if (!sh.flag) continue;

    // ---- last task of the request: decide
    if (MODE == SV_MODE_STOCHASTIC)
      decide_stochastic(p, b, g, t0, d0, sh.dec);
    else if (MODE == SV_MODE_TREE_GREEDY)
      decide_tree(p, b, g, t0, d0, sh.dec, tree_info, tree_par);
    else
      decide_argmax_chain<MODE>(p, b, g, t0, d0, sh.dec);
    if (tid == 0) st_dev(p.cnt_req + b, 0u);
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------
// k_draw (stochastic mode)
// ----------------------------------------------------------------------------

struct DrawShared {
  double d[kWaves];
  float f[kWaves];
  int i[kWaves];
  int last;
  double ta[kThreads], tb[kThreads];  // one tile of chunk partials
  float tm[kThreads];
  double a_tot, b_tot, S, base;
  float mrow;
  int cstar, lastpos_chunk;
};

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_draw(Params p) {
  constexpr int P = Elem<DT>::P;
  constexpr int NE = kUC * P;
  constexpr int64_t CH = (int64_t)kThreads * NE;
  __shared__ DrawShared sh;
  if (p.hdr[0] != 0) return;
  const int tid = threadIdx.x;
  const int b = blockIdx.x / p.nch_c;
  const int chunk = blockIdx.x - b * p.nch_c;
  const int64_t V = p.V;
  const int g = p.gamma[b];
  const int t0 = p.t_off[b];
  const float T = p.temp[b];
  const float ur = p.ur[b];

  int kind, j, trow, drow;
  float Mt = 0.f, Md = 0.f, k0 = 0.f;
  if (g == 0) {
    // nothing drafted: the step is a plain draw from target row 0
    if (!temp_ok(T) || !unit_ok(ur)) {
      if (chunk == 0 && tid == 0) {
        p.out_num[b] = -1;
        p.out_tokens[t0] = -1;
        if (p.out_resid) p.out_resid[b] = __builtin_nanf("");
      }
      return;
    }
    kind = kTermBonus;
    j = 0;
    trow = t0;
    drow = -1;
  } else {
    const Term tm = p.term[b];
    kind = tm.kind;
    if (kind == kTermNone) return;
    j = tm.j;
    trow = tm.trow;
    drow = tm.drow;
    Mt = tm.m_t;
    Md = tm.m_d;
    k0 = tm.k0;
  }
  const double Ld = kLog2eD / (double)T;
  const float Lhi = (float)Ld;
  const float Llo = (float)(Ld - (double)Lhi);
  const int64_t e_chunk = (int64_t)chunk * CH;

  // ---- chunk partial sums
  uint4 qt[kUC], qd[kUC];
#pragma unroll
  for (int k = 0; k < kUC; ++k) qt[k] = fetch<DT, VEC>(p.target, trow, V, e_chunk + ((int64_t)k * kThreads + tid) * P);
  if (kind == kTermResidual) {
#pragma unroll
    for (int k = 0; k < kUC; ++k) qd[k] = fetch<DT, VEC>(p.draft, drow, V, e_chunk + ((int64_t)k * kThreads + tid) * P);
  }
  float vt[NE];
#pragma unroll
  for (int k = 0; k < kUC; ++k) unpack<DT>(qt[k], vt + k * P);
  double A = 0.0, Bs = 0.0, Ap = 0.0, Bp = 0.0;
  float mc = 0.f;
  if (kind == kTermResidual) {
    float vd[NE];
#pragma unroll
    for (int k = 0; k < kUC; ++k) unpack<DT>(qd[k], vd + k * P);
#pragma unroll
    for (int k = 0; k < kUC; ++k) {
      float sa = 0.f, sb = 0.f, sap = 0.f, sbp = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const float a = exp_hp(vt[k * P + e] - Mt, Lhi, Llo);
        const float bb = exp_hp(vd[k * P + e] - Md, Lhi, Llo);
        sa += a;
        sb += bb;
        const bool in = a > k0 * bb;
        sap += in ? a : 0.f;
        sbp += in ? bb : 0.f;
      }
      A += (double)sa;
      Bs += (double)sb;
      Ap += (double)sap;
      Bp += (double)sbp;
    }
  } else {
    float m = vt[0];
#pragma unroll
    for (int e = 1; e < NE; ++e) m = fmaxf(m, vt[e]);
    mc = block_max(m, sh.f);
#pragma unroll
    for (int k = 0; k < kUC; ++k) {
      float sa = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) sa += exp_hp(vt[k * P + e] - mc, Lhi, Llo);
      A += (double)sa;
    }
  }
  A = block_sum_d(A, sh.d);
  if (kind == kTermResidual) {
    Bs = block_sum_d(Bs, sh.d);
    Ap = block_sum_d(Ap, sh.d);
    Bp = block_sum_d(Bp, sh.d);
  }
  if (tid == 0) {
    PartC pc;
    pc.a = A;
    pc.b = Bs;
    pc.ap = Ap;
    pc.bp = Bp;
    pc.m = mc;
    pc.pad[0] = pc.pad[1] = pc.pad[2] = 0;
    put_part_c(p.part_c + (int64_t)b * p.nch_c + chunk, pc);
    const unsigned old = signal(p.cnt_draw + b);
    sh.last = (old == (unsigned)(p.nch_c - 1));
  }
  __syncthreads();
  if (!sh.last) return;

  // ---- last workgroup of the request: choose the chunk.  Chunk partials are
  // staged through LDS a tile at a time and combined by thread 0 in chunk
  // order, so the result does not depend on which workgroup finished last.
  PartC* pcs = p.part_c + (int64_t)b * p.nch_c;
  const int nch = p.nch_c;
  // stage 1: totals of a and b, and the row maximum (bonus)
  {
    double at = 0.0, bt = 0.0;
    float M = -FLT_MAX;
    for (int base = 0; base < nch; base += kThreads) {
      const int ch = base + tid;
      if (ch < nch) {
        const PartC q = get_part_c(pcs + ch);
        sh.ta[tid] = q.a;
        sh.tb[tid] = q.b;
        sh.tm[tid] = q.m;
      }
      __syncthreads();
      if (tid == 0) {
        const int n = min(kThreads, nch - base);
        for (int k = 0; k < n; ++k) {
          at += sh.ta[k];
          bt += sh.tb[k];
          M = fmaxf(M, sh.tm[k]);
        }
      }
      __syncthreads();
    }
    if (tid == 0) {
      sh.a_tot = at;
      sh.b_tot = bt;
      sh.mrow = M;
    }
    __syncthreads();
  }
  const double K = kind == kTermResidual ? sh.a_tot / sh.b_tot : 0.0;
  const float Mrow = sh.mrow;
  // chunk weight: residual  sum_{a > k0 b}(a - K b) = A+ - K B+ ; bonus  A_c exp((m_c - M)/T)
  auto weight = [&](const PartC& q, int fb) -> double {
    if (kind == kTermResidual) return fb ? q.a : q.ap - K * q.bp;
    return q.a * exp2(((double)q.m - (double)Mrow) * Ld);
  };
  int fallback = 0;
  // stage 2: total mass S
  double S;
  {
    double tot = 0.0;
    for (int base = 0; base < nch; base += kThreads) {
      const int ch = base + tid;
      if (ch < nch) sh.ta[tid] = weight(get_part_c(pcs + ch), 0);
      __syncthreads();
      if (tid == 0) {
        const int n = min(kThreads, nch - base);
        for (int k = 0; k < n; ++k) tot += sh.ta[k];
      }
      __syncthreads();
    }
    if (tid == 0) sh.S = tot;
    __syncthreads();
    S = sh.S;
    if (kind == kTermResidual && !(S > 0.0)) {
      // max(0, p - q) vanished numerically: draw from p_j instead
      fallback = 1;
      S = sh.a_tot;
    }
  }
  const double target = (double)ur * S;
  // stage 3: first chunk whose cumulative weight exceeds the target
  if (tid == 0) {
    sh.cstar = -1;
    sh.lastpos_chunk = -1;
    sh.base = 0.0;
  }
  __syncthreads();
  {
    double cum = 0.0;
    for (int base = 0; base < nch; base += kThreads) {
      const int ch = base + tid;
      if (ch < nch) sh.ta[tid] = weight(get_part_c(pcs + ch), fallback);
      __syncthreads();
      if (tid == 0 && sh.cstar < 0) {
        const int n = min(kThreads, nch - base);
        for (int k = 0; k < n; ++k) {
          if (sh.ta[k] > 0.0) sh.lastpos_chunk = base + k;
          const double nxt = cum + sh.ta[k];
          if (nxt > target) {
            sh.cstar = base + k;
            sh.base = cum;
            break;
          }
          cum = nxt;
        }
      }
      __syncthreads();
      if (sh.cstar >= 0) break;  // uniform: read after the barrier
    }
  }
  int cstar = sh.cstar;
  bool take_last = false;
  if (cstar < 0) {  // rounding left the target at/after the end: last token with mass
    cstar = sh.lastpos_chunk >= 0 ? sh.lastpos_chunk : nch - 1;
    take_last = true;
  }
  const double cbase = sh.base;

  // ---- re-read chunk c*: thread t owns NE consecutive tokens
  const int64_t y0 = (int64_t)cstar * CH + (int64_t)tid * NE;
  double r[NE];
  double tsum = 0.0;
  const double chunk_factor =
      (kind == kTermBonus) ? exp2(((double)ld_dev(&pcs[cstar].m) - (double)Mrow) * Ld) : 1.0;
  const float ref = (kind == kTermBonus) ? ld_dev(&pcs[cstar].m) : Mt;
#pragma unroll
  for (int k = 0; k < kUC; ++k) {
    const uint4 q = fetch<DT, VEC>(p.target, trow, V, y0 + k * P);
    float v[P];
    unpack<DT>(q, v);
    float vdd[P];
    if (kind == kTermResidual && !fallback) {
      const uint4 qq = fetch<DT, VEC>(p.draft, drow, V, y0 + k * P);
      unpack<DT>(qq, vdd);
    }
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const float a = exp_hp(v[e] - ref, Lhi, Llo);
      double rv;
      if (kind == kTermResidual && !fallback) {
        const float bb = exp_hp(vdd[e] - Md, Lhi, Llo);
        rv = (a > k0 * bb) ? (double)a - K * (double)bb : 0.0;
      } else {
        rv = (double)a * chunk_factor;
      }
      if (y0 + k * P + e >= V) rv = 0.0;
      r[k * P + e] = rv;
      tsum += rv;
    }
  }
  double tot;
  const double excl = block_exclusive_scan_d(tsum, sh.d, tot);
  (void)tot;
  int cand = INT_MAX;
  int lastpos = -1;
  {
    double cum = cbase + excl;
    const bool mine = !take_last && cum <= target && cum + tsum > target;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      if (r[e] > 0.0) lastpos = (int)(y0 + e);
      if (mine && cand == INT_MAX) {
        cum += r[e];
        if (cum > target) cand = (int)(y0 + e);
      }
    }
  }
  const int ystar0 = block_min_int(cand, sh.i);
  const int ylast = block_max_int(lastpos, sh.i);
  if (tid == 0) {
    int y = ystar0 != INT_MAX ? ystar0 : ylast;
    if (y < 0 || y >= p.V) y = (int)min<int64_t>(V - 1, (int64_t)cstar * CH);
    p.out_tokens[t0 + j] = y;
    if (g == 0) p.out_num[b] = 0;
    if (p.out_resid) p.out_resid[b] = (kind == kTermResidual && !fallback) ? (float)(S / sh.a_tot) : 1.0f;
    st_dev(p.cnt_draw + b, 0u);
  }
}

}  // namespace

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------

int launch_prep(const Params& p, void* stream) {
  hipLaunchKernelGGL(k_prep, dim3(1), dim3(kPrepThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

template <int DT, bool VEC, int MODE>
static void stats_launch(const Params& p, hipStream_t s) {
  // one resident wave of persistent workgroups (occupancy queried once per process)
  static int per_cu = 0, cus = 0;
  if (per_cu == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_stats<DT, VEC, MODE>, kThreads, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
  }
  const int64_t items = (int64_t)p.n_task * p.nch_a;
  int64_t grid = (int64_t)per_cu * cus;
  if (grid > items) grid = items;
  if (grid < 1) grid = 1;  // workgroup 0 also publishes the offsets
  hipLaunchKernelGGL((k_stats<DT, VEC, MODE>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
}

template <int DT, bool VEC>
static void rowstats_dispatch(const Params& p, hipStream_t s) {
  switch (p.mode) {
    case SV_MODE_STOCHASTIC: stats_launch<DT, VEC, SV_MODE_STOCHASTIC>(p, s); break;
    case SV_MODE_GREEDY: stats_launch<DT, VEC, SV_MODE_GREEDY>(p, s); break;
    case SV_MODE_NKL: stats_launch<DT, VEC, SV_MODE_NKL>(p, s); break;
    default: stats_launch<DT, VEC, SV_MODE_TREE_GREEDY>(p, s); break;
  }
}

int launch_rowstats(const Params& p, bool vec, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (p.dtype == SV_DTYPE_BF16) {
    if (vec) rowstats_dispatch<SV_DTYPE_BF16, true>(p, s);
    else rowstats_dispatch<SV_DTYPE_BF16, false>(p, s);
  } else {
    if (vec) rowstats_dispatch<SV_DTYPE_F32, true>(p, s);
    else rowstats_dispatch<SV_DTYPE_F32, false>(p, s);
  }
  return (int)hipGetLastError();
}

int launch_draw(const Params& p, bool vec, void* stream) {
  const int64_t n = (int64_t)p.B * p.nch_c;
  if (n <= 0) return 0;
  const dim3 grid((unsigned)n);
  hipStream_t s = (hipStream_t)stream;
  if (p.dtype == SV_DTYPE_BF16) {
    if (vec) hipLaunchKernelGGL((k_draw<SV_DTYPE_BF16, true>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((k_draw<SV_DTYPE_BF16, false>), grid, dim3(kThreads), 0, s, p);
  } else {
    if (vec) hipLaunchKernelGGL((k_draw<SV_DTYPE_F32, true>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((k_draw<SV_DTYPE_F32, false>), grid, dim3(kThreads), 0, s, p);
  }
  return (int)hipGetLastError();
}

}  // namespace sv
