// gfx950 kernels of the speculative-decoding verify step.
//
// Launches per call (all on the caller's stream):
//   k_prep      batches above kLdsBatch only: one workgroup scans gamma into
//               the packed offsets, builds the row -> request maps and checks
//               the layout.  Smaller batches do this scan in LDS inside
//               k_stats.
//   k_stats     the streaming pass over the logits (the HBM-bound part).  The
//               (task, vocabulary chunk) items are split into contiguous
//               ranges, one per workgroup of a grid sized to fill the GPU
//               once.  A task is a (target row, draft row) pair (stochastic,
//               NKL) or a target row (greedy, tree, NKL bonus row).  Each
//               workgroup folds its chunks into running (max, sum exp,
//               argmax, KL cross terms) and writes one partial per task
//               segment with plain stores: no atomics, no waiting.
//   k_decide    one workgroup per request: merges the partials of its tasks,
//               evaluates acceptance (alpha = min(1, p/q) against u, argmax
//               match, NKL < delta, tree paths), refines KL values whose
//               one-pass form is not accurate enough with a second pass, and
//               writes tokens, counts and diagnostics.  Stochastic requests
//               leave the terminal slot to k_draw.
//   k_draw      stochastic mode only: one workgroup per (request, chunk) of
//               the terminal row; float64 chunk sums of the residual
//               max(0, p - q) (or of p for a bonus token); the last workgroup
//               of a request picks the chunk and draws the token by a
//               workgroup-wide prefix sum.
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
//
// Every exponential of the path is 2^((x - m) * Lhi) with Lhi = fl32(log2(e)/T),
// in the statistics, decision and draw passes alike, so the three passes see
// the same distributions.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cstdint>

#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kWaves = kThreads / 64;
constexpr double kLog2eD = 1.44269504088896340736;
constexpr double kLn2D = 0.693147180559945309417;

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
// pad pattern.  Addresses are clamped into the row and the pad is selected
// after the load, so every lane issues its loads unconditionally.
// VEC: rows are a whole number of 16-byte vectors and 16-byte aligned.
// Raw 16 bytes at clamped addresses: positions >= V hold copies of elements
// of the row, which the caller masks by position (mask_tail) where the data is
// consumed, so that no wait is placed right behind the load.
template <int DT, bool VEC>
__device__ __forceinline__ uint4 fetch_raw(const void* base, int64_t row, int64_t V, int64_t e0) {
  if (VEC) {
    const int64_t ec = e0 < V ? e0 : V - Elem<DT>::P;
    return *reinterpret_cast<const uint4*>(static_cast<const char*>(base) +
                                           (row * V + ec) * (DT == SV_DTYPE_BF16 ? 2 : 4));
  }
  uint32_t w[4];
  if (DT == SV_DTYPE_BF16) {
    const uint16_t* r = static_cast<const uint16_t*>(base) + row * V;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = r[e0 + e < V ? e0 + e : V - 1];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = h[2 * e] | (h[2 * e + 1] << 16);
  } else {
    const uint32_t* r = static_cast<const uint32_t*>(base) + row * V;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = r[e0 + e < V ? e0 + e : V - 1];
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Sets the unpacked elements of vector positions >= V to the pad value.
// v[k * P + e] is the element at e0(k) + e, e0(k) = base + k * stride.
template <int DT, int NV>
__device__ __forceinline__ void mask_tail(float* v, int64_t base, int64_t stride, int64_t V) {
  constexpr int P = Elem<DT>::P;
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int e = 0; e < P; ++e)
      if (base + k * stride + e >= V) v[k * P + e] = Elem<DT>::kPad;
}

template <int DT, bool VEC>
__device__ __forceinline__ uint4 fetch(const void* base, int64_t row, int64_t V, int64_t e0) {
  constexpr int P = Elem<DT>::P;
  constexpr uint32_t pp = Elem<DT>::kPadPair;
  if (VEC) {
    const int64_t ec = e0 < V ? e0 : V - P;  // a vector is entirely inside or past the row
    const char* ptr = static_cast<const char*>(base) + (row * V + ec) * (DT == SV_DTYPE_BF16 ? 2 : 4);
    uint4 q = *reinterpret_cast<const uint4*>(ptr);
    if (e0 >= V) q = make_uint4(pp, pp, pp, pp);
    return q;
  }
  uint32_t w[4];
  if (DT == SV_DTYPE_BF16) {
    const uint16_t* r = static_cast<const uint16_t*>(base) + row * V;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t y = e0 + e;
      h[e] = r[y < V ? y : V - 1];
      if (y >= V) h[e] = pp & 0xFFFFu;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = h[2 * e] | (h[2 * e + 1] << 16);
  } else {
    const uint32_t* r = static_cast<const uint32_t*>(base) + row * V;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t y = e0 + e;
      w[e] = r[y < V ? y : V - 1];
      if (y >= V) w[e] = pp;
    }
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

__device__ __forceinline__ bool unit_ok(float u) { return u >= 0.0f && u < 1.0f; }
__device__ __forceinline__ bool temp_ok(float t) { return t > 0.0f && t <= FLT_MAX; }

// 2^(dx * Lhi); dx = x - m <= 0 is the distance to a running maximum (exact
// for bf16 inputs), Lhi = fl32(log2(e)/T).  dx = -inf gives 0.
__device__ __forceinline__ float ex2(float dx, float Lhi) { return __builtin_amdgcn_exp2f(dx * Lhi); }
// ----------------------------------------------------------------------------
// k_prep (batches above kLdsBatch)
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
    // values are only used when the whole layout checks out (sum == R_d < 2^31)
    if (b < p.B) p.d_off[b] = (int)(carry + before + incl - g);
    carry += tile;
    __syncthreads();
  }
  if (tid == 0) p.d_off[p.B] = (int)carry;
  const bool bad = sh_bad != 0 || carry != (long long)p.R_d;
  if (tid == 0) {
    p.hdr[0] = bad ? 1 : 0;
    p.hdr[1] = 0;  // queue of the KL second pass
  }
  if (bad) return;
  __syncthreads();  // offsets written by other threads of this workgroup
  for (int b = tid; b < p.B; b += kPrepThreads) {
    const int g = p.gamma[b], d0 = p.d_off[b], t0 = d0 + b;
    if (p.mode == SV_MODE_STOCHASTIC)
      for (int k = 0; k < g; ++k) p.pair2req[d0 + k] = b;
    if (p.mode == SV_MODE_NKL)
      for (int k = 0; k <= g; ++k) p.row2req[t0 + k] = b;
  }
}

// ----------------------------------------------------------------------------
// k_stats: the streaming pass
// ----------------------------------------------------------------------------

// Items (task, chunk) are numbered task * nch + chunk; workgroup w of G
// streams items [w N / G, (w + 1) N / G).  The workgroup that streams item i
// is floor(((i + 1) G - 1) / N).  The float64 quotient floors exactly here:
// the numerator is an integer below 2^53, and the quotient is below 2^13, so
// its rounding error (< 2^-39) is far below the distance 1/N >= 2^-31 of any
// non-integer quotient to the next integer.
__device__ __forceinline__ int wg_of(int64_t item, int64_t N, int G) {
  return (int)floor((double)((item + 1) * G - 1) / (double)N);
}

struct StatsShared {
  int off[kLdsBatch + 1];  // packed draft-row offsets (small batches)
  float temp[kLdsBatch];
  long long wsum[kWaves];
  float m[2][kWaves];
  int i[kWaves];
  double d[4][kWaves];
  int bad;
};

// Packed offsets of a batch of at most kLdsBatch requests, scanned in LDS:
// off[b] = sum of gamma over the requests before b.  Returns whether the layout
// is valid (every gamma >= 0, sum == total_draft_rows).  `publish`: also write
// the offsets and the layout flag for the later kernels.
__device__ bool scan_offsets_lds(const Params& p, StatsShared& sh, bool soft, bool publish) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  long long g[4], loc = 0;
  bool bad = false;
  // all loads first (clamped indices, no branches), so they are in flight together
  int gl[4];
  float tl[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int bc = min(4 * tid + k, p.B - 1);
    gl[k] = p.gamma[bc];
    tl[k] = soft ? p.temp[bc] : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int b = 4 * tid + k;
    long long v = 0;
    if (b < p.B) {
      v = gl[k];
      if (v < 0) {
        bad = true;
        v = 0;
      }
      if (soft) sh.temp[b] = tl[k];
    }
    g[k] = v;
    loc += v;
  }
  long long incl = loc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) sh.wsum[w] = incl;
  if (tid == 0) sh.bad = 0;
  __syncthreads();
  long long before = 0, total = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    if (k < w) before += sh.wsum[k];
    total += sh.wsum[k];
  }
  long long run = before + incl - loc;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int b = 4 * tid + k;
    if (b < p.B) sh.off[b] = (int)run;
    run += g[k];
  }
  if (tid == 0) {
    sh.off[p.B] = (int)total;
    if (total != (long long)p.R_d) sh.bad = 1;
  }
  if (bad) sh.bad = 1;  // benign race: every writer stores 1
  __syncthreads();
  const bool ok = sh.bad == 0;
  if (publish) {
    for (int b = tid; b <= p.B; b += kThreads) p.d_off[b] = sh.off[b];
    if (tid == 0) {
      p.hdr[0] = ok ? 0 : 1;
      p.hdr[1] = 0;  // queue of the KL second pass
    }
  }
  return ok;
}

// Request of a statistics task: the last b with key(b) <= task, where
// key(b) = d_off[b] for pair tasks (stochastic: task = draft row) and
// d_off[b] + b for row tasks (NKL: task = target row).  `hint` is the request
// of this workgroup's previous (smaller) task, or -1.
template <int MODE>
__device__ __forceinline__ int find_req(const int* off, int B, int task, int hint) {
  if (hint < 0) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      const int key = MODE == SV_MODE_STOCHASTIC ? off[mid] : off[mid] + mid;
      if (key <= task) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  }
  int b = hint;
  while (b + 1 < B && (MODE == SV_MODE_STOCHASTIC ? off[b + 1] : off[b + 1] + b + 1) <= task) ++b;
  return b;
}

// Per-lane running statistics of the segment a workgroup streams.
struct Lane {
  float mt, md;  // running maxima of the target / draft elements seen
  int idx;       // lowest position attaining mt
  double st, sd, w, z;
};

template <int NV>
struct Vecs {
  uint4 v[NV];
};

// Rows and vocabulary chunk of one item of the statistics pass.  The second
// row of a pair is read from `dbase` (the draft logits; for the bonus row of an
// NKL request the target row itself, whose pair statistics are not used).
struct Desc {
  int task, chunk;
  int64_t trow, drow;
  const void* dbase;
  float Lhi;
};

// Loads of one chunk: thread t takes 16-byte vectors k * kThreads + t.
template <int DT, bool VEC, int NV, bool PAIR>
__device__ __forceinline__ void issue_chunk(const Params& p, const Desc& d, Vecs<NV>& qt, Vecs<NV>& qd) {
  constexpr int P = Elem<DT>::P;
  const int64_t e_chunk = (int64_t)d.chunk * kThreads * NV * P;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int64_t e0 = e_chunk + ((int64_t)k * kThreads + threadIdx.x) * P;
    qt.v[k] = fetch_raw<DT, VEC>(p.target, d.trow, p.V, e0);
    if (PAIR) qd.v[k] = fetch_raw<DT, VEC>(d.dbase, d.drow, p.V, e0);
  }
}

// Folds one chunk into the lane state.  SOFT: sums of exponentials; IDX:
// argmax of the target row; WZ: the KL cross terms of the draft row; PAIR: a
// draft row is streamed beside the target row.  Target and draft sums use the
// same accumulation pattern, so identical rows give bit-identical statistics.
template <int DT, int NV, bool SOFT, bool IDX, bool WZ, bool PAIR>
__device__ __forceinline__ void fold_chunk(Lane& L, const Vecs<NV>& qt, const Vecs<NV>& qd, const Desc& d,
                                           int64_t V) {
  constexpr int P = Elem<DT>::P;
  constexpr int NE = NV * P;
  const int64_t e_chunk = (int64_t)d.chunk * kThreads * NE;
  const float Lhi = d.Lhi;
  constexpr float pad = Elem<DT>::kPad;
  const int64_t lane_base = e_chunk + (int64_t)threadIdx.x * P;
  const bool tail = e_chunk + (int64_t)kThreads * NE > V;  // uniform: the chunk runs past the row end
  float vt[NE];
#pragma unroll
  for (int k = 0; k < NV; ++k) unpack<DT>(qt.v[k], vt + k * P);
  if (tail) mask_tail<DT, NV>(vt, lane_base, (int64_t)kThreads * P, V);
  float mc = vt[0];
#pragma unroll
  for (int e = 1; e < NE; ++e) mc = fmaxf(mc, vt[e]);
  if (mc > pad) {  // the lane holds positions < V in this chunk
    if (IDX && mc > L.mt) {
      int ic = NE - 1;
#pragma unroll
      for (int e = NE - 1; e >= 0; --e)
        if (vt[e] == mc) ic = e;
      L.idx = (int)(e_chunk + ((int64_t)(ic / P) * kThreads + threadIdx.x) * P + ic % P);
    }
    if (SOFT) {
      const float M = fmaxf(L.mt, mc);
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int e = 0; e < NE; e += 4) {
        a0 += ex2(vt[e] - M, Lhi);
        a1 += ex2(vt[e + 1] - M, Lhi);
        a2 += ex2(vt[e + 2] - M, Lhi);
        a3 += ex2(vt[e + 3] - M, Lhi);
      }
      const float f = ex2(L.mt - M, Lhi);  // 0 on the first chunk (L.mt = -inf)
      L.st = L.st * (double)f + (double)((a0 + a1) + (a2 + a3));
      L.mt = M;
    } else {
      L.mt = fmaxf(L.mt, mc);
    }
  }
  if (PAIR) {
    float vd[NE];
#pragma unroll
    for (int k = 0; k < NV; ++k) unpack<DT>(qd.v[k], vd + k * P);
    if (tail) mask_tail<DT, NV>(vd, lane_base, (int64_t)kThreads * P, V);
    float md = vd[0];
#pragma unroll
    for (int e = 1; e < NE; ++e) md = fmaxf(md, vd[e]);
    if (md > pad) {
      const float M = fmaxf(L.md, md);
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f, w0 = 0.f, w1 = 0.f, z0 = 0.f, z1 = 0.f;
#pragma unroll
      for (int e = 0; e < NE; e += 4) {
        const float e0 = ex2(vd[e] - M, Lhi);
        const float e1 = ex2(vd[e + 1] - M, Lhi);
        const float e2 = ex2(vd[e + 2] - M, Lhi);
        const float e3 = ex2(vd[e + 3] - M, Lhi);
        a0 += e0;
        a1 += e1;
        a2 += e2;
        a3 += e3;
        if (WZ) {
          // positions past the end hold the pad in both rows: difference 0
          const float g0 = vd[e] - vt[e], g1 = vd[e + 1] - vt[e + 1];
          const float g2 = vd[e + 2] - vt[e + 2], g3 = vd[e + 3] - vt[e + 3];
          w0 = fmaf(e0, g0, fmaf(e1, g1, w0));
          w1 = fmaf(e2, g2, fmaf(e3, g3, w1));
          z0 = fmaf(e0, fabsf(g0), fmaf(e1, fabsf(g1), z0));
          z1 = fmaf(e2, fabsf(g2), fmaf(e3, fabsf(g3), z1));
        }
      }
      const double f = (double)ex2(L.md - M, Lhi);
      L.sd = L.sd * f + (double)((a0 + a1) + (a2 + a3));
      if (WZ) {
        L.w = L.w * f + (double)(w0 + w1);
        L.z = L.z * f + (double)(z0 + z1);
      }
      L.md = M;
    }
  }
}

// Reduces the lane states over the workgroup and writes the segment's partial
// (thread 0, plain stores: the consumer is a later kernel).
template <bool SOFT, bool IDX, bool WZ, bool PAIR>
__device__ __forceinline__ void reduce_store(const Lane& L, float Lhi, PartA* dst, StatsShared& sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float wt = wave_max(L.mt);
  const float wd = PAIR ? wave_max(L.md) : 0.f;
  if (lane == 0) {
    sh.m[0][w] = wt;
    sh.m[1][w] = wd;
  }
  __syncthreads();
  float Mt = sh.m[0][0], Md = sh.m[1][0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) {
    Mt = fmaxf(Mt, sh.m[0][k]);
    Md = fmaxf(Md, sh.m[1][k]);
  }
  int idx = INT_MAX;
  if (IDX) idx = wave_min_int(L.mt == Mt ? L.idx : INT_MAX);
  double v0 = 0.0, v1 = 0.0, v2 = 0.0, v3 = 0.0;
  if (SOFT) {
    const double ft = L.mt == Mt ? 1.0 : (double)ex2(L.mt - Mt, Lhi);
    v0 = wave_sum_d(L.st * ft);
    if (PAIR) {
      const double fd = L.md == Md ? 1.0 : (double)ex2(L.md - Md, Lhi);
      v1 = wave_sum_d(L.sd * fd);
      if (WZ) {
        v2 = wave_sum_d(L.w * fd);
        v3 = wave_sum_d(L.z * fd);
      }
    }
  }
  if (lane == 0) {
    sh.i[w] = idx;
    sh.d[0][w] = v0;
    sh.d[1][w] = v1;
    sh.d[2][w] = v2;
    sh.d[3][w] = v3;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int I = sh.i[0];
    double s0 = sh.d[0][0], s1 = sh.d[1][0], s2 = sh.d[2][0], s3 = sh.d[3][0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) {
      I = min(I, sh.i[k]);
      s0 += sh.d[0][k];
      s1 += sh.d[1][k];
      s2 += sh.d[2][k];
      s3 += sh.d[3][k];
    }
    dst->m_t = Mt;
    if (IDX) dst->idx = I;
    if (SOFT) dst->s_t = s0;
    if (PAIR) {
      dst->m_d = Md;
      dst->s_d = s1;
      if (WZ) {
        dst->w = s2;
        dst->z = s3;
      }
    }
  }
  // the next segment writes sh.m before its first barrier and sh.i / sh.d only
  // after it, by which time thread 0 has read them: no barrier needed here
}

__device__ __forceinline__ void lane_reset(Lane& L) {
  L.mt = L.md = -INFINITY;
  L.idx = INT_MAX;
  L.st = L.sd = L.w = L.z = 0.0;
}

// Rows of task d.task (request lookup for the modes whose tasks pair rows).
template <int MODE, bool LDS>
__device__ __forceinline__ void set_rows(const Params& p, const StatsShared& sh, int& b, Desc& d) {
  if (MODE == SV_MODE_GREEDY || MODE == SV_MODE_TREE_GREEDY) {
    d.trow = d.task;
    d.drow = 0;
    d.dbase = p.target;
    d.Lhi = 0.0f;
    return;
  }
  float T;
  if constexpr (LDS) {
    b = find_req<MODE>(sh.off, p.B, d.task, b);
    T = sh.temp[b];
  } else {
    b = MODE == SV_MODE_STOCHASTIC ? p.pair2req[d.task] : p.row2req[d.task];
    T = p.temp[b];
  }
  d.Lhi = (float)(kLog2eD / (double)T);
  if (MODE == SV_MODE_STOCHASTIC) {
    d.trow = (int64_t)d.task + b;
    d.drow = d.task;
    d.dbase = p.draft;
  } else {
    int d0, d1;
    if constexpr (LDS) {
      d0 = sh.off[b];
      d1 = sh.off[b + 1];
    } else {
      d0 = p.d_off[b];
      d1 = p.d_off[b + 1];
    }
    const bool pair = d.task - (d0 + b) < d1 - d0;
    d.trow = d.task;
    d.drow = pair ? (int64_t)d.task - b : d.task;
    d.dbase = pair ? p.draft : p.target;
  }
}

template <int MODE, bool LDS>
__device__ __forceinline__ void next_desc(const Params& p, const StatsShared& sh, int& b, Desc& d) {
  if (++d.chunk == p.nch) {
    d.chunk = 0;
    ++d.task;
    set_rows<MODE, LDS>(p, sh, b, d);
  }
}

// WZ (stochastic only): also the KL cross terms, for the optional NKL output.
// Each workgroup streams its item range with two register buffers in turn:
// the loads of item i + 1 (also across a task boundary) are in flight while
// item i is folded; a task segment ends with a workgroup reduction whose
// barriers wait on LDS only, so the next loads stay in flight through it.
// LDS: the batch is small enough for the offsets to be scanned in LDS.
template <int DT, bool VEC, int MODE, bool WZ, bool LDS>
__global__ __launch_bounds__(kThreads) void k_stats(Params p) {
  constexpr bool SOFT = MODE == SV_MODE_STOCHASTIC || MODE == SV_MODE_NKL;
  constexpr int NV = SOFT ? 2 : 4;
  constexpr bool IDX = MODE != SV_MODE_STOCHASTIC;
  constexpr bool WZM = MODE == SV_MODE_NKL || WZ;
  __shared__ StatsShared sh;
  const int G = (int)gridDim.x, wg = (int)blockIdx.x;
  const int64_t N = (int64_t)p.n_task * p.nch;
  if (LDS) {
    // greedy and tree tasks are target rows: only workgroup 0 needs the scan,
    // to publish the offsets for the decision kernel
    if ((SOFT || wg == 0) && !scan_offsets_lds(p, sh, SOFT, wg == 0)) return;
  } else if (SOFT && p.hdr[0] != 0) {
    return;  // the prep kernel found a layout error
  }
  const int64_t i_end = (int64_t)(wg + 1) * N / G;
  int64_t i = (int64_t)wg * N / G;
  if (i >= i_end) return;
  int b = -1;
  Desc dA, dB;
  dA.task = (int)(i / p.nch);
  dA.chunk = (int)(i - (int64_t)dA.task * p.nch);
  set_rows<MODE, LDS>(p, sh, b, dA);
  Vecs<NV> At, Ad, Bt, Bd;
  issue_chunk<DT, VEC, NV, SOFT>(p, dA, At, Ad);
  Lane L;
  lane_reset(L);
  for (;;) {
    dB = dA;
    if (i + 1 < i_end) next_desc<MODE, LDS>(p, sh, b, dB);
    issue_chunk<DT, VEC, NV, SOFT>(p, dB, Bt, Bd);  // the last item reloads itself (cache hit)
    fold_chunk<DT, NV, SOFT, IDX, WZM, SOFT>(L, At, Ad, dA, p.V);
    if (dA.chunk == p.nch - 1 || i + 1 == i_end) {
      reduce_store<SOFT, IDX, WZM, SOFT>(L, dA.Lhi, p.part_a + (int64_t)dA.task * p.nch +
                                                        (wg - wg_of((int64_t)dA.task * p.nch, N, G)), sh);
      lane_reset(L);
    }
    if (++i >= i_end) break;
    dA = dB;
    if (i + 1 < i_end) next_desc<MODE, LDS>(p, sh, b, dA);
    issue_chunk<DT, VEC, NV, SOFT>(p, dA, At, Ad);
    fold_chunk<DT, NV, SOFT, IDX, WZM, SOFT>(L, Bt, Bd, dB, p.V);
    if (dB.chunk == p.nch - 1 || i + 1 == i_end) {
      reduce_store<SOFT, IDX, WZM, SOFT>(L, dB.Lhi, p.part_a + (int64_t)dB.task * p.nch +
                                                        (wg - wg_of((int64_t)dB.task * p.nch, N, G)), sh);
      lane_reset(L);
    }
    if (++i >= i_end) break;
  }
}

// ----------------------------------------------------------------------------
// k_decide: per-request merge and decision
// ----------------------------------------------------------------------------

// One-pass KL values whose estimated error exceeds kKlRel of the value, or
// that sit within the estimate of the NKL threshold, are recomputed in a
// second pass.  The estimate is kKlErr * (E_q|d - t| / T + 1): the cross term
// carries relative errors of a few float32 roundings per element against
// sum q |d - t| / T, the log normaliser ratio a few roundings absolute.
// Measured against the float64 reference over 6000 row pairs of several
// shapes (V from 1000 to 152064, bf16 and float32, T from 0.3 to 2, draft
// noise 0.003 to 1.5), the one-pass error stayed below 1.3e-7 times this
// scale; kKlErr keeps a margin above that.
constexpr double kKlErr = 3e-7;
constexpr double kKlRel = 1e-5;

// Merged statistics of one task.
struct Merged {
  float mt, md;
  int idx;
  double st, sd, w, z;
};

__device__ __forceinline__ double rescale(float m, float M, float Lhi) {
  return m == M ? 1.0 : (double)ex2(m - M, Lhi);
}

// Merges the partials of `task` over a group of S = 2^glog lanes: lane l of
// the group takes partial slots l, l + S, ... (vocabulary order), then the
// group combines by an xor butterfly, so every lane of the group ends with the
// same values.  `pair`: the task has draft statistics.  All lanes of the
// wave must call this.
template <bool SOFT>
__device__ __forceinline__ Merged merge_task(const Params& p, int64_t task, bool has, bool pair, int l, int glog,
                                             float Lhi) {
  const int S = 1 << glog;
  Merged r;
  r.mt = r.md = -INFINITY;
  r.idx = INT_MAX;
  r.st = r.sd = r.w = r.z = 0.0;
  if (has) {
    const int64_t N = (int64_t)p.n_task * p.nch;
    const int w_lo = wg_of(task * p.nch, N, p.stats_grid);
    const int nseg = wg_of((task + 1) * p.nch - 1, N, p.stats_grid) - w_lo + 1;
    const PartA* src = p.part_a + task * p.nch;
    for (int s = l; s < nseg; s += S) {
      const float mt = src[s].m_t;
      const int ix = src[s].idx;
      if (mt > r.mt || (mt == r.mt && ix < r.idx)) r.idx = ix;
      if (SOFT && pair) {
        const float Mt = fmaxf(r.mt, mt), md = src[s].m_d, Md = fmaxf(r.md, md);
        const double fo = rescale(r.md, Md, Lhi), fn = rescale(md, Md, Lhi);
        r.st = r.st * rescale(r.mt, Mt, Lhi) + src[s].s_t * rescale(mt, Mt, Lhi);
        r.sd = r.sd * fo + src[s].s_d * fn;
        r.w = r.w * fo + src[s].w * fn;
        r.z = r.z * fo + src[s].z * fn;
        r.md = Md;
      }
      r.mt = fmaxf(r.mt, mt);
    }
  }
  float Mt = r.mt, Md = r.md;
  for (int m = 1; m < S; m <<= 1) {
    Mt = fmaxf(Mt, __shfl_xor(Mt, m, 64));
    if (SOFT) Md = fmaxf(Md, __shfl_xor(Md, m, 64));
  }
  int ix = r.mt == Mt ? r.idx : INT_MAX;
  for (int m = 1; m < S; m <<= 1) ix = min(ix, __shfl_xor(ix, m, 64));
  if (SOFT) {
    const double ft = rescale(r.mt, Mt, Lhi), fd = rescale(r.md, Md, Lhi);
    double st = r.st * ft, sd = r.sd * fd, w = r.w * fd, z = r.z * fd;
    for (int m = 1; m < S; m <<= 1) {
      st += __shfl_xor(st, m, 64);
      sd += __shfl_xor(sd, m, 64);
      w += __shfl_xor(w, m, 64);
      z += __shfl_xor(z, m, 64);
    }
    r.st = st;
    r.sd = sd;
    r.w = w;
    r.z = z;
  }
  r.mt = Mt;
  r.md = Md;
  r.idx = ix;
  return r;
}

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

// KL(q || p) of one row pair in a second pass, as the sum of the non-negative
// terms q_y g(w_y), w_y = log(p_y / q_y), over one chunk of kThreads x kUR
// vectors.  Because sum q e^w = sum p = 1, the sum over the row equals
// sum q log(q/p) exactly, has no cancellation, and an error eps in the log
// normaliser ratio only adds O(eps^2).  All threads of the workgroup call.
template <int DT, bool VEC>
__device__ double kl_chunk(const Params& p, const RefIn& ri, int64_t drow, int64_t e_chunk, double* shd) {
  constexpr int P = Elem<DT>::P;
  const int64_t V = p.V;
  const float Lhi = ri.Lhi;
  const float c = (float)((double)Lhi * kLn2D);  // d(log p)/d(logit)
  const float lr = (float)log(ri.s_d / ri.s_t);
  const float inv_sd = (float)(1.0 / ri.s_d), inv_st = (float)(1.0 / ri.s_t);
  uint4 qt[kUR], qd[kUR];
#pragma unroll
  for (int k = 0; k < kUR; ++k) {
    const int64_t e0 = e_chunk + ((int64_t)k * kThreads + threadIdx.x) * P;
    qt[k] = fetch<DT, VEC>(p.target, ri.trow, V, e0);
    qd[k] = fetch<DT, VEC>(p.draft, drow, V, e0);
  }
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < kUR; ++k) {
    float vt[P], vd[P];
    unpack<DT>(qt[k], vt);
    unpack<DT>(qd[k], vd);
    float part = 0.f;  // P non-negative terms in float32, then float64
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const float dt = vt[e] - ri.m_t, dd = vd[e] - ri.m_d;
      const float q = ex2(dd, Lhi) * inv_sd;
      const float w = fmaf(dt - dd, c, lr);
      float term;
      if (fabsf(w) < 0.5f) {
        term = q * g_small(w);
      } else {
        // q g(w) = p - q - q w; also right where q underflows but p does not
        term = (ex2(dt, Lhi) * inv_st - q) - q * w;
      }
      part += term;  // positions past the end of the row give p = q = 0
    }
    acc += (double)part;
  }
  return block_sum_d(acc, shd);
}

struct DecideShared {
  float mt[kThreads], md[kThreads];
  double st[kThreads], sd[kThreads];
  int idx[kThreads];
  int acc[kThreads];
  double kl1[kThreads];
  int need[kThreads];
  int red_i[kWaves];
  double red_d[kWaves];
};

template <int MODE>
struct TreeShared {
  int16_t info[1];
  int16_t par[1];
  int idx[1];
};
template <>
struct TreeShared<SV_MODE_TREE_GREEDY> {
  int16_t info[SV_MAX_GAMMA + 1];  // (depth << 1) | accepted
  int16_t par[SV_MAX_GAMMA + 1];
  int idx[SV_MAX_GAMMA + 1];  // argmax of each node's target row
};

__device__ void finish_invalid(const Params& p, int b, int t0, int d0, int g) {
  for (int k = threadIdx.x; k <= g; k += kThreads) p.out_tokens[t0 + k] = -1;
  for (int k = threadIdx.x; k < g; k += kThreads) {
    if (p.out_nkl) p.out_nkl[d0 + k] = __builtin_nanf("");
    if (p.out_p_x) p.out_p_x[d0 + k] = __builtin_nanf("");
    if (p.out_q_x) p.out_q_x[d0 + k] = __builtin_nanf("");
  }
  if (threadIdx.x == 0) {
    p.out_num[b] = -1;
    if (p.out_resid) p.out_resid[b] = __builtin_nanf("");
    if (p.out_tree_node) p.out_tree_node[b] = -1;
    if (p.mode == SV_MODE_STOCHASTIC) p.term[b].kind = kTermNone;
  }
}

// Tree resolve over the node argmaxes in `tr.idx`: a node is accepted when its
// token is the argmax of its parent's target row and its parent is accepted;
// the deepest accepted node (lowest id on ties) ends the path.  Parents
// precede children, so one ordered pass settles every node.
__device__ void resolve_tree(const Params& p, int b, int g, int t0, int d0, TreeShared<SV_MODE_TREE_GREEDY>& tr,
                             DecideShared& sh) {
  const int N = g + 1;
  for (int n = 1 + threadIdx.x; n < N; n += kThreads) {
    const int pa = p.parents[d0 + n - 1];
    tr.par[n] = (int16_t)pa;
    tr.info[n] = (int16_t)(p.tokens[d0 + n - 1] == tr.idx[pa] ? 1 : 0);  // edge match, before ancestry
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    tr.info[0] = 1;  // root: depth 0, accepted
    for (int n = 1; n < N; ++n) {
      const int pi = tr.info[tr.par[n]];
      tr.info[n] = (int16_t)((((pi >> 1) + 1) << 1) | (pi & tr.info[n] & 1));
    }
  }
  __syncthreads();
  int key = -1;
  for (int n = threadIdx.x; n < N; n += kThreads) {
    const int ni = tr.info[n];
    if (ni & 1) key = max(key, ((ni >> 1) << 13) | (8191 - n));
  }
  const int best_key = block_max_int(key, sh.red_i);
  const int best = 8191 - (best_key & 8191);
  const int depth = best_key >> 13;
  for (int k = depth + 1 + threadIdx.x; k <= g; k += kThreads) p.out_tokens[t0 + k] = -1;
  if (threadIdx.x == 0) {
    for (int v = best; v != 0; v = tr.par[v]) p.out_tokens[t0 + (tr.info[v] >> 1) - 1] = p.tokens[d0 + v - 1];
    p.out_tokens[t0 + depth] = tr.idx[best];
    p.out_num[b] = depth;
    if (p.out_tree_node) p.out_tree_node[b] = best;
  }
}

template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void k_decide(Params p) {
  constexpr bool SOFT = MODE == SV_MODE_STOCHASTIC || MODE == SV_MODE_NKL;
  __shared__ DecideShared sh;
  __shared__ TreeShared<MODE> tr;
  const int b = blockIdx.x, tid = threadIdx.x;
  const bool want_kl = SOFT && p.want_kl;
  if (want_kl && tid == 0) p.pending[b] = 0;
  // independent loads first, so that they are in flight together
  const int hdr = p.hdr[0];
  const int d0 = p.d_off[b];
  const int d1 = p.d_off[b + 1];
  const float T = SOFT ? p.temp[b] : 1.0f;
  const float ur = MODE == SV_MODE_STOCHASTIC ? p.ur[b] : 0.0f;
  if (hdr != 0) {  // layout error: only the counts are written
    if (tid == 0) {
      p.out_num[b] = -1;
      if (MODE == SV_MODE_STOCHASTIC) p.term[b].kind = kTermNone;
    }
    return;
  }
  const int g = d1 - d0;
  const int t0 = d0 + b;
  const int64_t V = p.V;
  const float Lhi = SOFT ? (float)(kLog2eD / (double)T) : 0.0f;
  // request-level checks; the per-position ones follow the decision passes
  // (which only read inside the rows for valid token ids), and overwrite
  // everything the passes wrote if they fail
  if (g > p.max_gamma || (SOFT && !temp_ok(T)) || (MODE == SV_MODE_STOCHASTIC && !unit_ok(ur))) {
    finish_invalid(p, b, t0, d0, g);
    return;
  }

  const int glog = p.grp_log2, S = 1 << glog, TPP = kThreads >> glog;
  const int ntask = MODE == SV_MODE_STOCHASTIC ? g : g + 1;
  const int64_t tbase = MODE == SV_MODE_STOCHASTIC ? d0 : t0;
  const bool diag = SOFT && (p.out_p_x || p.out_q_x || p.out_nkl);
  const double c = (double)Lhi * kLn2D;  // d(log p)/d(logit)
  const double lnV = log((double)p.V);
  int j = -1;
  float jm_t = 0.f, jm_d = 0.f;
  double js_t = 1.0, js_d = 1.0;
  int jidx = 0;
  bool any_need = false, bad = false;
  int checked = 0;  // positions [0, checked) were checked inside the passes
  for (int base = 0; base < ntask; base += TPP) {
    const int q = tid >> glog, l = tid & (S - 1);
    const int ti = base + q;
    const bool has = ti < ntask;
    const bool pair = SOFT && ti < g;
    // the group leader's position data, issued before the partial loads
    // and the per-position input checks (node ti of a tree is position ti - 1)
    int x = -1;
    float tx = 0.f, dx = 0.f, u = 0.f;
    if (l == 0 && MODE != SV_MODE_TREE_GREEDY && ti < g) {
      x = p.tokens[d0 + ti];
      const bool xok = x >= 0 && x < p.V;
      if (SOFT && xok) {
        tx = load_scalar<DT>(p.target, t0 + ti, V, x);
        dx = load_scalar<DT>(p.draft, d0 + ti, V, x);
      }
      if (MODE == SV_MODE_STOCHASTIC) {
        u = p.ua[d0 + ti];
        if (!unit_ok(u)) bad = true;
      }
      if (!xok) bad = true;
    }
    if (l == 0 && MODE == SV_MODE_TREE_GREEDY && ti >= 1 && ti <= g) {
      const int xn = p.tokens[d0 + ti - 1], pa = p.parents[d0 + ti - 1];
      if (xn < 0 || xn >= p.V || pa < 0 || pa >= ti) bad = true;
    }
    const Merged r = merge_task<SOFT>(p, tbase + ti, has, pair, l, glog, Lhi);
    if (l == 0 && has) {
      const int idx = r.idx == INT_MAX ? 0 : r.idx;  // no element above the pad value: position 0
      if constexpr (MODE == SV_MODE_TREE_GREEDY) tr.idx[ti] = idx;
      sh.mt[q] = r.mt;
      sh.md[q] = r.md;
      sh.st[q] = r.st;
      sh.sd[q] = r.sd;
      sh.idx[q] = idx;
      if (MODE == SV_MODE_NKL) p.tidx[t0 + ti] = idx;
      int acc = 0, need = 0;
      double kl = 0.0;  // KL(q||p) = 0 for V == 1: both rows are the same point mass
      if (pair) {
        // log2 p(x) and log2 q(x) from the merged statistics (float32: the
        // relative error of p(x), q(x) and alpha stays near 1e-7)
        const float lpx = (tx - r.mt) * Lhi - __log2f((float)r.st);
        const float lqx = (dx - r.md) * Lhi - __log2f((float)r.sd);
        if (p.out_p_x) p.out_p_x[d0 + ti] = exp2f(lpx);
        if (p.out_q_x) p.out_q_x[d0 + ti] = exp2f(lqx);
        if (MODE == SV_MODE_STOCHASTIC) acc = u <= fminf(1.0f, exp2f(lpx - lqx)) ? 1 : 0;
        if (want_kl && p.V > 1) {
          // KL(q||p) = E_q[d - t]/T - (m_d - m_t)/T - log(s_d / s_t)
          const double lg = log(r.sd / r.st);
          const double klv = r.w / r.sd * c - (double)(r.md - r.mt) * c - lg;
          const double err = kKlErr * (r.z / r.sd * c + 1.0);
          need = (err > kKlRel * klv) ? 1 : 0;
          if (MODE == SV_MODE_NKL && fabs(klv - (double)p.delta * lnV) <= err) need = 1;
          kl = klv;
        }
      } else if (MODE == SV_MODE_GREEDY) {
        acc = (ti < g && x == idx) ? 1 : 0;
      }
      sh.acc[q] = acc;
      sh.kl1[q] = kl;
      sh.need[q] = need;
    }
    __syncthreads();
    if (want_kl && tid < TPP && base + tid < g) {
      // positions whose one-pass KL is not accurate enough are queued for the
      // grid-wide second pass; the request then waits for k_finish
      const int pos = d0 + base + tid;
      const int need = sh.need[tid];
      p.kl_need[pos] = need;
      p.kl_val[pos] = sh.kl1[tid];
      if (need) {
        RefIn ri;
        ri.s_t = sh.st[tid];
        ri.s_d = sh.sd[tid];
        ri.m_t = sh.mt[tid];
        ri.m_d = sh.md[tid];
        ri.Lhi = Lhi;
        ri.trow = t0 + base + tid;
        p.ref_in[pos] = ri;
        p.ref_list[atomicAdd(p.hdr + 1, 1)] = pos;
        any_need = true;
        if (MODE == SV_MODE_NKL) sh.acc[tid] = 0;
      } else {
        const double nkl = p.V > 1 ? sh.kl1[tid] / lnV : 0.0;
        if (p.out_nkl) p.out_nkl[pos] = (float)nkl;
        if (MODE == SV_MODE_NKL) sh.acc[tid] = nkl < (double)p.delta ? 1 : 0;
      }
    }
    if (want_kl) __syncthreads();
    if (MODE != SV_MODE_TREE_GREEDY) {
      const int cand = (tid < TPP && base + tid < ntask && !sh.acc[tid]) ? base + tid : INT_MAX;
      const int jp = block_min_int(cand, sh.red_i);
      if (j < 0 && jp != INT_MAX) {
        j = jp;
        const int s = jp - base;
        jm_t = sh.mt[s];
        jm_d = sh.md[s];
        js_t = sh.st[s];
        js_d = sh.sd[s];
        jidx = sh.idx[s];
      }
      if (j >= 0 && !diag) {
        checked = min(g, base + TPP);
        break;
      }
    }
    checked = min(g, base + TPP);
    __syncthreads();  // LDS of this pass is reused by the next
  }

  // positions the passes did not reach (an early exit) are checked here
  for (int k = checked + tid; k < g; k += kThreads) {
    const int x = p.tokens[d0 + k];
    bool ok = x >= 0 && x < p.V;
    if (MODE == SV_MODE_STOCHASTIC) ok = ok && unit_ok(p.ua[d0 + k]);
    if (MODE == SV_MODE_TREE_GREEDY) {
      const int pa = p.parents[d0 + k];  // parent of node k + 1
      ok = ok && pa >= 0 && pa <= k;
    }
    if (!ok) bad = true;
  }
  if (__syncthreads_or(bad)) {
    finish_invalid(p, b, t0, d0, g);
    return;
  }
  if constexpr (MODE == SV_MODE_TREE_GREEDY) {
    resolve_tree(p, b, g, t0, d0, tr, sh);
    return;
  }
  if (want_kl && __syncthreads_or(any_need)) {
    if (tid == 0) p.pending[b] = 1;
    if (MODE == SV_MODE_NKL) return;  // the decision needs the second-pass values: k_finish
  }
  if (j < 0) j = g;  // stochastic: every draft accepted
  for (int k = tid; k <= g; k += kThreads) {
    if (k < j) p.out_tokens[t0 + k] = p.tokens[d0 + k];
    else if (k > j) p.out_tokens[t0 + k] = -1;
    else if (MODE != SV_MODE_STOCHASTIC) p.out_tokens[t0 + k] = jidx;  // stochastic: the draw pass writes it
  }
  if (tid == 0) {
    p.out_num[b] = j;
    if (MODE == SV_MODE_STOCHASTIC) {
      Term tm;
      tm.j = j;
      tm.trow = t0 + j;
      tm.Lhi = Lhi;
      if (j < g) {
        tm.kind = kTermResidual;
        tm.drow = d0 + j;
        tm.m_t = jm_t;
        tm.m_d = jm_d;
        tm.k0 = (float)(js_t / js_d);
      } else {
        tm.kind = kTermBonus;
        tm.drow = -1;
        tm.m_t = tm.m_d = tm.k0 = 0.0f;
      }
      p.term[b] = tm;
    }
  }
}

// ----------------------------------------------------------------------------
// k_refine and k_finish (when KL values are computed)
//
// k_refine: the queued positions x chunks are split into contiguous ranges,
// one per workgroup; every (position, chunk) sum is written to its own slot,
// so the values do not depend on the queue order.  k_finish: one workgroup
// per request that waits for second-pass values adds the chunk sums in chunk
// order, writes the NKL values and, in NKL mode, the decision.
// ----------------------------------------------------------------------------

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_refine(Params p) {
  __shared__ double shd[kWaves];
  constexpr int64_t CHR = (int64_t)kThreads * kUR * Elem<DT>::P;
  const int64_t N = (int64_t)p.hdr[1] * p.nch_r;
  const int G = (int)gridDim.x, wg = (int)blockIdx.x;
  const int64_t i_end = (int64_t)(wg + 1) * N / G;
  for (int64_t i = (int64_t)wg * N / G; i < i_end; ++i) {
    const int k = (int)(i / p.nch_r);
    const int c = (int)(i - (int64_t)k * p.nch_r);
    const int pos = p.ref_list[k];
    const RefIn ri = p.ref_in[pos];
    const double v = kl_chunk<DT, VEC>(p, ri, pos, (int64_t)c * CHR, shd);
    if (threadIdx.x == 0) p.kl_part[(int64_t)pos * p.nch_r + c] = v;
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void k_finish(Params p) {
  __shared__ int red[kWaves];
  const int b = blockIdx.x, tid = threadIdx.x;
  if (!p.pending[b]) return;
  const int d0 = p.d_off[b];
  const int g = p.d_off[b + 1] - d0;
  const int t0 = d0 + b;
  const double lnV = log((double)p.V);
  int first = INT_MAX;
  for (int i = tid; i < g; i += kThreads) {
    const int pos = d0 + i;
    double kl = p.kl_val[pos];
    if (p.kl_need[pos]) {
      kl = 0.0;
      for (int c = 0; c < p.nch_r; ++c) kl += p.kl_part[(int64_t)pos * p.nch_r + c];
    }
    const double nkl = p.V > 1 ? kl / lnV : 0.0;
    p.out_nkl[pos] = (float)nkl;
    if (!(nkl < (double)p.delta)) first = min(first, i);
  }
  if (MODE == SV_MODE_NKL) {
    const int j0 = block_min_int(first, red);
    const int j = j0 == INT_MAX ? g : j0;
    for (int k = tid; k <= g; k += kThreads)
      p.out_tokens[t0 + k] = k < j ? p.tokens[d0 + k] : (k == j ? p.tidx[t0 + j] : -1);
    if (tid == 0) p.out_num[b] = j;
  }
}

// ----------------------------------------------------------------------------
// k_draw and k_select (stochastic mode)
//
// k_draw: items are (request, wave-chunk) pairs numbered b * nch_c + c; a
// wave-chunk is 64 lanes x kUC 16-byte vectors of the terminal row (and of the
// draft row for a residual).  Every wave of the grid streams a contiguous
// range of items on its own, without workgroup barriers, and writes one record
// of float64 sums per item.  k_select: one wave per request combines the
// records, picks the wave-chunk holding the draw and re-reads it.
// ----------------------------------------------------------------------------

__device__ __forceinline__ double wave_incl_scan_d(double v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Record of one wave-chunk: a_y = 2^((t_y - m_t) L) and b_y = 2^((d_y - m_d) L)
// are p_y and q_y up to the factors s_t, s_d; the residual record also holds
// the sums over {y : a_y > k0 b_y}, the support of max(0, p - q).  A bonus
// record holds the chunk maximum and sum_y 2^((t_y - m_c) L).
template <int DT, bool RESID>
__device__ __forceinline__ void draw_record(const Vecs<kUC>& qt, const Vecs<kUC>& qd, const Term& tm, float Lhi,
                                            PartC* dst) {
  constexpr int P = Elem<DT>::P;
  double A = 0.0, Bs = 0.0, Ap = 0.0, Bp = 0.0;
  float mc = 0.f;
  if (RESID) {
#pragma unroll
    for (int k = 0; k < kUC; ++k) {
      float vt[P], vd[P];
      unpack<DT>(qt.v[k], vt);
      unpack<DT>(qd.v[k], vd);
      float sa = 0.f, sb = 0.f, sap = 0.f, sbp = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const float a = ex2(vt[e] - tm.m_t, Lhi);
        const float bb = ex2(vd[e] - tm.m_d, Lhi);
        sa += a;
        sb += bb;
        const bool in = a > tm.k0 * bb;
        sap += in ? a : 0.f;
        sbp += in ? bb : 0.f;
      }
      A += (double)sa;
      Bs += (double)sb;
      Ap += (double)sap;
      Bp += (double)sbp;
    }
    A = wave_sum_d(A);
    Bs = wave_sum_d(Bs);
    Ap = wave_sum_d(Ap);
    Bp = wave_sum_d(Bp);
  } else {
    float vt[kUC * P];
#pragma unroll
    for (int k = 0; k < kUC; ++k) unpack<DT>(qt.v[k], vt + k * P);
    float m = vt[0];
#pragma unroll
    for (int e = 1; e < kUC * P; ++e) m = fmaxf(m, vt[e]);
    mc = wave_max(m);  // a wave-chunk starts inside the row: mc is a logit
#pragma unroll
    for (int k = 0; k < kUC; ++k) {
      float sa = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) sa += ex2(vt[k * P + e] - mc, Lhi);
      A += (double)sa;
    }
    A = wave_sum_d(A);
  }
  if ((threadIdx.x & 63) == 0) {  // plain stores: the reader is the next kernel
    dst->a = A;
    dst->b = Bs;
    dst->ap = Ap;
    dst->bp = Bp;
    dst->m = mc;
  }
}

template <int DT, bool VEC, bool RESID>
__device__ __forceinline__ void draw_issue(const Params& p, const Term& tm, int64_t e_chunk, Vecs<kUC>& qt,
                                           Vecs<kUC>& qd) {
  constexpr int P = Elem<DT>::P;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < kUC; ++k) {
    const int64_t e0 = e_chunk + ((int64_t)k * 64 + lane) * P;
    qt.v[k] = fetch<DT, VEC>(p.target, tm.trow, p.V, e0);
    if (RESID) qd.v[k] = fetch<DT, VEC>(p.draft, tm.drow, p.V, e0);
  }
}

// Streams wave-chunks [c0, c1) of request b (loads of chunk c + 1 in flight
// while chunk c is reduced).
template <int DT, bool VEC, bool RESID>
__device__ __forceinline__ void draw_segment(const Params& p, int b, const Term& tm, int c0, int c1, float Lhi) {
  constexpr int64_t CHW = (int64_t)64 * kUC * Elem<DT>::P;
  PartC* rec = p.part_c + (int64_t)b * p.nch_c;
  Vecs<kUC> ct, cd;
  draw_issue<DT, VEC, RESID>(p, tm, (int64_t)c0 * CHW, ct, cd);
  for (int c = c0; c < c1 - 1; ++c) {
    Vecs<kUC> nt, nd;
    draw_issue<DT, VEC, RESID>(p, tm, (int64_t)(c + 1) * CHW, nt, nd);
    draw_record<DT, RESID>(ct, cd, tm, Lhi, rec + c);
    ct = nt;
    cd = nd;
  }
  draw_record<DT, RESID>(ct, cd, tm, Lhi, rec + (c1 - 1));
}

// Residual chunk weight sum_{a > k0 b} (a - K b) = A+ - K B+, K = A/B, i.e.
// max(0, p - q) in units of 1/A; `fb`: the fallback draw from p_j; bonus:
// sum_y 2^((t_y - M) L) with M the row maximum.
__device__ __forceinline__ double chunk_weight(double a, double ap, double bp, float m, bool resid, bool fb, double K,
                                               float M, double Ld) {
  if (resid) return fb ? a : ap - K * bp;
  return a * exp2(((double)m - (double)M) * Ld);
}

// Residual weight of one token (units of 1/A), or its bonus / fallback weight.
__device__ __forceinline__ double token_weight(float t, float d, bool two, const Term& tm, float ref, float Lhi,
                                               double K, double cf) {
  const float a = ex2(t - ref, Lhi);
  if (two) {
    const float bb = ex2(d - tm.m_d, Lhi);
    return (a > tm.k0 * bb) ? (double)a - K * (double)bb : 0.0;
  }
  return (double)a * cf;
}

// Token draw of request b by one wave.  CACHED: the request has at most 256
// records; their fields are kept in registers (4 per lane) instead of being
// read again for each sweep.  Records are combined by fixed wave-wide
// reductions and scans in chunk order.
template <int DT, bool VEC, bool CACHED>
__device__ __forceinline__ void draw_select(const Params& p, int b, const Term& tm, float Lhi) {
  constexpr int P = Elem<DT>::P;
  constexpr int NE = kUC * P;
  constexpr int64_t CHW = (int64_t)64 * NE;
  constexpr int R = CACHED ? 4 : 1;
  const int lane = threadIdx.x & 63;
  const int nch = p.nch_c;
  PartC* pcs = p.part_c + (int64_t)b * nch;
  const bool resid = tm.kind == kTermResidual;
  const double Ld = (double)Lhi;
  double ca[R], cap[R], cbp[R];
  float cm[R];
  double at = 0.0, bt = 0.0;
  float M = -INFINITY;
  if constexpr (CACHED) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int ch = lane + 64 * r;
      ca[r] = cap[r] = cbp[r] = 0.0;
      cm[r] = -INFINITY;
      if (ch < nch) {
        const PartC q = pcs[ch];
        ca[r] = q.a;
        cap[r] = q.ap;
        cbp[r] = q.bp;
        cm[r] = q.m;
        at += q.a;
        bt += q.b;
        M = fmaxf(M, q.m);
      }
    }
  } else {
    for (int ch = lane; ch < nch; ch += 64) {
      const PartC q = pcs[ch];
      at += q.a;
      bt += q.b;
      M = fmaxf(M, q.m);
    }
  }
  at = wave_sum_d(at);
  bt = wave_sum_d(bt);
  M = wave_max(M);
  const double K = resid ? at / bt : 0.0;
  double S = 0.0;
  if constexpr (CACHED) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (lane + 64 * r < nch) S += chunk_weight(ca[r], cap[r], cbp[r], cm[r], resid, false, K, M, Ld);
  } else {
    for (int ch = lane; ch < nch; ch += 64) {
      const PartC q = pcs[ch];
      S += chunk_weight(q.a, q.ap, q.bp, q.m, resid, false, K, M, Ld);
    }
  }
  S = wave_sum_d(S);
  bool fb = false;
  if (resid && !(S > 0.0)) {
    // max(0, p - q) vanished numerically: draw from p_j instead
    fb = true;
    S = at;
  }
  const double target = (double)p.ur[b] * S;

  // the wave-chunk whose cumulative weight first exceeds the target: one
  // round per 64 consecutive chunks
  int cstar = -1, clast = -1;
  double cbase = 0.0, carry = 0.0;
  const int rounds = (nch + 63) / 64;
  for (int r = 0; r < rounds; ++r) {
    const int ch = lane + 64 * r;
    double w = 0.0;
    if (ch < nch) {
      if constexpr (CACHED) {
        // r < R here; select the round's register without dynamic indexing
        double a = ca[0], ap = cap[0], bp = cbp[0];
        float m = cm[0];
#pragma unroll
        for (int k = 1; k < R; ++k)
          if (r == k) {
            a = ca[k];
            ap = cap[k];
            bp = cbp[k];
            m = cm[k];
          }
        w = chunk_weight(a, ap, bp, m, resid, fb, K, M, Ld);
      } else {
        const PartC q = pcs[ch];
        w = chunk_weight(q.a, q.ap, q.bp, q.m, resid, fb, K, M, Ld);
      }
    }
    const double incl = wave_incl_scan_d(w);
    const double excl = carry + incl - w;
    const bool hit = w > 0.0 && excl <= target && target < excl + w;
    const int first = wave_min_int(hit ? ch : INT_MAX);
    const int lp = wave_max_int(w > 0.0 ? ch : -1);
    if (lp >= 0) clast = lp;
    if (first != INT_MAX) {
      cstar = first;
      cbase = __shfl(excl, first - 64 * r, 64);
      break;
    }
    carry += __shfl(incl, 63, 64);
  }
  const bool take_last = cstar < 0;  // rounding left the target at the end
  if (take_last) {
    cstar = clast >= 0 ? clast : nch - 1;
    cbase = 0.0;
  }

  // re-read wave-chunk c*: lane l owns NE consecutive tokens
  const int64_t V = p.V;
  const int64_t y0 = (int64_t)cstar * CHW + (int64_t)lane * NE;
  const bool two = resid && !fb;
  const float ref = resid ? tm.m_t : pcs[cstar].m;
  const double cf = resid ? 1.0 : exp2(((double)ref - (double)M) * Ld);
  Vecs<kUC> qt, qd;
#pragma unroll
  for (int k = 0; k < kUC; ++k) {
    qt.v[k] = fetch<DT, VEC>(p.target, tm.trow, V, y0 + k * P);
    qd.v[k] = two ? fetch<DT, VEC>(p.draft, tm.drow, V, y0 + k * P) : qt.v[k];
  }
  // positions past the end hold the pad: a = 0 there, so their weight is 0
  double tsum = 0.0;
#pragma unroll
  for (int k = 0; k < kUC; ++k) {
    float vt[P], vd[P];
    unpack<DT>(qt.v[k], vt);
    unpack<DT>(qd.v[k], vd);
#pragma unroll
    for (int e = 0; e < P; ++e) tsum += token_weight(vt[e], vd[e], two, tm, ref, Lhi, K, cf);
  }
  double cum = cbase + (wave_incl_scan_d(tsum) - tsum);
  const bool mine = !take_last && cum <= target && cum + tsum > target;
  int cand = INT_MAX, lastpos = -1;
#pragma unroll
  for (int k = 0; k < kUC; ++k) {
    float vt[P], vd[P];
    unpack<DT>(qt.v[k], vt);
    unpack<DT>(qd.v[k], vd);
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const double rv = token_weight(vt[e], vd[e], two, tm, ref, Lhi, K, cf);
      const int y = (int)(y0 + k * P + e);
      if (rv > 0.0) lastpos = y;
      if (mine && cand == INT_MAX) {
        cum += rv;
        if (cum > target) cand = y;
      }
    }
  }
  const int ystar = wave_min_int(cand);
  const int ylast = wave_max_int(lastpos);
  if (lane == 0) {
    int y = ystar != INT_MAX ? ystar : ylast;
    if (y < 0 || y >= p.V) y = (int)min(V - 1, (int64_t)cstar * CHW);
    p.out_tokens[tm.trow] = y;
    if (p.out_resid) p.out_resid[b] = two ? (float)(S / at) : 1.0f;
  }
}

// A layout error leaves every Term at kTermNone: nothing to draw.
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_draw(Params p) {
  const int W = (int)gridDim.x * kWaves;
  const int wave = (int)blockIdx.x * kWaves + (int)(threadIdx.x >> 6);
  const int64_t N = (int64_t)p.B * p.nch_c;
  int64_t i = (int64_t)wave * N / W;
  const int64_t i_end = (int64_t)(wave + 1) * N / W;
  while (i < i_end) {
    const int b = (int)(i / p.nch_c);
    const int c0 = (int)(i - (int64_t)b * p.nch_c);
    const int c1 = (int)min((int64_t)p.nch_c, c0 + (i_end - i));
    i += c1 - c0;
    const Term tm = p.term[b];
    if (tm.kind == kTermResidual) draw_segment<DT, VEC, true>(p, b, tm, c0, c1, tm.Lhi);
    else if (tm.kind == kTermBonus) draw_segment<DT, VEC, false>(p, b, tm, c0, c1, tm.Lhi);
  }
}

// one wave (workgroup of 64) per request
template <int DT, bool VEC>
__global__ __launch_bounds__(64) void k_select(Params p) {
  const int b = blockIdx.x;
  const Term tm = p.term[b];
  if (tm.kind == kTermNone) return;
  if (p.nch_c <= 256) draw_select<DT, VEC, true>(p, b, tm, tm.Lhi);
  else draw_select<DT, VEC, false>(p, b, tm, tm.Lhi);
}

}  // namespace

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------

int launch_prep(const Params& p, void* stream) {
  hipLaunchKernelGGL(k_prep, dim3(1), dim3(kPrepThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

namespace {

int num_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const int slot = dev >= 0 && dev < 64 ? dev : 0;
  if (cache[slot] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 1;
    cache[slot] = n;
  }
  return cache[slot];
}

template <int DT, bool VEC, int MODE, bool WZ>
int stats_occupancy() {
  static int occ = 0;  // same value from every thread: a race is benign
  if (occ == 0) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, k_stats<DT, VEC, MODE, WZ, true>, kThreads, 0) !=
            hipSuccess ||
        o <= 0)
      o = 1;
    occ = o;
  }
  return occ;
}

template <int DT, bool VEC>
int draw_occupancy() {
  static int occ = 0;
  if (occ == 0) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, k_draw<DT, VEC>, kThreads, 0) != hipSuccess || o <= 0) o = 1;
    occ = o;
  }
  return occ;
}

template <int DT, bool VEC>
int stats_occupancy_mode(int mode, bool wz) {
  switch (mode) {
    case SV_MODE_STOCHASTIC:
      return wz ? stats_occupancy<DT, VEC, SV_MODE_STOCHASTIC, true>()
                : stats_occupancy<DT, VEC, SV_MODE_STOCHASTIC, false>();
    case SV_MODE_GREEDY: return stats_occupancy<DT, VEC, SV_MODE_GREEDY, false>();
    case SV_MODE_NKL: return stats_occupancy<DT, VEC, SV_MODE_NKL, false>();
    default: return stats_occupancy<DT, VEC, SV_MODE_TREE_GREEDY, false>();
  }
}

// With events, the dispatch itself stamps them (kernel start and end), so the
// timing excludes the queueing around the launch.
template <typename K>
void launch_timed(K kernel, dim3 grid, const Params& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (e0 && e1) hipExtLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, s, e0, e1, 0, p);
  else hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, s, p);
}
template <int DT, bool VEC, int MODE, bool WZ>
void stats_launch(const Params& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (p.B <= kLdsBatch) launch_timed(k_stats<DT, VEC, MODE, WZ, true>, dim3(p.stats_grid), p, s, e0, e1);
  else launch_timed(k_stats<DT, VEC, MODE, WZ, false>, dim3(p.stats_grid), p, s, e0, e1);
}
template <int DT, bool VEC>
void stats_dispatch(const Params& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (p.mode) {
    case SV_MODE_STOCHASTIC:
      if (p.want_kl) stats_launch<DT, VEC, SV_MODE_STOCHASTIC, true>(p, s, e0, e1);
      else stats_launch<DT, VEC, SV_MODE_STOCHASTIC, false>(p, s, e0, e1);
      break;
    case SV_MODE_GREEDY: stats_launch<DT, VEC, SV_MODE_GREEDY, false>(p, s, e0, e1); break;
    case SV_MODE_NKL: stats_launch<DT, VEC, SV_MODE_NKL, false>(p, s, e0, e1); break;
    default: stats_launch<DT, VEC, SV_MODE_TREE_GREEDY, false>(p, s, e0, e1); break;
  }
}
template <int DT, bool VEC>
void decide_dispatch(const Params& p, hipStream_t s) {
  const dim3 grid(p.B), blk(kThreads);
  switch (p.mode) {
    case SV_MODE_STOCHASTIC: hipLaunchKernelGGL((k_decide<DT, VEC, SV_MODE_STOCHASTIC>), grid, blk, 0, s, p); break;
    case SV_MODE_GREEDY: hipLaunchKernelGGL((k_decide<DT, VEC, SV_MODE_GREEDY>), grid, blk, 0, s, p); break;
    case SV_MODE_NKL: hipLaunchKernelGGL((k_decide<DT, VEC, SV_MODE_NKL>), grid, blk, 0, s, p); break;
    default: hipLaunchKernelGGL((k_decide<DT, VEC, SV_MODE_TREE_GREEDY>), grid, blk, 0, s, p); break;
  }
}

}  // namespace

int plan_stats(Params& p, bool vec) {
  int occ;
  const bool wz = p.want_kl != 0;
  if (p.dtype == SV_DTYPE_BF16)
    occ = vec ? stats_occupancy_mode<SV_DTYPE_BF16, true>(p.mode, wz)
              : stats_occupancy_mode<SV_DTYPE_BF16, false>(p.mode, wz);
  else
    occ = vec ? stats_occupancy_mode<SV_DTYPE_F32, true>(p.mode, wz)
              : stats_occupancy_mode<SV_DTYPE_F32, false>(p.mode, wz);
  const int64_t N = (int64_t)p.n_task * p.nch;
  int64_t G = (int64_t)occ * num_cus();
  if (G > N) G = N;  // every workgroup gets at least one item
  if (G < 1) G = 1;
  p.stats_grid = (int32_t)G;
  // a task's chunks are spread over at most this many workgroups
  int64_t maxseg = 1;
  if (N > 0) {
    const int64_t ipw = N / G;
    maxseg = 1 + (p.nch - 1 + ipw - 1) / ipw;
    if (maxseg > p.nch) maxseg = p.nch;
  }
  int glog = 0;
  while ((1 << glog) < maxseg && glog < 6) ++glog;
  p.grp_log2 = glog;
  return 0;
}

int launch_stats(const Params& p, bool vec, void* stream, void* ev_start, void* ev_stop) {
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0 = (hipEvent_t)ev_start, e1 = (hipEvent_t)ev_stop;
  if (p.dtype == SV_DTYPE_BF16) {
    if (vec) stats_dispatch<SV_DTYPE_BF16, true>(p, s, e0, e1);
    else stats_dispatch<SV_DTYPE_BF16, false>(p, s, e0, e1);
  } else {
    if (vec) stats_dispatch<SV_DTYPE_F32, true>(p, s, e0, e1);
    else stats_dispatch<SV_DTYPE_F32, false>(p, s, e0, e1);
  }
  return (int)hipGetLastError();
}

int launch_decide(const Params& p, bool vec, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (p.dtype == SV_DTYPE_BF16) {
    if (vec) decide_dispatch<SV_DTYPE_BF16, true>(p, s);
    else decide_dispatch<SV_DTYPE_BF16, false>(p, s);
  } else {
    if (vec) decide_dispatch<SV_DTYPE_F32, true>(p, s);
    else decide_dispatch<SV_DTYPE_F32, false>(p, s);
  }
  return (int)hipGetLastError();
}

int launch_refine(const Params& p, bool vec, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  // the queue length is only known on the device: one wave of workgroups
  const dim3 grid((unsigned)(4 * num_cus())), blk(kThreads), fgrid(p.B);
  if (p.dtype == SV_DTYPE_BF16) {
    if (vec) hipLaunchKernelGGL((k_refine<SV_DTYPE_BF16, true>), grid, blk, 0, s, p);
    else hipLaunchKernelGGL((k_refine<SV_DTYPE_BF16, false>), grid, blk, 0, s, p);
  } else {
    if (vec) hipLaunchKernelGGL((k_refine<SV_DTYPE_F32, true>), grid, blk, 0, s, p);
    else hipLaunchKernelGGL((k_refine<SV_DTYPE_F32, false>), grid, blk, 0, s, p);
  }
  if (p.mode == SV_MODE_NKL) hipLaunchKernelGGL((k_finish<SV_MODE_NKL>), fgrid, blk, 0, s, p);
  else hipLaunchKernelGGL((k_finish<SV_MODE_STOCHASTIC>), fgrid, blk, 0, s, p);
  return (int)hipGetLastError();
}

int launch_draw(const Params& p, bool vec, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  int occ;
  if (p.dtype == SV_DTYPE_BF16) occ = vec ? draw_occupancy<SV_DTYPE_BF16, true>() : draw_occupancy<SV_DTYPE_BF16, false>();
  else occ = vec ? draw_occupancy<SV_DTYPE_F32, true>() : draw_occupancy<SV_DTYPE_F32, false>();
  // every wave streams a contiguous range of (request, wave-chunk) items
  const int64_t N = (int64_t)p.B * p.nch_c;
  int64_t G = (int64_t)occ * num_cus();
  if (G > (N + kWaves - 1) / kWaves) G = (N + kWaves - 1) / kWaves;
  if (G < 1) G = 1;
  const dim3 grid((unsigned)G), blk(kThreads);
  const dim3 sgrid(p.B), sblk(64);
  if (p.dtype == SV_DTYPE_BF16) {
    if (vec) hipLaunchKernelGGL((k_draw<SV_DTYPE_BF16, true>), grid, blk, 0, s, p);
    else hipLaunchKernelGGL((k_draw<SV_DTYPE_BF16, false>), grid, blk, 0, s, p);
    if (vec) hipLaunchKernelGGL((k_select<SV_DTYPE_BF16, true>), sgrid, sblk, 0, s, p);
    else hipLaunchKernelGGL((k_select<SV_DTYPE_BF16, false>), sgrid, sblk, 0, s, p);
  } else {
    if (vec) hipLaunchKernelGGL((k_draw<SV_DTYPE_F32, true>), grid, blk, 0, s, p);
    else hipLaunchKernelGGL((k_draw<SV_DTYPE_F32, false>), grid, blk, 0, s, p);
    if (vec) hipLaunchKernelGGL((k_select<SV_DTYPE_F32, true>), sgrid, sblk, 0, s, p);
    else hipLaunchKernelGGL((k_select<SV_DTYPE_F32, false>), sgrid, sblk, 0, s, p);
  }
  return (int)hipGetLastError();
}

}  // namespace sv
