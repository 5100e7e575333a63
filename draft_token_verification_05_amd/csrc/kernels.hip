// gfx950 kernels of the speculative-decoding verify step.
//
// Launches per call (all on the caller's stream).  A batch of at most
// kLdsBatch requests with a short statistics pass and no KL output (any mode
// but NKL; tree and block requests of at most kFusedNodes - 1 positions) runs
// as ONE dispatch, k_fused: its workgroups stream the statistics pass exactly
// as k_stats does (partials tagged with the call's epoch), then take the
// helper roles of k_decide, each waiting (bounded) for its request's partials
// instead of a kernel boundary.  Every other call:
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
//   k_decide    H workgroups ("helpers") per request, H = 1 in greedy and tree
//               modes and one per vocabulary slice of kThreads x kUT vectors
//               in stochastic and NKL modes.  Every helper merges the
//               partials of the request's tasks and takes the same decision
//               (alpha = min(1, p/q) against u, argmax match, NKL < delta,
//               tree paths); helper 0 writes tokens, counts and diagnostics.
//               Helper h then streams slice h of the rows that need a second
//               look: the terminal row(s) of a stochastic request (float64
//               sums of the residual max(0, p - q), or of p for a bonus
//               token) and the row pairs whose one-pass KL is not accurate
//               enough.  The last helper of a request to finish combines the
//               slices in slice order, draws the terminal token by inverse
//               CDF (a workgroup-wide prefix sum over the slice that holds
//               it) and completes the KL values and the NKL decision.
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
// Every exponential of the path is 2^((x - m) * Lhi) with Lhi = fl32(log2(e)/T)
// (the statistics pass forms it as 2^(x Lhi - fl(m Lhi)) and corrects the
// rounding of m Lhi once per chunk sum), so all passes see the same
// distributions to within float32 rounding.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cstdint>
#include <type_traits>

#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kWaves = kThreads / 64;
constexpr double kLog2eD = 1.44269504088896340736;
constexpr double kLn2D = 0.693147180559945309417;
constexpr float kLn2F = 0.693147180559945309417f;

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
// 64-bit DPP moves: both 32-bit halves take the same lane pattern; a lane
// that the row / bank masks leave out, or whose source lies outside its row,
// gets 0.
template <int CTRL, int RM = 0xF, int BM = 0xF>
__device__ __forceinline__ long long dpp64(long long v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)v, CTRL, RM, BM, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(v >> 32), CTRL, RM, BM, false);
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
template <int CTRL, int RM = 0xF, int BM = 0xF>
__device__ __forceinline__ double dpp_d(double v) {
  return __longlong_as_double(dpp64<CTRL, RM, BM>(__double_as_longlong(v)));
}
__device__ __forceinline__ double lane_d(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, l), hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Sum over the wave.  Within each row of 16 lanes, partner groups of 1, 2, 4
// and 8 lanes are added (quad permutes, half-row mirror, row mirror), so
// every lane of a row holds the same bits (a + b == b + a in IEEE); the four
// row sums are then added in a fixed order.  The result is wave-uniform.
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<0xB1>(v);   // quad_perm(1,0,3,2)
  v += dpp_d<0x4E>(v);   // quad_perm(2,3,0,1)
  v += dpp_d<0x141>(v);  // row_half_mirror
  v += dpp_d<0x140>(v);  // row_mirror
  return (lane_d(v, 0) + lane_d(v, 16)) + (lane_d(v, 32) + lane_d(v, 48));
}

// Inclusive prefix sums over the wave in lane order: sums of 2, 3 and 4
// within a row (row shifts of 1..3), then of 8 and 16 (row shifts of 4 and 8
// on the upper banks), then the rows before (row broadcasts of lanes 15 and
// 31).  Lanes with no source add 0.
__device__ __forceinline__ double wave_incl_scan_d(double v) {
  double x = v + dpp_d<0x111>(v);  // row_shr:1
  x += dpp_d<0x112>(v);            // row_shr:2
  x += dpp_d<0x113>(v);            // row_shr:3
  x += dpp_d<0x114, 0xF, 0xE>(x);  // row_shr:4, lanes 4..15 of each row
  x += dpp_d<0x118, 0xF, 0xC>(x);  // row_shr:8, lanes 8..15 of each row
  x += dpp_d<0x142, 0xA, 0xF>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_d<0x143, 0xC, 0xF>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}
__device__ __forceinline__ long long wave_incl_scan_i64(long long v) {
  long long x = v + dpp64<0x111>(v);
  x += dpp64<0x112>(v);
  x += dpp64<0x113>(v);
  x += dpp64<0x114, 0xF, 0xE>(x);
  x += dpp64<0x118, 0xF, 0xC>(x);
  x += dpp64<0x142, 0xA, 0xF>(x);
  x += dpp64<0x143, 0xC, 0xF>(x);
  return x;
}

// Value of the partner group in a reduction over aligned groups of M lanes:
// groups of M = 1, 2, 4, 8 lanes meet their neighbour inside the row (quad
// permutes, half-row mirror, row mirror); 16 and 32 across rows.  Every lane
// of a group must hold the same value when M > 1.
template <int M>
__device__ __forceinline__ double partner_d(double v) {
  if constexpr (M == 1) return dpp_d<0xB1>(v);
  else if constexpr (M == 2) return dpp_d<0x4E>(v);
  else if constexpr (M == 4) return dpp_d<0x141>(v);
  else if constexpr (M == 8) return dpp_d<0x140>(v);
  else return __shfl_xor(v, M, 64);
}
template <int M>
__device__ __forceinline__ float partner_f(float v) {
  if constexpr (M == 1) return dpp<0xB1>(v, v);
  else if constexpr (M == 2) return dpp<0x4E>(v, v);
  else if constexpr (M == 4) return dpp<0x141>(v, v);
  else if constexpr (M == 8) return dpp<0x140>(v, v);
  else return __shfl_xor(v, M, 64);
}
template <int M>
__device__ __forceinline__ int partner_i(int v) {
  if constexpr (M == 1) return dppi<0xB1>(v, v);
  else if constexpr (M == 2) return dppi<0x4E>(v, v);
  else if constexpr (M == 4) return dppi<0x141>(v, v);
  else if constexpr (M == 8) return dppi<0x140>(v, v);
  else return __shfl_xor(v, M, 64);
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
    const long long incl = wave_incl_scan_i64(g);
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
    p.hdr[1] = 0;  // KL second-pass queue
  }
  if (p.cnt_kl)  // KL second-pass counters (verify calls)
    for (int b = tid; b < p.B; b += kPrepThreads) p.cnt_kl[(int64_t)b * kCntStride] = 0u;
  if (bad) return;
  __syncthreads();  // offsets written by other threads of this workgroup
  for (int b = tid; b < p.B; b += kPrepThreads) {
    const int g = p.gamma[b], d0 = p.d_off[b], t0 = d0 + b;
    if (p.mode == SV_MODE_STOCHASTIC || p.mode == kModeConsensus)
      for (int k = 0; k < g; ++k) p.pair2req[d0 + k] = b;
    if (p.mode == SV_MODE_NKL)
      for (int k = 0; k <= g; ++k) p.row2req[t0 + k] = b;
  }
}

// ----------------------------------------------------------------------------
// cross-workgroup hand-over inside one dispatch.  Values that another
// workgroup reads during the same dispatch are written and read at device
// scope (they bypass the per-XCD L2, which is not coherent between XCDs); a
// writer publishes a flag or counts itself only after all of its stores have
// completed.
// ----------------------------------------------------------------------------

template <class T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Self-tagged words: (epoch << 32) | 32-bit payload, each written and read as
// one 64-bit device-scope access.  A reader that finds its call's epoch in a
// word also holds that word's payload, so fields need no ordering between
// them and a writer never waits for its stores to complete.
__device__ __forceinline__ uint64_t tagged(uint32_t v, uint32_t epoch) { return ((uint64_t)epoch << 32) | v; }
__device__ __forceinline__ bool tag_ok(uint64_t w, uint32_t epoch) { return (uint32_t)(w >> 32) == epoch; }
__device__ __forceinline__ void st_tagged_f(uint64_t* p, float v, uint32_t epoch) {
  st_dev(p, tagged(__float_as_uint(v), epoch));
}
__device__ __forceinline__ void st_tagged_d(uint64_t* p, double v, uint32_t epoch) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  st_dev(p, tagged((uint32_t)b, epoch));
  st_dev(p + 1, tagged((uint32_t)(b >> 32), epoch));
}
__device__ __forceinline__ float tagged_f(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ double tagged_d(uint64_t lo, uint64_t hi) {
  return __longlong_as_double((long long)(((hi & 0xFFFFFFFFull) << 32) | (lo & 0xFFFFFFFFull)));
}

// A single-dispatch statistics partial (the 48-byte PartA slot as six
// self-tagged words): written by the streaming workgroup with plain stores of
// its six words, read by the helpers in one round of loads.
__device__ __forceinline__ void st_tagged_part(uint64_t* t, float mt, double st, float md, double sd,
                                               uint32_t epoch) {
  st_tagged_f(t + 0, mt, epoch);
  st_tagged_d(t + 1, st, epoch);
  st_tagged_f(t + 3, md, epoch);
  st_tagged_d(t + 4, sd, epoch);
}
struct PartVals {
  float mt, md;
  double st, sd;
};
// A greedy-family partial in the single dispatch: the target row maximum and
// its lowest index as two self-tagged words.
__device__ __forceinline__ void st_tagged_idx(uint64_t* t, float mt, int idx, uint32_t epoch) {
  st_tagged_f(t + 0, mt, epoch);
  st_dev(t + 1, tagged((uint32_t)idx, epoch));
}
__device__ __forceinline__ bool ld_tagged_idx(const uint64_t* t, uint32_t epoch, float& mt, int& idx) {
  const uint64_t w0 = ld_dev(t + 0), w1 = ld_dev(t + 1);
  const bool ok = ((int)tag_ok(w0, epoch) & (int)tag_ok(w1, epoch)) != 0;
  mt = tagged_f(w0);
  idx = (int)(uint32_t)w1;
  return ok;
}
__device__ __forceinline__ bool ld_tagged_part(const uint64_t* t, uint32_t epoch, PartVals& v) {
  const uint64_t w0 = ld_dev(t + 0), w1 = ld_dev(t + 1), w2 = ld_dev(t + 2);
  const uint64_t w3 = ld_dev(t + 3), w4 = ld_dev(t + 4), w5 = ld_dev(t + 5);
  // bitwise: one test of all six tags, no branches between them
  const bool ok = ((int)tag_ok(w0, epoch) & (int)tag_ok(w1, epoch) & (int)tag_ok(w2, epoch) &
                   (int)tag_ok(w3, epoch) & (int)tag_ok(w4, epoch) & (int)tag_ok(w5, epoch)) != 0;
  v.mt = tagged_f(w0);
  v.st = tagged_d(w1, w2);
  v.md = tagged_f(w3);
  v.sd = tagged_d(w4, w5);
  return ok;
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
  PartA scratch;  // fused kernel: a recomputed partial on its way to the workspace
  int64_t pick_task;  // fused kernel: the missing partial the workgroup computes next
  int pick_seg;
  int sel;            // lowest thread with a missing partial (INT_MAX: none)
};

// Packed offsets of a batch of at most kLdsBatch requests, scanned in LDS:
// off[b] = sum of gamma over the requests before b.  Returns whether the layout
// is valid (every gamma >= 0, sum == total_draft_rows).  `publish`: also write
// the offsets and the layout flag for the later kernels.
// Loads of gamma (and the temperatures) for the scan: issued on their own,
// ahead of other loads, since vector loads complete in issue order.
struct ScanIn {
  int gl[4];
  float tl[4];
};
__device__ __forceinline__ ScanIn scan_load(const Params& p, bool soft) {
  ScanIn in;
  // clamped indices, no branches: all loads in flight together
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int bc = min(4 * (int)threadIdx.x + k, p.B - 1);
    in.gl[k] = p.gamma[bc];
    in.tl[k] = soft ? p.temp[bc] : 0.0f;
  }
  return in;
}

__device__ bool scan_offsets_lds(const Params& p, StatsShared& sh, const ScanIn& in, bool soft, bool publish) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  long long g[4], loc = 0;
  bool bad = false;
  const int* gl = in.gl;
  const float* tl = in.tl;
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
  const long long incl = wave_incl_scan_i64(loc);
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
    for (int b = tid; b < p.B; b += kThreads) p.cnt_kl[(int64_t)b * kCntStride] = 0u;  // KL second-pass counters
    if (tid == 0) {
      p.hdr[0] = ok ? 0 : 1;
      p.hdr[1] = 0;  // KL second-pass queue
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

// Rows and vocabulary chunk of one item of the statistics pass.  `pair`: a
// draft row is streamed beside the target row (every stochastic task; NKL
// tasks except the bonus rows).
struct Desc {
  int task, chunk;
  int64_t trow, drow;
  int pair;  // int, not bool: keeps the struct in registers
  float Lhi;
};

// Loads of one chunk of one row: thread t takes 16-byte vectors k * kThreads + t.
template <int DT, bool VEC, int NV>
__device__ __forceinline__ void issue_row(const void* base, int64_t row, int chunk, int64_t V, Vecs<NV>& q) {
  constexpr int P = Elem<DT>::P;
  const int64_t e_chunk = (int64_t)chunk * kThreads * NV * P;
#pragma unroll
  for (int k = 0; k < NV; ++k)
    q.v[k] = fetch_raw<DT, VEC>(base, row, V, e_chunk + ((int64_t)k * kThreads + threadIdx.x) * P);
}

template <int DT, bool VEC, int NV, bool PAIR>
__device__ __forceinline__ void issue_chunk(const Params& p, const Desc& d, Vecs<NV>& qt, Vecs<NV>& qd) {
  issue_row<DT, VEC, NV>(p.target, d.trow, d.chunk, p.V, qt);
  if (PAIR && d.pair) issue_row<DT, VEC, NV>(p.draft, d.drow, d.chunk, p.V, qd);
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
      // 2^(x L - c) with c = fl(M L): one FMA per element; the chunk sum is
      // scaled by 2^(-c_lo) ~ 1 - c_lo ln2, c_lo = M L - c (exact by FMA),
      // so the sums are those of 2^((x - M) L)
      const float M = fmaxf(L.mt, mc);
      const float c = M * Lhi;
      const float corr = fmaf(-fmaf(M, Lhi, -c), kLn2F, 1.0f);
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int e = 0; e < NE; e += 4) {
        a0 += __builtin_amdgcn_exp2f(fmaf(vt[e], Lhi, -c));
        a1 += __builtin_amdgcn_exp2f(fmaf(vt[e + 1], Lhi, -c));
        a2 += __builtin_amdgcn_exp2f(fmaf(vt[e + 2], Lhi, -c));
        a3 += __builtin_amdgcn_exp2f(fmaf(vt[e + 3], Lhi, -c));
      }
      const float f = ex2(L.mt - M, Lhi);  // 0 on the first chunk (L.mt = -inf)
      L.st = L.st * (double)f + (double)(((a0 + a1) + (a2 + a3)) * corr);
      L.mt = M;
    } else {
      L.mt = fmaxf(L.mt, mc);
    }
  }
  if (PAIR && d.pair) {
    float vd[NE];
#pragma unroll
    for (int k = 0; k < NV; ++k) unpack<DT>(qd.v[k], vd + k * P);
    if (tail) mask_tail<DT, NV>(vd, lane_base, (int64_t)kThreads * P, V);
    float md = vd[0];
#pragma unroll
    for (int e = 1; e < NE; ++e) md = fmaxf(md, vd[e]);
    if (md > pad) {
      const float M = fmaxf(L.md, md);
      const float c = M * Lhi;
      const float corr = fmaf(-fmaf(M, Lhi, -c), kLn2F, 1.0f);
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f, w0 = 0.f, w1 = 0.f, z0 = 0.f, z1 = 0.f;
#pragma unroll
      for (int e = 0; e < NE; e += 4) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(vd[e], Lhi, -c));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(vd[e + 1], Lhi, -c));
        const float e2 = __builtin_amdgcn_exp2f(fmaf(vd[e + 2], Lhi, -c));
        const float e3 = __builtin_amdgcn_exp2f(fmaf(vd[e + 3], Lhi, -c));
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
      L.sd = L.sd * f + (double)(((a0 + a1) + (a2 + a3)) * corr);
      if (WZ) {
        L.w = L.w * f + (double)((w0 + w1) * corr);
        L.z = L.z * f + (double)((z0 + z1) * corr);
      }
      L.md = M;
    }
  }
}

// Reduces the lane states over the workgroup and writes the segment's partial
// (thread 0).  Plain stores when the consumer is a later kernel.  FUSED
// (consumers in the same dispatch): self-tagged words, (m_t, s_t, m_d, s_d)
// for a stochastic pair, (m_t, argmax) for a greedy-family row.
template <bool SOFT, bool IDX, bool WZ, bool PAIR, bool FUSED = false>
__device__ __forceinline__ void reduce_store(const Lane& L, float Lhi, PartA* dst, StatsShared& sh,
                                             uint32_t epoch = 0) {
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
    if constexpr (FUSED) {
      // self-tagged words: no wait for the stores, the next loads stay in flight
      if constexpr (SOFT) st_tagged_part(reinterpret_cast<uint64_t*>(dst), Mt, s0, Md, s1, epoch);
      else st_tagged_idx(reinterpret_cast<uint64_t*>(dst), Mt, I, epoch);
    } else {
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
  if (MODE == SV_MODE_GREEDY || MODE == SV_MODE_TREE_GREEDY || MODE == SV_MODE_BLOCK) {
    d.trow = d.task;
    d.drow = 0;
    d.pair = 0;
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
    d.pair = 1;
  } else {
    int d0, d1;
    if constexpr (LDS) {
      d0 = sh.off[b];
      d1 = sh.off[b + 1];
    } else {
      d0 = p.d_off[b];
      d1 = p.d_off[b + 1];
    }
    d.pair = d.task - (d0 + b) < d1 - d0 ? 1 : 0;  // the bonus row (position gamma) has no draft row
    d.trow = d.task;
    d.drow = d.pair ? (int64_t)d.task - b : 0;
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

// The streaming pass of one workgroup.  WZ (stochastic only): also the KL
// cross terms, for the optional NKL output.  Each workgroup streams its item
// range with two register buffers in turn: the loads of item i + 1 (also
// across a task boundary) are in flight while item i is folded; a task segment
// ends with a workgroup reduction whose barriers wait on LDS only, so the next
// loads stay in flight through it.  LDS: the batch is small enough for the
// offsets to be scanned in LDS.  FUSED (LDS, not NKL): partials are tagged
// for helpers of the same dispatch, workgroups numbered
// p.stats_grid and above stream nothing, and nothing is published for later
// kernels.  Returns false when the offsets scan found a layout error.
// Issue priority of a streaming wave from the share of its work still left
// (rem of tot items): the waves resident on a compute unit are otherwise
// served oldest first, so the youngest workgroups fall behind and finish last
// with little company to keep the memory pipeline full.  Waves that are behind
// rank first; four levels, the last for the final twentieth of the work.
__device__ __forceinline__ void pace(int64_t rem, int64_t tot) {
  if (rem * 2 > tot) __builtin_amdgcn_s_setprio(3);
  else if (rem * 5 > tot) __builtin_amdgcn_s_setprio(2);
  else if (rem * 20 > tot) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

template <int DT, bool VEC, int MODE, bool WZ, bool LDS, bool FUSED>
__device__ __forceinline__ bool stats_phase(const Params& p, StatsShared& sh) {
  constexpr bool SOFT = MODE == SV_MODE_STOCHASTIC || MODE == SV_MODE_NKL;
  constexpr int NV = SOFT ? 2 : 4;
  constexpr bool IDX = MODE != SV_MODE_STOCHASTIC;
  constexpr bool WZM = MODE == SV_MODE_NKL || WZ;
  static_assert(!FUSED || (LDS && MODE != SV_MODE_NKL && !WZ), "fused: LDS scan, no KL");
  const int G = p.stats_grid, wg = (int)blockIdx.x;
  const bool streams = !FUSED || wg < G;
  const int64_t N = (int64_t)p.n_task * p.nch;
  const int64_t i_end = streams ? (int64_t)(wg + 1) * N / G : 0;
  int64_t i = streams ? (int64_t)wg * N / G : 0;
  const int64_t tot = i_end - i;
  Desc dA, dB;
  Vecs<NV> At, Ad, Bt, Bd;
  int b = -1;
  // soft modes with the offsets scan in LDS: the first chunk's row whose index
  // needs no request lookup (the draft row of a stochastic pair, the target
  // row of an NKL task) is requested right behind the scan's own loads, so
  // that it is in flight while the scan runs
  constexpr bool EARLY = LDS && SOFT;
  if constexpr (EARLY) {
    dA.task = (int)(i / p.nch);
    dA.chunk = (int)(i - (int64_t)dA.task * p.nch);
    const ScanIn scan_in = scan_load(p, SOFT);
    __asm__ volatile("" ::: "memory");  // keeps the scan's loads ahead in issue order
    // unconditional, so that the scan's waits count these loads exactly: a
    // workgroup without items reads target row 0 (always present) instead
    const bool has = i < i_end;
    const void* base = (MODE == SV_MODE_STOCHASTIC && has) ? p.draft : p.target;
    issue_row<DT, VEC, NV>(base, has ? dA.task : 0, has ? dA.chunk : 0, p.V, MODE == SV_MODE_STOCHASTIC ? Ad : At);
    if (!scan_offsets_lds(p, sh, scan_in, SOFT, !FUSED && wg == 0)) return false;
    if (!has) return true;
    set_rows<MODE, LDS>(p, sh, b, dA);
    if (MODE == SV_MODE_STOCHASTIC) issue_row<DT, VEC, NV>(p.target, dA.trow, dA.chunk, p.V, At);
    else if (dA.pair) issue_row<DT, VEC, NV>(p.draft, dA.drow, dA.chunk, p.V, Ad);
  } else if constexpr (FUSED) {
    // greedy family in one dispatch: tasks are target rows (no lookup), so the
    // first item's loads go out right behind the offsets scan's own; only the
    // helper workgroups need the scan, for their decisions
    const bool helper = wg < p.B * p.helpers;
    ScanIn scan_in{};
    if (helper) scan_in = scan_load(p, SOFT);
    __asm__ volatile("" ::: "memory");  // keeps the scan's loads ahead in issue order
    // unconditional, so that the scan's waits count these loads exactly: a
    // workgroup without items reads the first chunk of target row 0 instead
    const bool has = i < i_end;
    dA.task = has ? (int)(i / p.nch) : 0;
    dA.chunk = has ? (int)(i - (int64_t)dA.task * p.nch) : 0;
    set_rows<MODE, LDS>(p, sh, b, dA);
    issue_chunk<DT, VEC, NV, SOFT>(p, dA, At, Ad);
    if (helper && !scan_offsets_lds(p, sh, scan_in, SOFT, false)) return false;
    if (!has) return true;
  } else {
    if (LDS) {
      // greedy and tree tasks are target rows: only workgroup 0 needs the
      // scan, to publish the offsets for the decision kernel
      if (wg == 0 && !scan_offsets_lds(p, sh, scan_load(p, SOFT), SOFT, true)) return false;
    } else if (SOFT && p.hdr[0] != 0) {
      return false;  // the prep kernel found a layout error
    }
    if (i >= i_end) return true;
    dA.task = (int)(i / p.nch);
    dA.chunk = (int)(i - (int64_t)dA.task * p.nch);
    set_rows<MODE, LDS>(p, sh, b, dA);
    issue_chunk<DT, VEC, NV, SOFT>(p, dA, At, Ad);
  }
  Lane L;
  lane_reset(L);
  const auto store = [&](const Desc& d) {
    const int w_lo = wg_of((int64_t)d.task * p.nch, N, G);
    PartA* dst = p.part_a + (int64_t)d.task * p.nch + (wg - w_lo);
    reduce_store<SOFT, IDX, WZM, SOFT, FUSED>(L, d.Lhi, dst, sh, p.epoch);
    lane_reset(L);
  };
  // issue priorities by remaining work: always in the soft modes; in the
  // greedy family only for the single dispatch's shares of five items or more
  // (measured: the separate greedy pass, and single-dispatch shares of four
  // items or fewer, stream faster without)
  const bool paced = SOFT || (FUSED && tot >= 5);
  for (;;) {
    dB = dA;
    if (i + 1 < i_end) next_desc<MODE, LDS>(p, sh, b, dB);
    if (paced) pace(i_end - i, tot);
    issue_chunk<DT, VEC, NV, SOFT>(p, dB, Bt, Bd);  // the last item reloads itself (cache hit)
    fold_chunk<DT, NV, SOFT, IDX, WZM, SOFT>(L, At, Ad, dA, p.V);
    if (dA.chunk == p.nch - 1 || i + 1 == i_end) store(dA);
    if (++i >= i_end) break;
    dA = dB;
    if (i + 1 < i_end) next_desc<MODE, LDS>(p, sh, b, dA);
    if (paced) pace(i_end - i, tot);
    issue_chunk<DT, VEC, NV, SOFT>(p, dA, At, Ad);
    fold_chunk<DT, NV, SOFT, IDX, WZM, SOFT>(L, Bt, Bd, dB, p.V);
    if (dB.chunk == p.nch - 1 || i + 1 == i_end) store(dB);
    if (++i >= i_end) break;
  }
  return true;
}

template <int DT, bool VEC, int MODE, bool WZ, bool LDS>
__global__ __launch_bounds__(kThreads) void k_stats(Params p) {
  __shared__ StatsShared sh;
  stats_phase<DT, VEC, MODE, WZ, LDS, false>(p, sh);
}

// ----------------------------------------------------------------------------
// k_decide: per-request merge, decision, terminal draw and KL second pass
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

// NKL threshold of draft row `row`: delta, or with generation positions
// ("Chain of Draft" page, section 4.3, position-adaptive threshold)
// min(delta_max, delta * (1 + alpha * log2(pos + 1))) for the row's 0-based
// position pos, in float64.  k_decide and k_refine take it from here; POS:
// the call has positions (kernels compiled without them keep the registers
// the float64 log2 would take).
template <bool POS>
__device__ __forceinline__ double nkl_delta(const Params& p, int64_t row) {
  if (!POS || !p.nkl_pos) return (double)p.delta;
  const double pos = (double)p.nkl_pos[row];
  return fmin((double)p.nkl_dmax, (double)p.delta * (1.0 + (double)p.nkl_alpha * log2(pos + 1.0)));
}

// Merged statistics of one task.
struct Merged {
  float mt, md;
  int idx;
  double st, sd, w, z;
};

__device__ __forceinline__ double rescale(float m, float M, float Lhi) {
  return m == M ? 1.0 : (double)ex2(m - M, Lhi);
}

// Folds one partial (m_t, s_t, m_d, s_d, w, z, argmax) into a lane's running
// merge; slots are folded in vocabulary order.
template <bool SOFT>
__device__ __forceinline__ void merge_fold(Merged& r, float mt, int ix, double st, float md, double sd, double w,
                                           double z, bool pair, float Lhi) {
  if (mt > r.mt || (mt == r.mt && ix < r.idx)) r.idx = ix;
  if (SOFT && pair) {
    const float Mt = fmaxf(r.mt, mt), Md = fmaxf(r.md, md);
    const double fo = rescale(r.md, Md, Lhi), fn = rescale(md, Md, Lhi);
    r.st = r.st * rescale(r.mt, Mt, Lhi) + st * rescale(mt, Mt, Lhi);
    r.sd = r.sd * fo + sd * fn;
    r.w = r.w * fo + w * fn;
    r.z = r.z * fo + z * fn;
    r.md = Md;
  }
  r.mt = fmaxf(r.mt, mt);
}

__device__ __forceinline__ Merged merge_identity() {
  Merged r;
  r.mt = r.md = -INFINITY;
  r.idx = INT_MAX;
  r.st = r.sd = r.w = r.z = 0.0;
  return r;
}

// Combines the lanes' running merges over aligned groups of S = 2^glog lanes
// by an xor butterfly, so every lane of a group ends with the same values.
// All lanes of the wave must call this.
template <bool SOFT>
__device__ __forceinline__ Merged merge_group(Merged r, int glog, float Lhi) {
  const int S = 1 << glog;
  // group reductions: f is applied for M = 1, 2, 4, ... below S (uniform branches)
  const auto levels = [S](auto&& f) {
    if (S > 1) f(std::integral_constant<int, 1>{});
    if (S > 2) f(std::integral_constant<int, 2>{});
    if (S > 4) f(std::integral_constant<int, 4>{});
    if (S > 8) f(std::integral_constant<int, 8>{});
    if (S > 16) f(std::integral_constant<int, 16>{});
    if (S > 32) f(std::integral_constant<int, 32>{});
  };
  float Mt = r.mt, Md = r.md;
  levels([&](auto m) {
    Mt = fmaxf(Mt, partner_f<decltype(m)::value>(Mt));
    if (SOFT) Md = fmaxf(Md, partner_f<decltype(m)::value>(Md));
  });
  int ix = r.mt == Mt ? r.idx : INT_MAX;
  levels([&](auto m) { ix = min(ix, partner_i<decltype(m)::value>(ix)); });
  if (SOFT) {
    const double ft = rescale(r.mt, Mt, Lhi), fd = rescale(r.md, Md, Lhi);
    double st = r.st * ft, sd = r.sd * fd, w = r.w * fd, z = r.z * fd;
    levels([&](auto m) {
      constexpr int M = decltype(m)::value;
      st += partner_d<M>(st);
      sd += partner_d<M>(sd);
      w += partner_d<M>(w);
      z += partner_d<M>(z);
    });
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

// Merges the partials of `task` (written by an earlier kernel) over a group of
// S = 2^glog lanes: lane l of the group takes partial slots l, l + S, ...
// (vocabulary order), then the group combines by an xor butterfly.  `pair`:
// the task has draft statistics.  All lanes of the wave must call this.
template <bool SOFT>
__device__ __forceinline__ Merged merge_task(const Params& p, int64_t task, bool has, bool pair, int l, int glog,
                                             float Lhi) {
  const int S = 1 << glog;
  Merged r = merge_identity();
  if (has) {
    const int64_t N = (int64_t)p.n_task * p.nch;
    const int nseg = wg_of((task + 1) * p.nch - 1, N, p.stats_grid) - wg_of(task * p.nch, N, p.stats_grid) + 1;
    const PartA* src = p.part_a + task * p.nch;
    for (int s = l; s < nseg; s += S)
      merge_fold<SOFT>(r, src[s].m_t, src[s].idx, src[s].s_t, src[s].m_d, src[s].s_d, src[s].w, src[s].z, pair, Lhi);
  }
  return merge_group<SOFT>(r, glog, Lhi);
}

// ----------------------------------------------------------------------------
// fused kernel: the wait of a helper for its request's statistics
// ----------------------------------------------------------------------------

// Partial of segment `seg` of task `task` (a stochastic pair or a
// greedy-family row; the chunks of the task that statistics workgroup
// w_lo(task) + seg streams), computed again by the calling workgroup with the
// same chunk order, lane mapping and reduction as the statistics pass, so it
// is bit-identical to the original: left in
// sh.scratch and published as self-tagged words.  All threads call.
template <int DT, bool VEC, int MODE>
__device__ void recompute_segment(const Params& p, StatsShared& sh, int task, int seg) {
  constexpr bool SOFT = MODE == SV_MODE_STOCHASTIC;
  constexpr int NV = SOFT ? 2 : 4;
  const int G = p.stats_grid;
  const int64_t N = (int64_t)p.n_task * p.nch;
  const int64_t first = (int64_t)task * p.nch;
  const int w = wg_of(first, N, G) + seg;
  const int64_t lo = max(first, (int64_t)w * N / G);
  const int64_t hi = min(first + p.nch, (int64_t)(w + 1) * N / G);
  Desc d;
  int b = -1;
  d.task = task;
  d.chunk = (int)(lo - first);
  set_rows<MODE, true>(p, sh, b, d);
  Lane L;
  lane_reset(L);
  for (int64_t i = lo; i < hi; ++i, ++d.chunk) {
    Vecs<NV> qt, qd;
    issue_chunk<DT, VEC, NV, SOFT>(p, d, qt, qd);
    fold_chunk<DT, NV, SOFT, !SOFT, false, SOFT>(L, qt, qd, d, p.V);
  }
  reduce_store<SOFT, !SOFT, false, SOFT>(L, d.Lhi, &sh.scratch, sh);  // into LDS first
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t* t = reinterpret_cast<uint64_t*>(p.part_a + first + seg);
    if (SOFT) st_tagged_part(t, sh.scratch.m_t, sh.scratch.s_t, sh.scratch.m_d, sh.scratch.s_d, p.epoch);
    else st_tagged_idx(t, sh.scratch.m_t, sh.scratch.idx, p.epoch);
  }
}

// The running merge of this lane's partial slots of one task in the single
// dispatch: lane l of a group of S = 2^glog lanes takes slots l, l + S, ...,
// each read from its self-tagged words once they carry this call's epoch (one
// round of loads, then a poll while they do not).  A slot still missing after
// p.wait_polls polls (its workgroup is not resident, or slow) is computed by
// this workgroup itself, so the wait is bounded and the result does not
// depend on which workgroups run when.  All threads call (the slot rounds are
// uniform: ceil(maxseg / S)).
template <int DT, bool VEC, int MODE>
__device__ Merged fused_task_merge(const Params& p, StatsShared& ssh, int64_t task, bool has, int l, int glog,
                                   float Lhi) {
  constexpr bool SOFT = MODE == SV_MODE_STOCHASTIC;
  const int G = p.stats_grid, S = 1 << glog;
  const int64_t N = (int64_t)p.n_task * p.nch;
  const int nseg = has ? wg_of((task + 1) * p.nch - 1, N, G) - wg_of(task * p.nch, N, G) + 1 : 0;
  const int rounds = (p.maxseg + S - 1) >> glog;
  Merged r = merge_identity();
  for (int k = 0; k < rounds; ++k) {
    const int seg = l + k * S;
    const bool active = seg < nseg;
    const uint64_t* t = reinterpret_cast<const uint64_t*>(p.part_a + task * p.nch + seg);
    PartVals v{-INFINITY, -INFINITY, 0.0, 0.0};
    int vix = INT_MAX;
    const auto load = [&]() { return SOFT ? ld_tagged_part(t, p.epoch, v) : ld_tagged_idx(t, p.epoch, v.mt, vix); };
    bool ready = !active || load();
    for (int n = 0; !ready && n < p.wait_polls; ++n) {
      __builtin_amdgcn_s_sleep(2);
      ready = load();
    }
    // the fallback: missing slots are computed by the whole workgroup, one by one
    bool miss = !ready;
    while (__syncthreads_or(miss)) {
      if (threadIdx.x == 0) ssh.sel = INT_MAX;
      __syncthreads();
      if (miss) atomicMin(&ssh.sel, (int)threadIdx.x);  // the lowest missing thread goes first
      __syncthreads();
      const int owner = ssh.sel;
      if ((int)threadIdx.x == owner) {
        ssh.pick_task = task;
        ssh.pick_seg = seg;
      }
      __syncthreads();
      recompute_segment<DT, VEC, MODE>(p, ssh, (int)ssh.pick_task, ssh.pick_seg);
      __syncthreads();
      if ((int)threadIdx.x == owner) {
        v.mt = ssh.scratch.m_t;
        v.st = ssh.scratch.s_t;
        v.md = ssh.scratch.m_d;
        v.sd = ssh.scratch.s_d;
        vix = ssh.scratch.idx;
        miss = false;
      }
    }
    if (active) merge_fold<SOFT>(r, v.mt, SOFT ? INT_MAX : vix, v.st, v.md, v.sd, 0.0, 0.0, SOFT, Lhi);
  }
  return merge_group<SOFT>(r, glog, Lhi);
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

// Loads of one vocabulary slice: wave w covers the contiguous wave-chunk w of
// the slice (64 x kUT vectors); its lane l takes vectors k * 64 + l, k < kUT,
// of the target row and (TWO) of the draft row.
template <int DT, bool VEC, bool TWO>
__device__ __forceinline__ void slice_issue(const Params& p, int64_t trow, int64_t drow, int sl, uint4* qt,
                                            uint4* qd) {
  constexpr int P = Elem<DT>::P;
  const int64_t e_base = (int64_t)sl * kThreads * kUT * P;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < kUT; ++k) {
    const int64_t e0 = e_base + ((int64_t)(w * kUT + k) * 64 + lane) * P;
    qt[k] = fetch<DT, VEC>(p.target, trow, p.V, e0);
    if (TWO) qd[k] = fetch<DT, VEC>(p.draft, drow, p.V, e0);
  }
}

// Streams slices [s0, s1) of the rows with the loads of slice s + 1 in flight
// while slice s is consumed by f(qt, qd, s).  All threads call; f may hold
// workgroup barriers.
template <int DT, bool VEC, bool TWO, class F>
__device__ __forceinline__ void slice_stream(const Params& p, int64_t trow, int64_t drow, int s0, int s1, F&& f) {
  uint4 at[kUT], ad[kUT], bt[kUT], bd[kUT];
  if (s0 >= s1) return;
  slice_issue<DT, VEC, TWO>(p, trow, drow, s0, at, ad);
  for (int sl = s0; sl < s1; sl += 2) {
    if (sl + 1 < s1) slice_issue<DT, VEC, TWO>(p, trow, drow, sl + 1, bt, bd);
    f(at, ad, sl);
    if (sl + 1 >= s1) break;
    if (sl + 2 < s1) slice_issue<DT, VEC, TWO>(p, trow, drow, sl + 2, at, ad);
    f(bt, bd, sl + 1);
  }
}

// KL(q || p) of one row pair in a second pass, as the sum of the non-negative
// terms q_y g(w_y), w_y = log(p_y / q_y), over slices of the vocabulary.  Because sum q e^w = sum p = 1, the sum over the row equals
// sum q log(q/p) exactly, has no cancellation, and an error eps in the log
// normaliser ratio only adds O(eps^2).  All threads of the workgroup call.
// Per position constants: p_y = 2^(t_y L - ct) kt and q_y = 2^(d_y L - cd) kd
// (ct = fl(m_t L), kt = 2^(-(m_t L - ct)) / s_t, the same for the draft row),
// and w_y = log(p_y / q_y) = (t_y - d_y) c + lw, c = L ln 2.
struct KlIn {
  float ct, cd, kt, kd, lw;
};

__device__ __forceinline__ KlIn kl_in(float m_t, float m_d, double s_t, double s_d, float Lhi) {
  KlIn r;
  r.ct = m_t * Lhi;
  r.cd = m_d * Lhi;
  const double lo_t = (double)fmaf(m_t, Lhi, -r.ct), lo_d = (double)fmaf(m_d, Lhi, -r.cd);
  r.kt = (float)(exp2(-lo_t) / s_t);
  r.kd = (float)(exp2(-lo_d) / s_d);
  const double c = (double)Lhi * kLn2D;
  r.lw = (float)(((double)m_d - (double)m_t) * c + log(s_d / s_t));
  return r;
}

// Sum over one slice (thread-local part) of q_y g(w_y).  Both forms of the
// term are evaluated and one is selected (no divergent branch).
template <int DT>
__device__ __forceinline__ double kl_terms(const uint4* qt, const uint4* qd, const KlIn& ri, float Lhi) {
  constexpr int P = Elem<DT>::P;
  const float c = (float)((double)Lhi * kLn2D);  // d(log p)/d(logit)
  double acc = 0.0;
#pragma unroll
  for (int k = 0; k < kUT; ++k) {
    float vt[P], vd[P];
    unpack<DT>(qt[k], vt);
    unpack<DT>(qd[k], vd);
    float part = 0.f;  // P non-negative terms in float32, then float64
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const float q = __builtin_amdgcn_exp2f(fmaf(vd[e], Lhi, -ri.cd)) * ri.kd;
      const float pp = __builtin_amdgcn_exp2f(fmaf(vt[e], Lhi, -ri.ct)) * ri.kt;
      const float w = fmaf(vt[e] - vd[e], c, ri.lw);
      const float small = q * g_small(w);
      const float large = (pp - q) - q * w;  // q g(w) = p - q - q w; right also where q underflows
      part += fabsf(w) < 0.5f ? small : large;  // positions past the end give p = q = 0
    }
    acc += (double)part;
  }
  return acc;
}


struct DecideShared {
  float mt[kThreads], md[kThreads];
  double st[kThreads], sd[kThreads];
  int idx[kThreads];
  int acc[kThreads];
  double kl1[kThreads];
  int need[kThreads];
  int qbase, qcount;  // queue slots of a pass's positions for the KL second pass
  // draw records of the request kept by the token selection (one wave)
  double sel_s[kSelCache], sel_a[kSelCache];
  float sel_m[kSelCache];
  int red_i[kWaves];
  float red_f[kWaves];
  double red_d[kWaves];
  int flag;
  // what the draw's wave 0 hands to the workgroup
  int sel_cstar, sel_flags;
  float sel_ref, sel_M;
  double sel_cbase, sel_target, sel_ratio;
};

// Rank of this thread among the threads with `flag` (thread order), and one
// reservation of that many slots at the end of the KL queue (sh.qbase,
// sh.qcount).  All threads call.
__device__ __forceinline__ int block_excl_count(bool flag, int* tail, DecideShared& sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned long long m = __ballot(flag);
  const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
  __syncthreads();
  if (lane == 0) sh.red_i[w] = __popcll(m);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    if (k < w) before += sh.red_i[k];
    tot += sh.red_i[k];
  }
  if (threadIdx.x == 0) {
    sh.qcount = tot;
    sh.qbase = tot > 0 ? atomicAdd(tail, tot) : 0;
  }
  __syncthreads();
  return before + in_wave;
}

// Counts this workgroup on a KL second-pass counter (zeroed by the same
// call's offsets scan) once every store of the workgroup has completed; true
// in the last of the `H` arrivals.  The counter wraps to zero on the last
// arrival (atomic increment modulo H).
template <class SH>
__device__ __forceinline__ bool arrive_last(uint32_t* cnt, int H, SH& sh) {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
  __asm__ __volatile__("" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __builtin_amdgcn_atomic_inc32(cnt, (uint32_t)H - 1u, __ATOMIC_RELAXED, "agent");
    sh.flag = old + 1 == (uint32_t)H ? 1 : 0;
  }
  __syncthreads();
  return sh.flag != 0;
}

// Helper arrival counters: (epoch << 32) | arrivals.  The thread kClaimThread
// (lane 0 of the last wave) loads the request's word early (claim_load) and,
// before its workgroup counts itself, claims it for this call (claim): a word
// that carries another epoch -- left by an earlier call, or any other bytes --
// is replaced by (epoch << 32) with a compare-and-swap.  The first helper's
// swap succeeds; every other helper's fails or is skipped because the word
// already carries the epoch, and from then on only this call's increments
// change it.  No reset is needed and nothing in the workspace must start at a
// particular value.
constexpr int kClaimThread = kThreads - 64;

__device__ __forceinline__ uint64_t claim_load(const uint64_t* c) {
  return ld_dev(c);
}
__device__ __forceinline__ void claim(uint64_t* c, uint64_t cur, uint32_t epoch) {
  const uint64_t mine = (uint64_t)epoch << 32;
  // a failed swap returns the current word; within one call that word carries
  // the epoch, so the loop ends after at most two swaps (bounded regardless)
  for (int k = 0; k < 4 && (uint32_t)(cur >> 32) != epoch; ++k)
    if (__hip_atomic_compare_exchange_strong(c, &cur, mine, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      break;
}

// The same claim without waiting for the swap's result: only a word that
// carries another epoch is swapped, and a swap that fails because another
// workgroup of the call claimed the word first changes nothing.  The swap
// still completes before the workgroup counts itself (arrive_last waits for
// all of its memory operations).
__device__ __forceinline__ void claim_nowait(uint64_t* c, uint64_t cur, uint32_t epoch) {
  if ((uint32_t)(cur >> 32) != epoch)
    __hip_atomic_compare_exchange_strong(c, &cur, (uint64_t)epoch << 32, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
}

// Counts this workgroup on the request's claimed counter once every memory
// operation of the workgroup (its stores and the claim) has completed; true in
// the last of the `H` arrivals.
template <class SH>
__device__ __forceinline__ bool arrive_last(uint64_t* cnt, int H, SH& sh) {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores (and the claim) have completed
  __asm__ __volatile__("" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t old = __hip_atomic_fetch_add(cnt, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.flag = (uint32_t)old + 1u == (uint32_t)H ? 1 : 0;
  }
  __syncthreads();
  return sh.flag != 0;
}

// Decision scratch of the tree and block modes for requests of up to N - 1
// draft positions (N nodes).
template <int MODE, int N = SV_MAX_GAMMA + 1>
struct TreeShared {
  int16_t info[1];
  int16_t par[1];
  int idx[1];
};
template <int N>
struct TreeShared<SV_MODE_TREE_GREEDY, N> {
  int16_t info[N];  // (depth << 1) | accepted
  int16_t par[N];
  int idx[N];  // argmax of each node's target row
};
template <int N>
struct TreeShared<SV_MODE_BLOCK, N> {
  int idx[N];  // argmax of each position's target row
  int keep;    // the kept prefix e, from thread 0's run scan
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
  }
}

// Tree resolve over the node argmaxes in `tr.idx`: a node is accepted when its
// token is the argmax of its parent's target row and its parent is accepted;
// the deepest accepted node (lowest id on ties) ends the path.  Parents
// precede children, so one ordered pass settles every node.
template <class TS>
__device__ void resolve_tree(const Params& p, int b, int g, int t0, int d0, TS& tr, DecideShared& sh) {
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

// ----------------------------------------------------------------------------
// terminal draw of a stochastic request
// ----------------------------------------------------------------------------

// Terminal distribution of a stochastic request, taken by every helper from
// its own copy of the decision.
struct Term {
  int kind;      // TermKind
  int64_t trow;  // target row of the terminal distribution
  int64_t drow;  // draft row (residual only)
  float m_t;     // maximum of the target row (residual only)
  float m_d;     // maximum of the draft row (residual only)
  float k0;      // s_t / s_d from the statistics pass (residual only)
  float Lhi;     // fl32(log2(e) / T) of the request
};

// Draw record of one (request, wave-chunk); each wave of a helper covers one
// contiguous wave-chunk of a slice (64 lanes x kUT vectors).  With
// a_y = 2^((t_y - m_t) L) and b_y = 2^((d_y - m_d) L), i.e. p_y and q_y up to
// the factors 1/s_t and 1/s_d, and k0 = s_t / s_d:
//   residual: s = sum_y max(0, a_y - k0 b_y)  (max(0, p - q) in units of
//             1/s_t: one ratio decides both the support and the weight),
//             a = sum_y a_y (for the fallback draw from p_j);
//   bonus:    s = sum_y 2^((t_y - m) L) with m the chunk maximum
//             (m = -inf and s = 0 for a chunk past the end of the row).
// Sums: float over a lane's P elements of one vector, then float64.  Written
// with device-scope stores; a helper counts itself only once they have
// completed.
struct DrawRec {
  double s, a;
  float m;
  int32_t pad;
};
static_assert(sizeof(DrawRec) <= sizeof(PartC), "a draw record fits its workspace slot");

__device__ __forceinline__ float resid_weight(float t, float d, const Term& tm) {
  const float a = ex2(t - tm.m_t, tm.Lhi), bb = ex2(d - tm.m_d, tm.Lhi);
  return fmaxf(fmaf(-tm.k0, bb, a), 0.0f);  // one rounding of a - k0 b: its sign is exact
}

// OWN: the record goes to this workgroup's LDS cache (slot ch) instead of the
// workspace (the request's only helper keeps its records).
template <int DT, bool RESID, bool OWN = false>
__device__ __forceinline__ void draw_record(const uint4* qt, const uint4* qd, const Term& tm, DrawRec* dst,
                                            DecideShared* own = nullptr, int ch = 0) {
  constexpr int P = Elem<DT>::P;
  const float Lhi = tm.Lhi;
  const int lane = threadIdx.x & 63;
  if (RESID) {
    double S = 0.0, A = 0.0;
#pragma unroll
    for (int k = 0; k < kUT; ++k) {
      float vt[P], vd[P];
      unpack<DT>(qt[k], vt);
      unpack<DT>(qd[k], vd);
      float sr = 0.f, sa = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        sa += ex2(vt[e] - tm.m_t, Lhi);
        sr += resid_weight(vt[e], vd[e], tm);
      }
      S += (double)sr;
      A += (double)sa;
    }
    S = wave_sum_d(S);
    A = wave_sum_d(A);
    if (lane == 0) {
      if (OWN) {
        own->sel_s[ch] = S;
        own->sel_a[ch] = A;
      } else {
        st_dev(&dst->s, S);
        st_dev(&dst->a, A);
      }
    }
  } else {
    float vt[kUT * P];
#pragma unroll
    for (int k = 0; k < kUT; ++k) unpack<DT>(qt[k], vt + k * P);
    float mx = vt[0];
#pragma unroll
    for (int e = 1; e < kUT * P; ++e) mx = fmaxf(mx, vt[e]);
    const float mc = wave_max(mx);
    const bool empty = !(mc > Elem<DT>::kPad);  // the chunk lies past the end of the row
    double S = 0.0;
#pragma unroll
    for (int k = 0; k < kUT; ++k) {
      float sa = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) sa += ex2(vt[k * P + e] - mc, Lhi);
      S += (double)sa;
    }
    S = wave_sum_d(S);
    if (lane == 0) {
      if (OWN) {
        own->sel_s[ch] = empty ? 0.0 : S;
        own->sel_m[ch] = empty ? -INFINITY : mc;
      } else {
        st_dev(&dst->s, empty ? 0.0 : S);
        st_dev(&dst->m, empty ? -INFINITY : mc);
      }
    }
  }
}

// Token draw of request b by its last helper, from the NW wave-chunk records
// in token order: y* = min{y : C_y > u * C_{V-1}}.  Wave 0 combines the
// records by fixed wave-wide reductions and scans in chunk order and finds the
// wave-chunk that holds the draw (CACHED: at most kSelCache records, kept in
// LDS after the first sweep; OWN: all of them already there, written by this
// workgroup before a barrier).  The whole workgroup then reads that wave-chunk
// again, thread t taking its t-th vector (P consecutive tokens), and a
// workgroup scan of the threads' weights, in token order, leads to the thread
// and then the token that hold the draw.  All threads call.
template <int DT, bool VEC, bool CACHED, bool OWN = false>
__device__ __forceinline__ void draw_select(const Params& p, int b, const Term& tm, int NW, float ur,
                                            DecideShared& sh) {
  static_assert(CACHED || !OWN, "own records live in the LDS cache");
  constexpr int P = Elem<DT>::P;
  constexpr int64_t CHW = (int64_t)64 * kUT * P;  // tokens of one wave-chunk: kThreads vectors
  static_assert(64 * kUT == kThreads, "one vector of the wave-chunk per thread");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool resid = tm.kind == kTermResidual;
  const float Lhi = tm.Lhi;
  const double Ld = (double)Lhi;
  if (tid < 64) {
    const DrawRec* rec = reinterpret_cast<const DrawRec*>(p.part_c) + (int64_t)b * NW;
    double st = 0.0, at = 0.0;
    float M = -INFINITY;
    for (int ch = lane; ch < NW; ch += 64) {
      const double s0 = OWN ? sh.sel_s[ch] : ld_dev(&rec[ch].s);
      const double a0 = resid ? (OWN ? sh.sel_a[ch] : ld_dev(&rec[ch].a)) : 0.0;
      const float m0 = resid ? 0.0f : (OWN ? sh.sel_m[ch] : ld_dev(&rec[ch].m));
      st += s0;
      at += a0;
      M = fmaxf(M, m0);
      if (CACHED && !OWN) {  // each lane reads back only the records it wrote: no barrier needed
        sh.sel_s[ch] = s0;
        sh.sel_a[ch] = a0;
        sh.sel_m[ch] = m0;
      }
    }
    st = wave_sum_d(st);
    at = wave_sum_d(at);
    M = wave_max(M);
    const bool fb = resid && !(st > 0.0);  // max(0, p - q) vanished numerically: draw from p_j instead
    const auto weight = [&](int ch) {
      const double s0 = CACHED ? sh.sel_s[ch] : ld_dev(&rec[ch].s);
      if (resid) return fb ? (CACHED ? sh.sel_a[ch] : ld_dev(&rec[ch].a)) : s0;
      const float m0 = CACHED ? sh.sel_m[ch] : ld_dev(&rec[ch].m);
      return s0 > 0.0 ? s0 * exp2(((double)m0 - (double)M) * Ld) : 0.0;
    };
    const int rounds = (NW + 63) / 64;
    double S = resid ? (fb ? at : st) : 0.0;
    if (!resid) {
      for (int r = 0; r < rounds; ++r)
        if (lane + 64 * r < NW) S += weight(lane + 64 * r);
      S = wave_sum_d(S);
    }
    const double target = (double)ur * S;
    // the wave-chunk whose cumulative weight first exceeds the target: one
    // round per 64 consecutive chunks
    int cstar = -1, clast = -1;
    double cbase = 0.0, carry = 0.0;
    for (int r = 0; r < rounds; ++r) {
      const int ch = lane + 64 * r;
      const double w = ch < NW ? weight(ch) : 0.0;
      const double incl = wave_incl_scan_d(w);
      const double excl = carry + incl - w;
      const bool hit = w > 0.0 && excl <= target && target < excl + w;
      const int first = wave_min_int(hit ? ch : INT_MAX);
      const int lp = wave_max_int(w > 0.0 ? ch : -1);
      if (lp >= 0) clast = lp;
      if (first != INT_MAX) {
        cstar = first;
        cbase = lane_d(excl, first - 64 * r);
        break;
      }
      carry += lane_d(incl, 63);
    }
    const bool take_last = cstar < 0;  // rounding left the target at the end
    if (take_last) {
      cstar = clast >= 0 ? clast : NW - 1;
      cbase = 0.0;
    }
    if (lane == 0) {
      sh.sel_cstar = cstar;
      sh.sel_flags = (take_last ? 1 : 0) | (fb ? 2 : 0);
      sh.sel_cbase = cbase;
      sh.sel_target = target;
      sh.sel_M = M;
      sh.sel_ratio = resid && !fb ? st / at : 1.0;
      sh.sel_ref = resid ? tm.m_t : (CACHED ? sh.sel_m[cstar] : ld_dev(&rec[cstar].m));
    }
  }
  __syncthreads();
  const int cstar = sh.sel_cstar;
  const bool take_last = (sh.sel_flags & 1) != 0, fb = (sh.sel_flags & 2) != 0;
  const double cbase = sh.sel_cbase, target = sh.sel_target;
  // wave-chunk c* again: thread t owns tokens y0 .. y0 + P - 1
  const int64_t V = p.V;
  const int64_t y0 = (int64_t)cstar * CHW + (int64_t)tid * P;
  const bool two = resid && !fb;
  const float ref = sh.sel_ref;
  const double cf = resid ? 1.0 : exp2(((double)ref - (double)sh.sel_M) * Ld);
  const uint4 qt = fetch<DT, VEC>(p.target, tm.trow, V, y0);
  const uint4 qd = two ? fetch<DT, VEC>(p.draft, tm.drow, V, y0) : qt;
  // positions past the end hold the pad: their weight is 0
  float vt[P], vd[P], wt[P];
  unpack<DT>(qt, vt);
  unpack<DT>(qd, vd);
  float ls = 0.f;
  int lastpos = -1;  // the last token with a positive weight (the fallback)
#pragma unroll
  for (int e = 0; e < P; ++e) {
    wt[e] = two ? resid_weight(vt[e], vd[e], tm) : ex2(vt[e] - ref, Lhi);
    ls += wt[e];
    if (wt[e] > 0.f) lastpos = (int)(y0 + e);
  }
  const double tsum = (double)ls * cf;
  // workgroup exclusive scan of the threads' sums, in thread (= token) order
  const double incl = wave_incl_scan_d(tsum);
  if (lane == 63) sh.red_d[wv] = incl;
  __syncthreads();
  double before = 0.0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k)
    if (k < wv) before += sh.red_d[k];
  const double cum0 = cbase + (before + (incl - tsum));
  int cand = INT_MAX;
  if (!take_last && tsum > 0.0 && cum0 <= target && cum0 + tsum > target) {
    double cum = cum0;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      cum += (double)wt[e] * cf;
      if (cand == INT_MAX && cum > target) cand = (int)(y0 + e);
    }
    if (cand == INT_MAX) cand = lastpos;  // rounding inside the thread: its last positive token
  }
  const int ystar = block_min_int(cand, sh.red_i);
  const int ylast = block_max_int(lastpos, sh.red_i);
  if (tid == 0) {
    int y = ystar != INT_MAX ? ystar : ylast;
    if (y < 0 || y >= p.V) y = (int)min(V - 1, (int64_t)cstar * CHW);
    p.out_tokens[tm.trow] = y;
    if (p.out_resid) p.out_resid[b] = (float)sh.sel_ratio;
  }
}

// The terminal draw of one request by its helper h (slices [s0, s1) of the
// terminal row or row pair): stream the slices and write one record per
// wave-chunk, then count in on the request's arrival counter (claimed for this
// call: `arr_cur` is its early load); the last helper to arrive selects the
// token.  A request's only helper keeps its records in LDS and selects at
// once.  All threads call.
template <int DT, bool VEC>
__device__ __forceinline__ void terminal_draw(const Params& p, int b, const Term& tm, int s0, int s1, float ur,
                                              DecideShared& sh, uint64_t* arr, uint64_t arr_cur) {
  const int NS = p.nslices, NW = NS * kWaves;
  const int wv = threadIdx.x >> 6;
  if (p.helpers == 1 && NW <= kSelCache) {
    // the request's only helper (slices [0, NS)): its records stay in LDS,
    // with no counter and no round trip through the workspace
    if (tm.kind == kTermResidual)
      slice_stream<DT, VEC, true>(p, tm.trow, tm.drow, s0, s1, [&](const uint4* qt, const uint4* qd, int sl) {
        draw_record<DT, true, true>(qt, qd, tm, nullptr, &sh, sl * kWaves + wv);
      });
    else
      slice_stream<DT, VEC, false>(p, tm.trow, tm.drow, s0, s1, [&](const uint4* qt, const uint4* qd, int sl) {
        draw_record<DT, false, true>(qt, qd, tm, nullptr, &sh, sl * kWaves + wv);
      });
    __syncthreads();
    draw_select<DT, VEC, true, true>(p, b, tm, NW, ur, sh);
    return;
  }
  if (threadIdx.x == kClaimThread) claim(arr, arr_cur, p.epoch);  // completes before this helper counts itself
  DrawRec* rec = reinterpret_cast<DrawRec*>(p.part_c) + (int64_t)b * NW + wv;
  if (tm.kind == kTermResidual)
    slice_stream<DT, VEC, true>(p, tm.trow, tm.drow, s0, s1, [&](const uint4* qt, const uint4* qd, int sl) {
      draw_record<DT, true>(qt, qd, tm, rec + sl * kWaves);
    });
  else
    slice_stream<DT, VEC, false>(p, tm.trow, tm.drow, s0, s1, [&](const uint4* qt, const uint4* qd, int sl) {
      draw_record<DT, false>(qt, qd, tm, rec + sl * kWaves);
    });
  if (arrive_last(arr, p.helpers, sh)) {
    if (NW <= kSelCache) draw_select<DT, VEC, true>(p, b, tm, NW, ur, sh);
    else draw_select<DT, VEC, false>(p, b, tm, NW, ur, sh);
  }
}

// Second-pass KL values of request b from the slice sums, added in slice
// order.  NKL mode: k_decide wrote the outputs with every queued position
// accepted (decision jnn); the first queued position that the second-pass
// value rejects, if it precedes jnn, becomes the decision.
template <int MODE, bool POS, class SH>
__device__ __forceinline__ void kl_finish(const Params& p, int b, const ReqFin& f, SH& sh) {
  const int t0 = f.d0 + b, NS = p.nslices;
  const double lnV = log((double)p.V);
  int first = INT_MAX;
  for (int i = threadIdx.x; i < f.g; i += kThreads) {
    const int pos = f.d0 + i;
    const bool need = p.kl_need[pos] != 0;
    double kl = 0.0;  // the slots of positions not queued hold older values: not used
    for (int s = 0; s < NS; ++s) kl += ld_dev(&p.kl_part[(int64_t)pos * NS + s]);
    if (!need) continue;
    const double nkl = p.V > 1 ? kl / lnV : 0.0;
    p.out_nkl[pos] = (float)nkl;  // the other positions were written by k_decide
    if (!(nkl < nkl_delta<POS>(p, pos))) first = min(first, i);
  }
  if (MODE == SV_MODE_NKL) {
    const int jr = block_min_int(first, sh.red_i);
    if (jr < f.jnn) {
      for (int k = jr + threadIdx.x; k <= f.jnn; k += kThreads) p.out_tokens[t0 + k] = k == jr ? p.tidx[t0 + jr] : -1;
      if (threadIdx.x == 0) p.out_num[b] = jr;
    }
  }
}

// ----------------------------------------------------------------------------
// k_decide
// ----------------------------------------------------------------------------

// The decision and terminal draw of request b by its helper h.  ok: the
// packed layout is valid; d0, d1: the request's draft-row offsets; T, ur: its
// temperature and resample uniform (ur is first used after the decision, so
// its load may still be in flight).  FUSED (any mode but NKL): called in the
// statistics kernel itself, where it waits for the request's partials.  TS:
// the tree / block decision scratch, sized for the call's requests.
// POS (NKL): per-position thresholds from generation positions.
template <int DT, bool VEC, int MODE, bool FUSED, bool POS = false, class TS>
__device__ __forceinline__ void decide_request(const Params& p, int b, int h, bool ok, int d0, int d1, float T,
                                               float ur, DecideShared& sh, TS& tr, StatsShared* ssh) {
  constexpr bool SOFT = MODE == SV_MODE_STOCHASTIC || MODE == SV_MODE_NKL;
  const int NS = p.nslices;
  // helper h streams slices [s0, s1) wherever rows get a second look
  const int s0 = h * p.slices_per_helper, s1 = min(NS, s0 + p.slices_per_helper);
  const bool writer = h == 0;  // helper 0 writes the outputs of the decision
  const int tid = threadIdx.x;
  const bool want_kl = SOFT && !FUSED && p.want_kl;  // the single dispatch has no KL output
  // the request's arrival counter, loaded now and claimed before the draw
  uint64_t* const arr = p.cnt + (int64_t)b * kArrStride;
  uint64_t arr_cur = 0;
  if (MODE == SV_MODE_STOCHASTIC && tid == kClaimThread) arr_cur = claim_load(arr);
  if (!ok) {  // layout error: only the counts are written
    if (writer && tid == 0) p.out_num[b] = -1;
    return;
  }
  const int g = d1 - d0;
  const int t0 = d0 + b;
  const int64_t V = p.V;
  const float Lhi = SOFT ? (float)(kLog2eD / (double)T) : 0.0f;
  // request-level checks; the per-position ones (and the resample uniform's)
  // follow the decision passes (which only read inside the rows for valid
  // token ids), and overwrite everything the passes wrote if they fail
  if (g > p.max_gamma || (SOFT && !temp_ok(T))) {
    if (writer) finish_invalid(p, b, t0, d0, g);
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
  bool bad = false;
  int n_queued = 0;  // positions queued for the KL second pass (helper 0)
  int run = 0, best_run = 0, best_end = 0;  // block mode: agreeing runs (thread 0)
  int checked = 0;  // positions [0, checked) were checked inside the passes
  // the group leader's position data of the pass starting at `base`
  // (node ti of a tree is position ti - 1), and the per-position input checks
  struct Pos {
    int x;
    float tx, dx, u;
  };
  const auto load_pos = [&](int base) {
    const int ti = base + (tid >> glog);
    Pos ps{-1, 0.f, 0.f, 0.f};
    if ((tid & (S - 1)) == 0 && MODE != SV_MODE_TREE_GREEDY && ti < g) {
      ps.x = p.tokens[d0 + ti];
      const bool xok = ps.x >= 0 && ps.x < p.V;
      // the logits at the drafted token: the stochastic test, and p(x), q(x)
      // when asked for (the NKL decision does not use them)
      if (SOFT && xok && (MODE == SV_MODE_STOCHASTIC || p.out_p_x || p.out_q_x)) {
        ps.tx = load_scalar<DT>(p.target, t0 + ti, V, ps.x);
        ps.dx = load_scalar<DT>(p.draft, d0 + ti, V, ps.x);
      }
      if (MODE == SV_MODE_STOCHASTIC) {
        ps.u = p.ua[d0 + ti];
        if (!unit_ok(ps.u)) bad = true;
      }
      if (!xok) bad = true;
      if (MODE == SV_MODE_NKL && POS && p.nkl_pos[d0 + ti] < 0) bad = true;
    }
    if ((tid & (S - 1)) == 0 && MODE == SV_MODE_TREE_GREEDY && ti >= 1 && ti <= g) {
      const int xn = p.tokens[d0 + ti - 1], pa = p.parents[d0 + ti - 1];
      if (xn < 0 || xn >= p.V || pa < 0 || pa >= ti) bad = true;
    }
    return ps;
  };
  for (int base = 0; base < ntask; base += TPP) {
    const int q = tid >> glog, l = tid & (S - 1);
    const int ti = base + q;
    const bool has = ti < ntask;
    const bool pair = SOFT && ti < g;
    // issued before the partial loads
    const Pos ps = load_pos(base);
    const int x = ps.x;
    const float tx = ps.tx, dx = ps.dx, u = ps.u;
    Merged r;
    if constexpr (FUSED) r = fused_task_merge<DT, VEC, MODE>(p, *ssh, tbase + ti, has, l, glog, Lhi);
    else r = merge_task<SOFT>(p, tbase + ti, has, pair, l, glog, Lhi);
    if (l == 0 && has) {
      const int idx = r.idx == INT_MAX ? 0 : r.idx;  // no element above the pad value: position 0
      if constexpr (MODE == SV_MODE_TREE_GREEDY || MODE == SV_MODE_BLOCK) tr.idx[ti] = idx;
      sh.mt[q] = r.mt;
      sh.md[q] = r.md;
      sh.st[q] = r.st;
      sh.sd[q] = r.sd;
      sh.idx[q] = idx;
      if (MODE == SV_MODE_NKL && writer) p.tidx[t0 + ti] = idx;
      int acc = 0, need = 0;
      double kl = 0.0;  // KL(q||p) = 0 for V == 1: both rows are the same point mass
      if (pair) {
        // log2 p(x) and log2 q(x) from the merged statistics (float32: the
        // relative error of p(x), q(x) and alpha stays near 1e-7)
        const float lpx = (tx - r.mt) * Lhi - __log2f((float)r.st);
        const float lqx = (dx - r.md) * Lhi - __log2f((float)r.sd);
        if (writer && p.out_p_x) p.out_p_x[d0 + ti] = exp2f(lpx);
        if (writer && p.out_q_x) p.out_q_x[d0 + ti] = exp2f(lqx);
        if (MODE == SV_MODE_STOCHASTIC) acc = u <= fminf(1.0f, exp2f(lpx - lqx)) ? 1 : 0;
        if (want_kl && p.V > 1) {
          // KL(q||p) = E_q[d - t]/T - (m_d - m_t)/T - log(s_d / s_t)
          const double lg = log(r.sd / r.st);
          const double klv = r.w / r.sd * c - (double)(r.md - r.mt) * c - lg;
          const double err = kKlErr * (r.z / r.sd * c + 1.0);
          need = (err > kKlRel * klv) ? 1 : 0;
          if (MODE == SV_MODE_NKL && fabs(klv - nkl_delta<POS>(p, d0 + ti) * lnV) <= err) need = 1;
          kl = klv;
        }
      } else if (MODE == SV_MODE_GREEDY || MODE == SV_MODE_BLOCK) {
        acc = (ti < g && x == idx) ? 1 : 0;
      }
      sh.acc[q] = acc;
      sh.kl1[q] = kl;
      sh.need[q] = need;
    }
    __syncthreads();
    if (want_kl) {
      if (tid < TPP && base + tid < g) {
        const int pos = d0 + base + tid;
        const int need = sh.need[tid];
        if (writer) p.kl_need[pos] = need;
        if (need) {
          // NKL: taken as accepted here; k_refine corrects the outputs if the
          // second-pass value rejects it
          if (MODE == SV_MODE_NKL) sh.acc[tid] = 1;
        } else {
          const double nkl = p.V > 1 ? sh.kl1[tid] / lnV : 0.0;
          if (writer && p.out_nkl) p.out_nkl[pos] = (float)nkl;
          if (MODE == SV_MODE_NKL) sh.acc[tid] = nkl < nkl_delta<POS>(p, pos) ? 1 : 0;
        }
      }
      if (writer) {
        // queue the positions of this pass whose one-pass KL is not accurate
        // enough for the second pass (k_refine), with their merged statistics
        const int need = (tid < TPP && base + tid < g) ? sh.need[tid] : 0;
        const int rank = block_excl_count(need != 0, p.hdr + 1, sh);
        if (need) {
          const KlIn ri = kl_in(sh.mt[tid], sh.md[tid], sh.st[tid], sh.sd[tid], Lhi);
          RefItem e;
          e.pos = d0 + base + tid;
          e.b = b;
          e.trow = t0 + base + tid;
          e.Lhi = Lhi;
          e.ct = ri.ct;
          e.cd = ri.cd;
          e.kt = ri.kt;
          e.kd = ri.kd;
          e.lw = ri.lw;
          e.pad = 0;
          p.ref_list[sh.qbase + rank] = e;
        }
        n_queued += sh.qcount;
      }
    }
    if (MODE == SV_MODE_BLOCK) {
      // runs of agreeing positions, continued across passes by thread 0: a run
      // replaces the best one only when strictly longer (the first longest wins)
      if (tid == 0)
        for (int q = 0; q < TPP && base + q < g; ++q) {
          run = sh.acc[q] ? run + 1 : 0;
          if (run > best_run) {
            best_run = run;
            best_end = base + q + 1;
          }
        }
    } else if (MODE != SV_MODE_TREE_GREEDY) {
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

  if (MODE == SV_MODE_STOCHASTIC && tid == 0 && !unit_ok(ur)) bad = true;
  // positions the passes did not reach (an early exit) are checked here
  for (int k = checked + tid; k < g; k += kThreads) {
    const int x = p.tokens[d0 + k];
    bool ok = x >= 0 && x < p.V;
    if (MODE == SV_MODE_STOCHASTIC) ok = ok && unit_ok(p.ua[d0 + k]);
    if (MODE == SV_MODE_TREE_GREEDY) {
      const int pa = p.parents[d0 + k];  // parent of node k + 1
      ok = ok && pa >= 0 && pa <= k;
    }
    if (MODE == SV_MODE_NKL && POS) ok = ok && p.nkl_pos[d0 + k] >= 0;
    if (!ok) bad = true;
  }
  if (__syncthreads_or(bad)) {
    if (writer) finish_invalid(p, b, t0, d0, g);
    if (want_kl && writer && tid == 0) p.req_fin[b] = ReqFin{d0, g, g, -1};  // k_refine leaves the request alone
    return;
  }
  if constexpr (MODE == SV_MODE_TREE_GREEDY) {
    resolve_tree(p, b, g, t0, d0, tr, sh);
    return;
  }
  if constexpr (MODE == SV_MODE_BLOCK) {
    if (tid == 0) tr.keep = best_run >= p.block_min_len ? best_end : 0;
    __syncthreads();
    const int e = tr.keep;
    for (int k = tid; k <= g; k += kThreads) p.out_tokens[t0 + k] = k < e ? p.tokens[d0 + k] : k == e ? tr.idx[e] : -1;
    if (tid == 0) p.out_num[b] = e;
    return;
  }
  if (j < 0) j = g;  // every draft accepted
  if (want_kl && writer && tid == 0) p.req_fin[b] = ReqFin{d0, g, j, n_queued};
  if (writer) {
    for (int k = tid; k <= g; k += kThreads) {
      if (k < j) p.out_tokens[t0 + k] = p.tokens[d0 + k];
      else if (k > j) p.out_tokens[t0 + k] = -1;
      else if (MODE != SV_MODE_STOCHASTIC) p.out_tokens[t0 + k] = jidx;  // stochastic: the draw writes it
    }
    if (tid == 0) p.out_num[b] = j;
  }
  if constexpr (MODE == SV_MODE_STOCHASTIC) {
    Term tm;
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
    terminal_draw<DT, VEC>(p, b, tm, s0, s1, ur, sh, arr, arr_cur);
  }
}

// H workgroups ("helpers") per request (see decide_request), after k_stats.
// POS: NKL with generation positions.
template <int DT, bool VEC, int MODE, bool POS = false>
__global__ __launch_bounds__(kThreads) void k_decide(Params p) {
  constexpr bool SOFT = MODE == SV_MODE_STOCHASTIC || MODE == SV_MODE_NKL;
  __shared__ DecideShared sh;
  __shared__ TreeShared<MODE> tr;
  const int b = (int)(blockIdx.x % (unsigned)p.B);
  const int h = (int)(blockIdx.x / (unsigned)p.B);
  // independent loads first, so that they are in flight together
  const int hdr = p.hdr[0];
  const int d0 = p.d_off[b];
  const int d1 = p.d_off[b + 1];
  const float T = SOFT ? p.temp[b] : 1.0f;
  const float ur = MODE == SV_MODE_STOCHASTIC ? p.ur[b] : 0.0f;
  decide_request<DT, VEC, MODE, false, POS>(p, b, h, hdr == 0, d0, d1, T, ur, sh, tr, nullptr);
}

// Draft-side sampling: row b's token is the inverse-CDF draw from
// softmax(x_b / T_b) with the uniform u_b, by the same records and selection as
// the bonus draw of the verify step.  Workgroup (row b, helper h) streams its
// slices of the row; the last helper of the row to arrive selects the token.
// A row with a bad temperature or uniform gets -1 (every helper of the row
// sees the same inputs, so none of them arrives).
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void k_sample(Params p) {
  __shared__ DecideShared sh;
  const int b = (int)(blockIdx.x % (unsigned)p.B), h = (int)(blockIdx.x / (unsigned)p.B);
  uint64_t* const arr = p.cnt + (int64_t)b * kArrStride;
  const uint64_t arr_cur = threadIdx.x == kClaimThread ? claim_load(arr) : 0;
  const float T = p.temp[b], u = p.ur[b];
  if (!temp_ok(T) || !unit_ok(u)) {
    if (h == 0 && threadIdx.x == 0) p.out_tokens[b] = -1;
    return;
  }
  Term tm;
  tm.kind = kTermBonus;
  tm.trow = b;
  tm.drow = -1;
  tm.m_t = tm.m_d = tm.k0 = 0.0f;
  tm.Lhi = (float)(kLog2eD / (double)T);
  const int NS = p.nslices, s0 = h * p.slices_per_helper, s1 = min(NS, s0 + p.slices_per_helper);
  terminal_draw<DT, VEC>(p, b, tm, s0, s1, u, sh, arr, arr_cur);
}

// ----------------------------------------------------------------------------
// top-k of each row (the children of a tree-draft node)
// ----------------------------------------------------------------------------

// Ordering key of logit x at index y: a larger x first, the lower index first
// among equal x (-0 and +0 are equal).  0 is below every key: "no candidate".
__device__ __forceinline__ uint64_t topk_key(float x, int y) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);  // order-preserving map to unsigned
  return ((uint64_t)b << 32) | (uint32_t)(0x7FFFFFFF - y);
}
__device__ __forceinline__ int topk_index(uint64_t key) { return 0x7FFFFFFF - (int)(uint32_t)key; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const uint64_t o = __shfl_xor(v, m);
    v = o > v ? o : v;
  }
  return v;
}

// bf16 rows: a 32-bit key of the same order within one helper's range of at
// most 65536 elements, the order-mapped bf16 bits (topk_map16x2) above
// 0xFFFF - (index - base); back to the 64-bit key of the element (0 stays "no
// candidate"):
__device__ __forceinline__ uint64_t topk_key_from16(uint32_t k16, int base) {
  if (k16 == 0) return 0;
  uint32_t h = k16 >> 16;
  h = (h & 0x8000u) ? (h & 0x7FFFu) : ((0x10000u - h) & 0xFFFFu);
  return topk_key(__uint_as_float(h << 16), base + (int)(0xFFFFu - (k16 & 0xFFFFu)));
}
// Branchless insertion into a sorted (largest first) list of 32-bit keys:
// the new i-th key is the middle one of the old (i-1)-th, the old i-th and the
// new key (one median-of-three per entry).
__device__ __forceinline__ uint32_t med3u(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
}
template <int K>
__device__ __forceinline__ void topk_insert16(uint32_t (&lst)[K], uint32_t key) {
  if constexpr (K <= 4) {
    uint32_t nl[K];
    nl[0] = max(lst[0], key);
#pragma unroll
    for (int i = 1; i < K; ++i) nl[i] = med3u(lst[i - 1], lst[i], key);
#pragma unroll
    for (int i = 0; i < K; ++i) lst[i] = nl[i];
  } else {  // (longer lists: the compare-and-swap chain, which compiles far faster)
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const uint32_t hi = max(lst[i], key), lo = min(lst[i], key);
      lst[i] = hi;
      key = lo;
    }
  }
}

// The order-preserving 16-bit maps of the two bf16 values of a word, both at
// once with 16-bit lane arithmetic: h -> h | 0x8000 for h >= +0 and h ->
// 0x10000 - h for negative h.  -0 and +0 both map to 0x8000, and no value maps
// to 0 (the "no candidate" key).
typedef short sv_i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short sv_u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t topk_map16x2(uint32_t wd) {
  const sv_i16x2 sgn = __builtin_bit_cast(sv_i16x2, wd) >> (short)15;  // per half: all ones if negative
  const sv_u16x2 h = __builtin_bit_cast(sv_u16x2, wd);
  const sv_u16x2 neg = (unsigned short)0 - h, pos = h | (unsigned short)0x8000;
  const uint32_t m = __builtin_bit_cast(uint32_t, sgn);
  return (__builtin_bit_cast(uint32_t, neg) & m) | (__builtin_bit_cast(uint32_t, pos) & ~m);
}

// Keeps the K largest keys seen by this thread, sorted, largest first.
template <int K>
__device__ __forceinline__ void topk_insert(uint64_t (&lst)[K], uint64_t key) {
  if (key <= lst[K - 1]) return;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const uint64_t hi = lst[i] > key ? lst[i] : key, lo = lst[i] > key ? key : lst[i];
    lst[i] = hi;
    key = lo;
  }
}

// The k largest of the keys the threads hold (each thread's list sorted,
// largest first): k rounds of a workgroup maximum over the list heads; the
// holder of the maximum drops its head.  Thread 0 gets them in out[0..k).
template <int K>
__device__ __forceinline__ void topk_merge(uint64_t (&lst)[K], int k, uint64_t* out, uint64_t* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int r = 0; r < k; ++r) {
    const uint64_t m = wave_max_u64(lst[0]);
    if (lane == 0) red[w] = m;
    __syncthreads();
    uint64_t best = red[0];
#pragma unroll
    for (int j = 1; j < kWaves; ++j) best = red[j] > best ? red[j] : best;
    if (lst[0] == best && best != 0) {  // keys are unique: one holder
#pragma unroll
      for (int i = 0; i + 1 < K; ++i) lst[i] = lst[i + 1];
      lst[K - 1] = 0;
    }
    if (threadIdx.x == 0) out[r] = best;
    __syncthreads();
  }
}

// Top-k of row b: helper h streams its slices of the row, keeping each
// thread's K best keys (K: k rounded up to a power of two), merges them over
// the workgroup and stores its k best; the last helper of the row to arrive
// merges the helpers' candidates and writes the k indices.
struct TopkShared {
  uint64_t best[kTopkMax], red[kWaves];
  int flag;
};

template <int DT, bool VEC, int K>
__global__ __launch_bounds__(kThreads) void k_topk(Params p) {
  __shared__ TopkShared sh;
  constexpr int P = Elem<DT>::P;
  const int b = (int)(blockIdx.x % (unsigned)p.B), h = (int)(blockIdx.x / (unsigned)p.B);
  const int k = p.topk, H = p.helpers, NS = p.nslices;
  const int s0 = h * p.slices_per_helper, s1 = min(NS, s0 + p.slices_per_helper);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint64_t* const arr = p.cnt + (int64_t)b * kArrStride;
  const uint64_t arr_cur = threadIdx.x == kClaimThread ? claim_load(arr) : 0;
  uint64_t lst[K];
#pragma unroll
  for (int i = 0; i < K; ++i) lst[i] = 0;
  constexpr int CH = kThreads * kUT * P;  // elements of one slice
  if (DT == SV_DTYPE_BF16 && (s1 - s0) * CH <= 65536) {
    // 32-bit keys relative to the helper's first element, straight from the
    // bf16 bits; converted to the 64-bit keys for the merges
    const int base = s0 * CH;
    uint32_t l16[K];
#pragma unroll
    for (int i = 0; i < K; ++i) l16[i] = 0;
    // element y gets the key (map16(x_y) << 16) | (0xFFFF - (y - base)), 0 past the row's end
    slice_stream<DT, VEC, false>(p, b, -1, s0, s1, [&](const uint4* qt, const uint4*, int sl) {
      if (sl == s0 && threadIdx.x == kClaimThread) claim(arr, arr_cur, p.epoch);
#pragma unroll
      for (int j = 0; j < kUT; ++j) {
        const int y0 = sl * CH + ((w * kUT + j) * 64 + lane) * P;
        const uint32_t c0 = 0xFFFFu - (uint32_t)(y0 - base);
        const int lim = p.V - y0;  // elements e < lim lie inside the row
        const uint32_t wd[4] = {topk_map16x2(qt[j].x), topk_map16x2(qt[j].y), topk_map16x2(qt[j].z),
                                topk_map16x2(qt[j].w)};
#pragma unroll
        for (int e = 0; e < P; ++e) {
          const uint32_t hi = (e & 1) ? (wd[e >> 1] & 0xFFFF0000u) : (wd[e >> 1] << 16);
          topk_insert16<K>(l16, e < lim ? (hi | (c0 - (uint32_t)e)) : 0u);
        }
      }
    });
#pragma unroll
    for (int i = 0; i < K; ++i) lst[i] = topk_key_from16(l16[i], base);
  } else {
    slice_stream<DT, VEC, false>(p, b, -1, s0, s1, [&](const uint4* qt, const uint4*, int sl) {
      if (sl == s0 && threadIdx.x == kClaimThread) claim(arr, arr_cur, p.epoch);
      const int64_t e_base = (int64_t)sl * CH;
#pragma unroll
      for (int j = 0; j < kUT; ++j) {
        float v[P];
        unpack<DT>(qt[j], v);
        const int64_t y0 = e_base + ((int64_t)(w * kUT + j) * 64 + lane) * P;
#pragma unroll
        for (int e = 0; e < P; ++e)
          if (y0 + e < p.V) topk_insert<K>(lst, topk_key(v[e], (int)(y0 + e)));
      }
    });
  }
  if (s0 >= s1 && threadIdx.x == kClaimThread) claim(arr, arr_cur, p.epoch);
  topk_merge<K>(lst, k, sh.best, sh.red);
  // row b's candidates: kThreads slots, helper h's k of them at h * k (H * k <= kThreads)
  uint64_t* cand = p.topk_cand + (int64_t)b * kThreads;
  const int tid = (int)threadIdx.x;
  if (tid < k) st_dev(&cand[h * k + tid], sh.best[tid]);
  if (!arrive_last(arr, H, sh)) return;
  // the row's last helper: one candidate per thread, then the same merge
  uint64_t c1[1] = {0};
  if (tid < H * k) c1[0] = ld_dev(&cand[tid]);
  topk_merge<1>(c1, k, sh.best, sh.red);
  if (tid < k) p.out_tokens[(int64_t)b * k + tid] = topk_index(sh.best[tid]);
}

// The whole step in one dispatch (batches up to kLdsBatch; stochastic without
// KL output, greedy, tree and block).  Every workgroup first streams its share
// of the statistics pass (stats_phase: partials tagged with the call's epoch);
// then workgroup r below B x H takes the helper role (request r mod B, helper
// r / B; H = 1 outside the stochastic mode) of the decision kernel: it reads
// its request's partials as they arrive (fused_task_merge, a bounded wait with
// its own fallback) instead of after a kernel boundary, and takes the offsets
// and temperatures from its own LDS scan.  Tree and block requests hold at
// most kFusedNodes - 1 positions here.  Vector-load variants are held to 128
// registers (4 waves per SIMD) without spilling.
template <int DT, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(VEC ? 4 : 1))) void k_fused(Params p) {
  constexpr bool SOFT = MODE == SV_MODE_STOCHASTIC;
  __shared__ StatsShared ssh;
  __shared__ DecideShared sh;
  __shared__ TreeShared<MODE, kFusedNodes> tr;
  const bool ok = stats_phase<DT, VEC, MODE, false, true, true>(p, ssh);
  const int r = (int)blockIdx.x;
  if (r < p.B * p.helpers) {
    const int b = r % p.B, h = r / p.B;
    const float ur = SOFT ? p.ur[b] : 0.0f;
    decide_request<DT, VEC, MODE, true>(p, b, h, ok, ssh.off[b], ssh.off[b + 1], SOFT ? ssh.temp[b] : 1.0f, ur, sh,
                                        tr, &ssh);
  }
}

// ----------------------------------------------------------------------------
// k_refine: the KL second pass over the queue that k_decide filled.  Items
// (queued position, vocabulary slice) are dealt round-robin to the
// workgroups and stream with the loads of the next item in flight; every
// item's sum has its own slot, so the result does not depend on the order.
// The workgroup that completes a request's last item (per-request counter)
// adds the sums and writes the NKL values and, in NKL mode, the decision.
// ----------------------------------------------------------------------------

// workgroup scratch of k_refine
struct RefineShared {
  int red_i[kWaves];
  double red_d[kWaves];
  int flag;
};

template <int DT, bool VEC, int MODE, bool POS = false>
__global__ __launch_bounds__(kThreads) void k_refine(Params p) {
  __shared__ RefineShared sh;
  const int NS = p.nslices;
  const int64_t G = gridDim.x, wg = blockIdx.x;
  // Items are dealt round-robin (item it to workgroup it mod G), so the queue
  // entry of this workgroup's first item is known before the queue length and
  // both loads are in flight together; the entry is used only if the item
  // exists (the index is clamped into the queue's storage).
  const RefItem first = p.ref_list[min(wg / NS, (int64_t)max(p.R_d, 1) - 1)];
  const int64_t N = (int64_t)p.hdr[1] * NS;
  if (wg >= N) return;
  uint4 at[kUT], ad[kUT], bt[kUT], bd[kUT];
  RefItem ea, eb;
  ReqFin fa, fb;
  // the request's completion record (its queued count, -1 if it failed its
  // input checks) travels with the item, then the slice
  const auto issue = [&](int64_t it, const RefItem& e, ReqFin& f, uint4* qt, uint4* qd) {
    f = p.req_fin[e.b];
    slice_issue<DT, VEC, true>(p, e.trow, e.pos, (int)(it % NS), qt, qd);
  };
  const auto consume = [&](const uint4* qt, const uint4* qd, const RefItem& e, const ReqFin& f, int64_t it) {
    const KlIn ri{e.ct, e.cd, e.kt, e.kd, e.lw};
    const double v = block_sum_d(kl_terms<DT>(qt, qd, ri, e.Lhi), sh.red_d);
    if (threadIdx.x == 0) st_dev(&p.kl_part[(int64_t)e.pos * NS + it % NS], v);
    if (f.pending > 0 && arrive_last(p.cnt_kl + (int64_t)e.b * kCntStride, f.pending * NS, sh))
      kl_finish<MODE, POS>(p, e.b, f, sh);
  };
  ea = first;
  issue(wg, ea, fa, at, ad);
  for (int64_t it = wg; it < N; it += 2 * G) {
    const bool second = it + G < N;
    if (second) {
      eb = p.ref_list[(it + G) / NS];
      issue(it + G, eb, fb, bt, bd);
    }
    consume(at, ad, ea, fa, it);
    if (!second) break;
    if (it + 2 * G < N) {
      ea = p.ref_list[(it + 2 * G) / NS];
      issue(it + 2 * G, ea, fa, at, ad);
    }
    consume(bt, bd, eb, fb, it + G);
  }
}

// ----------------------------------------------------------------------------
// consensus across K drafts ("Chain of Draft" page, section 4.4,
// Consensus-Aware Accept): per position, the NKL of every ordered pair of its
// K draft rows, M[a][b] = KL(q_a || q_b) / ln V, and the closest pair's
// symmetrised distance against the consensus and divergence thresholds.
//
// One dispatch (k_cons), one workgroup per (position, chunk).  One read of
// the rows gives per row s = sum 2^(x L - R) and per ordered pair t = sum
// 2^(x_a L - R_a) (x_a - x_b) and z, the same with |x_a - x_b| (R: integer
// reference exponents).  The position's last workgroup merges the chunks:
//   KL_ab = c T_ab / S_a - (R_a - R_b) ln 2 - ln(S_a / S_b),  c = L ln 2,
// with the one-pass error estimate kKlErr (c Z_ab / S_a + 1) of the verify
// KL.  It decides there unless an estimate exceeds kKlRel of its value or the
// decision (a threshold, the closest pair) lies within the estimates; then it
// sums the exact form q_a g(w), w = ln(q_b / q_a), g(w) = e^w - 1 - w >= 0
// (no cancellation) over the position's chunks itself -- a second read of that
// position's rows only -- and decides from those sums.
// ----------------------------------------------------------------------------

constexpr int kConsMaxPairs = kConsMaxDrafts * (kConsMaxDrafts - 1);
constexpr int kConsRing = 2;  // vectors of every row in flight per thread
static_assert(kConsVec % kConsRing == 0, "whole rounds of the ring");

struct ConsShared {
  float m[kConsMaxDrafts][kWaves];
  double d[kConsMaxDrafts + 2 * kConsMaxPairs][kWaves];
  float Mrow[kConsMaxDrafts];
  double Srow[kConsMaxDrafts];
  double tot[kConsMaxPairs];  // exact sums of the position (the last workgroup)
  long long scan[kWaves];
  float T;
  int req, bad, need, flag;
};

// Ordered pair (a, b), a != b, at a * (K - 1) + (b < a ? b : b - 1).
template <int K>
__device__ __forceinline__ constexpr int cons_pair_index(int a, int b) {
  return a * (K - 1) + (b < a ? b : b - 1);
}

// First element of vector k of chunk `chunk` for this thread.
template <int DT>
__device__ __forceinline__ int64_t cons_e0(int64_t chunk, int k) {
  return (chunk * kConsVec * kThreads + (int64_t)k * kThreads + threadIdx.x) * Elem<DT>::P;
}

// Sets the unpacked elements at positions >= V of the vector starting at e0
// to the pad.  The loads themselves (fetch_raw) take no select, so that no
// wait is placed between them.
template <int DT, bool VEC>
__device__ __forceinline__ void cons_mask(float* v, int64_t e0, int64_t V) {
  constexpr int P = Elem<DT>::P;
  if (VEC) {  // a vector lies wholly inside or wholly past the row
    const bool in = e0 < V;
#pragma unroll
    for (int e = 0; e < P; ++e) v[e] = in ? v[e] : Elem<DT>::kPad;
  } else {
#pragma unroll
    for (int e = 0; e < P; ++e)
      if (e0 + e >= V) v[e] = Elem<DT>::kPad;
  }
}

// Reference exponent of a row segment whose largest element is vm: an
// integer near vm L (clamped so that it stays exact in float32), so that the
// terms 2^(x L - R) are at most about 1 and rescaling between references is
// an exact power of two.
constexpr int kConsRNone = -(1 << 30);  // no element seen yet
__device__ __forceinline__ int cons_ref(float vm, float Lhi) {
  const float r = ceilf(vm * Lhi);
  return (int)fminf(fmaxf(r, -16000000.0f), 16000000.0f);  // NaN (an invalid T) gives the lower bound
}

// The request of position `pos` by a scan of gamma in LDS (batches of at most
// kLdsBatch requests: thread t holds requests 4t .. 4t + 3, whose gamma and
// temperature it loaded before the rows, so that the scan waits for those
// loads only), with the layout check: sh.bad = 1 for a negative gamma or
// sum(gamma) != R_d.  The thread that holds the request publishes its
// temperature in sh.T.  All threads call.
struct ConsReqIn {
  int g[4];
  float t[4];
};
__device__ __forceinline__ ConsReqIn cons_req_load(const Params& p) {
  ConsReqIn in;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = 4 * threadIdx.x + j;
    in.g[j] = b < p.B ? p.gamma[b] : 0;
    in.t[j] = b < p.B ? p.temp[b] : 1.0f;
  }
  return in;
}
__device__ __forceinline__ void cons_find_request(const Params& p, int64_t pos, const ConsReqIn& in, ConsShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) {
    sh.req = -1;
    sh.bad = 0;
  }
  long long g[4], tot = 0;
  bool neg = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    g[j] = in.g[j];
    neg = neg || g[j] < 0;
    g[j] = g[j] < 0 ? 0 : g[j];
    tot += g[j];
  }
  const long long incl = wave_incl_scan_i64(tot);
  if (lane == 63) sh.scan[w] = incl;
  __syncthreads();
  long long before = incl - tot, all = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    if (k < w) before += sh.scan[k];
    all += sh.scan[k];
  }
  if (neg) sh.bad = 1;  // benign race: every writer stores 1
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (pos >= before && pos < before + g[j]) {
      sh.req = 4 * tid + j;
      sh.T = in.t[j];
    }
    before += g[j];
  }
  __syncthreads();
  if (tid == 0 && (all != (long long)p.R_d || sh.req < 0)) sh.bad = 1;
  __syncthreads();
}

// Reference exponents and sums of the position's K rows, merged over the
// chunks: wave a < K takes row a, lane l the chunks l, l + 64, ..., then a
// fixed-order wave reduction, so the result does not depend on which
// workgroup computes it.  All threads call; results in sh.Mrow (R) / sh.Srow (S).
template <int K>
__device__ __forceinline__ void cons_row_stats(const Params& p, int64_t pos, int64_t nch, ConsShared& sh) {
  static_assert(K <= kWaves, "one wave per draft row");
  const int lane = threadIdx.x & 63, a = threadIdx.x >> 6;
  if (a < K) {
    const float* src = p.cons_stats + (pos * K + a) * nch * 4;
    float R = -INFINITY;
    for (int64_t c = lane; c < nch; c += 64) R = fmaxf(R, ld_dev(src + c * 4));
    R = wave_max(R);
    double S = 0.0;
    for (int64_t c = lane; c < nch; c += 64)
      S += ldexp(ld_dev(reinterpret_cast<const double*>(src + c * 4 + 2)), max((int)(ld_dev(src + c * 4) - R), -2000));
    S = wave_sum_d(S);
    if (lane == 0) {
      sh.Mrow[a] = R;
      sh.Srow[a] = S;
    }
  }
  __syncthreads();
}

// Writes the outputs of position `pos` from its K x K matrix (one thread):
// the closest pair a < b (lowest on ties) and its state.
template <int K>
__device__ __forceinline__ void cons_write(const Params& p, int64_t pos, const double (&m)[K][K]) {
  if (p.cons_nkl)
#pragma unroll
    for (int a = 0; a < K; ++a)
#pragma unroll
      for (int bb = 0; bb < K; ++bb) p.cons_nkl[pos * K * K + a * K + bb] = (float)m[a][bb];
  double best = INFINITY;
  int pair = -1;
#pragma unroll
  for (int a = 0; a < K; ++a)
#pragma unroll
    for (int bb = a + 1; bb < K; ++bb) {
      const double d = 0.5 * (m[a][bb] + m[bb][a]);
      if (d < best) {
        best = d;
        pair = a * K + bb;
      }
    }
  p.cons_pair[pos] = pair;
  p.cons_state[pos] = best < (double)p.cons_dc ? 1 : (best > (double)p.cons_dd ? 2 : 0);
}

// -1 (and NaN in the matrix) for a position that has no valid answer.
template <int K>
__device__ __forceinline__ void cons_write_invalid(const Params& p, int64_t pos) {
  p.cons_state[pos] = -1;
  p.cons_pair[pos] = -1;
  if (p.cons_nkl)
    for (int k = 0; k < K * K; ++k) p.cons_nkl[pos * K * K + k] = __builtin_nanf("");
}

// Merge of the position's chunk records (one wave; the lanes take chunks l,
// l + 64, ..., then fixed-order wave reductions) into the one-pass matrix
// and its error estimates.  With q_a = 2^(x_a L - R_a) / S_a:
//   KL_ab = c T_ab / S_a - (R_a - R_b) ln 2 - ln(S_a / S_b),
// estimate kKlErr (c Z_ab / S_a + 1) as for the verify KL.  Returns (in every
// lane) whether the exact pass is needed: an estimate above kKlRel of its
// value, or the decision -- a threshold, the closest pair -- within the
// estimates.  Otherwise lane 0 writes the outputs.
template <int K>
__device__ __forceinline__ bool cons_merge(const Params& p, int64_t pos, int64_t nch, float Lhi) {
  constexpr int NP = K * (K - 1);
  const int lane = threadIdx.x & 63;
  const double c = (double)Lhi * kLn2D;
  float R[K];
  double sl[K], tl[NP], zl[NP];
#pragma unroll
  for (int a = 0; a < K; ++a) sl[a] = 0.0;
#pragma unroll
  for (int q = 0; q < NP; ++q) tl[q] = zl[q] = 0.0;
  if (nch <= 64) {  // one chunk per lane: all records in one round of loads
    const int64_t ch = lane;
    const bool has = ch < nch;
    float rc[K];
    double sc[K], tc[NP], zc[NP];
#pragma unroll
    for (int a = 0; a < K; ++a) {
      const float* src = p.cons_stats + ((pos * K + a) * nch + (has ? ch : 0)) * 4;
      rc[a] = ld_dev(src);
      sc[a] = ld_dev(reinterpret_cast<const double*>(src + 2));
    }
    const double* tz = p.cons_tz + (pos * nch + (has ? ch : 0)) * 2 * NP;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      tc[q] = ld_dev(tz + 2 * q);
      zc[q] = ld_dev(tz + 2 * q + 1);
    }
#pragma unroll
    for (int a = 0; a < K; ++a) R[a] = wave_max(has ? rc[a] : -INFINITY);
    if (has) {
#pragma unroll
      for (int a = 0; a < K; ++a) {
        const double f = ldexp(1.0, max((int)(rc[a] - R[a]), -2000));  // exact
        sl[a] = sc[a] * f;
#pragma unroll
        for (int bb = 0; bb < K; ++bb)
          if (bb != a) {
            const int q = cons_pair_index<K>(a, bb);
            tl[q] = tc[q] * f;
            zl[q] = zc[q] * f;
          }
      }
    }
  } else {
#pragma unroll
    for (int a = 0; a < K; ++a) {
      const float* src = p.cons_stats + (pos * K + a) * nch * 4;
      float mx = -INFINITY;
      for (int64_t ch = lane; ch < nch; ch += 64) mx = fmaxf(mx, ld_dev(src + ch * 4));
      R[a] = wave_max(mx);
    }
    for (int64_t ch = lane; ch < nch; ch += 64) {
      double f[K];
#pragma unroll
      for (int a = 0; a < K; ++a) {
        const float* src = p.cons_stats + ((pos * K + a) * nch + ch) * 4;
        f[a] = ldexp(1.0, max((int)(ld_dev(src) - R[a]), -2000));  // exact
        sl[a] += ld_dev(reinterpret_cast<const double*>(src + 2)) * f[a];
      }
      const double* tz = p.cons_tz + (pos * nch + ch) * 2 * NP;
#pragma unroll
      for (int a = 0; a < K; ++a)
#pragma unroll
        for (int bb = 0; bb < K; ++bb)
          if (bb != a) {
            const int q = cons_pair_index<K>(a, bb);
            tl[q] += ld_dev(tz + 2 * q) * f[a];
            zl[q] += ld_dev(tz + 2 * q + 1) * f[a];
          }
    }
  }
  double S[K], T[NP], Z[NP];
#pragma unroll
  for (int a = 0; a < K; ++a) S[a] = wave_sum_d(sl[a]);
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    T[q] = wave_sum_d(tl[q]);
    Z[q] = wave_sum_d(zl[q]);
  }
  const double lnV = log((double)p.V);
  double m[K][K], err[K][K];
  bool need = false;
#pragma unroll
  for (int a = 0; a < K; ++a)
#pragma unroll
    for (int bb = 0; bb < K; ++bb) {
      m[a][bb] = 0.0;
      err[a][bb] = 0.0;
      if (a == bb || p.V == 1) continue;  // one token: both rows are the same point mass
      const int q = cons_pair_index<K>(a, bb);
      const double kl = T[q] / S[a] * c - (double)(R[a] - R[bb]) * kLn2D - log(S[a] / S[bb]);
      const double e = kKlErr * (Z[q] / S[a] * c + 1.0);
      need = need || !(e <= kKlRel * kl);
      m[a][bb] = kl / lnV;
      err[a][bb] = e / lnV;
    }
  double db = INFINITY, eb = 0.0;  // the closest pair's distance and estimate (lowest pair on ties)
  int best = -1;
#pragma unroll
  for (int a = 0; a < K; ++a)
#pragma unroll
    for (int bb = a + 1; bb < K; ++bb) {
      const double d = 0.5 * (m[a][bb] + m[bb][a]);
      if (d < db) {
        db = d;
        eb = 0.5 * (err[a][bb] + err[bb][a]);
        best = a * K + bb;
      }
    }
  need = need || best < 0 || fabs(db - (double)p.cons_dc) <= eb || fabs(db - (double)p.cons_dd) <= eb;
#pragma unroll
  for (int a = 0; a < K; ++a)
#pragma unroll
    for (int bb = a + 1; bb < K; ++bb)  // another pair within the estimates of the closest one
      if (a * K + bb != best && 0.5 * (m[a][bb] + m[bb][a]) - db <= 0.5 * (err[a][bb] + err[bb][a]) + eb) need = true;
  if (!need && lane == 0) cons_write<K>(p, pos, m);
  return need;
}

// Exact sums of one chunk of a position: per ordered pair (a, b), a != b,
// the sum of q_a g(w), w = ln(q_b / q_a) = (x_b - x_a) c + lw_ab, with
// q_a(y) = 2^(x_a L - R_a) / S_a (row statistics in sh.Mrow / sh.Srow).
// One vector of every row at a time, the next vector's loads in flight;
// q_a g(w_ab) and q_b g(w_ba) share the even and odd parts of g's series
// (w_ba = -w_ab exactly).  The workgroup's sums end in sh.d[q][wave].
template <int DT, bool VEC, int K>
__device__ __forceinline__ void cons_exact_chunk(const Params& p, int64_t pos, int64_t chunk, float Lhi, ConsShared& sh) {
  constexpr int P = Elem<DT>::P;
  constexpr int NP = K * (K - 1);
  constexpr int NU = NP / 2;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float c = (float)((double)Lhi * kLn2D);
  const auto load_vec = [&](int k, uint4* q) {
    const int64_t e0 = cons_e0<DT>(chunk, k);
#pragma unroll
    for (int a = 0; a < K; ++a) q[a] = fetch_raw<DT, VEC>(p.target, pos * K + a, p.V, e0);
  };
  uint4 cur[K], nxt[K];
  load_vec(0, cur);
  float ct[K], kt[K], lw[NU];
#pragma unroll
  for (int a = 0; a < K; ++a) {
    ct[a] = sh.Mrow[a];
    kt[a] = (float)(1.0 / sh.Srow[a]);
  }
  {
    int u = 0;
#pragma unroll
    for (int a = 0; a < K; ++a)
#pragma unroll
      for (int bb = a + 1; bb < K; ++bb)
        lw[u++] = (float)((double)(sh.Mrow[a] - sh.Mrow[bb]) * kLn2D + log(sh.Srow[a] / sh.Srow[bb]));
  }
  double acc[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) acc[q] = 0.0;
#pragma unroll 1
  for (int k = 0; k < kConsVec; ++k) {  // fp32 partial sums over one vector (P elements), fp64 beyond
    if (k + 1 < kConsVec) load_vec(k + 1, nxt);
    float v[K][P];
#pragma unroll
    for (int a = 0; a < K; ++a) {
      unpack<DT>(cur[a], v[a]);
      cons_mask<DT, VEC>(v[a], cons_e0<DT>(chunk, k), p.V);
    }
    float part[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) part[q] = 0.f;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      float qv[K];
#pragma unroll
      for (int a = 0; a < K; ++a) qv[a] = __builtin_amdgcn_exp2f(fmaf(v[a][e], Lhi, -ct[a])) * kt[a];
      int u = 0;
#pragma unroll
      for (int a = 0; a < K; ++a)
#pragma unroll
        for (int bb = a + 1; bb < K; ++bb) {
          const float wv = fmaf(v[bb][e] - v[a][e], c, lw[u++]);
          const float w2 = wv * wv;
          float ev = fmaf(w2, 1.0f / 40320.0f, 1.0f / 720.0f);  // g(w) = E + O, g(-w) = E - O (series to w^9)
          ev = fmaf(w2, ev, 1.0f / 24.0f);
          ev = fmaf(w2, ev, 0.5f) * w2;
          float od = fmaf(w2, 1.0f / 362880.0f, 1.0f / 5040.0f);
          od = fmaf(w2, od, 1.0f / 120.0f);
          od = fmaf(w2, od, 1.0f / 6.0f) * (w2 * wv);
          const bool sm = fabsf(wv) < 0.5f;
          const float dq = qv[bb] - qv[a];
          // q_a g(w) = q_b - q_a - q_a w and q_b g(-w) = q_a - q_b + q_b w away from 0
          const float ab = sm ? qv[a] * (ev + od) : fmaf(-qv[a], wv, dq);
          const float ba = sm ? qv[bb] * (ev - od) : fmaf(qv[bb], wv, -dq);
          part[cons_pair_index<K>(a, bb)] += ab;  // positions past the end give 0
          part[cons_pair_index<K>(bb, a)] += ba;
        }
    }
#pragma unroll
    for (int q = 0; q < NP; ++q) acc[q] += (double)part[q];
#pragma unroll
    for (int a = 0; a < K; ++a) cur[a] = nxt[a];
  }
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const double t = wave_sum_d(acc[q]);
    if (lane == 0) sh.d[q][w] = t;
  }
  __syncthreads();
}

// The whole consensus step in one dispatch: one workgroup per (position,
// chunk).  Each sums its chunk of the K rows in one read -- per row s =
// sum 2^(x L - R), per ordered pair t = sum 2^(x_a L - R_a) (x_a - x_b) and
// z, the same with |x_a - x_b| -- against a running integer reference
// exponent R per thread (fmaf(x, L, -R): the single rounding is relative to
// the small exponent where the mass is; when R grows the sums are rescaled by
// an exact power of two, and again to the chunk's largest R).  It writes the
// chunk's records at device scope and counts itself on the position's
// arrival counter; the last workgroup of the position merges the records
// (cons_merge) and, where the one-pass values are not accurate enough, sums
// the exact form over the position's chunks itself.  LDS: the request comes
// from a scan of gamma in LDS (else from k_prep's map and layout flag).
template <int DT, bool VEC, int K, bool LDS>
__global__ __launch_bounds__(kThreads) void k_cons(Params p) {
  __shared__ ConsShared sh;
  constexpr int P = Elem<DT>::P;
  constexpr int NP = K * (K - 1);
  constexpr int NV = K + 2 * NP;  // s per row, then t and z per ordered pair
  const int64_t nch = (p.V + chunk_cons(DT) - 1) / chunk_cons(DT);
  const int64_t pos = blockIdx.x / nch, chunk = blockIdx.x % nch;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t* cnt = p.cnt + pos * kArrStride;
  const uint64_t cnt_cur = threadIdx.x == kClaimThread ? claim_load(cnt) : 0;  // issued before the rows
  ConsReqIn rin{};
  if (LDS) rin = cons_req_load(p);  // issued before the rows: the scan waits for these only
  // a ring of kConsRing vectors of every row in flight: slot k % kConsRing
  // is reloaded with vector k + kConsRing as soon as vector k is unpacked
  uint4 raw[kConsRing][K];
#pragma unroll
  for (int k = 0; k < kConsRing; ++k) {
    const int64_t e0 = cons_e0<DT>(chunk, k);
#pragma unroll
    for (int a = 0; a < K; ++a) raw[k][a] = fetch_raw<DT, VEC>(p.target, pos * K + a, p.V, e0);
  }
  __builtin_amdgcn_sched_barrier(0);  // the loads go out before any of them is used
  // claimed now (its swap runs meanwhile), before this workgroup counts itself
  if (threadIdx.x == kClaimThread) claim_nowait(cnt, cnt_cur, p.epoch);
  bool bad;
  float T;
  if (LDS) {
    cons_find_request(p, pos, rin, sh);
    bad = sh.bad != 0;
    T = bad ? 1.0f : sh.T;
  } else {
    bad = p.hdr[0] != 0;
    T = bad ? 1.0f : p.temp[p.pair2req[pos]];
  }
  const bool valid = !bad && temp_ok(T);
  const float Lhi = valid ? (float)(kLog2eD / (double)T) : 1.0f;
  int R[K];
  double acc[NV];
#pragma unroll
  for (int a = 0; a < K; ++a) R[a] = kConsRNone;
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.0;
  const auto rescale = [&](int a, int sh_exp) {
    acc[a] = ldexp(acc[a], sh_exp);
#pragma unroll
    for (int bb = 0; bb < K; ++bb)
      if (bb != a) {
        const int q = K + 2 * cons_pair_index<K>(a, bb);
        acc[q] = ldexp(acc[q], sh_exp);
        acc[q + 1] = ldexp(acc[q + 1], sh_exp);
      }
  };
#pragma unroll
  for (int k = 0; k < kConsVec; ++k) {
    const int64_t e0 = cons_e0<DT>(chunk, k);
    float v[K][P];
#pragma unroll
    for (int a = 0; a < K; ++a) unpack<DT>(raw[k % kConsRing][a], v[a]);
    if (k + kConsRing < kConsVec) {
      const int64_t e1 = cons_e0<DT>(chunk, k + kConsRing);
#pragma unroll
      for (int a = 0; a < K; ++a) raw[k % kConsRing][a] = fetch_raw<DT, VEC>(p.target, pos * K + a, p.V, e1);
    }
    if (e0 < p.V) {  // vectors wholly past the row's end add nothing
      float nr[K];  // -R of each row after this vector
#pragma unroll
      for (int a = 0; a < K; ++a) {
        if (!VEC) cons_mask<DT, VEC>(v[a], e0, p.V);  // rows of whole vectors: this one is inside
        float vm = v[a][0];
#pragma unroll
        for (int e = 1; e < P; ++e) vm = fmaxf(vm, v[a][e]);
        const int rn = max(R[a], cons_ref(vm, Lhi));
        rescale(a, max(R[a] - rn, -2000));  // 0 when unchanged; the first vector scales zeros
        R[a] = rn;
        nr[a] = -(float)rn;
      }
      float part[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) part[i] = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        float ev[K];
#pragma unroll
        for (int a = 0; a < K; ++a) {
          ev[a] = __builtin_amdgcn_exp2f(fmaf(v[a][e], Lhi, nr[a]));
          part[a] += ev[a];
        }
#pragma unroll
        for (int a = 0; a < K; ++a)
#pragma unroll
          for (int bb = a + 1; bb < K; ++bb) {
            const float d = v[a][e] - v[bb][e];
            const int qa = K + 2 * cons_pair_index<K>(a, bb), qb = K + 2 * cons_pair_index<K>(bb, a);
            part[qa] = fmaf(ev[a], d, part[qa]);
            part[qa + 1] = fmaf(ev[a], fabsf(d), part[qa + 1]);
            part[qb] = fmaf(-ev[bb], d, part[qb]);
            part[qb + 1] = fmaf(ev[bb], fabsf(d), part[qb + 1]);
          }
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[i] += (double)part[i];
    }
    __builtin_amdgcn_sched_barrier(0);  // one vector's terms at a time: bounded registers
  }
  // the chunk's reference of every row, then each thread's sums rescaled to it
#pragma unroll
  for (int a = 0; a < K; ++a) {
    const int rw = wave_max_int(R[a]);
    if (lane == 0) sh.m[a][w] = (float)rw;  // integers below 2^24: exact
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < K; ++a) {
    float Rc = sh.m[a][0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) Rc = fmaxf(Rc, sh.m[a][k]);
    rescale(a, max(R[a] - (int)Rc, -2000));  // threads that saw no element hold zeros
    if (threadIdx.x == 0) sh.Mrow[a] = Rc;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const double t = wave_sum_d(acc[i]);
    if (lane == 0) sh.d[i][w] = t;
  }
  __syncthreads();
  if (threadIdx.x < NV) {  // the chunk's records, read by the position's last workgroup
    const int i = threadIdx.x;
    double t = sh.d[i][0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) t += sh.d[i][k];
    if (i < K) {
      float* dst = p.cons_stats + ((pos * K + i) * nch + chunk) * 4;
      st_dev(dst, sh.Mrow[i]);
      st_dev(reinterpret_cast<double*>(dst + 2), t);
    } else {
      st_dev(p.cons_tz + (pos * nch + chunk) * 2 * NP + (i - K), t);
    }
  }
  if (!arrive_last(cnt, (int)nch, sh)) return;
  // the position's last workgroup
  if (!valid) {
    if (threadIdx.x == 0) cons_write_invalid<K>(p, pos);
    return;
  }
  if (w == 0) {
    const bool need = cons_merge<K>(p, pos, nch, Lhi);
    if (lane == 0) sh.need = need ? 1 : 0;
  }
  __syncthreads();
  if (!sh.need) return;
  // exact form over the position's chunks, summed in chunk order
  cons_row_stats<K>(p, pos, nch, sh);
  if (threadIdx.x < NP) sh.tot[threadIdx.x] = 0.0;
  for (int64_t ch = 0; ch < nch; ++ch) {
    cons_exact_chunk<DT, VEC, K>(p, pos, ch, Lhi, sh);
    if (threadIdx.x < NP) {
      double t = sh.d[threadIdx.x][0];
#pragma unroll
      for (int k = 1; k < kWaves; ++k) t += sh.d[threadIdx.x][k];
      sh.tot[threadIdx.x] += t;
    }
    __syncthreads();  // sh.d is reused by the next chunk
  }
  if (threadIdx.x == 0) {
    const double lnV = log((double)p.V);
    double m[K][K];
#pragma unroll
    for (int a = 0; a < K; ++a)
#pragma unroll
      for (int bb = 0; bb < K; ++bb)
        m[a][bb] = (a == bb || p.V == 1) ? 0.0 : sh.tot[cons_pair_index<K>(a, bb)] / lnV;
    cons_write<K>(p, pos, m);
  }
}

// ----------------------------------------------------------------------------
// plain-read probe (measurement aid): streams a buffer with the statistics
// pass's partition -- static contiguous ranges of 16 KB items, one per
// workgroup, the next item's loads in flight while the current one is folded
// -- and does nothing with the data but an xor, so that its time is what the
// GPU needs to read that many bytes in that pattern.
// ----------------------------------------------------------------------------

constexpr int kProbeVecs = 4;  // 16-byte vectors per thread per item: 16 KB per item

__global__ __launch_bounds__(kThreads) void k_read_probe(const uint4* buf, int64_t nitems, uint32_t* sink) {
  const int64_t G = gridDim.x, wg = blockIdx.x;
  int64_t i = wg * nitems / G;
  const int64_t e = (wg + 1) * nitems / G;
  uint32_t acc = 0;
  uint4 a[kProbeVecs], b[kProbeVecs];
  const auto issue = [&](int64_t it, uint4* q) {
#pragma unroll
    for (int k = 0; k < kProbeVecs; ++k) q[k] = buf[(it * kProbeVecs + k) * kThreads + threadIdx.x];
  };
  const auto fold = [&](const uint4* q) {
#pragma unroll
    for (int k = 0; k < kProbeVecs; ++k) acc ^= q[k].x ^ q[k].y ^ q[k].z ^ q[k].w;
  };
  if (i < e) issue(i, a);
  for (; i < e; i += 2) {
    if (i + 1 < e) issue(i + 1, b);
    fold(a);
    if (i + 1 >= e) break;
    if (i + 2 < e) issue(i + 2, a);
    fold(b);
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads; any racing value will do
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

// Statistics partition over G workgroups (at most one per item): fills
// p.stats_grid and p.grp_log2, the lanes that merge one task's partials.
void set_stats_grid(Params& p, int64_t G) {
  const int64_t N = (int64_t)p.n_task * p.nch;
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
  p.maxseg = (int32_t)maxseg;
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
int stats_occupancy_mode(int mode, bool wz) {
  switch (mode) {
    case SV_MODE_STOCHASTIC:
      return wz ? stats_occupancy<DT, VEC, SV_MODE_STOCHASTIC, true>()
                : stats_occupancy<DT, VEC, SV_MODE_STOCHASTIC, false>();
    case SV_MODE_GREEDY:
    case SV_MODE_BLOCK: return stats_occupancy<DT, VEC, SV_MODE_GREEDY, false>();  // the same pass
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
    case SV_MODE_GREEDY:
    case SV_MODE_BLOCK: stats_launch<DT, VEC, SV_MODE_GREEDY, false>(p, s, e0, e1); break;  // argmax of every row
    case SV_MODE_NKL: stats_launch<DT, VEC, SV_MODE_NKL, false>(p, s, e0, e1); break;
    default: stats_launch<DT, VEC, SV_MODE_TREE_GREEDY, false>(p, s, e0, e1); break;
  }
}
template <int DT, bool VEC>
void decide_dispatch(const Params& p, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)p.B * p.helpers)), blk(kThreads);
  switch (p.mode) {
    case SV_MODE_STOCHASTIC: hipLaunchKernelGGL((k_decide<DT, VEC, SV_MODE_STOCHASTIC>), grid, blk, 0, s, p); break;
    case SV_MODE_GREEDY: hipLaunchKernelGGL((k_decide<DT, VEC, SV_MODE_GREEDY>), grid, blk, 0, s, p); break;
    case SV_MODE_BLOCK: hipLaunchKernelGGL((k_decide<DT, VEC, SV_MODE_BLOCK>), grid, blk, 0, s, p); break;
    case SV_MODE_NKL:
      if (p.nkl_pos) hipLaunchKernelGGL((k_decide<DT, VEC, SV_MODE_NKL, true>), grid, blk, 0, s, p);
      else hipLaunchKernelGGL((k_decide<DT, VEC, SV_MODE_NKL>), grid, blk, 0, s, p);
      break;
    default: hipLaunchKernelGGL((k_decide<DT, VEC, SV_MODE_TREE_GREEDY>), grid, blk, 0, s, p); break;
  }
}

}  // namespace

// Helpers per request: enough workgroups to fill the device once (resident
// k_decide workgroups / B), at most one per slice; each helper then streams a
// contiguous run of slices.
template <int DT, bool VEC, int MODE>
int decide_capacity() {
  static int occ = 0;  // same value from every thread: a race is benign
  if (occ == 0) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, k_decide<DT, VEC, MODE>, kThreads, 0) != hipSuccess || o <= 0)
      o = 1;
    occ = o;
  }
  return occ * num_cus();
}

int plan_decide(Params& p, bool vec) {
  p.nslices = (int32_t)((p.V + chunk_t(p.dtype) - 1) / chunk_t(p.dtype));
  if (p.mode != SV_MODE_STOCHASTIC) {
    p.helpers = 1;
    p.slices_per_helper = p.nslices;
    return 0;
  }
  int cap;
  if (p.dtype == SV_DTYPE_BF16)
    cap = vec ? decide_capacity<SV_DTYPE_BF16, true, SV_MODE_STOCHASTIC>()
              : decide_capacity<SV_DTYPE_BF16, false, SV_MODE_STOCHASTIC>();
  else
    cap = vec ? decide_capacity<SV_DTYPE_F32, true, SV_MODE_STOCHASTIC>()
              : decide_capacity<SV_DTYPE_F32, false, SV_MODE_STOCHASTIC>();
  int64_t H = ((int64_t)cap + p.B - 1) / p.B;
  if (H > p.nslices) H = p.nslices;
  if (H < 1) H = 1;
  const int64_t spp = (p.nslices + H - 1) / H;
  p.slices_per_helper = (int32_t)spp;
  p.helpers = (int32_t)((p.nslices + spp - 1) / spp);  // no helper without a slice
  return 0;
}

int plan_stats(Params& p, bool vec) {
  int occ;
  const bool wz = p.want_kl != 0;
  if (p.dtype == SV_DTYPE_BF16)
    occ = vec ? stats_occupancy_mode<SV_DTYPE_BF16, true>(p.mode, wz)
              : stats_occupancy_mode<SV_DTYPE_BF16, false>(p.mode, wz);
  else
    occ = vec ? stats_occupancy_mode<SV_DTYPE_F32, true>(p.mode, wz)
              : stats_occupancy_mode<SV_DTYPE_F32, false>(p.mode, wz);
  set_stats_grid(p, (int64_t)occ * num_cus());
  return 0;
}

template <int DT, bool VEC>
int fused_occupancy(int mode) {
  static int occ[SV_MODE_BLOCK + 1] = {0, 0, 0, 0, 0};  // same value from every thread: a race is benign
  int& o = occ[mode];
  if (o == 0) {
    int v = 0;
    hipError_t e;
    switch (mode) {
      case SV_MODE_STOCHASTIC:
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, k_fused<DT, VEC, SV_MODE_STOCHASTIC>, kThreads, 0);
        break;
      case SV_MODE_GREEDY:
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, k_fused<DT, VEC, SV_MODE_GREEDY>, kThreads, 0);
        break;
      case SV_MODE_TREE_GREEDY:
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, k_fused<DT, VEC, SV_MODE_TREE_GREEDY>, kThreads, 0);
        break;
      default:
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, k_fused<DT, VEC, SV_MODE_BLOCK>, kThreads, 0);
        break;
    }
    o = (e == hipSuccess && v > 0) ? v : 1;
  }
  return o;
}

int plan_fused(Params& p, bool vec) {
  if (p.mode == SV_MODE_NKL) return 0;
  // tree and block requests keep one entry per position in LDS
  if ((p.mode == SV_MODE_TREE_GREEDY || p.mode == SV_MODE_BLOCK) && p.max_gamma >= kFusedNodes) return 0;
  const int o = p.dtype == SV_DTYPE_BF16 ? (vec ? fused_occupancy<SV_DTYPE_BF16, true>(p.mode)
                                                : fused_occupancy<SV_DTYPE_BF16, false>(p.mode))
                                         : (vec ? fused_occupancy<SV_DTYPE_F32, true>(p.mode)
                                                : fused_occupancy<SV_DTYPE_F32, false>(p.mode));
  // at most kFusedPerCu workgroups per compute unit: the units serve their
  // workgroups' loads roughly in age order, so the newest stream last.  With
  // the statistics waves paced by their remaining work, four per unit measure
  // best on the Llama-3-shaped batch (31.5 us per step; 31.9 at three, 32.8
  // at two)
  const int64_t cap = (int64_t)(o < kFusedPerCu ? o : kFusedPerCu) * num_cus();
  // Single dispatch only while the statistics pass is short: it saves the
  // second launch and the hand-over to the decision (the 82 MB Llama-3-shaped
  // batch: 7 items per workgroup, about 2.5 us per step), but it streams with
  // fewer workgroups per CU than k_stats and its helpers poll while others
  // stream, which costs more than that on long passes (the 680 MB ragged
  // batch, 55 items per workgroup: about 10 us).
  if ((int64_t)p.n_task * p.nch > kFusedItemsPerWg * cap) return 0;
  set_stats_grid(p, cap);
  p.nslices = (int32_t)((p.V + chunk_t(p.dtype) - 1) / chunk_t(p.dtype));
  if (p.mode != SV_MODE_STOCHASTIC) {
    // one helper per request: no terminal draw
    p.helpers = 1;
    p.slices_per_helper = p.nslices;
  } else {
    // helpers per request: what the resident grid holds, at most one per slice
    int64_t H = cap / p.B;
    if (H > p.nslices) H = p.nslices;
    if (H < 1) H = 1;
    const int64_t spp = (p.nslices + H - 1) / H;
    p.slices_per_helper = (int32_t)spp;
    p.helpers = (int32_t)((p.nslices + spp - 1) / spp);
  }
  // one helper role per workgroup (a role loop would cost registers), so a
  // batch above the resident grid (B x H > cap) gets helpers that start as
  // others finish
  const int64_t roles = (int64_t)p.B * p.helpers;
  return (int)(roles > p.stats_grid ? roles : p.stats_grid);
}

template <int DT, bool VEC>
void fused_dispatch(const Params& p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (p.mode) {
    case SV_MODE_STOCHASTIC: launch_timed(k_fused<DT, VEC, SV_MODE_STOCHASTIC>, grid, p, s, e0, e1); break;
    case SV_MODE_GREEDY: launch_timed(k_fused<DT, VEC, SV_MODE_GREEDY>, grid, p, s, e0, e1); break;
    case SV_MODE_TREE_GREEDY: launch_timed(k_fused<DT, VEC, SV_MODE_TREE_GREEDY>, grid, p, s, e0, e1); break;
    default: launch_timed(k_fused<DT, VEC, SV_MODE_BLOCK>, grid, p, s, e0, e1); break;
  }
}

int launch_fused(const Params& p, bool vec, int grid, void* stream, void* ev_start, void* ev_stop) {
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0 = (hipEvent_t)ev_start, e1 = (hipEvent_t)ev_stop;
  if (p.dtype == SV_DTYPE_BF16) {
    if (vec) fused_dispatch<SV_DTYPE_BF16, true>(p, dim3(grid), s, e0, e1);
    else fused_dispatch<SV_DTYPE_BF16, false>(p, dim3(grid), s, e0, e1);
  } else {
    if (vec) fused_dispatch<SV_DTYPE_F32, true>(p, dim3(grid), s, e0, e1);
    else fused_dispatch<SV_DTYPE_F32, false>(p, dim3(grid), s, e0, e1);
  }
  return (int)hipGetLastError();
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

template <int DT, bool VEC>
int sample_capacity() {
  static int occ = 0;  // same value from every thread: a race is benign
  if (occ == 0) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, k_sample<DT, VEC>, kThreads, 0) != hipSuccess || o <= 0)
      o = 1;
    occ = o;
  }
  return occ * num_cus();
}

int plan_sample(Params& p, bool vec) {
  p.nslices = (int32_t)((p.V + chunk_t(p.dtype) - 1) / chunk_t(p.dtype));
  int cap;
  if (p.dtype == SV_DTYPE_BF16)
    cap = vec ? sample_capacity<SV_DTYPE_BF16, true>() : sample_capacity<SV_DTYPE_BF16, false>();
  else
    cap = vec ? sample_capacity<SV_DTYPE_F32, true>() : sample_capacity<SV_DTYPE_F32, false>();
  // enough helpers to fill the device once, at most one per slice
  int64_t H = ((int64_t)cap + p.B - 1) / p.B;
  if (H > p.nslices) H = p.nslices;
  if (H < 1) H = 1;
  const int64_t spp = (p.nslices + H - 1) / H;
  p.slices_per_helper = (int32_t)spp;
  p.helpers = (int32_t)((p.nslices + spp - 1) / spp);
  return 0;
}

int launch_sample(const Params& p, bool vec, void* stream, void* ev_start, void* ev_stop) {
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0 = (hipEvent_t)ev_start, e1 = (hipEvent_t)ev_stop;
  const dim3 grid((unsigned)((int64_t)p.B * p.helpers));
  if (p.dtype == SV_DTYPE_BF16) {
    if (vec) launch_timed(k_sample<SV_DTYPE_BF16, true>, grid, p, s, e0, e1);
    else launch_timed(k_sample<SV_DTYPE_BF16, false>, grid, p, s, e0, e1);
  } else {
    if (vec) launch_timed(k_sample<SV_DTYPE_F32, true>, grid, p, s, e0, e1);
    else launch_timed(k_sample<SV_DTYPE_F32, false>, grid, p, s, e0, e1);
  }
  return (int)hipGetLastError();
}

template <int DT, bool VEC, int K>
int topk_capacity() {
  static int occ = 0;  // same value from every thread: a race is benign
  if (occ == 0) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, k_topk<DT, VEC, K>, kThreads, 0) != hipSuccess || o <= 0)
      o = 1;
    occ = o;
  }
  return occ * num_cus();
}

// the per-thread list length: k rounded up to a power of two
int topk_lanes(int k) { return k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : 16; }

template <int DT, bool VEC>
void topk_dispatch(const Params& p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1, int* cap) {
  switch (topk_lanes(p.topk)) {
    case 1: if (cap) *cap = topk_capacity<DT, VEC, 1>(); else launch_timed(k_topk<DT, VEC, 1>, grid, p, s, e0, e1); break;
    case 2: if (cap) *cap = topk_capacity<DT, VEC, 2>(); else launch_timed(k_topk<DT, VEC, 2>, grid, p, s, e0, e1); break;
    case 4: if (cap) *cap = topk_capacity<DT, VEC, 4>(); else launch_timed(k_topk<DT, VEC, 4>, grid, p, s, e0, e1); break;
    case 8: if (cap) *cap = topk_capacity<DT, VEC, 8>(); else launch_timed(k_topk<DT, VEC, 8>, grid, p, s, e0, e1); break;
    default: if (cap) *cap = topk_capacity<DT, VEC, 16>(); else launch_timed(k_topk<DT, VEC, 16>, grid, p, s, e0, e1); break;
  }
}

void topk_any(const Params& p, bool vec, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1, int* cap) {
  if (p.dtype == SV_DTYPE_BF16) {
    if (vec) topk_dispatch<SV_DTYPE_BF16, true>(p, grid, s, e0, e1, cap);
    else topk_dispatch<SV_DTYPE_BF16, false>(p, grid, s, e0, e1, cap);
  } else {
    if (vec) topk_dispatch<SV_DTYPE_F32, true>(p, grid, s, e0, e1, cap);
    else topk_dispatch<SV_DTYPE_F32, false>(p, grid, s, e0, e1, cap);
  }
}

int plan_topk(Params& p, bool vec) {
  p.nslices = (int32_t)((p.V + chunk_t(p.dtype) - 1) / chunk_t(p.dtype));
  int cap = 1;
  topk_any(p, vec, dim3(1), nullptr, nullptr, nullptr, &cap);
  // enough helpers to fill the device once, at most one per slice, and at
  // most kThreads / k so that the last helper holds one candidate per thread
  int64_t H = ((int64_t)cap + p.B - 1) / p.B;
  if (H > p.nslices) H = p.nslices;
  if (p.dtype == SV_DTYPE_BF16 && H < (p.nslices + 7) / 8) H = (p.nslices + 7) / 8;  // 16-bit local indices
  if (H > kThreads / p.topk) H = kThreads / p.topk;
  if (H < 1) H = 1;
  const int64_t spp = (p.nslices + H - 1) / H;
  p.slices_per_helper = (int32_t)spp;
  p.helpers = (int32_t)((p.nslices + spp - 1) / spp);
  return 0;
}

int launch_topk(const Params& p, bool vec, void* stream, void* ev_start, void* ev_stop) {
  topk_any(p, vec, dim3((unsigned)((int64_t)p.B * p.helpers)), (hipStream_t)stream, (hipEvent_t)ev_start,
           (hipEvent_t)ev_stop, nullptr);
  return (int)hipGetLastError();
}

int launch_read_probe(const void* buf, int64_t bytes, int wgs_per_cu, void* sink, void* stream, void* ev_start,
                      void* ev_stop) {
  const int64_t item = (int64_t)kProbeVecs * kThreads * 16;
  const int64_t nitems = bytes / item;
  const dim3 grid((unsigned)((int64_t)wgs_per_cu * num_cus()));
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0 = (hipEvent_t)ev_start, e1 = (hipEvent_t)ev_stop;
  const uint4* b = static_cast<const uint4*>(buf);
  uint32_t* k = static_cast<uint32_t*>(sink);
  if (e0 && e1) hipExtLaunchKernelGGL(k_read_probe, grid, dim3(kThreads), 0, s, e0, e1, 0, b, nitems, k);
  else hipLaunchKernelGGL(k_read_probe, grid, dim3(kThreads), 0, s, b, nitems, k);
  return (int)hipGetLastError();
}

namespace {
template <int DT, bool VEC, int K>
void cons_launch(const Params& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int64_t nch = (p.V + chunk_cons(DT) - 1) / chunk_cons(DT);
  const dim3 grid((unsigned)((int64_t)p.R_d * nch)), blk(kThreads);
  // e0 / e1 take the dispatch's own start and end timestamps
  if (p.cons_lds) {
    if (e0 && e1) hipExtLaunchKernelGGL((k_cons<DT, VEC, K, true>), grid, blk, 0, s, e0, e1, 0, p);
    else hipLaunchKernelGGL((k_cons<DT, VEC, K, true>), grid, blk, 0, s, p);
  } else {
    if (e0 && e1) hipExtLaunchKernelGGL((k_cons<DT, VEC, K, false>), grid, blk, 0, s, e0, e1, 0, p);
    else hipLaunchKernelGGL((k_cons<DT, VEC, K, false>), grid, blk, 0, s, p);
  }
}
template <int DT, bool VEC>
void cons_k(const Params& p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (p.cons_k) {
    case 2: cons_launch<DT, VEC, 2>(p, s, e0, e1); break;
    case 3: cons_launch<DT, VEC, 3>(p, s, e0, e1); break;
    default: cons_launch<DT, VEC, 4>(p, s, e0, e1); break;
  }
}
}  // namespace

int launch_consensus(const Params& p, bool vec, void* stream, void* ev_start, void* ev_stop) {
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0 = (hipEvent_t)ev_start, e1 = (hipEvent_t)ev_stop;
  if (!p.cons_lds) hipLaunchKernelGGL(k_prep, dim3(1), dim3(kPrepThreads), 0, s, p);
  if (p.R_d == 0 && e0 && e1) {  // nothing to stream: the two events become plain markers
    hipError_t e = hipEventRecord(e0, s);
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e != hipSuccess) return (int)e;
  }
  if (p.R_d > 0) {
    if (p.dtype == SV_DTYPE_BF16) {
      if (vec) cons_k<SV_DTYPE_BF16, true>(p, s, e0, e1);
      else cons_k<SV_DTYPE_BF16, false>(p, s, e0, e1);
    } else {
      if (vec) cons_k<SV_DTYPE_F32, true>(p, s, e0, e1);
      else cons_k<SV_DTYPE_F32, false>(p, s, e0, e1);
    }
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

template <int DT, bool VEC>
static void refine_dispatch(const Params& p, hipStream_t s, dim3 grid) {
  if (p.mode == SV_MODE_NKL && p.nkl_pos)
    hipLaunchKernelGGL((k_refine<DT, VEC, SV_MODE_NKL, true>), grid, dim3(kThreads), 0, s, p);
  else if (p.mode == SV_MODE_NKL)
    hipLaunchKernelGGL((k_refine<DT, VEC, SV_MODE_NKL>), grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL((k_refine<DT, VEC, SV_MODE_STOCHASTIC>), grid, dim3(kThreads), 0, s, p);
}

int launch_refine(const Params& p, bool vec, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  // the queue length is known on the device only: one workgroup per resident slot
  const dim3 grid((unsigned)(4 * num_cus()));
  if (p.dtype == SV_DTYPE_BF16) {
    if (vec) refine_dispatch<SV_DTYPE_BF16, true>(p, s, grid);
    else refine_dispatch<SV_DTYPE_BF16, false>(p, s, grid);
  } else {
    if (vec) refine_dispatch<SV_DTYPE_F32, true>(p, s, grid);
    else refine_dispatch<SV_DTYPE_F32, false>(p, s, grid);
  }
  return (int)hipGetLastError();
}

}  // namespace sv
