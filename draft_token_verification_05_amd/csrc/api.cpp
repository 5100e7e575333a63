// C-ABI entry points of libspecverify: argument validation, workspace layout,
// launch sequence.  Declared in include/specverify.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "specverify_probe.h"
#include "sv_internal.h"

namespace {

thread_local char g_hip_error[256] = "";

// Polls of a statistics partial (single dispatch) before a helper computes it
// itself (when cfg->wait_polls is 0): a few milliseconds, far above the normal
// wait of a few microseconds.
constexpr int32_t kDefaultWaitPolls = 4096;

// Epochs that tag the fused kernel's partials and the helpers' arrival
// counters: one per call, never 0 or 0xFFFFFFFF (the words of a zero-filled
// or 0xFF-filled buffer).  The start differs between processes, so a
// workspace handed between them does not meet its own old tags.
uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{
      (uint32_t)std::chrono::steady_clock::now().time_since_epoch().count() * 2654435761u};
  uint32_t e;
  do e = counter.fetch_add(1u, std::memory_order_relaxed) + 1u;
  while (e == 0u || e == 0xFFFFFFFFu);
  return e;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Host-side checks of everything that needs no device data.
int validate(const void* target, const void* draft, const int32_t* tokens, const int32_t* gamma, const float* temp,
             const float* ua, const float* ur, int32_t mode, float delta, const int32_t* parents,
             const int32_t* out_tokens, const int32_t* out_num, const float* out_nkl, const sv_config* cfg) {
  if (!cfg || cfg->struct_size != sizeof(sv_config) || cfg->wait_polls < 0) return SV_EINVAL;
  if (cfg->batch <= 0 || cfg->vocab <= 0) return SV_EINVAL;
  if (cfg->dtype != SV_DTYPE_F32 && cfg->dtype != SV_DTYPE_BF16) return SV_EINVAL;
  if (mode < SV_MODE_STOCHASTIC || mode > SV_MODE_BLOCK) return SV_EINVAL;
  if (cfg->max_gamma < 0) return SV_EINVAL;
  if (mode == SV_MODE_BLOCK && cfg->block_min_len < 0) return SV_EINVAL;
  if (cfg->max_gamma > SV_MAX_GAMMA) return SV_EUNSUPPORTED;
  const int64_t R_d = cfg->total_draft_rows;
  if (R_d < 0 || R_d > (int64_t)cfg->batch * cfg->max_gamma) return SV_EINVAL;
  if (R_d + cfg->batch > INT32_MAX) return SV_EUNSUPPORTED;
  const int64_t nch_a = (cfg->vocab + sv::chunk_a(cfg->dtype) - 1) / sv::chunk_a(cfg->dtype);
  const int64_t nch_t = (cfg->vocab + sv::chunk_t(cfg->dtype) - 1) / sv::chunk_t(cfg->dtype);
  // grids and flat indices: statistics partials, decision helpers, KL slice sums
  if ((R_d + cfg->batch) * nch_a > INT32_MAX || (int64_t)cfg->batch * nch_t > INT32_MAX || R_d * nch_t > INT32_MAX)
    return SV_EUNSUPPORTED;

  const bool soft = mode == SV_MODE_STOCHASTIC || mode == SV_MODE_NKL;
  if (!target || !gamma || !out_tokens || !out_num) return SV_EINVAL;
  if (R_d > 0 && !tokens) return SV_EINVAL;
  if (soft && R_d > 0 && !draft) return SV_EINVAL;
  if (soft && !temp) return SV_EINVAL;
  if (mode == SV_MODE_STOCHASTIC && (!ur || (R_d > 0 && !ua))) return SV_EINVAL;
  if (mode == SV_MODE_NKL && (!std::isfinite(delta) || (R_d > 0 && !out_nkl))) return SV_EINVAL;
  if (mode == SV_MODE_NKL && cfg->nkl_position &&
      !(std::isfinite(cfg->nkl_alpha) && std::isfinite(cfg->nkl_delta_max) && aligned(cfg->nkl_position, 4)))
    return SV_EINVAL;
  if (mode == SV_MODE_TREE_GREEDY && R_d > 0 && !parents) return SV_EINVAL;

  const size_t es = (size_t)sv::elem_size(cfg->dtype);
  if (!aligned(target, es) || (draft && !aligned(draft, es))) return SV_EINVAL;
  const void* p4[] = {tokens, gamma, temp, ua, ur, parents, out_tokens, out_num, out_nkl, cfg->out_p_x,
                      cfg->out_q_x, cfg->out_resid_mass, cfg->out_tree_node};
  for (const void* p : p4)
    if (p && !aligned(p, 4)) return SV_EINVAL;

  const sv::Layout L = sv::make_layout(cfg->batch, cfg->vocab, cfg->dtype, R_d);
  if (!cfg->workspace || cfg->workspace_bytes < L.total || !aligned(cfg->workspace, 256)) return SV_EWORKSPACE;
  return SV_OK;
}

int hip_fail(hipError_t e) {
  std::snprintf(g_hip_error, sizeof(g_hip_error), "HIP error: %s (%d)", hipGetErrorString(e), (int)e);
  return SV_EHIP;
}

}  // namespace

// Scratch of spec_verify_noalloc: file-scope device memory, one copy on every
// GPU the library runs on, held until the process ends.  In host code this
// name is only a handle for hipGetSymbolAddress; the device address of the
// current GPU's copy comes from noalloc_scratch().
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current GPU's copy of `scratch`, looked up once per
// device (with that device current) and kept.
int noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return SV_EUNSUPPORTED;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e);
      if (!ptr) return hip_fail(hipErrorInvalidSymbol);
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return SV_OK;
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_size(const sv_config* cfg) {
  if (!cfg || cfg->struct_size != sizeof(sv_config)) return 0;
  if (cfg->batch <= 0 || cfg->vocab <= 0 || cfg->total_draft_rows < 0 || cfg->max_gamma < 0) return 0;
  if (cfg->dtype != SV_DTYPE_F32 && cfg->dtype != SV_DTYPE_BF16) return 0;
  return sv::make_layout(cfg->batch, cfg->vocab, cfg->dtype, cfg->total_draft_rows).total;
}

const char* spec_verify_status_string(int status) {
  switch (status) {
    case SV_OK: return "SV_OK: success";
    case SV_EINVAL: return "SV_EINVAL: invalid argument";
    case SV_EUNSUPPORTED: return "SV_EUNSUPPORTED: configuration not supported";
    case SV_EWORKSPACE:
      return "SV_EWORKSPACE: workspace missing, misaligned or too small (spec_verify_noalloc: the configuration "
             "needs more than SV_NOALLOC_SCRATCH_BYTES of scratch)";
    case SV_EHIP: return g_hip_error[0] ? g_hip_error : "SV_EHIP: HIP launch failure";
    default: return "unknown status";
  }
}

int spec_verify_version(void) { return SPECVERIFY_VERSION; }

int spec_verify_single_dispatch(const sv_config* cfg, int32_t mode, int32_t with_nkl) {
  if (!cfg || cfg->struct_size != sizeof(sv_config) || cfg->batch <= 0 || cfg->vocab <= 0 ||
      cfg->total_draft_rows < 0 || (cfg->dtype != SV_DTYPE_F32 && cfg->dtype != SV_DTYPE_BF16) ||
      mode < SV_MODE_STOCHASTIC || mode > SV_MODE_BLOCK)
    return SV_EINVAL;
  if (mode == SV_MODE_NKL || (mode == SV_MODE_STOCHASTIC && with_nkl) || cfg->batch > sv::kLdsBatch) return 0;
  if (cfg->total_draft_rows * (int64_t)((cfg->vocab + sv::chunk_stats(cfg->dtype, mode) - 1) /
                                        sv::chunk_stats(cfg->dtype, mode)) > INT32_MAX)
    return 0;
  sv::Params p{};
  p.B = cfg->batch;
  p.V = cfg->vocab;
  p.dtype = cfg->dtype;
  p.mode = mode;
  p.R_d = (int32_t)cfg->total_draft_rows;
  p.max_gamma = cfg->max_gamma;
  p.n_task = mode == SV_MODE_STOCHASTIC ? p.R_d : p.R_d + p.B;
  p.nch = (int32_t)((p.V + sv::chunk_stats(p.dtype, mode) - 1) / sv::chunk_stats(p.dtype, mode));
  // the vector-load variant: the one whose occupancy the plan uses for aligned rows
  const bool vec = ((size_t)p.V * (size_t)sv::elem_size(p.dtype)) % 16 == 0;
  return sv::plan_fused(p, vec) > 0 ? 1 : 0;
}

int spec_verify(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                const int32_t* gamma_per_req, const float* temperature, const float* u_accept,
                const float* u_resample, int32_t mode, float delta, const int32_t* tree_parents,
                int32_t* out_tokens, int32_t* out_num_accepted, float* out_nkl, const sv_config* cfg) {
  const int st = validate(target_logits, draft_logits, draft_tokens, gamma_per_req, temperature, u_accept,
                          u_resample, mode, delta, tree_parents, out_tokens, out_num_accepted, out_nkl, cfg);
  if (st != SV_OK) return st;

  const int32_t B = cfg->batch, V = cfg->vocab;
  const int64_t R_d = cfg->total_draft_rows;
  const sv::Layout L = sv::make_layout(B, V, cfg->dtype, R_d);
  char* ws = static_cast<char*>(cfg->workspace);

  sv::Params p{};
  p.target = target_logits;
  p.draft = draft_logits;
  p.tokens = draft_tokens;
  p.gamma = gamma_per_req;
  p.temp = temperature;
  p.ua = u_accept;
  p.ur = u_resample;
  p.parents = tree_parents;
  p.out_tokens = out_tokens;
  p.out_num = out_num_accepted;
  p.out_nkl = (mode == SV_MODE_STOCHASTIC || mode == SV_MODE_NKL) ? out_nkl : nullptr;
  const bool soft = mode == SV_MODE_STOCHASTIC || mode == SV_MODE_NKL;
  p.out_p_x = soft ? cfg->out_p_x : nullptr;
  p.out_q_x = soft ? cfg->out_q_x : nullptr;
  p.out_resid = mode == SV_MODE_STOCHASTIC ? cfg->out_resid_mass : nullptr;
  p.out_tree_node = mode == SV_MODE_TREE_GREEDY ? cfg->out_tree_node : nullptr;
  p.B = B;
  p.V = V;
  p.max_gamma = cfg->max_gamma;
  p.mode = mode;
  p.dtype = cfg->dtype;
  p.R_d = (int32_t)R_d;
  p.n_task = (int32_t)(mode == SV_MODE_STOCHASTIC ? R_d : R_d + B);
  p.nch = (int32_t)((V + sv::chunk_stats(cfg->dtype, mode) - 1) / sv::chunk_stats(cfg->dtype, mode));
  p.delta = delta;
  p.nkl_pos = mode == SV_MODE_NKL ? cfg->nkl_position : nullptr;
  p.nkl_alpha = cfg->nkl_alpha;
  p.nkl_dmax = cfg->nkl_delta_max;
  p.want_kl = (mode == SV_MODE_NKL || (mode == SV_MODE_STOCHASTIC && out_nkl)) ? 1 : 0;
  p.block_min_len = cfg->block_min_len > 0 ? cfg->block_min_len : 3;  // 3: the page's min_block_len
  p.hdr = reinterpret_cast<int32_t*>(ws + L.off_hdr);
  p.d_off = reinterpret_cast<int32_t*>(ws + L.off_doff);
  p.pair2req = reinterpret_cast<int32_t*>(ws + L.off_pair2req);
  p.row2req = reinterpret_cast<int32_t*>(ws + L.off_row2req);
  p.part_a = reinterpret_cast<sv::PartA*>(ws + L.off_part_a);
  p.cnt = reinterpret_cast<uint64_t*>(ws + L.off_cnt);
  p.cnt_kl = reinterpret_cast<uint32_t*>(ws + L.off_cnt_kl);
  p.req_fin = reinterpret_cast<sv::ReqFin*>(ws + L.off_req_fin);
  p.part_c = reinterpret_cast<sv::PartC*>(ws + L.off_part_c);
  p.ref_list = reinterpret_cast<sv::RefItem*>(ws + L.off_ref_list);
  p.kl_need = reinterpret_cast<int32_t*>(ws + L.off_kl_need);
  p.tidx = reinterpret_cast<int32_t*>(ws + L.off_tidx);
  p.kl_part = reinterpret_cast<double*>(ws + L.off_kl_part);

  // 16-byte vector loads need every row to start on a 16-byte boundary
  const size_t es = (size_t)sv::elem_size(cfg->dtype);
  const bool vec = ((size_t)V * es) % 16 == 0 && aligned(target_logits, 16) &&
                   (!draft_logits || aligned(draft_logits, 16));

  hipStream_t s = static_cast<hipStream_t>(cfg->stream);
  hipEvent_t* ev = static_cast<hipEvent_t*>(cfg->phase_events);
  hipError_t e;

  // batches that scan their offsets in LDS, want no KL output and have a
  // short statistics pass: the whole step in one dispatch (not NKL mode)
  const int fused_grid = (!p.want_kl && B <= sv::kLdsBatch) ? sv::plan_fused(p, vec) : 0;
  p.epoch = next_epoch();
  p.wait_polls = cfg->wait_polls > 0 ? cfg->wait_polls : kDefaultWaitPolls;
  if (fused_grid > 0) {
    const int grid = fused_grid;
    if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return hip_fail(e);
    if ((e = (hipError_t)sv::launch_fused(p, vec, grid, s, ev ? ev[1] : nullptr, ev ? ev[2] : nullptr)) !=
        hipSuccess)
      return hip_fail(e);
    if (ev && (e = hipEventRecord(ev[3], s)) != hipSuccess) return hip_fail(e);
    return SV_OK;
  }

  sv::plan_stats(p, vec);
  sv::plan_decide(p, vec);
  if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return hip_fail(e);
  // small batches scan their offsets inside the statistics kernel
  if (B > sv::kLdsBatch && (e = (hipError_t)sv::launch_prep(p, s)) != hipSuccess) return hip_fail(e);
  // ev[1] / ev[2] take the statistics dispatch's own start and end timestamps
  if ((e = (hipError_t)sv::launch_stats(p, vec, s, ev ? ev[1] : nullptr, ev ? ev[2] : nullptr)) != hipSuccess)
    return hip_fail(e);
  if ((e = (hipError_t)sv::launch_decide(p, vec, s)) != hipSuccess) return hip_fail(e);
  if (p.want_kl && (e = (hipError_t)sv::launch_refine(p, vec, s)) != hipSuccess) return hip_fail(e);
  if (ev && (e = hipEventRecord(ev[3], s)) != hipSuccess) return hip_fail(e);
  return SV_OK;
}

int spec_verify_noalloc(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                        const int32_t* gamma_per_req, const float* temperature, const float* u_accept,
                        const float* u_resample, int32_t mode, float delta, const int32_t* tree_parents,
                        int32_t* out_tokens, int32_t* out_num_accepted, float* out_nkl, const sv_config* cfg) {
  if (!cfg || cfg->struct_size != sizeof(sv_config)) return SV_EINVAL;
  sv_config c = *cfg;
  const size_t need = spec_verify_workspace_size(&c);
  if (need == 0) return SV_EINVAL;
  if (need > (size_t)SV_NOALLOC_SCRATCH_BYTES) return SV_EWORKSPACE;
  void* ptr = nullptr;
  const int st = noalloc_scratch(&ptr);
  if (st != SV_OK) return st;
  c.workspace = ptr;
  c.workspace_bytes = SV_NOALLOC_SCRATCH_BYTES;
  return spec_verify(target_logits, draft_logits, draft_tokens, gamma_per_req, temperature, u_accept, u_resample,
                     mode, delta, tree_parents, out_tokens, out_num_accepted, out_nkl, &c);
}

int spec_sample_rows(const void* logits, const float* temperature, const float* u, int32_t* out_tokens,
                     const sv_config* cfg) {
  if (!cfg || cfg->struct_size != sizeof(sv_config) || cfg->wait_polls < 0) return SV_EINVAL;
  if (cfg->batch <= 0 || cfg->vocab <= 0) return SV_EINVAL;
  if (cfg->dtype != SV_DTYPE_F32 && cfg->dtype != SV_DTYPE_BF16) return SV_EINVAL;
  if (!logits || !temperature || !u || !out_tokens) return SV_EINVAL;
  const size_t es = (size_t)sv::elem_size(cfg->dtype);
  if (!aligned(logits, es) || !aligned(temperature, 4) || !aligned(u, 4) || !aligned(out_tokens, 4))
    return SV_EINVAL;
  const int64_t nch_t = (cfg->vocab + sv::chunk_t(cfg->dtype) - 1) / sv::chunk_t(cfg->dtype);
  if ((int64_t)cfg->batch * nch_t * (sv::kThreads / 64) > INT32_MAX) return SV_EUNSUPPORTED;
  const sv::Layout L = sv::make_layout(cfg->batch, cfg->vocab, cfg->dtype, 0);
  if (!cfg->workspace || cfg->workspace_bytes < L.total || !aligned(cfg->workspace, 256)) return SV_EWORKSPACE;

  uint8_t* ws = static_cast<uint8_t*>(cfg->workspace);
  sv::Params p{};
  p.target = logits;
  p.temp = temperature;
  p.ur = u;
  p.out_tokens = out_tokens;
  p.B = cfg->batch;
  p.V = cfg->vocab;
  p.dtype = cfg->dtype;
  p.mode = SV_MODE_STOCHASTIC;
  p.hdr = reinterpret_cast<int32_t*>(ws + L.off_hdr);
  p.cnt = reinterpret_cast<uint64_t*>(ws + L.off_cnt);
  p.part_c = reinterpret_cast<sv::PartC*>(ws + L.off_part_c);
  p.epoch = next_epoch();
  p.wait_polls = cfg->wait_polls > 0 ? cfg->wait_polls : kDefaultWaitPolls;
  const bool vec = ((size_t)cfg->vocab * es) % 16 == 0 && aligned(logits, 16);
  sv::plan_sample(p, vec);
  hipStream_t s = static_cast<hipStream_t>(cfg->stream);
  hipEvent_t* ev = static_cast<hipEvent_t*>(cfg->phase_events);
  hipError_t e;
  if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return hip_fail(e);
  if ((e = (hipError_t)sv::launch_sample(p, vec, s, ev ? ev[1] : nullptr, ev ? ev[2] : nullptr)) != hipSuccess)
    return hip_fail(e);
  if (ev && (e = hipEventRecord(ev[3], s)) != hipSuccess) return hip_fail(e);
  return SV_OK;
}

int spec_topk_rows(const void* logits, int32_t k, int32_t* out_idx, const sv_config* cfg) {
  if (!cfg || cfg->struct_size != sizeof(sv_config) || cfg->wait_polls < 0) return SV_EINVAL;
  if (cfg->batch <= 0 || cfg->vocab <= 0) return SV_EINVAL;
  if (cfg->dtype != SV_DTYPE_F32 && cfg->dtype != SV_DTYPE_BF16) return SV_EINVAL;
  if (k < 1 || k > sv::kTopkMax || k > cfg->vocab) return SV_EINVAL;
  if (!logits || !out_idx) return SV_EINVAL;
  const size_t es = (size_t)sv::elem_size(cfg->dtype);
  if (!aligned(logits, es) || !aligned(out_idx, 4)) return SV_EINVAL;
  const int64_t nch_t = (cfg->vocab + sv::chunk_t(cfg->dtype) - 1) / sv::chunk_t(cfg->dtype);
  if ((int64_t)cfg->batch * nch_t > INT32_MAX || (int64_t)cfg->batch * k > INT32_MAX) return SV_EUNSUPPORTED;
  const sv::Layout L = sv::make_layout(cfg->batch, cfg->vocab, cfg->dtype, 0);
  if (!cfg->workspace || cfg->workspace_bytes < L.total || !aligned(cfg->workspace, 256)) return SV_EWORKSPACE;

  uint8_t* ws = static_cast<uint8_t*>(cfg->workspace);
  sv::Params p{};
  p.target = logits;
  p.out_tokens = out_idx;
  p.B = cfg->batch;
  p.V = cfg->vocab;
  p.dtype = cfg->dtype;
  p.topk = k;
  p.cnt = reinterpret_cast<uint64_t*>(ws + L.off_cnt);
  p.topk_cand = reinterpret_cast<uint64_t*>(ws + L.off_topk);
  p.epoch = next_epoch();
  const bool vec = ((size_t)cfg->vocab * es) % 16 == 0 && aligned(logits, 16);
  sv::plan_topk(p, vec);
  hipStream_t s = static_cast<hipStream_t>(cfg->stream);
  hipEvent_t* ev = static_cast<hipEvent_t*>(cfg->phase_events);
  hipError_t e;
  if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return hip_fail(e);
  if ((e = (hipError_t)sv::launch_topk(p, vec, s, ev ? ev[1] : nullptr, ev ? ev[2] : nullptr)) != hipSuccess)
    return hip_fail(e);
  if (ev && (e = hipEventRecord(ev[3], s)) != hipSuccess) return hip_fail(e);
  return SV_OK;
}

size_t spec_consensus_workspace_size(const sv_config* cfg, int32_t num_drafts) {
  if (!cfg || cfg->struct_size != sizeof(sv_config)) return 0;
  if (cfg->batch <= 0 || cfg->vocab <= 0 || cfg->total_draft_rows < 0) return 0;
  if (cfg->dtype != SV_DTYPE_F32 && cfg->dtype != SV_DTYPE_BF16) return 0;
  if (num_drafts < 2 || num_drafts > sv::kConsMaxDrafts) return 0;
  return sv::make_cons_layout(cfg->batch, cfg->vocab, cfg->dtype, cfg->total_draft_rows, num_drafts).total;
}

int spec_consensus(const void* draft_logits, int32_t num_drafts, const int32_t* gamma_per_req,
                   const float* temperature, float delta_c, float delta_d, float* out_nkl, int32_t* out_state,
                   int32_t* out_pair, const sv_config* cfg) {
  if (!cfg || cfg->struct_size != sizeof(sv_config)) return SV_EINVAL;
  if (cfg->batch <= 0 || cfg->vocab <= 0 || cfg->max_gamma < 0) return SV_EINVAL;
  if (cfg->dtype != SV_DTYPE_F32 && cfg->dtype != SV_DTYPE_BF16) return SV_EINVAL;
  if (num_drafts < 2 || num_drafts > sv::kConsMaxDrafts) return SV_EINVAL;
  if (!std::isfinite(delta_c) || !std::isfinite(delta_d)) return SV_EINVAL;
  if (cfg->max_gamma > SV_MAX_GAMMA) return SV_EUNSUPPORTED;
  const int64_t npos = cfg->total_draft_rows;
  if (npos < 0 || npos > (int64_t)cfg->batch * cfg->max_gamma) return SV_EINVAL;
  const int64_t K = num_drafts;
  const sv::ConsLayout L = sv::make_cons_layout(cfg->batch, cfg->vocab, cfg->dtype, npos, K);
  if (npos * K > INT32_MAX || npos * L.nch > INT32_MAX) return SV_EUNSUPPORTED;
  if (!gamma_per_req || !temperature || !out_state || !out_pair || (npos > 0 && !draft_logits)) return SV_EINVAL;
  const size_t es = (size_t)sv::elem_size(cfg->dtype);
  if ((draft_logits && !aligned(draft_logits, es)) || !aligned(gamma_per_req, 4) || !aligned(temperature, 4) ||
      !aligned(out_state, 4) || !aligned(out_pair, 4) || (out_nkl && !aligned(out_nkl, 4)))
    return SV_EINVAL;
  if (!cfg->workspace || cfg->workspace_bytes < L.total || !aligned(cfg->workspace, 256)) return SV_EWORKSPACE;

  char* ws = static_cast<char*>(cfg->workspace);
  sv::Params p{};
  p.target = draft_logits;
  p.gamma = gamma_per_req;
  p.temp = temperature;
  p.B = cfg->batch;
  p.V = cfg->vocab;
  p.dtype = cfg->dtype;
  p.max_gamma = cfg->max_gamma;
  p.mode = sv::kModeConsensus;
  p.R_d = (int32_t)npos;
  p.cons_k = num_drafts;
  p.cons_dc = delta_c;
  p.cons_dd = delta_d;
  p.cons_nkl = out_nkl;
  p.cons_state = out_state;
  p.cons_pair = out_pair;
  p.hdr = reinterpret_cast<int32_t*>(ws + L.off_hdr);
  p.d_off = reinterpret_cast<int32_t*>(ws + L.off_doff);
  p.pair2req = reinterpret_cast<int32_t*>(ws + L.off_pos2req);
  p.cons_stats = reinterpret_cast<float*>(ws + L.off_stats);
  p.cons_tz = reinterpret_cast<double*>(ws + L.off_tz);
  p.cnt = reinterpret_cast<uint64_t*>(ws + L.off_cnt);
  p.cons_lds = cfg->batch <= sv::kLdsBatch ? 1 : 0;
  p.epoch = next_epoch();
  p.wait_polls = kDefaultWaitPolls;
  const bool vec = ((size_t)cfg->vocab * es) % 16 == 0 && (!draft_logits || aligned(draft_logits, 16));
  hipStream_t s = static_cast<hipStream_t>(cfg->stream);
  hipEvent_t* ev = static_cast<hipEvent_t*>(cfg->phase_events);
  hipError_t e;
  if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return hip_fail(e);
  if ((e = (hipError_t)sv::launch_consensus(p, vec, s, ev ? ev[1] : nullptr, ev ? ev[2] : nullptr)) != hipSuccess)
    return hip_fail(e);
  if (ev && (e = hipEventRecord(ev[3], s)) != hipSuccess) return hip_fail(e);
  return SV_OK;
}

int spec_read_probe(const void* buf, uint64_t bytes, int32_t wgs_per_cu, void* sink, void* stream,
                    void* ev_start, void* ev_stop) {
  if (!buf || !sink || wgs_per_cu < 1 || wgs_per_cu > 32 || !aligned(buf, 16) || !aligned(sink, 4))
    return SV_EINVAL;
  if (bytes < 16384) return SV_EINVAL;
  const hipError_t e = (hipError_t)sv::launch_read_probe(buf, (int64_t)bytes, wgs_per_cu, sink, stream, ev_start,
                                                          ev_stop);
  return e == hipSuccess ? SV_OK : hip_fail(e);
}

}  // extern "C"
