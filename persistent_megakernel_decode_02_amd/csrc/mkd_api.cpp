// Host side of the C ABI declared in include/mkd.h.
//
// The host records pointers, computes the RoPE table, builds and uploads the
// instruction tensor and launches; it never needs to understand the model
// beyond shapes (Hyperkernel teardown, "What is in the repository": the host
// copies tensors to the addresses the plan names and launches).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "mkd_internal.h"

using namespace mkd;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MKD_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

size_t round16(size_t n) { return (n + 15) & ~(size_t)15; }

}  // namespace

// Byte layout of a handle's workspace (caller-owned device memory).  The
// tables init writes come first; the schedule and the tagged activation block
// of the loaded schedule follow.  Every region starts on a 256-byte boundary.
struct WsLayout {
  size_t wtab = 0, rope = 0, status = 0, zero = 0, fixed = 0;  // written by init
  size_t sched = 0, ll = 0, total = 0;                          // per schedule
  size_t sched_words = 0, ll_words = 0;
  int flag_stride = 0;
  size_t sz[9] = {};  // words of h, qkv, part, aout, hmid, act, route, lm, flags
  int32_t s_qkv = 0, s_part = 0;
};

struct mkd_model {
  mkd_config cfg{};
  int device = 0;
  int n_cu = 0;
  int32_t max_seq = 0;
  uint16_t* kv = nullptr;
  std::vector<uint64_t> wptr;
  char* ws = nullptr;            // borrowed workspace
  size_t ws_bytes = 0;
  WsLayout lay;
  uint64_t* d_wtab = nullptr;    // regions of the workspace
  float* d_rope = nullptr;
  int32_t* d_status = nullptr;
  void* d_zero = nullptr;        // 4 KiB of zeros: streamer loads past the end of a tile
  int32_t* h_ctrl = nullptr;     // borrowed pinned host control block; word 0 = stop
  const int32_t* d_stop = nullptr;  // its device-side address
  uint64_t* d_ll = nullptr;
  size_t ll_words = 0;
  // sub-buffers of d_ll
  uint64_t *h = nullptr, *qkv = nullptr, *part = nullptr, *aout = nullptr, *hmid = nullptr,
           *act = nullptr, *route = nullptr, *lm = nullptr, *flags = nullptr;
  int32_t* d_sched = nullptr;
  size_t sched_words = 0;
  int batch = 1;  // sequences decoded together
  int n_wg = 0, n_chunks = 0, max_instr = 0, n_lm = 0, x_floats = 0, out_floats = 0, res_floats = 0;
  int pre_units = 0, pre_off = 0, n_stages = 0;
  int32_t s_qkv = 0, s_part = 0;  // per-sequence strides of qkv and part (words)
  int flag_stride = 0;
  int x_cap = 0, pre_cap = -1;     // mkd_set_lds_limits
  bool predict = false;            // mkd_set_expert_prediction (MoE models)
  bool plain_launch = false;       // mkd_set_launch_mode
  bool static_ws = false;          // the workspace is the library's static array (mkd_init_static)
  int32_t spec_hit = 0, spec_n = 0;  // expert predictions of the last waited-for launch
  hipEvent_t done = nullptr;
  hipEvent_t k0 = nullptr, k1 = nullptr;  // timing events around the megakernel
  bool launched = false, timed = false;
  double clock_hz = 100e6;
  uint64_t watchdog_ticks = 0;
  uint64_t* trace = nullptr;
  size_t trace_cap = 0;
};

namespace {

constexpr size_t kWsAlign = 256;
constexpr size_t kZeroBytes = 4096;
constexpr size_t kCtrlWords = 16;   // host control block: int32 words the caller provides

size_t align_ws(size_t n) { return (n + kWsAlign - 1) & ~(kWsAlign - 1); }
int32_t round16i(int64_t n) { return (int32_t)((n + 15) / 16 * 16); }

// the tables init writes: pointer table, RoPE table, status words, zero page
void ws_fixed(const mkd_config* c, int32_t max_seq, WsLayout* L) {
  const size_t n_ptr = W_GLOBAL + (size_t)c->n_layers * layer_slots(c);
  L->wtab = 0;
  L->rope = align_ws(L->wtab + n_ptr * 8);
  L->status = align_ws(L->rope + (size_t)max_seq * c->head_dim * 4);   // cos and sin, hd/2 each
  L->zero = align_ws(L->status + S_WORDS * 4);
  L->fixed = align_ws(L->zero + kZeroBytes);
}

// The schedule and the tagged activation block of one schedule tensor: one
// completion flag per instruction of each stage; h, aout, hmid, act and lm
// interleave the sequences (element r of sequence b at r * batch + b); qkv
// and part hold one block per sequence, 128-byte aligned.
void ws_schedule(const mkd_config* c, const int32_t* words, size_t n, WsLayout* L) {
  const int n_wg = words[H_NWG], n_chunks = words[H_NCHUNKS], batch = words[H_BATCH];
  const int n_st = words[H_NSTAGES];
  int flag_stride = kFlagAlign;
  std::vector<int> per(n_st, 0);
  const int32_t* body = words + kWords + n_wg;
  for (int w = 0; w < n_wg; ++w)
    for (int j = 0; j < words[kWords + w]; ++j) {
      const int32_t* ins = body + ((size_t)w * words[H_MAXINSTR] + j) * kWords;
      per[ins[I_STAGE]] = std::max(per[ins[I_STAGE]], ins[I_INDEX] + 1);
    }
  for (int v : per) flag_stride = std::max(flag_stride, (v + kFlagAlign - 1) / kFlagAlign * kFlagAlign);
  const int n_lm = c->vocab < n_wg ? c->vocab : n_wg;
  const int qd = c->n_q_heads * c->head_dim, kvd = c->n_kv_heads * c->head_dim;
  L->s_qkv = round16i(qd + 2 * kvd);
  L->s_part = round16i((int64_t)c->n_q_heads * n_chunks * (c->head_dim + 2));
  const size_t sz[9] = {round16((size_t)c->d_model * batch), (size_t)batch * L->s_qkv, (size_t)batch * L->s_part,
                        round16((size_t)qd * batch), round16((size_t)c->d_model * batch),
                        round16((size_t)c->d_ff * (c->top_k ? c->top_k : 1) * batch),
                        16, round16(2 * (size_t)n_lm * batch),
                        round16((size_t)n_st * flag_stride / 2)};
  L->ll_words = 0;
  for (int i = 0; i < 9; ++i) {
    L->sz[i] = sz[i];
    // the flags start on a 256-byte boundary, as do their per-stage arrays
    if (i == 7) L->sz[i] += (32 - (L->ll_words + sz[i]) % 32) % 32;
    L->ll_words += L->sz[i];
  }
  L->flag_stride = flag_stride;
  L->sched_words = n;
  L->sched = L->fixed;
  L->ll = align_ws(L->sched + n * 4);
  L->total = align_ws(L->ll + L->ll_words * 8);
}

// split-KV chunks when the caller leaves the choice to the library
int default_chunks(const mkd_config* c, int n_wg, int n_positions) {
  // one chunk (one attention instruction per q head) up to 512 KiB of K and V
  // per head, else one chunk per workgroup and kv head (at most 64); measured
  // best on the 1B and 3B shapes at KV 1024-16384
  const double head_bytes = (double)n_positions * c->head_dim * 4.0;  // K and V rows
  int cap = n_wg / c->n_kv_heads;
  cap = cap < 1 ? 1 : (cap > 64 ? 64 : cap);
  return head_bytes <= 512.0 * 1024 ? 1 : cap;
}

}  // namespace

extern "C" {

int mkd_version(void) { return MKD_ABI_VERSION; }

const char* mkd_last_error(void) { return g_err.c_str(); }

int mkd_config_check(const mkd_config* cfg) {
  const char* why = "";
  const int rc = config_check(cfg, &why);
  if (rc) return fail(rc, why);
  return MKD_OK;
}

int mkd_weight_count(const mkd_config* cfg, size_t* n_out) {
  int rc = mkd_config_check(cfg);
  if (rc) return rc;
  if (!n_out) return fail(MKD_E_INVALID, "null n_out");
  *n_out = (size_t)(cfg->tied ? 2 : 3) + (size_t)cfg->n_layers * layer_slots(cfg);
  return MKD_OK;
}

int mkd_weight_shape(const mkd_config* cfg, size_t index, int64_t* rows, int64_t* cols) {
  size_t n = 0;
  int rc = mkd_weight_count(cfg, &n);
  if (rc) return rc;
  if (index >= n || !rows || !cols) return fail(MKD_E_INVALID, "weight index out of range");
  const int64_t d = cfg->d_model, F = cfg->d_ff, V = cfg->vocab;
  const int64_t qd = (int64_t)cfg->n_q_heads * cfg->head_dim, kvd = (int64_t)cfg->n_kv_heads * cfg->head_dim;
  const size_t g = cfg->tied ? 2 : 3;
  if (index < g) {
    if (index == 1) { *rows = d; *cols = 1; }
    else { *rows = V; *cols = d; }  // embed, lm_head
    return MKD_OK;
  }
  const int k = (int)((index - g) % layer_slots(cfg));
  switch (k) {
    case WL_ATTN_NORM: case WL_FFN_NORM: *rows = d; *cols = 1; return MKD_OK;
    case WL_Q: *rows = qd; *cols = d; return MKD_OK;
    case WL_K: case WL_V: *rows = kvd; *cols = d; return MKD_OK;
    case WL_O: *rows = d; *cols = qd; return MKD_OK;
    default: break;
  }
  if (!cfg->n_experts) {
    if (k == WL_DOWN) { *rows = d; *cols = F; }
    else { *rows = F; *cols = d; }
    return MKD_OK;
  }
  if (k == WL_ROUTER) { *rows = cfg->n_experts; *cols = d; return MKD_OK; }
  const int e = k - WL_EXPERTS;  // gate[E], up[E], down[E]
  if (e < 2 * cfg->n_experts) { *rows = F; *cols = d; }
  else { *rows = d; *cols = F; }
  return MKD_OK;
}

int mkd_kv_cache_bytes(const mkd_config* cfg, int32_t max_seq, size_t* bytes_out) {
  int rc = mkd_config_check(cfg);
  if (rc) return rc;
  if (max_seq < 1 || !bytes_out) return fail(MKD_E_INVALID, "max_seq must be >= 1");
  *bytes_out = (size_t)cfg->n_layers * 2 * cfg->n_kv_heads * (size_t)max_seq * cfg->head_dim * 2;
  return MKD_OK;
}

int mkd_schedule_build_batch(const mkd_config* cfg, int32_t n_wg, int32_t n_chunks, int32_t batch,
                             int32_t* out, size_t capacity, size_t* n_words) {
  const char* why = "";
  const int rc = schedule_build(cfg, n_wg, n_chunks, batch, out, capacity, n_words, &why);
  if (rc) return fail(rc, why);
  return MKD_OK;
}

int mkd_schedule_build(const mkd_config* cfg, int32_t n_wg, int32_t n_chunks, int32_t* out,
                       size_t capacity, size_t* n_words) {
  return mkd_schedule_build_batch(cfg, n_wg, n_chunks, 1, out, capacity, n_words);
}

int mkd_schedule_validate(const mkd_config* cfg, const int32_t* words, size_t n_words) {
  const char* why = "";
  const int rc = schedule_validate(cfg, words, n_words, &why);
  if (rc) return fail(rc, why);
  return MKD_OK;
}

int mkd_default_chunks(const mkd_config* cfg, int32_t n_wg, int32_t n_positions, int32_t* n_chunks) {
  const char* why = "";
  if (!cfg || !n_chunks) return fail(MKD_E_INVALID, "null argument");
  if (config_check(cfg, &why)) return fail(MKD_E_INVALID, why);
  if (n_wg < 1 || n_positions < 1) return fail(MKD_E_INVALID, "n_wg and n_positions must be >= 1");
  *n_chunks = default_chunks(cfg, n_wg, n_positions);
  return MKD_OK;
}

int mkd_workspace_bytes(const mkd_config* cfg, int32_t n_wg, int32_t n_chunks, int32_t batch, int32_t max_seq,
                        size_t* bytes_out) {
  const char* why = "";
  if (!cfg || !bytes_out) return fail(MKD_E_INVALID, "null argument");
  if (config_check(cfg, &why)) return fail(MKD_E_INVALID, why);
  if (max_seq < 1 || n_wg < 1) return fail(MKD_E_INVALID, "max_seq and n_wg must be >= 1");
  if (n_chunks == 0) n_chunks = default_chunks(cfg, n_wg, max_seq);
  size_t n = 0;
  if (schedule_build(cfg, n_wg, n_chunks, batch, nullptr, 0, &n, &why)) return fail(MKD_E_INVALID, why);
  std::vector<int32_t> w(n);
  if (schedule_build(cfg, n_wg, n_chunks, batch, w.data(), n, &n, &why)) return fail(MKD_E_INVALID, why);
  WsLayout L;
  ws_fixed(cfg, max_seq, &L);
  ws_schedule(cfg, w.data(), n, &L);
  *bytes_out = L.total;
  return MKD_OK;
}

int mkd_workspace_layout(const mkd_config* cfg, int32_t n_wg, int32_t n_chunks, int32_t batch, int32_t max_seq,
                         size_t* offsets_out) {
  size_t total = 0;
  int rc = mkd_workspace_bytes(cfg, n_wg, n_chunks, batch, max_seq, &total);
  if (rc) return rc;
  if (!offsets_out) return fail(MKD_E_INVALID, "null offsets_out");
  const char* why = "";
  if (n_chunks == 0) n_chunks = default_chunks(cfg, n_wg, max_seq);
  size_t n = 0;
  schedule_build(cfg, n_wg, n_chunks, batch, nullptr, 0, &n, &why);
  std::vector<int32_t> w(n);
  schedule_build(cfg, n_wg, n_chunks, batch, w.data(), n, &n, &why);
  WsLayout L;
  ws_fixed(cfg, max_seq, &L);
  ws_schedule(cfg, w.data(), n, &L);
  const size_t v[8] = {L.wtab, L.rope, L.status, L.zero, L.sched, L.ll, L.ll + (L.ll_words - L.sz[8]) * 8, L.total};
  for (int i = 0; i < 8; ++i) offsets_out[i] = v[i];
  return MKD_OK;
}

int mkd_init(const mkd_config* cfg, const void* const* weights, size_t n_weights, void* kv_cache,
             int32_t max_seq, void* workspace, size_t workspace_bytes, int32_t* host_control, int32_t device,
             mkd_model** out) {
  return mkd_init_batch(cfg, weights, n_weights, kv_cache, max_seq, 1, workspace, workspace_bytes, host_control,
                        device, out);
}

// mkd_init_batch and mkd_init_static; static_ws: the workspace is this
// library's static array on `device` (already known to be device memory)
static int init_common(const mkd_config* cfg, const void* const* weights, size_t n_weights, void* kv_cache,
                       int32_t max_seq, int32_t batch, void* workspace, size_t workspace_bytes,
                       int32_t* host_control, int32_t device, bool static_ws, mkd_model** out) {
  if (!out) return fail(MKD_E_INVALID, "null out");
  *out = nullptr;
  if (batch < 1 || batch > kMaxBatch) return fail(MKD_E_INVALID, "batch must be in [1, 8]");
  if (batch > 1 && cfg && cfg->n_experts)
    return fail(MKD_E_UNSUPPORTED, "batched decode is implemented for dense models only");
  if (batch > 1 && cfg && cfg->d_model > 16 * kThreads)
    return fail(MKD_E_UNSUPPORTED, "batched decode needs d_model <= 8192");
  size_t want = 0;
  int rc = mkd_weight_count(cfg, &want);
  if (rc) return rc;
  if (!weights || n_weights != want)
    return fail(MKD_E_INVALID, "expected " + std::to_string(want) + " weight pointers, got " +
                                   std::to_string(n_weights));
  for (size_t i = 0; i < n_weights; ++i) {
    if (!weights[i] || ((uintptr_t)weights[i] & 15))
      return fail(MKD_E_INVALID, "weight " + std::to_string(i) + " is null or not 16-byte aligned");
  }
  if (max_seq < 1) return fail(MKD_E_INVALID, "max_seq must be >= 1");
  if (!kv_cache || ((uintptr_t)kv_cache & 15)) return fail(MKD_E_INVALID, "kv_cache null or misaligned");
  const size_t head_bytes = (size_t)max_seq * cfg->head_dim * 2;
  if (head_bytes > 0x7fffffffull) return fail(MKD_E_INVALID, "max_seq * head_dim too large");
  WsLayout L;
  ws_fixed(cfg, max_seq, &L);
  if (!workspace || ((uintptr_t)workspace & (kWsAlign - 1)))
    return fail(MKD_E_INVALID, "workspace null or not 256-byte aligned");
  if (workspace_bytes < L.fixed)
    return fail(MKD_E_INVALID, std::string(static_ws ? "the static workspace" : "workspace") + " of " +
                                   std::to_string(workspace_bytes) + " bytes is smaller than the " +
                                   std::to_string(L.fixed) + " its tables need at max_seq " + std::to_string(max_seq) +
                                   (static_ws ? "" : " (mkd_workspace_bytes sizes it)"));
  if (!host_control || ((uintptr_t)host_control & 63))
    return fail(MKD_E_INVALID, "host_control null or not 64-byte aligned");

  hipError_t e = hipSetDevice(device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MKD_E_UNSUPPORTED, std::string("library is built for gfx950, device is ") + prop.gcnArchName);
  int coop = 0;
  hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, device);
  if (!coop) return fail(MKD_E_UNSUPPORTED, "device lacks cooperative launch");
  // the borrowed memory must be what the kernel can reach: device memory of
  // this device, and pinned (device-mapped) host memory for the control block
  hipPointerAttribute_t at{};
  if (!static_ws && (hipPointerGetAttributes(&at, workspace) != hipSuccess || at.type != hipMemoryTypeDevice ||
                     at.device != device)) {
    (void)hipGetLastError();
    return fail(MKD_E_INVALID, "workspace is not device memory of device " + std::to_string(device));
  }
  hipPointerAttribute_t hc{};
  if (hipPointerGetAttributes(&hc, host_control) != hipSuccess || hc.type != hipMemoryTypeHost ||
      !hc.devicePointer) {
    (void)hipGetLastError();
    return fail(MKD_E_INVALID, "host_control is not pinned host memory mapped for the device");
  }

  mkd_model* m = new mkd_model();
  m->cfg = *cfg;
  m->batch = batch;
  m->device = device;
  m->n_cu = prop.multiProcessorCount;
  m->max_seq = max_seq;
  m->kv = (uint16_t*)kv_cache;
  m->ws = (char*)workspace;
  m->ws_bytes = workspace_bytes;
  m->lay = L;
  m->d_wtab = (uint64_t*)(m->ws + L.wtab);
  m->d_rope = (float*)(m->ws + L.rope);
  m->d_status = (int32_t*)(m->ws + L.status);
  m->d_zero = m->ws + L.zero;
  m->h_ctrl = host_control;
  m->d_stop = (const int32_t*)hc.devicePointer;
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) == hipSuccess && khz > 0)
    m->clock_hz = (double)khz * 1e3;
  m->watchdog_ticks = (uint64_t)(2.0 * m->clock_hz);

  // pointer table: embed, final_norm, lm_head (embed when tied), then layers
  const int ls = layer_slots(cfg);
  m->wptr.assign(W_GLOBAL + (size_t)cfg->n_layers * ls, 0);
  size_t k = 0;
  m->wptr[W_EMBED] = (uint64_t)weights[k++];
  m->wptr[W_FINAL_NORM] = (uint64_t)weights[k++];
  m->wptr[W_LM_HEAD] = cfg->tied ? m->wptr[W_EMBED] : (uint64_t)weights[k++];
  for (int l = 0; l < cfg->n_layers; ++l)
    for (int s = 0; s < ls; ++s) m->wptr[W_GLOBAL + (size_t)l * ls + s] = (uint64_t)weights[k++];

  // RoPE table: angle = pos * theta^(-2i/hd) in fp64, cos and sin rounded to fp32
  const int half = cfg->head_dim / 2;
  std::vector<float> rope((size_t)2 * max_seq * half);
  for (int pos = 0; pos < max_seq; ++pos)
    for (int i = 0; i < half; ++i) {
      const double a = (double)pos * pow(cfg->rope_theta, (-2.0 * i) / cfg->head_dim);
      rope[(size_t)pos * half + i] = (float)cos(a);
      rope[(size_t)max_seq * half + (size_t)pos * half + i] = (float)sin(a);
    }

  auto cleanup = [&](int code, const std::string& msg) {
    mkd_destroy(m);
    return fail(code, msg);
  };
  for (size_t i = 0; i < kCtrlWords; ++i) __atomic_store_n(host_control + i, 0, __ATOMIC_SEQ_CST);
  if ((e = hipMemset(m->d_zero, 0, kZeroBytes)) != hipSuccess) return cleanup(MKD_E_HIP, "clear zero page");
  if ((e = hipMemcpy(m->d_wtab, m->wptr.data(), m->wptr.size() * 8, hipMemcpyHostToDevice)) != hipSuccess)
    return cleanup(MKD_E_HIP, "upload wtab");
  if ((e = hipMemcpy(m->d_rope, rope.data(), rope.size() * 4, hipMemcpyHostToDevice)) != hipSuccess)
    return cleanup(MKD_E_HIP, "upload rope");
  if ((e = hipMemset(m->d_status, 0, S_WORDS * 4)) != hipSuccess) return cleanup(MKD_E_HIP, "clear status");
  if ((e = hipEventCreateWithFlags(&m->done, hipEventDisableTiming)) != hipSuccess)
    return cleanup(MKD_E_HIP, "hipEventCreate");
  if ((e = hipEventCreate(&m->k0)) != hipSuccess || (e = hipEventCreate(&m->k1)) != hipSuccess)
    return cleanup(MKD_E_HIP, "hipEventCreate");
  *out = m;
  return MKD_OK;
}

int mkd_init_batch(const mkd_config* cfg, const void* const* weights, size_t n_weights, void* kv_cache,
                   int32_t max_seq, int32_t batch, void* workspace, size_t workspace_bytes, int32_t* host_control,
                   int32_t device, mkd_model** out) {
  return init_common(cfg, weights, n_weights, kv_cache, max_seq, batch, workspace, workspace_bytes, host_control,
                     device, false, out);
}

namespace {
// the handle that holds each device's static workspace (null: free)
std::mutex g_static_mu;
mkd_model* g_static_owner[64] = {};
}  // namespace

int mkd_init_static(const mkd_config* cfg, const void* const* weights, size_t n_weights, void* kv_cache,
                    int32_t max_seq, int32_t* host_control, int32_t device, mkd_model** out) {
  if (!out) return fail(MKD_E_INVALID, "null out");
  *out = nullptr;
  if (device < 0 || device >= 64) return fail(MKD_E_INVALID, "device index out of range");
  hipError_t e = hipSetDevice(device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (g_static_owner[device])
    return fail(MKD_E_INVALID, "the static workspace of device " + std::to_string(device) +
                                   " is held by another handle (mkd_destroy it first)");
  void* ws = nullptr;
  const char* why = "";
  int rc = static_workspace(device, &ws, &why);
  if (rc) return fail(rc, why);
  rc = init_common(cfg, weights, n_weights, kv_cache, max_seq, 1, ws, kStaticWorkspaceBytes, host_control, device,
                   true, out);
  if (rc) return rc;
  (*out)->static_ws = true;
  g_static_owner[device] = *out;
  return MKD_OK;
}

// LDS floats for the GEMV row results of the largest tile (x2 for the
// opcodes that stream two rows per output row), for every sequence
static int out_floats_for(const mkd_config* c, int n_wg, int n_chunks, int batch) {
  const int n_st = stage_count(c, n_chunks);
  std::vector<StageDesc> st(n_st);
  int got = 0;
  stage_list(c, n_chunks, batch, st.data(), &got, n_st);
  int best = 4;
  for (int i = 0; i < n_st; ++i) {
    const StageDesc& s = st[i];
    if (!is_tiled(s.op)) continue;
    int avail = n_wg, first = 0;
    placement(st, i, n_wg, &avail, &first);
    const int n = s.size < avail ? s.size : avail;
    int rows = (s.size + n - 1) / n;
    if (s.op == OP_UPGATE || s.op == OP_MOE_UPGATE || s.op == OP_MOE_DOWN) rows *= 2;
    best = rows > best ? rows : best;
  }
  // several sequences: plus the partial sums of tiles whose rows are split
  // over K between wavefronts (fewer than 64 partial rows per tile)
  if (batch > 1) best += 64;
  return ((best * batch) + 3) & ~3;
}

// LDS floats for the residual rows of a tile: the whole vector (as before)
// with one sequence, the largest O-projection or down tile for each of several
static int res_floats_for(const mkd_config* c, int n_wg, int n_chunks, int batch) {
  if (batch == 1) return (c->d_model + 3) & ~3;
  const int n_st = stage_count(c, n_chunks);
  std::vector<StageDesc> st(n_st);
  int got = 0;
  stage_list(c, n_chunks, batch, st.data(), &got, n_st);
  int best = 4;
  for (int i = 0; i < n_st; ++i) {
    const StageDesc& s = st[i];
    if (s.op != OP_OPROJ && s.op != OP_DOWN && s.op != OP_MOE_DOWN) continue;
    int avail = n_wg, first = 0;
    placement(st, i, n_wg, &avail, &first);
    const int n = s.size < avail ? s.size : avail;
    const int rows = (s.size + n - 1) / n;
    best = rows > best ? rows : best;
  }
  return ((best + 3) & ~3) * batch;
}

// Limits a caller may put on the LDS plan (mkd_set_lds_limits): the batched
// input area in floats (0 = none) and the staged gate/up units per wavefront
// (-1 = none).  They only ever shrink what the plan would use.
struct LdsCaps {
  int x_cap = 0, pre_cap = -1;
};

// Dense gate/up weights staged in LDS ahead of the instruction: as many
// 1 KiB units per wavefront as the LDS left over holds, up to kPreMax (and
// the caller's cap).  They are loaded while the workgroup waits out the
// attention phase, when its own load queue is otherwise empty.
static int pre_units_for(const mkd_config* c, size_t lds_used, int lds_max, const LdsCaps& caps) {
  if (c->n_experts > 0 || lds_max <= 0 || lds_used >= (size_t)lds_max) return 0;
  int n = (int)(((size_t)lds_max - lds_used) / ((size_t)kWaves * 1024));
  if (n > kPreMax) n = kPreMax;
  if (caps.pre_cap >= 0 && caps.pre_cap < n) n = caps.pre_cap;
  return n;
}

// LDS floats of one input vector of n elements per sequence: one sequence
// reads x in 512-wide segments; with several sequences, interleaved, every
// 8-element slice (8 * batch floats) is followed by 4 padding floats
static int vec_floats(int n, int batch) {
  const int padded = (n + 511) & ~511;
  return batch == 1 ? padded : padded / 8 * (8 * batch + 4);
}

// LDS floats for the staged input vectors (and the other staging uses of
// that area); with_act false leaves out the down projection's input, which
// several sequences may stream in passes over K (one segment at least)
static int x_floats_for(const mkd_config* c, int n_chunks, int n_lm, int batch, bool with_act = true) {
  const int G = c->n_q_heads / c->n_kv_heads, hd = c->head_dim;
  const int qd = c->n_q_heads * hd;
  auto vec = [&](int n) { return vec_floats(n, batch); };
  int x = vec(c->d_model);
  x = x > vec(qd) ? x : vec(qd);
  const int act = with_act ? vec(c->d_ff) * (c->top_k ? c->top_k : 1) : vec(512);
  x = x > act ? x : act;
  const int lm = 2 * n_lm * batch;                      // every sequence's LM-head partials
  x = x > lm ? x : lm;
  const int ared = n_chunks * (hd + 2) + 4 * hd;   // a head's chunk partials, then quarter sums
  x = x > ared ? x : ared;
  const int attn = (G + 2) * hd + kWaves * G * (hd + 2);
  x = x > attn ? x : attn;
  return (x + 3) & ~3;
}

constexpr size_t kLdsSlack = 256;  // static LDS of the kernel and a margin

// Several sequences: when the interleaved down-projection input does not fit
// in LDS next to everything else, shrink the input area to what fits, in
// whole 512-element segments per sequence; the down projection then runs in
// passes over K.  The other inputs (normalised as a whole) are never split:
// if even they do not fit, the area is left as is and the LDS check fails.
// The caller's cap shrinks the area further (within the same bounds), so
// that the passes can be exercised on small models.
static void fit_x(KParams& p, const mkd_config* c, int n_chunks, int n_lm, int batch, int lds_max,
                  const LdsCaps& caps) {
  if (batch == 1) return;
  if (caps.x_cap > 0) {
    const int seg = 64 * (8 * batch + 4);   // one 512-element segment of every sequence, padded
    const int cap = caps.x_cap / seg * seg;
    if (cap > 0 && cap < p.x_floats && cap >= x_floats_for(c, n_chunks, n_lm, batch, false)) {
      p.x_floats = cap;
      return;
    }
  }
  if (lds_max <= 0) return;
  const size_t other = lds_bytes(p) - (size_t)p.x_floats * sizeof(float);
  if (other + kLdsSlack >= (size_t)lds_max) return;
  const int fill = (int)(((size_t)lds_max - kLdsSlack - other) / sizeof(float)) & ~3;
  if (fill >= p.x_floats) {
    // it fits: the area grows to the whole LDS left, and the part past the
    // gate/up and O-projection inputs holds staged gate/up weights
    p.x_floats = fill;
    return;
  }
  const int seg = 64 * (8 * batch + 4);
  const int x = fill / seg * seg;
  if (x >= x_floats_for(c, n_chunks, n_lm, batch, false)) p.x_floats = x;
}

// Gate/up weight units staged in LDS ahead of their instruction.  One
// sequence: the LDS left after everything else (pre_units_for).  Several:
// the input area past the two inputs that are live while the units are
// (the O-projection's, read while they load, and gate/up's own); the down
// projection's longer input reuses that space after gate/up has read them.
static void set_pre(KParams& p, const mkd_config* c, int batch, int lds_max, const LdsCaps& caps) {
  p.pre_off = 0;
  if (c->n_experts > 0) {
    // MoE: nothing is staged (the expert prediction requests its rows into
    // registers at the start of the gate/up tile)
    p.pre_units = 0;
    return;
  }
  if (batch == 1) {
    p.pre_units = pre_units_for(c, lds_bytes(p), lds_max, caps);
    return;
  }
  p.pre_units = 0;
  // measured: with the down projection in passes over K (larger batches)
  // staging slows the step down
  if (p.x_floats < vec_floats(c->d_ff, batch)) return;
  const int qd = c->n_q_heads * c->head_dim;
  const int off = (std::max(vec_floats(c->d_model, batch), vec_floats(qd, batch)) + 3) & ~3;
  if (off >= p.x_floats) return;
  int n = (p.x_floats - off) / (kWaves * 256);   // 1 KiB units per wavefront
  n = std::min(n, kPreMax);
  if (caps.pre_cap >= 0 && caps.pre_cap < n) n = caps.pre_cap;
  if (n < 4) return;   // the batched streamer stages whole groups of 4 rows
  p.pre_off = off;
  p.pre_units = n;
}

// The per-workgroup LDS areas of a schedule (n_wg workgroups, n_chunks
// split-KV chunks, batch sequences) on a device with lds_max bytes per
// workgroup (0: unknown, no fitting).
static KParams lds_plan(const mkd_config* c, int n_wg, int n_chunks, int batch, int lds_max,
                        const LdsCaps& caps = LdsCaps()) {
  const int n_lm = c->vocab < n_wg ? c->vocab : n_wg;
  KParams p{};
  p.x_floats = x_floats_for(c, n_chunks, n_lm, batch);
  p.out_floats = out_floats_for(c, n_wg, n_chunks, batch);
  p.res_floats = res_floats_for(c, n_wg, n_chunks, batch);
  p.d = c->d_model;
  fit_x(p, c, n_chunks, n_lm, batch, lds_max, caps);
  set_pre(p, c, batch, lds_max, caps);
  return p;
}

int mkd_lds_plan(const mkd_config* cfg, int32_t batch, int32_t n_wg, int32_t n_chunks, int32_t lds_max,
                 int32_t* out) {
  const char* why = "";
  if (!cfg || !out) return fail(MKD_E_INVALID, "null argument");
  if (config_check(cfg, &why)) return fail(MKD_E_INVALID, why);
  if (batch < 1 || batch > kMaxBatch || n_wg < 1 || n_chunks < 1 || n_chunks > 64 || lds_max < 0)
    return fail(MKD_E_INVALID, "batch, n_wg, n_chunks or lds_max out of range");
  const KParams p = lds_plan(cfg, n_wg, n_chunks, batch, lds_max);
  out[0] = p.x_floats;
  out[1] = p.out_floats;
  out[2] = p.res_floats;
  out[3] = p.pre_units;
  out[4] = p.pre_off;
  out[5] = (int32_t)lds_bytes(p);
  return MKD_OK;
}

int mkd_device_info(mkd_model* m, int32_t* n_cu, int32_t* max_coop_wg) {
  if (!m) return fail(MKD_E_INVALID, "null model");
  if (n_cu) *n_cu = m->n_cu;
  if (max_coop_wg) {
    int lds_max = 0;
    hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, m->device);
    const KParams p = lds_plan(&m->cfg, m->n_cu, 1, m->batch, lds_max);
    int mx = 0;
    const int rc = max_coop_blocks(m->device, lds_bytes(p), m->batch, m->cfg.n_experts > 0, &mx);
    if (rc) return fail(rc, "occupancy query failed");
    *max_coop_wg = mx;
  }
  return MKD_OK;
}

static int upload_schedule(mkd_model* m, const int32_t* words, size_t n) {
  const mkd_config* c = &m->cfg;
  const int n_wg = words[H_NWG], n_chunks = words[H_NCHUNKS], batch = words[H_BATCH];
  if (n_chunks > 64) return fail(MKD_E_UNSUPPORTED, "n_chunks > 64 is not supported by the device code");
  if (n_wg > 4096) return fail(MKD_E_UNSUPPORTED, "n_wg > 4096 is not supported by the device code");
  if (batch != m->batch)
    return fail(MKD_E_INVALID, "schedule is for " + std::to_string(batch) + " sequences, the model decodes " +
                                   std::to_string(m->batch));
  const int n_lm = c->vocab < n_wg ? c->vocab : n_wg;
  int lds_max = 0;
  hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, m->device);
  LdsCaps caps;
  caps.x_cap = m->x_cap;
  caps.pre_cap = m->pre_cap;
  const KParams p = lds_plan(c, n_wg, n_chunks, batch, lds_max, caps);
  const size_t lds = lds_bytes(p);
  if (lds_max > 0 && lds > (size_t)lds_max)
    return fail(MKD_E_UNSUPPORTED, "schedule needs " + std::to_string(lds) + " bytes of LDS per workgroup, device has " +
                                       std::to_string(lds_max) + " (use more workgroups)");
  int mx = 0;
  int rc = max_coop_blocks(m->device, lds, batch, c->n_experts > 0, &mx);
  if (rc) return fail(rc, "occupancy query failed");
  if (n_wg > mx)
    return fail(MKD_E_COOPERATIVE, "n_wg " + std::to_string(n_wg) + " exceeds the " +
                                       std::to_string(mx) + " workgroups that can be co-resident");
  WsLayout L = m->lay;
  ws_schedule(c, words, n, &L);
  if (L.total > m->ws_bytes)
    return fail(MKD_E_INVALID, "this schedule needs a workspace of " + std::to_string(L.total) + " bytes, the handle has " +
                                   std::to_string(m->ws_bytes) +
                                   (m->static_ws ? " (the static workspace's fixed size)" : " (mkd_workspace_bytes sizes it)"));
  hipError_t e = hipSetDevice(m->device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  if (m->launched) hipEventSynchronize(m->done);
  m->lay = L;
  m->d_sched = (int32_t*)(m->ws + L.sched);
  if ((e = hipMemcpy(m->d_sched, words, n * 4, hipMemcpyHostToDevice)) != hipSuccess)
    return hip_fail(e, "upload schedule");
  m->sched_words = n;
  // the tagged activation block, cleared before each launch
  m->d_ll = (uint64_t*)(m->ws + L.ll);
  m->ll_words = L.ll_words;
  uint64_t* q = m->d_ll;
  uint64_t** dst[9] = {&m->h, &m->qkv, &m->part, &m->aout, &m->hmid, &m->act, &m->route, &m->lm, &m->flags};
  for (int i = 0; i < 9; ++i) { *dst[i] = q; q += L.sz[i]; }
  m->n_stages = words[H_NSTAGES];
  m->flag_stride = L.flag_stride;
  m->n_wg = n_wg;
  m->n_chunks = n_chunks;
  m->max_instr = words[H_MAXINSTR];
  m->n_lm = n_lm;
  m->x_floats = p.x_floats;
  m->out_floats = p.out_floats;
  m->res_floats = p.res_floats;
  m->pre_units = p.pre_units;
  m->pre_off = p.pre_off;
  m->s_qkv = L.s_qkv; m->s_part = L.s_part;
  return MKD_OK;
}

int mkd_load_schedule(mkd_model* m, const int32_t* words, size_t n_words) {
  if (!m) return fail(MKD_E_INVALID, "null model");
  int rc = mkd_schedule_validate(&m->cfg, words, n_words);
  if (rc) return rc;
  return upload_schedule(m, words, n_words);
}

int mkd_build_schedule(mkd_model* m, int32_t n_wg, int32_t n_chunks, int32_t* host_out,
                       size_t capacity, size_t* n_words) {
  if (!m) return fail(MKD_E_INVALID, "null model");
  if (n_wg == 0) n_wg = m->n_cu;
  if (n_chunks == 0) n_chunks = default_chunks(&m->cfg, n_wg, m->max_seq);
  size_t n = 0;
  int rc = mkd_schedule_build_batch(&m->cfg, n_wg, n_chunks, m->batch, nullptr, 0, &n);
  if (rc) return rc;
  std::vector<int32_t> w(n);
  rc = mkd_schedule_build_batch(&m->cfg, n_wg, n_chunks, m->batch, w.data(), n, &n);
  if (rc) return rc;
  if (n_words) *n_words = n;
  if (host_out) {
    if (capacity < n) return fail(MKD_E_INVALID, "host_out too small for the schedule");
    memcpy(host_out, w.data(), n * 4);
  }
  return upload_schedule(m, w.data(), n);
}

// one launch of n_steps decode steps for every sequence of the model
static int decode_launch(mkd_model* m, const int32_t* first_tokens, const int32_t* start_pos, int32_t n_steps,
                         const int32_t* forced_dev, int32_t* tokens_out_dev, float* logits_out_dev,
                         void* stream) {
  if (!m->d_sched) return fail(MKD_E_INVALID, "no schedule loaded");
  const mkd_config* c = &m->cfg;
  if (!first_tokens || !start_pos) return fail(MKD_E_INVALID, "null first_tokens or start_pos");
  for (int b = 0; b < m->batch; ++b) {
    if (first_tokens[b] < 0 || first_tokens[b] >= c->vocab) return fail(MKD_E_INVALID, "first token out of range");
    if (start_pos[b] < 0 || n_steps < 1 || (int64_t)start_pos[b] + n_steps > m->max_seq)
      return fail(MKD_E_INVALID, "need start_pos >= 0, n_steps >= 1, start_pos + n_steps <= max_seq");
  }
  if (!tokens_out_dev) return fail(MKD_E_INVALID, "null tokens_out_dev");
  if (m->trace && m->trace_cap < (size_t)m->n_wg * n_steps * m->max_instr * kTraceWords)
    return fail(MKD_E_INVALID, "trace buffer too small for this launch");
  if ((int64_t)n_steps * (c->n_layers + 1) >= 0xffffffffll) return fail(MKD_E_INVALID, "n_steps too large");
  hipError_t e = hipSetDevice(m->device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  if (m->launched) {
    // the reset kernel of a new launch would clear the flags and activations
    // a running one still uses (on another stream it would not wait for it)
    const hipError_t q = hipEventQuery(m->done);
    if (q == hipErrorNotReady) return fail(MKD_E_INVALID, "the previous launch is still running: mkd_wait first");
    if (q != hipSuccess) return hip_fail(q, "previous launch");
    m->launched = false;   // finished; its status is superseded by this launch
  }
  // a stop requested while no launch was running must not end this one
  __atomic_store_n(m->h_ctrl, 0, __ATOMIC_SEQ_CST);
  KParams p{};
  p.sched = m->d_sched;
  p.wtab = m->d_wtab;
  p.kv = m->kv;
  p.rope = m->d_rope;
  p.h = m->h; p.qkv = m->qkv; p.part = m->part; p.aout = m->aout;
  p.hmid = m->hmid; p.act = m->act; p.route = m->route; p.lm = m->lm;
  p.flags = (uint32_t*)m->flags;
  p.flag_stride = m->flag_stride;
  p.zero = m->d_zero;
  p.n_stages = m->n_stages;
  p.forced = forced_dev;
  p.tokens_out = tokens_out_dev;
  p.logits_out = logits_out_dev;
  p.status = m->d_status;
  p.stop = m->d_stop;
  p.trace = m->trace;
  p.watchdog_ticks = m->watchdog_ticks;
  p.n_wg = m->n_wg; p.max_instr = m->max_instr; p.n_chunks = m->n_chunks; p.n_lm_tiles = m->n_lm;
  p.n_steps = n_steps; p.max_seq = m->max_seq;
  p.B = m->batch;
  for (int b = 0; b < m->batch; ++b) {
    p.first_tok[b] = first_tokens[b];
    p.start[b] = start_pos[b];
  }
  p.s_qkv = m->s_qkv; p.s_part = m->s_part;
  p.s_kv = (int64_t)c->n_layers * 2 * c->n_kv_heads * m->max_seq * c->head_dim;
  p.L = c->n_layers; p.d = c->d_model; p.hq = c->n_q_heads; p.hkv = c->n_kv_heads; p.hd = c->head_dim;
  p.F = c->d_ff; p.V = c->vocab; p.E = c->n_experts; p.topk = c->top_k;
  p.qd = c->n_q_heads * c->head_dim; p.kvd = c->n_kv_heads * c->head_dim;
  p.G = c->n_q_heads / c->n_kv_heads; p.tied = c->tied; p.lslots = layer_slots(c);
  p.x_floats = m->x_floats;
  p.out_floats = m->out_floats;
  p.res_floats = m->res_floats;
  p.pre_units = m->pre_units;
  p.pre_off = m->pre_off;
  // the prediction's router scoring takes one expert row per wavefront, d <= 4096
  p.predict = m->predict && c->n_experts > 0 && c->n_experts <= kWaves && c->d_model <= 4096;
  p.eps = c->rms_eps;
  const char* why = "";
  const int rc = launch(p, m->ll_words, stream, m->k0, m->k1, !m->plain_launch, &why);
  if (rc) return fail(rc, why);
  m->timed = true;
  if ((e = hipEventRecord(m->done, (hipStream_t)stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  m->launched = true;
  return MKD_OK;
}

int mkd_decode(mkd_model* m, int32_t first_token, int32_t start_pos, int32_t n_steps,
               const int32_t* forced_dev, int32_t* tokens_out_dev, float* logits_out_dev, void* stream) {
  if (!m) return fail(MKD_E_INVALID, "null model");
  if (m->batch != 1) return fail(MKD_E_INVALID, "the model decodes several sequences: use mkd_decode_batch");
  return decode_launch(m, &first_token, &start_pos, n_steps, forced_dev, tokens_out_dev, logits_out_dev, stream);
}

int mkd_decode_batch(mkd_model* m, const int32_t* first_tokens, const int32_t* start_pos, int32_t n_steps,
                     int32_t* tokens_out_dev, float* logits_out_dev, void* stream) {
  if (!m) return fail(MKD_E_INVALID, "null model");
  return decode_launch(m, first_tokens, start_pos, n_steps, nullptr, tokens_out_dev, logits_out_dev, stream);
}

int mkd_wait(mkd_model* m, int32_t timeout_ms, mkd_status* out) {
  if (!m) return fail(MKD_E_INVALID, "null model");
  if (out) *out = mkd_status{MKD_OK, -1, -1, -1};
  if (!m->launched) return MKD_OK;
  hipSetDevice(m->device);
  const auto t0 = std::chrono::steady_clock::now();
  for (;;) {
    const hipError_t q = hipEventQuery(m->done);
    if (q == hipSuccess) break;
    if (q != hipErrorNotReady) return hip_fail(q, "launch failed");
    if (timeout_ms >= 0 &&
        std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(timeout_ms))
      return fail(MKD_E_TIMEOUT, "decode launch still running after the host timeout");
    std::this_thread::sleep_for(std::chrono::microseconds(200));
  }
  int32_t st[S_WORDS];
  hipError_t e = hipMemcpy(st, m->d_status, sizeof(st), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "read status");
  m->launched = false;
  __atomic_store_n(m->h_ctrl, 0, __ATOMIC_SEQ_CST);
  m->spec_hit = st[S_SPEC_HIT];
  m->spec_n = st[S_SPEC_N];
  if (out) *out = mkd_status{st[S_CODE], st[S_WG], st[S_INSTR], st[S_TOKEN]};
  if (st[S_CODE] != MKD_OK) {
    return fail(st[S_CODE], "device reported error " + std::to_string(st[S_CODE]) + " at workgroup " +
                                std::to_string(st[S_WG]) + ", instruction " + std::to_string(st[S_INSTR]) +
                                ", step " + std::to_string(st[S_TOKEN]));
  }
  return MKD_OK;
}

int mkd_abort(mkd_model* m) {
  if (!m) return fail(MKD_E_INVALID, "null model");
  // only a launch that is in flight can be stopped; the next launch clears
  // the word again before it starts
  if (m->launched) __atomic_store_n(m->h_ctrl, 1, __ATOMIC_SEQ_CST);
  return MKD_OK;
}

int mkd_set_lds_limits(mkd_model* m, int32_t max_input_floats, int32_t max_staged_units) {
  if (!m) return fail(MKD_E_INVALID, "null model");
  if (max_input_floats < 0 || max_staged_units < -1) return fail(MKD_E_INVALID, "limits out of range");
  m->x_cap = max_input_floats;
  m->pre_cap = max_staged_units;
  return MKD_OK;
}

}  // extern "C"

namespace mkd {
// csrc/mkd_probe.hip: a plain streaming read of buf (bytes, a multiple of 16) on `stream`
int read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream, const char** why);
}  // namespace mkd

extern "C" {

int mkd_read_probe(const void* buf_dev, size_t bytes, uint32_t* sink_dev, void* stream) {
  if (!buf_dev || !sink_dev) return fail(MKD_E_INVALID, "null buffer or sink");
  if (bytes < 16 || bytes % 16) return fail(MKD_E_INVALID, "bytes must be a positive multiple of 16");
  if ((uintptr_t)buf_dev % 16) return fail(MKD_E_INVALID, "the buffer must be 16-byte aligned");
  const char* why = "";
  const int rc = read_probe(buf_dev, bytes, sink_dev, stream, &why);
  return rc == MKD_OK ? MKD_OK : fail(rc, why);
}

int mkd_set_expert_prediction(mkd_model* m, int32_t on) {
  if (!m) return fail(MKD_E_INVALID, "null model");
  if (on != 0 && on != 1) return fail(MKD_E_INVALID, "on must be 0 or 1");
  m->predict = on != 0;
  return MKD_OK;
}

int mkd_spec_stats(mkd_model* m, int32_t* hits, int32_t* predictions) {
  if (!m || !hits || !predictions) return fail(MKD_E_INVALID, "null argument");
  *hits = m->spec_hit;
  *predictions = m->spec_n;
  return MKD_OK;
}

int mkd_set_launch_mode(mkd_model* m, int32_t cooperative) {
  if (!m) return fail(MKD_E_INVALID, "null model");
  if (cooperative != 0 && cooperative != 1) return fail(MKD_E_INVALID, "cooperative must be 0 or 1");
  m->plain_launch = cooperative == 0;
  return MKD_OK;
}

int mkd_set_watchdog(mkd_model* m, int32_t watchdog_ms) {
  if (!m) return fail(MKD_E_INVALID, "null model");
  if (watchdog_ms < 1) return fail(MKD_E_INVALID, "watchdog_ms must be >= 1");
  m->watchdog_ticks = (uint64_t)((double)watchdog_ms * 1e-3 * m->clock_hz);
  return MKD_OK;
}

int mkd_set_trace(mkd_model* m, uint64_t* trace_dev, size_t capacity_words) {
  if (!m) return fail(MKD_E_INVALID, "null model");
  m->trace = trace_dev;
  m->trace_cap = trace_dev ? capacity_words : 0;
  return MKD_OK;
}

int mkd_kernel_ms(mkd_model* m, float* ms) {
  if (!m || !ms) return fail(MKD_E_INVALID, "null argument");
  if (!m->timed) return fail(MKD_E_INVALID, "no launch has been timed");
  hipSetDevice(m->device);
  const hipError_t e = hipEventElapsedTime(ms, m->k0, m->k1);
  if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
  return MKD_OK;
}

int mkd_clock_hz(mkd_model* m, double* hz) {
  if (!m || !hz) return fail(MKD_E_INVALID, "null argument");
  *hz = m->clock_hz;
  return MKD_OK;
}

void mkd_destroy(mkd_model* m) {
  if (!m) return;
  hipSetDevice(m->device);
  if (m->launched && m->done) hipEventSynchronize(m->done);
  if (m->static_ws) {
    std::lock_guard<std::mutex> lock(g_static_mu);
    if (g_static_owner[m->device] == m) g_static_owner[m->device] = nullptr;
  }
  if (m->done) hipEventDestroy(m->done);
  if (m->k0) hipEventDestroy(m->k0);
  if (m->k1) hipEventDestroy(m->k1);
  delete m;
}

}  // extern "C"
