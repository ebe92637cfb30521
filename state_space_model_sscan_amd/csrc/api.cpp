// api.cpp -- the C ABI of libsscan: argument validation and kernel dispatch.
// Every check runs before anything is launched; see include/sscan.h.
#include "sscan.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "launch.hpp"
#include "mixer_ops.hpp"

namespace {

thread_local std::string g_last_error;
std::atomic<int> g_pointer_checks{1};
std::atomic<int64_t> g_knobs[sscan::kKnobCount];  // zero-initialised: every knob at the library's choice

sscan_status fail(sscan_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sscan_status ok() {
  g_last_error.clear();
  return SSCAN_OK;
}

constexpr int64_t kMaxDim = int64_t(1) << 31;

struct Buf {
  const char* name;
  const void* p;
  size_t bytes;
  bool out;
};

bool is_device_ptr(const void* p) {
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // do not leave the error for the caller's next HIP call
    return false;
  }
  return attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged;
}

bool overlap(const Buf& a, const Buf& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes, b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
  return a0 < b1 && b0 < a1;
}

// Null, alignment, alias and device checks over a list of buffers. `required`
// buffers must be non-null when they have bytes. inplace_out / inplace_in name one
// output/input pair that may be the same buffer (exactly, not partially).
sscan_status check_buffers(const Buf* bufs, int n, const bool* required, const void* inplace_out,
                           const void* inplace_in) {
  for (int i = 0; i < n; ++i) {
    if (bufs[i].bytes == 0) continue;
    if (!bufs[i].p) {
      if (required[i]) return fail(SSCAN_ERR_NULL, "%s is NULL", bufs[i].name);
      continue;
    }
    if ((uintptr_t)bufs[i].p % 16 != 0)
      return fail(SSCAN_ERR_ALIGN, "%s (%p) is not 16-byte aligned", bufs[i].name, bufs[i].p);
  }
  for (int i = 0; i < n; ++i) {
    if (!bufs[i].out) continue;
    for (int j = 0; j < n; ++j) {
      if (i == j || !overlap(bufs[i], bufs[j])) continue;
      if (bufs[j].out && j < i) continue;  // reported once per pair
      // in place means the very same buffer: identical base pointer and size
      const bool allowed = inplace_out && inplace_out == inplace_in && bufs[i].p == inplace_out &&
                           bufs[j].p == inplace_in && bufs[i].bytes == bufs[j].bytes;
      if (!allowed) return fail(SSCAN_ERR_ALIAS, "%s overlaps %s", bufs[i].name, bufs[j].name);
    }
  }
  if (g_pointer_checks.load(std::memory_order_relaxed)) {
    for (int i = 0; i < n; ++i) {
      if (!bufs[i].p || bufs[i].bytes == 0) continue;
      if (!is_device_ptr(bufs[i].p))
        return fail(SSCAN_ERR_NOT_DEVICE, "%s (%p) is not device memory", bufs[i].name, bufs[i].p);
    }
  }
  return SSCAN_OK;
}

sscan_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SSCAN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

sscan_status check_mamba1_desc(const sscan_mamba1_desc* d, bool step) {
  if (!d) return fail(SSCAN_ERR_NULL, "descriptor is NULL");
  if (d->batch < 0 || d->seqlen < 0 || d->channels <= 0 || d->state_dim <= 0 || d->ngroups <= 0)
    return fail(SSCAN_ERR_SHAPE, "need batch >= 0, seqlen >= 0, channels, state_dim, ngroups > 0");
  if (d->batch >= kMaxDim || d->seqlen >= kMaxDim || d->channels >= kMaxDim)
    return fail(SSCAN_ERR_SHAPE, "a size exceeds 2^31");
  if (d->channels % d->ngroups != 0) return fail(SSCAN_ERR_SHAPE, "ngroups must divide channels");
  if (step && d->seqlen != 1) return fail(SSCAN_ERR_SHAPE, "sscan_step needs seqlen == 1");
  if (d->act != SSCAN_F32 && d->act != SSCAN_BF16) return fail(SSCAN_ERR_DTYPE, "act must be F32 or BF16");
  if (d->state_dim > 256) return fail(SSCAN_ERR_UNSUPPORTED, "Mamba-1 state_dim must be <= 256");
  if (d->ngroups > 1 && (d->channels / d->ngroups) % 64 != 0)
    return fail(SSCAN_ERR_UNSUPPORTED, "with ngroups > 1, channels / ngroups must be a multiple of 64");
  if (d->batch > 65535) return fail(SSCAN_ERR_UNSUPPORTED, "batch must be <= 65535");
  return SSCAN_OK;
}

// map_only: the descriptor of sscan_ssd_attention, which does not read head_dim
sscan_status check_ssd_desc(const sscan_ssd_desc* d, bool step, bool map_only = false) {
  if (!d) return fail(SSCAN_ERR_NULL, "descriptor is NULL");
  if (d->batch < 0 || d->seqlen < 0 || d->nheads <= 0 || d->head_dim <= 0 || d->state_dim <= 0 ||
      d->ngroups <= 0)
    return fail(SSCAN_ERR_SHAPE, "need batch >= 0, seqlen >= 0, nheads, head_dim, state_dim, ngroups > 0");
  if (d->batch >= kMaxDim || d->seqlen >= kMaxDim || d->nheads * d->head_dim >= kMaxDim)
    return fail(SSCAN_ERR_SHAPE, "a size exceeds 2^31");
  if (d->nheads % d->ngroups != 0) return fail(SSCAN_ERR_SHAPE, "ngroups must divide nheads");
  if (d->chunk != 0 && (d->chunk < 16 || d->chunk > 256 || (d->chunk & (d->chunk - 1)) != 0))
    return fail(SSCAN_ERR_SHAPE, "chunk must be 0 or a power of two in 16..256");
  if (d->reserved != 0) return fail(SSCAN_ERR_SHAPE, "reserved must be 0");
  if (step && d->seqlen != 1) return fail(SSCAN_ERR_SHAPE, "sscan_ssd_step needs seqlen == 1");
  if (d->act != SSCAN_F32 && d->act != SSCAN_BF16) return fail(SSCAN_ERR_DTYPE, "act must be F32 or BF16");
  if (d->state_dim > 128) return fail(SSCAN_ERR_UNSUPPORTED, "SSD state_dim must be <= 128");
  if (!map_only && d->ngroups > 1 && ((d->nheads / d->ngroups) * d->head_dim) % 64 != 0)
    return fail(SSCAN_ERR_UNSUPPORTED,
                "with ngroups > 1, (nheads / ngroups) * head_dim must be a multiple of 64");
  if (d->batch > 65535) return fail(SSCAN_ERR_UNSUPPORTED, "batch must be <= 65535");
  return SSCAN_OK;
}

sscan::SSDArgs ssd_args(const sscan_ssd_desc* d) {
  sscan::SSDArgs a{};
  a.batch = d->batch; a.L = d->seqlen; a.H = d->nheads; a.P = d->head_dim; a.N = d->state_dim;
  a.G = d->ngroups; a.chunk = d->chunk; a.bf16 = d->act == SSCAN_BF16;
  return a;
}

}  // namespace

int64_t sscan::knob(int which) {
  return which > 0 && which < kKnobCount ? g_knobs[which].load(std::memory_order_relaxed) : 0;
}

extern "C" {

int sscan_abi_version(void) { return SSCAN_ABI_VERSION; }

int sscan_set_pointer_checks(int enabled) { return g_pointer_checks.exchange(enabled ? 1 : 0); }

int64_t sscan_set_tuning(int knob, int64_t value) {
  if (knob <= 0 || knob >= sscan::kKnobCount || value < 0) return -1;
  return g_knobs[knob].exchange(value);
}

const char* sscan_last_error(void) { return g_last_error.c_str(); }

const char* sscan_status_string(int st) {
  switch (st) {
    case SSCAN_OK: return "ok";
    case SSCAN_ERR_NULL: return "null pointer";
    case SSCAN_ERR_SHAPE: return "invalid shape";
    case SSCAN_ERR_DTYPE: return "invalid dtype";
    case SSCAN_ERR_UNSUPPORTED: return "unsupported variant";
    case SSCAN_ERR_NOT_DEVICE: return "not device memory";
    case SSCAN_ERR_ALIGN: return "misaligned pointer";
    case SSCAN_ERR_ALIAS: return "output overlaps input";
    case SSCAN_ERR_WORKSPACE: return "workspace missing or too small";
    case SSCAN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t sscan_mamba1_workspace_size(const sscan_mamba1_desc* d) {
  if (check_mamba1_desc(d, false) != SSCAN_OK) return 0;
  return sscan::mamba1_plan(d->batch, d->seqlen, d->channels, d->state_dim, d->ngroups,
                            d->act == SSCAN_BF16 ? 2 : 4)
      .ws_bytes;
}

sscan_status sscan_mamba1_fwd(const sscan_mamba1_desc* d, const void* x, const void* dt_raw,
                              const float* dt_bias, const float* A_log, const void* B, const void* C,
                              const float* D, const void* z, const float* state_input, void* y,
                              float* state_output, float* states, void* workspace, size_t workspace_bytes,
                              void* stream) {
  sscan_status st = check_mamba1_desc(d, false);
  if (st != SSCAN_OK) return st;
  const int64_t b = d->batch, L = d->seqlen, Dc = d->channels, N = d->state_dim, G = d->ngroups;
  const size_t es = d->act == SSCAN_BF16 ? 2 : 4;
  const sscan::Mamba1Plan plan = sscan::mamba1_plan(b, L, Dc, N, G, (int64_t)es);
  const size_t act_bytes = (size_t)(b * L * Dc) * es, bc_bytes = (size_t)(b * L * G * N) * es;
  const size_t st_bytes = (size_t)(b * Dc * N) * 4;
  const Buf bufs[] = {
      {"x", x, act_bytes, false},
      {"dt_raw", dt_raw, act_bytes, false},
      {"dt_bias", dt_bias, (size_t)Dc * 4, false},
      {"A_log", A_log, (size_t)(Dc * N) * 4, false},
      {"B", B, bc_bytes, false},
      {"C", C, bc_bytes, false},
      {"D", D, (size_t)Dc * 4, false},
      {"z", z, act_bytes, false},
      {"state_input", state_input, st_bytes, false},
      {"y", y, act_bytes, true},
      {"state_output", state_output, st_bytes, true},
      {"states", states, (size_t)(b * L * Dc * N) * 4, true},
      {"workspace", workspace, plan.ws_bytes, true},
  };
  const bool req[] = {true, true, true, true, true, true, true, false, false, true, true, false, true};
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return fail(SSCAN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", plan.ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  st = check_buffers(bufs, 13, req, nullptr, nullptr);
  if (st != SSCAN_OK) return st;
  sscan::Mamba1Args a{};
  a.batch = b; a.L = L; a.Dc = Dc; a.N = N; a.G = G; a.bf16 = d->act == SSCAN_BF16;
  a.bc_eps = d->bc_rms_eps > 0.0f ? d->bc_rms_eps : 0.0f;
  a.x = x; a.dt = dt_raw; a.dt_bias = dt_bias; a.A_log = A_log; a.B = B; a.C = C; a.D = D; a.z = z;
  a.h0 = state_input; a.y = y; a.h_out = state_output; a.states = states;
  return hip_status(sscan::launch_mamba1_fwd(a, plan, workspace, (hipStream_t)stream), "sscan_mamba1_fwd launch");
}

sscan_status sscan_step(const sscan_mamba1_desc* d, const float* state_input, float* state_output,
                        const void* x, const void* dt_raw, const float* dt_bias, const float* A_log,
                        const void* B, const void* C, const float* D, const void* z, void* y, void* stream) {
  sscan_status st = check_mamba1_desc(d, true);
  if (st != SSCAN_OK) return st;
  const int64_t b = d->batch, Dc = d->channels, N = d->state_dim, G = d->ngroups;
  const size_t es = d->act == SSCAN_BF16 ? 2 : 4;
  const size_t act_bytes = (size_t)(b * Dc) * es, st_bytes = (size_t)(b * Dc * N) * 4;
  const Buf bufs[] = {
      {"x", x, act_bytes, false},
      {"dt_raw", dt_raw, act_bytes, false},
      {"dt_bias", dt_bias, (size_t)Dc * 4, false},
      {"A_log", A_log, (size_t)(Dc * N) * 4, false},
      {"B", B, (size_t)(b * G * N) * es, false},
      {"C", C, (size_t)(b * G * N) * es, false},
      {"D", D, (size_t)Dc * 4, false},
      {"z", z, act_bytes, false},
      {"state_input", state_input, st_bytes, false},
      {"y", y, act_bytes, true},
      {"state_output", state_output, st_bytes, true},
  };
  const bool req[] = {true, true, true, true, true, true, true, false, true, true, true};
  st = check_buffers(bufs, 11, req, state_output, state_input);
  if (st != SSCAN_OK) return st;
  sscan::Mamba1Args a{};
  a.batch = b; a.L = 1; a.Dc = Dc; a.N = N; a.G = G; a.bf16 = d->act == SSCAN_BF16;
  a.bc_eps = d->bc_rms_eps > 0.0f ? d->bc_rms_eps : 0.0f;
  a.x = x; a.dt = dt_raw; a.dt_bias = dt_bias; a.A_log = A_log; a.B = B; a.C = C; a.D = D; a.z = z;
  a.h0 = state_input; a.y = y; a.h_out = state_output; a.states = nullptr;
  return hip_status(sscan::launch_mamba1_step(a, (hipStream_t)stream), "sscan_step launch");
}

size_t sscan_ssd_workspace_size(const sscan_ssd_desc* d) {
  if (check_ssd_desc(d, false) != SSCAN_OK) return 0;
  const sscan::SSDArgs a = ssd_args(d);
  size_t w = sscan::ssd_tokenloop_ws(a);
  if (sscan::ssd_chunk_supported(a)) {
    const size_t wc = sscan::ssd_chunk_ws(a);
    if (wc > w) w = wc;
  }
  return w;
}

}  // extern "C"

namespace {

// sscan_ssd_fwd and sscan_ssd_fwd_noalloc: noalloc takes the library's static
// device scratch instead of a caller's workspace.
sscan_status ssd_fwd(const sscan_ssd_desc* d, const void* x, const void* dt_raw, const float* dt_bias,
                     const float* A_log, const void* B, const void* C, const float* D, const void* z,
                     const float* state_input, void* y, float* state_output, float* states, void* workspace,
                     size_t workspace_bytes, void* stream, bool noalloc, const char* what) {
  sscan_status st = check_ssd_desc(d, false);
  if (st != SSCAN_OK) return st;
  sscan::SSDArgs a = ssd_args(d);
  if (noalloc) a.ws_cap = sscan::kScratchBytes;  // the plan fits the static scratch where it can
  const int64_t b = a.batch, L = a.L, H = a.H, P = a.P, N = a.N, G = a.G;
  const size_t es = a.bf16 ? 2 : 4;
  const size_t act_bytes = (size_t)(b * L * H * P) * es, bc_bytes = (size_t)(b * L * G * N) * es;
  const size_t st_bytes = (size_t)(b * H * P * N) * 4;
  const bool chunk = states == nullptr && sscan::ssd_chunk_supported(a);
  const size_t need = chunk ? sscan::ssd_chunk_ws(a) : sscan::ssd_tokenloop_ws(a);
  const Buf bufs[] = {
      {"x", x, act_bytes, false},
      {"dt_raw", dt_raw, (size_t)(b * L * H) * es, false},
      {"dt_bias", dt_bias, (size_t)H * 4, false},
      {"A_log", A_log, (size_t)H * 4, false},
      {"B", B, bc_bytes, false},
      {"C", C, bc_bytes, false},
      {"D", D, (size_t)H * 4, false},
      {"z", z, act_bytes, false},
      {"state_input", state_input, st_bytes, false},
      {"y", y, act_bytes, true},
      {"state_output", state_output, st_bytes, true},
      {"states", states, (size_t)(b * L * H * P * N) * 4, true},
      {"workspace", workspace, noalloc ? 0 : need, true},
  };
  const bool req[] = {true, true, true, true, true, true, true, false, false, true, true, false, true};
  if (noalloc) {
    if (need > sscan::kScratchBytes)
      return fail(SSCAN_ERR_UNSUPPORTED, "this problem needs %zu bytes of scratch; the static scratch holds %zu",
                  need, sscan::kScratchBytes);
  } else if (need > 0 && (!workspace || workspace_bytes < need)) {
    return fail(SSCAN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  }
  st = check_buffers(bufs, 13, req, nullptr, nullptr);
  if (st != SSCAN_OK) return st;
  if (noalloc && need > 0) {
    const hipError_t e = sscan::scratch_ptr(&workspace);
    if (e != hipSuccess) return hip_status(e, "the static scratch's device address");
  }
  a.x = x; a.dt = dt_raw; a.dt_bias = dt_bias; a.A_log = A_log; a.B = B; a.C = C; a.D = D; a.z = z;
  a.h0 = state_input; a.y = y; a.h_out = state_output; a.states = states;
  const hipError_t e = chunk ? sscan::launch_ssd_chunk(a, workspace, (hipStream_t)stream)
                             : sscan::launch_ssd_tokenloop(a, workspace, (hipStream_t)stream);
  return hip_status(e, what);
}

}  // namespace

extern "C" {

sscan_status sscan_ssd_fwd(const sscan_ssd_desc* d, const void* x, const void* dt_raw, const float* dt_bias,
                           const float* A_log, const void* B, const void* C, const float* D, const void* z,
                           const float* state_input, void* y, float* state_output, float* states,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return ssd_fwd(d, x, dt_raw, dt_bias, A_log, B, C, D, z, state_input, y, state_output, states, workspace,
                 workspace_bytes, stream, false, "sscan_ssd_fwd launch");
}

sscan_status sscan_ssd_fwd_noalloc(const sscan_ssd_desc* d, const void* x, const void* dt_raw, const float* dt_bias,
                                   const float* A_log, const void* B, const void* C, const float* D, const void* z,
                                   const float* state_input, void* y, float* state_output, float* states,
                                   void* stream) {
  return ssd_fwd(d, x, dt_raw, dt_bias, A_log, B, C, D, z, state_input, y, state_output, states, nullptr, 0, stream,
                 true, "sscan_ssd_fwd_noalloc launch");
}

sscan_status sscan_ssd_step(const sscan_ssd_desc* d, const float* state_input, float* state_output, const void* x,
                            const void* dt_raw, const float* dt_bias, const float* A_log, const void* B,
                            const void* C, const float* D, const void* z, void* y, void* stream) {
  sscan_status st = check_ssd_desc(d, true);
  if (st != SSCAN_OK) return st;
  sscan::SSDArgs a = ssd_args(d);
  const int64_t b = a.batch, H = a.H, P = a.P, N = a.N, G = a.G;
  const size_t es = a.bf16 ? 2 : 4;
  const size_t act_bytes = (size_t)(b * H * P) * es, st_bytes = (size_t)(b * H * P * N) * 4;
  const Buf bufs[] = {
      {"x", x, act_bytes, false},
      {"dt_raw", dt_raw, (size_t)(b * H) * es, false},
      {"dt_bias", dt_bias, (size_t)H * 4, false},
      {"A_log", A_log, (size_t)H * 4, false},
      {"B", B, (size_t)(b * G * N) * es, false},
      {"C", C, (size_t)(b * G * N) * es, false},
      {"D", D, (size_t)H * 4, false},
      {"z", z, act_bytes, false},
      {"state_input", state_input, st_bytes, false},
      {"y", y, act_bytes, true},
      {"state_output", state_output, st_bytes, true},
  };
  const bool req[] = {true, true, true, true, true, true, true, false, true, true, true};
  st = check_buffers(bufs, 11, req, state_output, state_input);
  if (st != SSCAN_OK) return st;
  a.x = x; a.dt = dt_raw; a.dt_bias = dt_bias; a.A_log = A_log; a.B = B; a.C = C; a.D = D; a.z = z;
  a.h0 = state_input; a.y = y; a.h_out = state_output; a.states = nullptr;
  return hip_status(sscan::launch_ssd_step(a, (hipStream_t)stream), "sscan_ssd_step launch");
}

static sscan::AttnArgs attn_args(const sscan_ssd_desc* d) {
  sscan::AttnArgs a{};
  a.batch = d->batch; a.L = d->seqlen; a.H = d->nheads; a.N = d->state_dim; a.G = d->ngroups;
  a.bf16 = d->act == SSCAN_BF16;
  return a;
}

size_t sscan_ssd_attention_workspace_size(const sscan_ssd_desc* d) {
  if (check_ssd_desc(d, false, true) != SSCAN_OK) return 0;
  return sscan::ssd_attention_ws(attn_args(d));
}

sscan_status sscan_ssd_attention(const sscan_ssd_desc* d, const void* dt_raw, const float* dt_bias,
                                 const float* A_log, const void* B, const void* C, float* alpha, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  sscan_status st = check_ssd_desc(d, false, true);
  if (st != SSCAN_OK) return st;
  const int64_t b = d->batch, L = d->seqlen, H = d->nheads, N = d->state_dim, G = d->ngroups;
  const size_t es = d->act == SSCAN_BF16 ? 2 : 4;
  // the map's size must fit a size_t and the kernel's 64-bit indexing
  const double map_elems = (double)b * (double)L * (double)L * (double)H;
  if (map_elems * 4.0 > 9.0e18) return fail(SSCAN_ERR_SHAPE, "the attention map exceeds 2^63 bytes");
  sscan::AttnArgs a = attn_args(d);
  if (!sscan::ssd_attention_supported(a))
    return fail(SSCAN_ERR_UNSUPPORTED, "the map needs fewer than 2^31 tiles of 32 x 32 tokens x 128 heads");
  const size_t need = sscan::ssd_attention_ws(a);
  const Buf bufs[] = {
      {"dt_raw", dt_raw, (size_t)(b * L * H) * es, false},
      {"dt_bias", dt_bias, (size_t)H * 4, false},
      {"A_log", A_log, (size_t)H * 4, false},
      {"B", B, (size_t)(b * L * G * N) * es, false},
      {"C", C, (size_t)(b * L * G * N) * es, false},
      {"alpha", alpha, (size_t)b * (size_t)L * (size_t)L * (size_t)H * 4, true},
      {"workspace", workspace, need, true},
  };
  const bool req[] = {true, true, true, true, true, true, true};
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(SSCAN_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  st = check_buffers(bufs, 7, req, nullptr, nullptr);
  if (st != SSCAN_OK) return st;
  a.dt = dt_raw; a.dt_bias = dt_bias; a.A_log = A_log; a.B = B; a.C = C; a.alpha = alpha;
  a.ws_P = (double*)workspace;
  a.ws_beta = (float*)(a.ws_P + b * L * H);
  return hip_status(sscan::launch_ssd_attention(a, (hipStream_t)stream), "sscan_ssd_attention launch");
}

sscan_status sscan_conv1d_silu(const sscan_conv_desc* d, const void* x, const float* weight, const float* bias,
                               const float* conv_state_in, void* out, float* conv_state_out, void* stream) {
  if (!d) return fail(SSCAN_ERR_NULL, "descriptor is NULL");
  if (d->batch < 0 || d->seqlen < 0 || d->channels <= 0 || d->width <= 0)
    return fail(SSCAN_ERR_SHAPE, "need batch >= 0, seqlen >= 0, channels > 0, width > 0");
  if (d->batch >= kMaxDim || d->seqlen >= kMaxDim || d->channels >= kMaxDim)
    return fail(SSCAN_ERR_SHAPE, "a size exceeds 2^31");
  if (d->reserved != 0) return fail(SSCAN_ERR_SHAPE, "reserved must be 0");
  if (d->act != SSCAN_F32 && d->act != SSCAN_BF16) return fail(SSCAN_ERR_DTYPE, "act must be F32 or BF16");
  if (d->width > 8) return fail(SSCAN_ERR_UNSUPPORTED, "width must be <= 8");
  if (d->batch > 65535) return fail(SSCAN_ERR_UNSUPPORTED, "batch must be <= 65535");
  const int64_t b = d->batch, L = d->seqlen, Dc = d->channels, W = d->width;
  const size_t es = d->act == SSCAN_BF16 ? 2 : 4;
  const size_t act_bytes = (size_t)(b * L * Dc) * es, st_bytes = (size_t)(b * Dc * (W - 1)) * 4;
  const Buf bufs[] = {
      {"x", x, act_bytes, false},
      {"weight", weight, (size_t)(Dc * W) * 4, false},
      {"bias", bias, (size_t)Dc * 4, false},
      {"conv_state_in", conv_state_in, st_bytes, false},
      {"out", out, act_bytes, true},
      {"conv_state_out", conv_state_out, st_bytes, true},
  };
  const bool req[] = {true, true, false, false, true, false};
  sscan_status st = check_buffers(bufs, 6, req, nullptr, nullptr);
  if (st != SSCAN_OK) return st;
  sscan::ConvArgs a{};
  a.batch = b; a.L = L; a.Dc = Dc; a.W = W; a.bf16 = d->act == SSCAN_BF16;
  a.x = x; a.weight = weight; a.bias = bias; a.state_in = conv_state_in; a.out = out; a.state_out = conv_state_out;
  return hip_status(sscan::launch_conv1d_silu(a, (hipStream_t)stream), "sscan_conv1d_silu launch");
}

sscan_status sscan_gated_rmsnorm(int64_t rows, int64_t width, int32_t act, const void* y, const void* z,
                                 const float* weight, float eps, void* out, void* stream) {
  if (rows < 0 || width <= 0) return fail(SSCAN_ERR_SHAPE, "need rows >= 0 and width > 0");
  if (rows >= kMaxDim || width >= kMaxDim) return fail(SSCAN_ERR_SHAPE, "a size exceeds 2^31");
  if (!(eps > 0.0f)) return fail(SSCAN_ERR_SHAPE, "eps must be > 0");
  if (act != SSCAN_F32 && act != SSCAN_BF16) return fail(SSCAN_ERR_DTYPE, "act must be F32 or BF16");
  const size_t es = act == SSCAN_BF16 ? 2 : 4;
  const size_t bytes = (size_t)(rows * width) * es;
  const Buf bufs[] = {
      {"y", y, bytes, false},
      {"z", z, bytes, false},
      {"weight", weight, (size_t)width * 4, false},
      {"out", out, bytes, true},
  };
  const bool req[] = {true, true, true, true};
  sscan_status st = check_buffers(bufs, 4, req, nullptr, nullptr);
  if (st != SSCAN_OK) return st;
  sscan::NormArgs a{};
  a.rows = rows; a.width = width; a.bf16 = act == SSCAN_BF16; a.eps = eps;
  a.y = y; a.z = z; a.weight = weight; a.out = out;
  return hip_status(sscan::launch_gated_rmsnorm(a, (hipStream_t)stream), "sscan_gated_rmsnorm launch");
}

}  // extern "C"
